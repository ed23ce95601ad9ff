"""Host-side checks of the meta-cache's stream/event protocol (no GPU).

A fake backend simulates two in-order streams with random operation durations:
every op starts when its stream is free and all events it waits on have fired.
Buffers carry (layer, version) tags; the test replays the trajectory call
pattern and checks that every reuse reads the entry of the right layer from its
latest anchor, and that no copy or kernel overlaps a conflicting access."""
import random

import pytest

from sparse_attention_diffusion_amd import MCS_COPY_D2H, MCS_COPY_H2D
from sparse_attention_diffusion_amd.cache import MetaCache
from sparse_attention_diffusion_amd.trajectory import step_kind


class Buf:
    def __init__(self, name):
        self.name = name
        self.writes = [(0.0, None)]   # (time, tag)
        self.accesses = []            # (t0, t1, kind)

    def value_at(self, t):
        return max((w for w in self.writes if w[0] <= t), key=lambda w: w[0])[1]

    def access(self, t0, t1, kind):
        for a0, a1, k in self.accesses:
            if (kind == "w" or k == "w") and a0 < t1 and t0 < a1:
                raise AssertionError(f"{self.name}: {kind} [{t0:.2f},{t1:.2f}) overlaps {k} [{a0:.2f},{a1:.2f})")
        self.accesses.append((t0, t1, kind))

    def numel(self):
        return 1

    def element_size(self):
        return 1


class Stream:
    def __init__(self, name):
        self.name = name
        self.t = 0.0


class Event:
    def __init__(self):
        self.time = None


class LazyFuture:
    def __init__(self, ex, fn):
        self.ex, self.fn, self.done, self.value = ex, fn, False, None

    def result(self):
        self.ex.run_until(self)
        return self.value


class LazyExecutor:
    """One worker, submission order, but a job runs only when some thread needs its
    result (or a later job's): the compute thread must never use an event before
    the job that records it has run."""

    def __init__(self):
        self.queue = []

    def submit(self, fn):
        f = LazyFuture(self, fn)
        self.queue.append(f)
        return f

    def run_until(self, f):
        while not f.done:
            g = self.queue.pop(0)
            g.value = g.fn()
            g.done = True


class HostChunk:
    def __init__(self, name, size):
        self.name, self.size, self.views = name, size, []


class FakeBackend:
    def __init__(self, seed, pinned_ok=True):
        self.rng = random.Random(seed)
        self.compute = Stream("compute")
        self.side = Stream("side")
        self.n = 0
        self.ex = LazyExecutor()
        self.chunks = []
        self.pageable = []
        self.pinned_ok = pinned_ok

    def submit(self, fn):
        return self.ex.submit(fn)

    def nbytes(self, shape, dtype):
        return 1000  # every tensor of an entry: 1,000 bytes

    def empty_pageable(self, shape, dtype):
        self.n += 1
        b = Buf(f"host{self.n}")
        self.pageable.append(b)
        return b

    def empty_pinned_bytes(self, nbytes):
        assert self.pinned_ok, "pinned memory requested with a zero budget"
        assert nbytes & (nbytes - 1) == 0, "pinned chunks must be powers of two"
        self.n += 1
        c = HostChunk(f"chunk{self.n}", nbytes)
        self.chunks.append(c)
        return c

    def host_size(self, buf):
        return buf.size

    def host_view(self, buf, offset, nbytes):
        if isinstance(buf, HostChunk):
            assert 0 <= offset and offset + nbytes <= buf.size
            assert all(offset + nbytes <= o or o + n <= offset for o, n, _ in buf.views), "overlapping views"
            v = Buf(f"{buf.name}[{offset}:{offset + nbytes}]")
            buf.views.append((offset, nbytes, v))
            return v
        return Buf(f"{buf.name}.{offset}")  # sub-view of a view: the entry's tensors

    def typed(self, raw, shape, dtype):
        return raw

    def compute_stream(self):
        return self.compute

    def event(self):
        return Event()

    def record(self, ev, stream):
        ev.time = stream.t

    def wait(self, stream, ev):
        assert ev.time is not None, "waiting on an event that was never recorded"
        stream.t = max(stream.t, ev.time)

    def copy(self, dst, src, kind, stream):
        dur = self.rng.uniform(0.5, 4.0)
        t0, t1 = stream.t, stream.t + dur
        src.access(t0, t1, "r")
        dst.access(t0, t1, "w")
        dst.writes.append((t1, src.value_at(t0)))
        stream.t = t1

    def kernel(self, reads=(), writes=(), tag=None):
        dur = self.rng.uniform(0.5, 3.0)
        t0, t1 = self.compute.t, self.compute.t + dur
        vals = [b.value_at(t0) for b in reads]
        for b in reads:
            b.access(t0, t1, "r")
        for b in writes:
            b.access(t0, t1, "w")
            b.writes.append((t1, tag))
        self.compute.t = t1
        return vals

    def empty_device(self, shape, dtype):
        self.n += 1
        return Buf(f"dev{self.n}")

    def empty_host(self, shape, dtype):
        self.n += 1
        return Buf(f"host{self.n}")


SHAPES = {"perm": ((1,), None), "idx": ((1,), None), "resid": ((1,), None)}


def replay(cache, be, layers, steps, warmup=2, interval=3):
    version = {}
    for step in range(steps):
        kind = step_kind(step, warmup, interval)
        for layer in range(layers):
            if kind == "anchor":
                buf = cache.anchor_buffers(layer, busy_layer=layer - 1)
                version[layer] = (layer, step)
                be.kernel(writes=list(buf.values()), tag=version[layer])
                cache.commit_anchor(layer)
                cache.release(layer)
            elif kind == "reuse":
                buf = cache.get(layer)
                vals = be.kernel(reads=list(buf.values()))
                assert vals == [version[layer]] * 3, (step, layer, vals, version[layer])
                cache.release(layer)
            nxt_step, nxt_layer = (step, layer + 1) if layer + 1 < layers else (step + 1, 0)
            if nxt_step < steps and step_kind(nxt_step, warmup, interval) == "reuse":
                cache.prefetch(nxt_layer, busy_layer=layer)
    cache.drain()  # run the side-stream jobs nobody waited for (their copies are checked too)


@pytest.mark.parametrize("seed", range(20))
@pytest.mark.parametrize("layers,slots", [(1, 1), (2, 2), (5, 2), (6, 3)])
def test_offload_protocol_orders_every_access(seed, layers, slots):
    be = FakeBackend(seed)
    cache = MetaCache(layers, SHAPES, be, offload=True, device_slots=slots)
    replay(cache, be, layers, steps=12)
    assert cache.bytes_d2h > 0 and (layers <= slots or cache.bytes_h2d > 0)


def test_resident_mode_needs_no_copies():
    be = FakeBackend(0)
    cache = MetaCache(4, SHAPES, be, offload=False)
    replay(cache, be, 4, steps=10)
    assert cache.bytes_d2h == 0 and cache.bytes_h2d == 0


def test_reuse_before_any_anchor_is_an_error():
    be = FakeBackend(0)
    cache = MetaCache(2, SHAPES, be, offload=True)
    with pytest.raises(RuntimeError):
        cache.get(0)
    with pytest.raises(RuntimeError):
        cache.prefetch(1)


def test_a_dropped_wait_is_detected():
    # Plant a mistake in the protocol (the reuse no longer waits for the prefetch)
    # and check that the simulation catches the race.
    be = FakeBackend(3)
    cache = MetaCache(4, SHAPES, be, offload=True, device_slots=2)
    real_wait = be.wait

    def lazy_wait(stream, ev):
        if stream is be.compute:
            return  # compute stream ignores every event
        real_wait(stream, ev)

    be.wait = lazy_wait
    with pytest.raises(AssertionError):
        replay(cache, be, 4, steps=12)


def test_copy_kinds():
    be = FakeBackend(1)
    kinds = []
    orig = be.copy
    be.copy = lambda d, s, k, st: (kinds.append(k), orig(d, s, k, st))
    cache = MetaCache(3, SHAPES, be, offload=True, device_slots=2)
    replay(cache, be, 3, steps=8)
    assert set(kinds) == {MCS_COPY_D2H, MCS_COPY_H2D}


@pytest.mark.parametrize("seed", range(12))
@pytest.mark.parametrize("layers,resident,slots", [(5, 2, 2), (6, 3, 2), (4, 3, 2), (4, 4, 2), (7, 1, 3)])
def test_mixed_residency_orders_every_access_and_copies_only_offloaded_layers(seed, layers, resident, slots):
    be = FakeBackend(seed)
    copied = []
    orig = be.copy

    def copy(d, s, k, st):
        copied.append((d.name, s.name, k))
        orig(d, s, k, st)

    be.copy = copy
    cache = MetaCache(layers, SHAPES, be, offload=True, device_slots=slots, resident_layers=resident)
    assert cache.resident == frozenset(range(resident))
    host_names = {b.name for e in cache.entries for b in e.host.values()}
    assert all(not cache.entries[l].host for l in range(resident))
    steps, warmup, interval = 12, 2, 3
    replay(cache, be, layers, steps=steps, warmup=warmup, interval=interval)
    anchors = sum(1 for s in range(steps) if step_kind(s, warmup, interval) == "anchor")
    offloaded = layers - resident
    # every device -> host copy is of an offloaded layer, once per anchor and tensor
    assert cache.bytes_d2h == anchors * offloaded * len(SHAPES) * 1000
    assert all((k == MCS_COPY_D2H) == (d in host_names) for d, _, k in copied)
    if offloaded == 0:
        assert copied == []


def test_resident_layers_bounds():
    be = FakeBackend(0)
    with pytest.raises(ValueError):
        MetaCache(3, SHAPES, be, offload=True, resident_layers=-1)
    cache = MetaCache(3, SHAPES, be, offload=True, resident_layers=10)
    assert cache.resident == frozenset(range(3)) and cache.slots == []


def test_entry_bytes_of_the_trajectory_layer():
    from sparse_attention_diffusion_amd import workloads as W
    from sparse_attention_diffusion_amd.trajectory import entry_bytes
    wl = W.WORKLOADS["hunyuan_trajectory"]
    # perm 11.4 MB + lists 3.18 GB + residual 730 MB; with bitmaps 1.40 GB
    assert entry_bytes(wl, 0.15, False) == 24 * (4 * 118800 + 4 * 1857 * 17824 + 118800 * 128 * 2)
    assert entry_bytes(wl, 0.15, True) == 1403235936


@pytest.mark.parametrize("seed", range(8))
@pytest.mark.parametrize("budget_entries", [0, 1, 3, 100])
def test_pinned_budget_splits_host_copies_and_orders_every_access(seed, budget_entries):
    # one entry = 3 tensors of 1,000 bytes, padded to 3 x 1,024; chunks of 4,096 bytes
    # hold one entry each (two would need 6,144)
    be = FakeBackend(seed, pinned_ok=budget_entries > 0)
    layers = 6
    cache = MetaCache(layers, SHAPES, be, offload=True, device_slots=2, pinned_budget=4096 * budget_entries,
                      pinned_chunk=4096)
    pinned = [l for l in range(layers) if cache.entries[l].pinned]
    assert pinned == list(range(min(budget_entries, layers)))
    assert cache.arena.reserved <= 4096 * budget_entries
    assert all(c.size == 4096 for c in be.chunks)
    assert cache.host_pinned_bytes == 3000 * len(pinned)
    assert cache.host_pageable_bytes == 3000 * (layers - len(pinned))
    assert len(be.pageable) == 3 * (layers - len(pinned))
    replay(cache, be, layers, steps=12)
    assert cache.bytes_h2d > 0


def test_pinned_chunks_pack_several_entries():
    be = FakeBackend(0)
    cache = MetaCache(8, SHAPES, be, offload=True, device_slots=2, pinned_budget=1 << 20, pinned_chunk=1 << 15)
    # all eight entries (3 x 1,024 bytes each) fit one chunk (views checked for overlap)
    assert len(be.chunks) == 1 and be.chunks[0].size == 1 << 15
    assert len(be.chunks[0].views) == 8
    assert all(e.pinned for e in cache.entries)


def test_lazy_worker_is_needed_by_the_protocol():
    # a compute-thread wait on an event whose job never ran is caught by the fake
    be = FakeBackend(1)
    cache = MetaCache(4, SHAPES, be, offload=True, device_slots=2)
    real_await = cache._await
    cache._await = lambda fut: None if fut is None else (fut.value if fut.done else be.event())
    with pytest.raises(AssertionError, match="never recorded"):
        replay(cache, be, 4, steps=12)
    cache._await = real_await


def test_bad_pinned_arguments():
    be = FakeBackend(0)
    with pytest.raises(ValueError):
        MetaCache(3, SHAPES, be, offload=True, pinned_budget=-1)
    with pytest.raises(ValueError):
        MetaCache(3, SHAPES, be, offload=True, pinned_chunk=3000)
