"""Meta-cache of the MC-Sparse hot path: per-layer {perm, idx, resid} (or, compact,
{perm, bits, resid} with the kept-key lists as per-group key bitmaps).

MC-Sparse summary page, residual paragraph: groups, indices and the residual are
produced together on anchor steps and reused on later steps; when GPU memory is
tight, inactive entries move to host memory and the next layer's entry is
prefetched so that the transfer hides behind compute.

Two modes:
* resident: every layer keeps its own device buffers;
* offload: layers share a small pool of device slots; after an anchor the entry
  is copied to host memory (device -> host) on a side stream, and before a layer
  runs its entry is copied back into a free slot (host -> device) on the side
  stream, gated by events so that the compute stream never reads a slot whose
  copy has not finished and the side stream never overwrites a slot the compute
  stream may still read.
Offload can keep the first `resident_layers` layers resident (the layers that fit
a device-memory budget): those have their own buffers and are never copied, and
only the others go through the slot pool and the host.

Host memory.  Pinned (page-locked) host memory is what lets a copy run
asynchronously at full link rate, but a process can only pin so much of it
(about 64 GiB on the MI355X hosts used here), far less than a 40-layer cache of
kept-key lists (157 GB).  Host copies are therefore pinned while they fit a
budget (`pinned_budget` bytes, packed into power-of-two chunks so that the
pinned allocator rounds nothing up) and pageable beyond it; a copy to or from
pageable memory goes through the HIP runtime's own staging and blocks the thread
that issues it.  So that such a copy never stalls the thread that enqueues the
attention kernels, every side-stream operation is issued, in order, by one
worker thread; the compute thread only records events on its own stream and
waits (on the host) for the worker's event of a copy before it makes the compute
stream depend on it.

All copies go through `mcs_copy_async` of the C ABI (or an injected copier with
the same signature for host-only tests); streams and events are torch's
(default priority).
"""
from __future__ import annotations

import threading
import time
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field

from . import MCS_COPY_D2H, MCS_COPY_H2D, mcs_copy_async

GiB = 1 << 30
DEFAULT_PINNED_BUDGET = 48 * GiB
PINNED_CHUNK = 8 * GiB


@dataclass
class _Slot:
    tensors: dict
    layer: int = -1          # layer whose entry the slot holds (or is receiving)
    side_last: object = None  # future -> event: last side-stream access (host copy read or prefetch write)
    released: object = None   # event: compute stream finished its last use of this slot


@dataclass
class _Entry:
    state: str = "empty"     # empty | device | host
    slot: int = -1           # device slot while on device
    host: dict = field(default_factory=dict)
    pinned: bool = False     # host copies in pinned memory
    d2h_done: object = None  # future -> event: host copy complete


class _Done:
    """A future that is already resolved."""

    def __init__(self, value):
        self.value = value

    def result(self):
        return self.value


class PinnedArena:
    """Pinned host buffers carved from chunks of `chunk` bytes (a power of two, so
    the pinned allocator rounds nothing up), at most `budget` bytes in total."""

    def __init__(self, backend, budget, chunk=PINNED_CHUNK):
        self.be = backend
        self.budget = int(budget)
        self.chunk = int(chunk)
        self.chunks = []   # (buffer, used bytes)
        self.reserved = 0  # bytes of chunks allocated

    def take(self, nbytes):
        """A pinned uint8 buffer of nbytes (256-byte aligned offsets) or None when
        the budget cannot hold it."""
        need = (nbytes + 255) & ~255
        for i, (buf, used) in enumerate(self.chunks):
            if used + need <= self.be.host_size(buf):
                self.chunks[i] = (buf, used + need)
                return self.be.host_view(buf, used, nbytes)
        left = self.budget - self.reserved
        if left < need:
            return None
        # a full chunk while the budget allows one, else the largest power of two left
        size = max(1 << (need - 1).bit_length(), min(self.chunk, 1 << (left.bit_length() - 1)))
        if size > left:
            return None
        buf = self.be.empty_pinned_bytes(size)
        self.reserved += size
        self.chunks.append((buf, need))
        return self.be.host_view(buf, 0, nbytes)


class TorchBackend:
    """Streams and events of torch on one device; side-stream work runs on one
    worker thread, in submission order."""

    def __init__(self, device):
        import torch
        self.torch = torch
        self.device = device
        self.side = torch.cuda.Stream(device=device)  # default priority
        self.pool = ThreadPoolExecutor(max_workers=1, thread_name_prefix="mcs-cache",
                                       initializer=lambda: torch.cuda.set_device(device))

    def compute_stream(self):
        return self.torch.cuda.current_stream(self.device)

    def event(self):
        return self.torch.cuda.Event()

    def record(self, event, stream):
        event.record(stream)

    def wait(self, stream, event):
        stream.wait_event(event)

    def copy(self, dst, src, kind, stream):
        mcs_copy_async(dst, src, kind, stream=stream)

    def submit(self, fn):
        return self.pool.submit(fn)

    def empty_device(self, shape, dtype):
        return self.torch.empty(shape, dtype=dtype, device=self.device)

    def empty_pageable(self, shape, dtype):
        return self.torch.empty(shape, dtype=dtype)

    def empty_pinned_bytes(self, nbytes):
        return self.torch.empty(nbytes, dtype=self.torch.uint8, pin_memory=True)

    def host_size(self, buf):
        return buf.numel()

    def host_view(self, buf, offset, nbytes):
        return buf[offset:offset + nbytes]

    def typed(self, raw, shape, dtype):
        return raw.view(dtype).view(shape)

    def nbytes(self, shape, dtype):
        import math
        return math.prod(shape) * self.torch.empty((), dtype=dtype).element_size()

    def close(self):
        self.pool.shutdown(wait=True)


class MetaCache:
    """Per-layer cache of named device tensors (perm, idx or bits, resid) with
    optional host offload."""

    def __init__(self, layers, shapes, backend, offload=False, device_slots=2, resident_layers=0,
                 pinned_budget=DEFAULT_PINNED_BUDGET, pinned_chunk=PINNED_CHUNK):
        """shapes: {name: (shape, dtype)} of one layer's entry, e.g. {"perm": ...,
        "idx": ..., "resid": ...}.  With offload, layers 0 .. resident_layers-1
        stay resident; the rest share `device_slots` device slots, and their host
        copies are pinned while `pinned_budget` bytes hold them (in chunks of
        `pinned_chunk` bytes, a power of two), pageable beyond."""
        if pinned_chunk <= 0 or pinned_chunk & (pinned_chunk - 1):
            raise ValueError("pinned_chunk must be a power of two")
        if resident_layers < 0:
            raise ValueError("resident_layers must be >= 0")
        if pinned_budget < 0:
            raise ValueError("pinned_budget must be >= 0")
        self.layers = layers
        self.shapes = shapes
        self.keys = tuple(shapes)
        self.be = backend
        self.offload = offload
        self.resident = frozenset(range(min(layers, resident_layers) if offload else layers))
        self.own = {layer: {k: backend.empty_device(*shapes[k]) for k in self.keys} for layer in sorted(self.resident)}
        pooled = layers - len(self.resident)
        nslots = min(pooled, device_slots)
        if pooled > 1 and nslots < 2:
            raise ValueError("offload needs at least two device slots")
        self.slots = [_Slot({k: backend.empty_device(*shapes[k]) for k in self.keys}) for _ in range(nslots)]
        self.entries = [_Entry() for _ in range(layers)]
        sizes = {k: backend.nbytes(*shapes[k]) for k in self.keys}
        entry = sum((b + 255) & ~255 for b in sizes.values())
        # chunks no larger than what all offloaded entries need together
        total = max(1, entry * (layers - len(self.resident)))
        self.arena = PinnedArena(backend, pinned_budget, min(pinned_chunk, 1 << (total - 1).bit_length()))
        self.host_pinned_bytes = 0
        self.host_pageable_bytes = 0
        for layer, e in enumerate(self.entries):
            if layer in self.resident:
                continue
            raw = self.arena.take(entry)
            if raw is not None:
                off = 0
                for k in self.keys:
                    e.host[k] = backend.typed(backend.host_view(raw, off, sizes[k]), *shapes[k])
                    off += (sizes[k] + 255) & ~255
                e.pinned = True
                self.host_pinned_bytes += sum(sizes.values())
            else:
                e.host = {k: backend.empty_pageable(*shapes[k]) for k in self.keys}
                self.host_pageable_bytes += sum(sizes.values())
        self.bytes_d2h = 0
        self.bytes_h2d = 0
        self.host_wait_s = 0.0  # compute thread blocked on the worker's events
        self._lock = threading.Lock()

    # -- helpers -------------------------------------------------------------
    def _await(self, fut):
        """Event of a side-stream job; blocks the calling thread until the worker
        has issued the job's copies (and, for pageable memory, run them)."""
        if fut is None:
            return None
        t0 = time.perf_counter()
        ev = fut.result()
        self.host_wait_s += time.perf_counter() - t0
        return ev

    def _slot_of(self, layer):
        """Pool slot holding `layer`'s entry, or -1 (resident layers hold none)."""
        e = self.entries[layer]
        return e.slot if e.state == "device" and layer not in self.resident else -1

    def _take_slot(self, layer, avoid=()):
        """A device slot for `layer`: its own if resident, else a slot not in `avoid`
        (preferring one whose owner already left); the slot's previous owner leaves
        the device.  Returns (slot, future of the previous owner's host copy or
        None): whoever overwrites the slot must wait for that copy to have read it."""
        own = self._slot_of(layer)
        if own >= 0:
            return own, None
        cands = [i for i in range(len(self.slots)) if i not in avoid]
        # prefer a slot whose owner is already on the host (or empty)
        cands.sort(key=lambda i: (self.slots[i].layer >= 0 and self.entries[self.slots[i].layer].state == "device",
                                  i))
        i = cands[0]
        prev = self.slots[i].layer
        pending = None
        if prev >= 0 and prev != layer and self.entries[prev].state == "device":
            if self.entries[prev].d2h_done is None:
                raise RuntimeError(f"layer {prev} would be evicted before its host copy was enqueued")
            pending = self.entries[prev].d2h_done
            self.entries[prev].state = "host"
            self.entries[prev].slot = -1
        self.slots[i].layer = layer
        return i, pending

    # -- public API ----------------------------------------------------------
    def anchor_buffers(self, layer, busy_layer=-1):
        """Device tensors the anchor of `layer` writes into (on the compute stream).
        `busy_layer` is a layer whose slot the compute stream is still using."""
        if layer in self.resident:
            self.entries[layer].state = "device"
            return self.own[layer]
        avoid = () if busy_layer < 0 or self._slot_of(busy_layer) < 0 else (self._slot_of(busy_layer),)
        i, pending = self._take_slot(layer, avoid)
        s = self.slots[i]
        comp = self.be.compute_stream()
        if pending is not None:  # the evicted entry's host copy must have read the slot
            self.be.wait(comp, self._await(pending))
        if s.side_last is not None:  # no host copy or prefetch of this slot may still be running
            self.be.wait(comp, self._await(s.side_last))
        e = self.entries[layer]
        e.state, e.slot, e.d2h_done = "device", i, None
        return s.tensors

    def commit_anchor(self, layer):
        """Call after the anchor of `layer` was enqueued: in offload mode start the
        device -> host copy of its entry on the side stream."""
        if layer in self.resident:
            return
        e = self.entries[layer]
        s = self.slots[e.slot]
        written = self.be.event()
        self.be.record(written, self.be.compute_stream())
        src = dict(s.tensors)
        for k in self.keys:
            self.bytes_d2h += self.be.nbytes(*self.shapes[k])

        def job():
            self.be.wait(self.be.side, written)
            for k in self.keys:
                self.be.copy(e.host[k], src[k], MCS_COPY_D2H, self.be.side)
            done = self.be.event()
            self.be.record(done, self.be.side)
            return done

        e.d2h_done = self.be.submit(job)
        s.side_last = e.d2h_done

    def prefetch(self, layer, busy_layer=-1):
        """Start bringing `layer`'s entry to the device (no-op if resident)."""
        if layer in self.resident:
            return
        e = self.entries[layer]
        if e.state == "device":
            return
        if e.state != "host":
            raise RuntimeError(f"layer {layer} has no cached entry to prefetch")
        avoid = () if busy_layer < 0 or self._slot_of(busy_layer) < 0 else (self._slot_of(busy_layer),)
        i, pending = self._take_slot(layer, avoid)
        s = self.slots[i]
        released = s.released    # the compute stream's last use of the slot must be over
        own_copy = e.d2h_done    # the entry's own host copy must be complete
        dst = dict(s.tensors)
        for k in self.keys:
            self.bytes_h2d += self.be.nbytes(*self.shapes[k])

        def job():
            # earlier jobs ran first (one worker, submission order): their futures are resolved
            for fut in (pending, own_copy):
                if fut is not None:
                    self.be.wait(self.be.side, fut.result())
            if released is not None:
                self.be.wait(self.be.side, released)
            for k in self.keys:
                self.be.copy(dst[k], e.host[k], MCS_COPY_H2D, self.be.side)
            done = self.be.event()
            self.be.record(done, self.be.side)
            return done

        s.side_last = self.be.submit(job)
        e.state, e.slot = "device", i

    def get(self, layer):
        """Device tensors of `layer`'s entry for a reuse step on the compute stream
        (prefetching on the side stream first if it was not prefetched)."""
        e = self.entries[layer]
        if e.state == "empty":
            raise RuntimeError(f"layer {layer} has no anchor yet")
        if layer in self.resident:
            return self.own[layer]
        if e.state != "device":
            self.prefetch(layer)
        s = self.slots[e.slot]
        if s.side_last is not None:
            self.be.wait(self.be.compute_stream(), self._await(s.side_last))
        return s.tensors

    def release(self, layer):
        """Mark the end of the compute stream's use of `layer`'s slot."""
        if layer in self.resident:
            return
        e = self.entries[layer]
        if e.state != "device":
            return
        s = self.slots[e.slot]
        s.released = self.be.event()
        self.be.record(s.released, self.be.compute_stream())

    def drain(self):
        """Block until every side-stream job has been issued (host side)."""
        for s in self.slots:
            self._await(s.side_last)
        for e in self.entries:
            self._await(e.d2h_done)
