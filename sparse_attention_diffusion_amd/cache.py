"""Meta-cache of the MC-Sparse hot path: per-layer {perm, idx, resid} (or, compact,
{perm, bits, resid} with the kept-key lists as per-group key bitmaps).

MC-Sparse summary page, residual paragraph: groups, indices and the residual are
produced together on anchor steps and reused on later steps; when GPU memory is
tight, inactive entries move to host memory and the next layer's entry is
prefetched so that the transfer hides behind compute.

Two modes:
* resident: every layer keeps its own device buffers;
* offload: layers share a small pool of device slots; after an anchor the entry
  is copied to pinned host memory (device -> host) on a side stream, and before a
  layer runs its entry is copied back into a free slot (host -> device) on the
  side stream, gated by events so that the compute stream never reads a slot
  whose copy has not finished and the side stream never overwrites a slot the
  compute stream may still read.
Offload can keep the first `resident_layers` layers resident (the layers that fit
a device-memory budget): those have their own buffers and are never copied, and
only the others go through the slot pool and the host.

All copies go through `mcs_copy_async` of the C ABI (or an injected copier with
the same signature for host-only tests); streams and events are torch's
(default priority).
"""
from __future__ import annotations

from dataclasses import dataclass, field

from . import MCS_COPY_D2H, MCS_COPY_H2D, mcs_copy_async


@dataclass
class _Slot:
    tensors: dict
    layer: int = -1           # layer whose entry the slot holds (or is receiving)
    side_last: object = None  # event: last side-stream access (host copy read or prefetch write) done
    released: object = None   # event: compute stream finished its last use of this slot


@dataclass
class _Entry:
    state: str = "empty"      # empty | device | host
    slot: int = -1            # device slot while on device
    host: dict = field(default_factory=dict)
    d2h_done: object = None   # event: host copy complete


class TorchBackend:
    """Streams and events of torch on one device."""

    def __init__(self, device):
        import torch
        self.torch = torch
        self.device = device
        self.side = torch.cuda.Stream(device=device)  # default priority

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

    def empty_device(self, shape, dtype):
        return self.torch.empty(shape, dtype=dtype, device=self.device)

    def empty_host(self, shape, dtype):
        return self.torch.empty(shape, dtype=dtype, pin_memory=True)


class MetaCache:
    """Per-layer cache of named device tensors (perm, idx or bits, resid) with
    optional host offload."""

    def __init__(self, layers, shapes, backend, offload=False, device_slots=2, resident_layers=0):
        """shapes: {name: (shape, dtype)} of one layer's entry, e.g. {"perm": ...,
        "idx": ..., "resid": ...}.  With offload, layers 0 .. resident_layers-1
        stay resident; the rest share `device_slots` device slots."""
        if resident_layers < 0:
            raise ValueError("resident_layers must be >= 0")
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
        for layer, e in enumerate(self.entries):
            if layer not in self.resident:
                e.host = {k: backend.empty_host(*shapes[k]) for k in self.keys}
        self.bytes_d2h = 0
        self.bytes_h2d = 0

    # -- slot management ---------------------------------------------------
    def _slot_of(self, layer):
        """Pool slot holding `layer`'s entry, or -1 (resident layers hold none)."""
        e = self.entries[layer]
        return e.slot if e.state == "device" and layer not in self.resident else -1

    def _take_slot(self, layer, avoid=()):
        """A device slot for `layer`: its own if resident, else a slot not in `avoid`
        (preferring one whose owner already left); the slot's previous owner leaves
        the device.  Returns (slot, event of the previous owner's host copy or None):
        whoever overwrites the slot must wait for that copy to have read it."""
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
        if pending is not None:  # the evicted entry's host copy must have read the slot
            self.be.wait(self.be.compute_stream(), pending)
        if s.side_last is not None:  # no host copy or prefetch of this slot may still be running
            self.be.wait(self.be.compute_stream(), s.side_last)
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
        self.be.wait(self.be.side, written)
        for k in self.keys:
            self.be.copy(e.host[k], s.tensors[k], MCS_COPY_D2H, self.be.side)
            self.bytes_d2h += s.tensors[k].numel() * s.tensors[k].element_size()
        e.d2h_done = self.be.event()
        self.be.record(e.d2h_done, self.be.side)
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
        if pending is not None:  # same stream already orders it; explicit for clarity
            self.be.wait(self.be.side, pending)
        if s.released is not None:  # the compute stream's last use of the slot must be over
            self.be.wait(self.be.side, s.released)
        self.be.wait(self.be.side, e.d2h_done)
        for k in self.keys:
            self.be.copy(s.tensors[k], e.host[k], MCS_COPY_H2D, self.be.side)
            self.bytes_h2d += s.tensors[k].numel() * s.tensors[k].element_size()
        s.side_last = self.be.event()
        self.be.record(s.side_last, self.be.side)
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
            self.be.wait(self.be.compute_stream(), s.side_last)
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
