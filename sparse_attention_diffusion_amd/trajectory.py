"""Denoising-trajectory harness of the MC-Sparse hot path (one GPU).

Schedule (MC-Sparse summary page, method and kernel-speed paragraphs; the pages
leave the exact schedule open): the first `warmup` steps run dense attention, then
an anchor step every `interval` steps (grouping, selection, dense attention and
residual), and reuse steps in between (gather-sparse attention + cached
residual).  Every layer has its own drifting Q/K/V (a random walk per step) and
its own meta-cache entry, optionally offloaded to pinned host memory with
next-layer prefetch on a side stream.

Usage: python -m sparse_attention_diffusion_amd.trajectory [--layers L] [--steps S]
       [--offload] [--density RHO]   (prints one JSON line)
"""
from __future__ import annotations

import argparse
import json
import math
import sys
import time

import numpy as np


def step_kind(step, warmup, interval):
    if step < warmup:
        return "dense"
    return "anchor" if (step - warmup) % interval == 0 else "reuse"


class LayerInputs:
    """Q/K/V of every layer: float32 masters on the device, advanced by one
    random-walk step at a time and rounded once into the storage-dtype buffers a
    layer call reads, so that layer l at step t holds exactly
    ``make_qkv_torch(wl, step=t, layer=l)`` (drift applied before rounding)."""

    def __init__(self, wl, layers, device):
        from .workloads import base_qkv_torch, storage_dtype_torch
        self.wl = wl
        self.device = device
        self.master = [base_qkv_torch(wl, device, layer=l) for l in range(layers)]
        dt = storage_dtype_torch(wl)
        self.work = tuple(torch_empty_like(self.master[0][0], dt) for _ in range(3))

    def advance(self, layer, step):
        from .workloads import drift_torch_
        drift_torch_(*self.master[layer], self.wl, layer, step)

    def get(self, layer):
        """Storage-dtype Q, K, V of `layer` at its current step (shared buffers: valid
        until the next call)."""
        for w, m in zip(self.work, self.master[layer]):
            w.copy_(m)
        return self.work


def torch_empty_like(t, dtype):
    import torch
    return torch.empty(t.shape, dtype=dtype, device=t.device)


def entry_bytes(wl, density, compact):
    """Bytes of one layer's cache entry: perm (int32 [H][N]), the kept keys (int32
    lists [H][G][kpad], or bitmaps [H][G][ceil(N/32)] when compact) and the
    residual ([H][N][D] in the workload's dtype)."""
    h, n, d, g = wl.heads, wl.n, wl.head_dim, wl.groups
    kpad = -(-wl.topk(density) // 32) * 32
    keys = g * ((n + 31) // 32) if compact else g * kpad
    return h * (4 * n + 4 * keys + n * d * (4 if wl.dtype == "f32" else 2))


def run(wl, layers, steps, warmup=5, interval=5, density=0.15, offload=False, device_slots=2, heads_per_pass=4,
        record_outputs=None, log=None, compact=False, resident_layers=0, pinned_budget=None, record_inputs=None,
        record_entries=None):
    """compact: cache the kept-key sets as per-group key bitmaps (encoded after
    each anchor, decoded before each reuse into one shared list buffer).
    resident_layers: with offload, the first that many layers keep their entries
    on the device (the layers that fit a memory budget); only the rest are
    offloaded.  pinned_budget: bytes of pinned host memory for the offloaded
    entries (default: the cache's), pageable beyond.
    record_outputs / record_inputs: dicts keyed by (step, layer) whose values are
    filled with the layer call's output / its (q, k, v) on the device;
    record_entries: dict filled, at every anchor of a (step, layer) key present
    in it, with the cache entry the anchor wrote ({"perm", "idx", "resid"}, idx
    decoded when compact)."""
    import torch

    import sparse_attention_diffusion_amd as mcs
    from .cache import DEFAULT_PINNED_BUDGET, MetaCache, TorchBackend

    dev = torch.device("cuda:0")
    kk = wl.topk(density)
    inputs = LayerInputs(wl, layers, dev)
    q0 = inputs.get(0)[0]
    d = mcs.make_dims(q0, topk=kk)
    h, n, dd = q0.shape
    g = wl.groups
    if compact:
        shapes = {"perm": ((h, n), torch.int32), "bits": ((h, g, mcs.bits_words(n)), torch.int32),
                  "resid": ((h, n, dd), q0.dtype)}
        idx_scratch = torch.empty((h, g, d.kpad), dtype=torch.int32, device=dev)
    else:
        shapes = {"perm": ((h, n), torch.int32), "idx": ((h, g, d.kpad), torch.int32),
                  "resid": ((h, n, dd), q0.dtype)}
    be = TorchBackend(dev)
    cache = MetaCache(layers, shapes, be, offload=offload, device_slots=device_slots,
                      resident_layers=resident_layers,
                      pinned_budget=DEFAULT_PINNED_BUDGET if pinned_budget is None else pinned_budget)
    ws = torch.empty(mcs.mcs_workspace_bytes(d, mcs.MCS_OP_ANCHOR, heads_per_pass), dtype=torch.uint8, device=dev)
    o_dense = torch.empty_like(q0)
    out = torch.empty_like(q0)
    stream = torch.cuda.current_stream(dev)
    times = {"dense": [], "anchor": [], "reuse": []}
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for step in range(steps):
        kind = step_kind(step, warmup, interval)
        for layer in range(layers):
            if step > 0:
                inputs.advance(layer, step)
            q, k, v = inputs.get(layer)
            a = torch.cuda.Event(enable_timing=True)
            b = torch.cuda.Event(enable_timing=True)
            a.record(stream)
            if kind == "dense":
                mcs.mcs_dense_attn(q, k, v, o=out)
            elif kind == "anchor":
                buf = cache.anchor_buffers(layer, busy_layer=layer - 1)
                res = dict(buf, o_dense=o_dense, lse=None)
                if compact:
                    res["idx"] = idx_scratch
                mcs.mcs_anchor(q, k, v, kk, ws=ws, heads_per_pass=heads_per_pass, out=res)
                if compact:
                    mcs.mcs_idx_to_bits(idx_scratch, n, kk, bits=buf["bits"])
                if record_entries is not None and (step, layer) in record_entries:
                    idx_rec = mcs.mcs_bits_to_idx(buf["bits"], n, kk, kpad=d.kpad) if compact else buf["idx"]
                    record_entries[(step, layer)] = {"perm": buf["perm"].clone(), "idx": idx_rec.clone(),
                                                     "resid": buf["resid"].clone()}
                cache.commit_anchor(layer)
                cache.release(layer)
            else:
                buf = cache.get(layer)
                idx = mcs.mcs_bits_to_idx(buf["bits"], n, kk, idx=idx_scratch) if compact else buf["idx"]
                mcs.mcs_reuse(q, k, v, buf["perm"], idx, buf["resid"], kk, o=out)
                cache.release(layer)
            b.record(stream)
            times[kind].append((a, b))
            # prefetch the entry the next layer-call will need
            nxt_step, nxt_layer = (step, layer + 1) if layer + 1 < layers else (step + 1, 0)
            if nxt_step < steps and step_kind(nxt_step, warmup, interval) == "reuse":
                cache.prefetch(nxt_layer, busy_layer=layer)
            if record_outputs is not None and (step, layer) in record_outputs:
                record_outputs[(step, layer)] = (o_dense if kind == "anchor" else out).clone()
            if record_inputs is not None and (step, layer) in record_inputs:
                record_inputs[(step, layer)] = tuple(t.clone() for t in (q, k, v))
        if log:
            torch.cuda.synchronize()
            log(f"[trajectory] step {step + 1}/{steps} ({kind}) done")
    cache.drain()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    be.close()
    ms = {kk_: [x.elapsed_time(y) for x, y in v_] for kk_, v_ in times.items()}
    t_dense_call = float(np.mean(ms["dense"])) if ms["dense"] else float("nan")
    total_attn = sum(sum(v_) for v_ in ms.values())
    all_dense = t_dense_call * steps * layers
    anchors = sum(1 for s in range(steps) if step_kind(s, warmup, interval) == "anchor")
    reuses = steps - warmup - anchors
    # effective density of the whole trajectory (dense = 1) and its amortised
    # overhead over the sparse steps, in density points
    eff = total_attn / all_dense if all_dense == all_dense else float("nan")
    overhead = ((eff * steps - warmup - (steps - warmup) * density) / (steps - warmup) * 100.0
                if steps > warmup else float("nan"))
    return {
        "workload": wl.name, "layers": layers, "steps": steps, "warmup": warmup, "interval": interval,
        "density": density, "topk": kk, "offload": offload, "compact": compact,
        "resident_layers": len(cache.resident), "anchors": anchors,
        "reuse_steps": reuses,
        "wall_s": round(wall, 3),
        "attention_ms": round(total_attn, 1),
        "all_dense_ms_estimate": round(all_dense, 1),
        "speedup_vs_dense": round(all_dense / total_attn, 3) if total_attn else None,
        "mean_ms": {k_: round(float(np.mean(v_)), 3) for k_, v_ in ms.items() if v_},
        "anchor_overhead_density_points": round(overhead, 2) if overhead == overhead else None,
        "cache_bytes_per_layer": sum(math.prod(s_) * torch.empty((), dtype=t_).element_size()
                                     for s_, t_ in shapes.values()),
        "bytes_d2h": cache.bytes_d2h, "bytes_h2d": cache.bytes_h2d,
        "host_pinned_bytes": cache.host_pinned_bytes, "host_pageable_bytes": cache.host_pageable_bytes,
        "host_wait_s": round(cache.host_wait_s, 3),
        "h2d_gbps_if_serial": round(cache.bytes_h2d / 1e9 / wall, 2) if wall > 0 else None,
    }


def main():
    from .workloads import WORKLOADS
    ap = argparse.ArgumentParser()
    ap.add_argument("--workload", default="hunyuan_trajectory")
    ap.add_argument("--layers", type=int, default=4)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--interval", type=int, default=5)
    ap.add_argument("--density", type=float, default=0.15)
    ap.add_argument("--offload", action="store_true")
    ap.add_argument("--compact", action="store_true", help="cache kept-key sets as per-group key bitmaps")
    ap.add_argument("--heads-per-pass", type=int, default=4)
    ap.add_argument("--resident-gb", type=float, default=0.0,
                    help="with --offload: keep resident as many layers' entries as fit in this many GB")
    ap.add_argument("--pinned-gb", type=float, default=None,
                    help="with --offload: pinned host memory for the offloaded entries (GiB), pageable beyond")
    args = ap.parse_args()
    wl = WORKLOADS[args.workload]
    resident = 0
    if args.offload and args.resident_gb > 0:
        resident = min(args.layers, int(args.resident_gb * 1e9 // entry_bytes(wl, args.density, args.compact)))
    res = run(wl, args.layers, args.steps, args.warmup, args.interval, args.density, args.offload,
              heads_per_pass=args.heads_per_pass, log=lambda m: print(m, file=sys.stderr, flush=True),
              compact=args.compact, resident_layers=resident,
              pinned_budget=None if args.pinned_gb is None else int(args.pinned_gb * (1 << 30)))
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
