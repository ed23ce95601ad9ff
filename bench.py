"""Benchmark of the MC-Sparse hot path on one MI355X.

Workload: the Wan2.1-14B-like 720p attention layer (21x45x80 latent grid ->
75,600 tokens, 40 heads, head_dim 128, bf16, C = 64, density 0.2 -> K = 15,120),
synthetic inputs drawn on the GPU (see sparse_attention_diffusion_amd/workloads.py).

One timed step is one pass of the whole hot path over that layer:
  anchor  = PDDP grouping + dense attention (with row statistics, doubling as
            selection pass 1) + selection pass 2 / top-K + residual (sparse),
  reuse   = gather-sparse attention + cached residual,
  kernel  = gather-sparse attention alone on the cached indices (the metric's
            kernel-only figure; the pages time the kernel without selection and
            grouping, MC-Sparse summary page, kernel-speed paragraph);
  pairs   = the pair plan and the pair-shared variant of the sparse kernel on
            the same indices (reported under "pairs" and stage_ms, not in value).
`value` is the gather-sparse attention throughput in useful TFLOP/s
(4*N*K*D*H per launch over the kernel's average launch time, HIP events on the
launch stream); `x_vs_dense` compares with this library's own dense attention on
the same tensors.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--density RHO] [--cold]

--cold writes a 512 MB scratch buffer (twice the 256 MB MALL) before every timed
call, outside its events, so each stage starts with cold caches.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

MFMA_BF16_PEAK_TFLOPS = 2500.0   # MI355X dense bf16 MFMA (published)
HBM_PEAK_GBPS = 8000.0           # MI355X HBM3E (published)

# Sources of the gather-sparse kernel: the committed counter summary applies only
# while these are byte-identical to the ones it was taken from.
KERNEL_SOURCES = ("sparse_attention_diffusion_amd/csrc/attn.hip", "sparse_attention_diffusion_amd/csrc/ldstile.hpp",
                  "sparse_attention_diffusion_amd/csrc/common.hpp", "sparse_attention_diffusion_amd/csrc/kernels.hpp")


def sources_sha256() -> str:
    import hashlib
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def committed_traffic(workload: str, density: float):
    """Memory-fabric bytes per launch of the gather-sparse kernel (L2 misses,
    MALL hits included, plus writes) from the committed FETCH_SIZE / WRITE_SIZE
    summary (calibrated against a copy of known size), or None when there is none
    or the kernel sources changed since it was taken."""
    path = os.path.join(ROOT, "profiles", f"counters_gather_sparse_{workload}_density{density:g}.md")
    try:
        with open(path) as f:
            for line in f:
                if line.startswith("traffic-json: "):
                    rec = json.loads(line[len("traffic-json: "):])
                    if rec.get("sources_sha256") == sources_sha256():
                        return int(rec["bytes_per_launch"])
                    return None
    except OSError:
        return None
    return None


def pct_of_ideal(speedup: float, density: float) -> float:
    """Fraction of the ideal 1/density speedup (4.79x at density 0.2 is 0.958)."""
    return speedup * density


def _timed(fn, stream):
    import torch
    a = torch.cuda.Event(enable_timing=True)
    b = torch.cuda.Event(enable_timing=True)
    a.record(stream)
    out = fn()
    b.record(stream)
    return out, (a, b)


def cpu_baseline(q, k, v, perm, idx, kk, scale, budget_s=12.0):
    """The fp64 oracle's gather-sparse attention on a bounded sample (groups of one
    head of the same workload), as useful TFLOP/s."""
    import numpy as np
    from oracle import ref

    qh = q[0].float().cpu().numpy()
    kh = k[0].float().cpu().numpy()
    vh = v[0].float().cpu().numpy()
    ph = perm[0].cpu().numpy()
    ih = idx[0].cpu().numpy()
    d = qh.shape[1]
    done, flops = 0, 0.0
    t0 = time.perf_counter()
    g = 0
    while True:
        mem = ph[g * 64:(g + 1) * 64]
        ref.sparse_attention_group(qh, kh, vh, mem, ih[g, :kk].astype(np.int64), scale)
        flops += 4.0 * len(mem) * kk * d
        done += 1
        g += 1
        if time.perf_counter() - t0 > budget_s or g >= ih.shape[0]:
            break
    dt = time.perf_counter() - t0
    try:
        cores = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        cores = os.cpu_count()
    threads = int(os.environ.get("OMP_NUM_THREADS", cores))
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": min(cores, threads), "kind": "oracle",
            "sample": f"fp64 numpy gather-sparse attention of {done} query groups (64 queries x {kk} keys x "
                      f"D={d}) of head 0, {dt:.1f} s; host {_host_info(cores)}"}


def _host_info(cores: int) -> str:
    """CPU model, usable cores and BLAS threads of the machine running the oracle."""
    model = "unknown CPU"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    blas = "?"
    try:
        from threadpoolctl import threadpool_info
        pools = [p for p in threadpool_info() if p.get("user_api") == "blas"]
        if pools:
            blas = f"{pools[0].get('internal_api')} x{pools[0].get('num_threads')}"
    except Exception:  # threadpoolctl missing or failing: leave it unknown
        pass
    return f"{model}, {cores} usable cores, BLAS {blas}"


def sdpa_context(q, k, v, reps=3):
    """torch SDPA (flash / efficient backends only) on the same tensors, for context."""
    import torch
    from torch.nn.attention import SDPBackend, sdpa_kernel
    try:
        with sdpa_kernel([SDPBackend.FLASH_ATTENTION, SDPBackend.EFFICIENT_ATTENTION]):
            f = lambda: torch.nn.functional.scaled_dot_product_attention(q[None], k[None], v[None])
            f()
            torch.cuda.synchronize()
            s = torch.cuda.current_stream()
            evs = [_timed(f, s)[1] for _ in range(reps)]
            torch.cuda.synchronize()
            return sum(a.elapsed_time(b) for a, b in evs) / reps
    except Exception as e:  # backend unavailable in this torch: report nothing
        print(f"[bench] torch SDPA context unavailable: {type(e).__name__}: {e}", file=sys.stderr)
        return None


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=5)
    ap.add_argument("--warmup", type=int, default=1)
    ap.add_argument("--workload", default="wan14b_720p")
    ap.add_argument("--density", type=float, default=0.2)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-sdpa", action="store_true")
    ap.add_argument("--cold", action="store_true",
                    help="write a 512 MB scratch buffer before every timed call (cold L2 and MALL)")
    ap.add_argument("--copy-probe", action="store_true",
                    help="copy 1 GiB once before the workload (calibrates FETCH_SIZE/WRITE_SIZE counters)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: the MC-Sparse hot path runs and is timed on a single MI355X "
              "(heads shard across GPUs without any exchange; there is no multi-GPU code path).",
              file=sys.stderr)
        sys.exit(2)

    import torch
    import sparse_attention_diffusion_amd as mcs
    from sparse_attention_diffusion_amd import workloads as W

    wl = W.WORKLOADS[args.workload]
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    n, h, d = wl.n, wl.heads, wl.head_dim
    kk = wl.topk(args.density)
    print(f"[bench] {wl.name}: N={n} H={h} D={d} {wl.dtype} C={wl.group} density={args.density} K={kk}",
          file=sys.stderr, flush=True)
    if args.copy_probe:
        src = torch.ones(1 << 28, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    q, k, v = W.make_qkv_torch(wl, dev)
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream(dev)

    d_ = mcs.make_dims(q, topk=kk)
    ws = torch.empty(mcs.mcs_workspace_bytes(d_, mcs.MCS_OP_ANCHOR), dtype=torch.uint8, device=dev)
    gws = torch.empty(mcs.mcs_workspace_bytes(d_, mcs.MCS_OP_GROUP), dtype=torch.uint8, device=dev)
    swsz = mcs.mcs_workspace_bytes(d_, mcs.MCS_OP_SELECT)
    g = wl.groups
    cache = dict(perm=torch.empty((h, n), dtype=torch.int32, device=dev),
                 idx=torch.empty((h, g, d_.kpad), dtype=torch.int32, device=dev),
                 resid=torch.empty_like(q), o_dense=torch.empty_like(q), lse=None)
    o_reuse = torch.empty_like(q)
    o_sparse = torch.empty_like(q)
    o_pairs = torch.empty_like(q)
    pidx = torch.empty_like(cache["idx"])
    ncommon = torch.empty((h, mcs.pairs_of(n)), dtype=torch.int32, device=dev)
    o_dense = torch.empty_like(q)
    lse = torch.empty((h, n), dtype=torch.float32, device=dev)

    scratch = torch.empty(512 << 20, dtype=torch.uint8, device=dev) if args.cold else None

    def timed(fn):
        if scratch is not None:
            scratch.fill_(1)  # same stream, before the start event: not timed
        return _timed(fn, stream)

    def step(record):
        ev = {}
        # anchor (composite entry point), then its stages one by one for the breakdown
        _, ev["anchor"] = timed(lambda: mcs.mcs_anchor(q, k, v, kk, ws=ws, out=cache))
        _, ev["group"] = timed(lambda: mcs.mcs_group(q, ws=gws, perm=cache["perm"]))
        _, ev["dense"] = timed(lambda: mcs.mcs_dense_attn(q, k, v, want_lse=False, o=o_dense))
        _, ev["select"] = timed(lambda: mcs.mcs_select(q, k, cache["perm"], kk, lse=None, ws=ws[:swsz],
                                                       idx=cache["idx"]))
        _, ev["reuse"] = timed(lambda: mcs.mcs_reuse(q, k, v, cache["perm"], cache["idx"], cache["resid"], kk,
                                                     o=o_reuse))
        _, ev["sparse"] = timed(lambda: mcs.mcs_sparse_attn(q, k, v, cache["perm"], cache["idx"], kk,
                                                            o=o_sparse))
        # pair-shared gathers (reported beside the headline kernel, not in `value`)
        _, ev["pair_plan"] = timed(lambda: mcs.mcs_pair_plan(cache["idx"], n, kk, pidx=pidx, ncommon=ncommon))
        _, ev["sparse_pairs"] = timed(lambda: mcs.mcs_sparse_attn_pairs(q, k, v, cache["perm"], pidx, ncommon, kk,
                                                                        o=o_pairs))
        if record is not None:
            record.append(ev)

    for _ in range(args.warmup):
        step(None)
    torch.cuda.synchronize()
    recs = []
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(recs)
        torch.cuda.synchronize()
        print(f"[bench] step {i + 1}/{args.steps} done", file=sys.stderr, flush=True)
    wall = time.perf_counter() - t0
    ms = {key: sum(r[key][0].elapsed_time(r[key][1]) for r in recs) / len(recs) for key in recs[0]}

    flops_sparse = 4.0 * n * kk * d * h
    flops_dense = 4.0 * n * n * d * h
    t_sparse, t_dense = ms["sparse"] / 1e3, ms["dense"] / 1e3
    value = flops_sparse / t_sparse / 1e12
    speedup = t_dense / t_sparse
    # Reference work of the other stages (per layer):
    #   PDDP: per level of the split tree, two reads of Q (statistics, projections)
    #         plus ~6 4-byte scalars per token (perm, keys, partition);
    #   selection: two N^2 D contractions (pass 1 LSE, pass 2 group mass).
    levels = max(1, (g - 1).bit_length())
    pddp_bytes = levels * (2.0 * n * d * h * q.element_size() + 24.0 * n * h)
    flops_select = 4.0 * n * n * d * h
    # K and V rows the sparse kernel gathers into LDS (mostly served by L2 / MALL)
    gather_bytes = 2.0 * g * kk * d * q.element_size() * h
    sdpa_ms = None if args.no_sdpa else sdpa_context(q, k, v)
    out = {
        "metric": "gather-sparse attn TFLOP/s, % MFMA peak, x vs dense @ density 0.2, 75,600 tok",
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(wall / args.steps * 1e3, 2),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": f"{wl.name}: {wl.grid[0]}x{wl.grid[1]}x{wl.grid[2]} grid, N={n}, H={h}, D={d}, "
                               f"bf16, C={wl.group}, density={args.density}, K={kk}",
                   "tokens": n, "heads": h, "head_dim": d, "group": wl.group, "density": args.density, "topk": kk},
        "pct_mfma_peak": round(100.0 * value / MFMA_BF16_PEAK_TFLOPS, 2),
        "x_vs_dense": round(speedup, 3),
        "pct_of_ideal": round(100.0 * pct_of_ideal(speedup, args.density), 1),
        "dense_tflops": round(flops_dense / t_dense / 1e12, 2),
        "stage_ms": {key: round(val, 3) for key, val in ms.items()},
        "cache": "cold (512 MB written before every timed call)" if args.cold else "warm",
        "stage_rates": {"sparse_gather_tbps": round(gather_bytes / t_sparse / 1e12, 2),
                        "group_ref_gbps": round(pddp_bytes / (ms["group"] / 1e3) / 1e9, 1),
                        "group_ref_frac_hbm": round(pddp_bytes / (ms["group"] / 1e3) / 1e9 / HBM_PEAK_GBPS, 4),
                        "select_tflops": round(flops_select / (ms["select"] / 1e3) / 1e12, 1),
                        "select_frac_mfma": round(flops_select / (ms["select"] / 1e3) / 1e12 / MFMA_BF16_PEAK_TFLOPS,
                                                  4)},
        "torch_sdpa_ms": None if sdpa_ms is None else round(sdpa_ms, 3),
        "pairs": {"shared_fraction": round(float(ncommon.double().sum().item()) / (h * (g // 2) * kk), 4),
                  "sparse_pairs_tflops": round(flops_sparse / (ms["sparse_pairs"] / 1e3) / 1e12, 2)},
        "roofline": {"bound": "mfma", "achieved": round(value, 2), "peak": MFMA_BF16_PEAK_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(value / MFMA_BF16_PEAK_TFLOPS, 4),
                     "traffic": committed_traffic(wl.name, args.density)},
    }
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(q, k, v, cache["perm"], cache["idx"], kk, 1.0 / d ** 0.5)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
