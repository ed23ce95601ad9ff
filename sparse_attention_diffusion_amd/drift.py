"""Anchor-interval and drift study (MC-Sparse summary page, residual and
limitations paragraphs: reuse steps assume that attention changes slowly, the
residual changes less across denoising steps than the output, and every anchor
still costs a full dense attention plus selection).

One attention layer drifts for T steps after an anchor at step 0 (the workload
generator's per-step random walk).  At every step t it measures, against fresh
dense attention O_t:
  * the reuse output (sparse attention on the anchor's groups and keys, plus the
    anchor's residual R_0), and the same without the residual;
  * how far a freshly computed residual R_t = O_t - sparse_t (same groups and
    keys) has moved from R_0, next to how far the output itself has moved,
    ||R_t - R_0|| / ||R_0|| and ||O_t - O_0|| / ||O_0||.
From the measured times of the anchor entry point, the reuse step and dense
attention it derives, for anchor gaps g = 1..T+1, the cost of a step averaged over
one gap, (t_anchor + (g - 1) t_reuse) / g, as an effective density (that cost
over t_dense), and the overhead in density points, (effective density - density)
* 100.  The warm-up sweep applies the same costs to a whole trajectory of S
steps (S = 50 by default) that starts with W dense warm-up steps and then runs
an anchor every g steps: speed-up against S dense steps and the overhead of the
sparse steps in density points, ((cost / t_dense) - W - (S - W) * density) /
(S - W) * 100, the figure the trajectory harness reports.

Usage: python -m sparse_attention_diffusion_amd.drift [--workload NAME] [--density RHO]
       [--steps T] [--drift SIGMA] [--heads H]
"""
from __future__ import annotations

import argparse
import json
import sys


def _rel(a, b):
    """||a - b|| / ||b|| over the whole tensor (Frobenius), in fp32."""
    a, b = a.float(), b.float()
    return ((a - b).norm() / b.norm()).item()


def _mean_max(a, b):
    d = (a.float() - b.float()).abs()
    return round(d.mean().item(), 6), round(d.max().item(), 5)


WARMUPS = (0, 1, 2, 5, 10, 15)
GAPS = (1, 2, 3, 5, 8, 10, 15, 20, 25)


def schedule_cost(t_dense, t_anchor, t_reuse, total_steps, warmup, gap, density):
    """Attention cost of a trajectory: `warmup` dense steps, then an anchor every
    `gap` steps and reuse steps in between.  Returns (speed-up against all-dense,
    overhead of the sparse steps in density points)."""
    sparse = total_steps - warmup
    anchors = -(-sparse // gap) if sparse > 0 else 0
    cost = warmup * t_dense + anchors * t_anchor + (sparse - anchors) * t_reuse
    speedup = total_steps * t_dense / cost
    overhead = ((cost / t_dense - warmup - sparse * density) / sparse * 100.0) if sparse > 0 else float("nan")
    return speedup, overhead


def run(workload="hunyuan_trajectory", density=0.15, steps=25, drift=None, heads=None, reps=3, device="cuda:0",
        capture=None, total_steps=50):
    """capture: optional dict that receives the anchor's device tensors (perm, idx,
    resid, o_dense) for checks against the oracle."""
    import dataclasses

    import torch

    import sparse_attention_diffusion_amd as mcs
    from sparse_attention_diffusion_amd import workloads as W

    wl = W.WORKLOADS[workload]
    if drift is not None:
        wl = dataclasses.replace(wl, drift_sigma=drift)
    if heads is not None:
        wl = dataclasses.replace(wl, heads=heads)
    dev = torch.device(device)
    kk = wl.topk(density)
    q, k, v = W.make_qkv_torch(wl, dev)
    anchor = mcs.mcs_anchor(q, k, v, kk)
    perm, idx, r0, o0 = anchor["perm"], anchor["idx"], anchor["resid"], anchor["o_dense"]
    if capture is not None:
        capture.update(perm=perm, idx=idx, resid=r0, o_dense=o0)

    def timed(fn):
        fn()
        torch.cuda.synchronize()
        ts = []
        for _ in range(reps):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            fn()
            b.record()
            b.synchronize()
            ts.append(a.elapsed_time(b))
        return sorted(ts)[len(ts) // 2]

    ws = torch.empty(mcs.mcs_workspace_bytes(mcs.make_dims(q, topk=kk), mcs.MCS_OP_ANCHOR), dtype=torch.uint8,
                     device=dev)
    out_buf = {key: torch.empty_like(val) if val is not None else None for key, val in anchor.items()}
    o_buf = torch.empty_like(q)
    t_anchor = timed(lambda: mcs.mcs_anchor(q, k, v, kk, ws=ws, out=out_buf))
    t_reuse = timed(lambda: mcs.mcs_reuse(q, k, v, perm, idx, r0, kk, o=o_buf))
    t_dense = timed(lambda: mcs.mcs_dense_attn(q, k, v, o=o_buf))
    del out_buf, ws

    res = {"workload": wl.name, "tokens": wl.n, "heads": wl.heads, "density": density, "topk": kk,
           "drift_sigma": wl.drift_sigma, "ms": {"anchor": round(t_anchor, 3), "reuse": round(t_reuse, 3),
                                                 "dense": round(t_dense, 3)},
           "steps": []}
    for t in range(1, steps + 1):
        qt, kt, vt = W.make_qkv_torch(wl, dev, step=t)
        o_t, _ = mcs.mcs_dense_attn(qt, kt, vt)
        sp = mcs.mcs_sparse_attn(qt, kt, vt, perm, idx, kk)
        reuse = mcs.mcs_reuse(qt, kt, vt, perm, idx, r0, kk)
        r_t = o_t.float() - sp.float()
        e_r, m_r = _mean_max(reuse, o_t)
        e_s, m_s = _mean_max(sp, o_t)
        res["steps"].append({"step": t, "reuse_mean_abs": e_r, "reuse_max_abs": m_r,
                             "no_residual_mean_abs": e_s, "no_residual_max_abs": m_s,
                             "resid_change_rel": round(_rel(r_t, r0), 5), "output_change_rel": round(_rel(o_t, o0), 5)})
        del qt, kt, vt, o_t, sp, reuse, r_t
    res["gap"] = []
    for g in range(1, steps + 2):
        per_step = (t_anchor + (g - 1) * t_reuse) / g
        eff = per_step / t_dense
        res["gap"].append({"gap": g, "effective_density": round(eff, 4), "overhead_points": round((eff - density) * 100, 2),
                           "speedup_vs_dense": round(1.0 / eff, 3)})
    res["warmup_sweep"] = []
    for w in WARMUPS:
        for g in GAPS:
            sp_, ov = schedule_cost(t_dense, t_anchor, t_reuse, total_steps, w, g, density)
            res["warmup_sweep"].append({"steps": total_steps, "warmup": w, "gap": g, "speedup_vs_dense": round(sp_, 3),
                                        "overhead_points": round(ov, 2)})
    torch.cuda.synchronize()
    return res


def main(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("--workload", default="hunyuan_trajectory")
    ap.add_argument("--density", type=float, default=0.15)
    ap.add_argument("--steps", type=int, default=25)
    ap.add_argument("--drift", type=float, default=None)
    ap.add_argument("--heads", type=int, default=None)
    args = ap.parse_args(argv)
    res = run(args.workload, args.density, args.steps, args.drift, args.heads)
    print(json.dumps(res))
    ms = res["ms"]
    print(f"[drift] {res['workload']}: anchor {ms['anchor']:.1f} ms, reuse {ms['reuse']:.1f} ms, dense {ms['dense']:.1f} ms",
          file=sys.stderr)
    for s in res["steps"]:
        if s["step"] in (1, 4, 9, 14, 19, 24) or s["step"] == len(res["steps"]):
            g = res["gap"][s["step"]]
            print(f"[drift] step {s['step']:2d}: reuse mean-abs {s['reuse_mean_abs']:.2e} (no residual "
                  f"{s['no_residual_mean_abs']:.2e}); residual moved {s['resid_change_rel']:.3f}, output "
                  f"{s['output_change_rel']:.3f}; gap {g['gap']}: {g['overhead_points']:.1f} density points, "
                  f"{g['speedup_vs_dense']:.2f}x dense", file=sys.stderr)
    for row in res["warmup_sweep"]:
        if row["gap"] in (5, 10, 25):
            print(f"[drift] {row['steps']} steps, warm-up {row['warmup']:2d}, gap {row['gap']:2d}: "
                  f"{row['speedup_vs_dense']:.2f}x dense, {row['overhead_points']:.1f} density points", file=sys.stderr)


if __name__ == "__main__":
    main()
