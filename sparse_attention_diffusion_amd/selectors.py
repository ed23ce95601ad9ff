"""Matched-density comparison of selectors on synthetic DiT-like attention
(MC-Sparse summary page, block-sparsity and gap paragraphs: at the same
density, block selection from mean-pooled scores loses mass that a token-level
selection keeps, and the tail that any selection drops is what the residual
stores).

Both selectors keep the same number of keys, K = density * N (a whole number of
64-token blocks), and run through the same gather kernel:
  * ours:  PDDP groups of 64 similar queries, exact per-group top-K by summed
           softmax mass (the anchor step);
  * block: vanilla block sparsity, query blocks of 64 consecutive tokens scoring
           key blocks by mean-pooled vectors (mcs_block_select);
  * per-query oracle, on a sample: one query per PDDP group (its group's first
           slot) keeps its own top K keys, by running the same exact selection
           on a perm that holds only that query in each group (empty slots
           carry no weight).  All three selectors are also reported on this
           sample, for a like-for-like comparison.
Reported per selector, over all heads and queries:
  * captured mass: the share of each query's dense softmax weight on its kept
    keys, exp(lse_sparse - lse_dense) (mcs_sparse_lse, mcs_dense_attn);
  * output error against dense attention at the anchor step (no residual), and
    at drifted reuse steps with and without the anchor's residual
    (dense - sparse at the anchor, added unscaled).

Inputs come from the workload generator (random Fourier features of the latent
grid plus noise, V ~ N(0, 1), per-step random-walk drift).  The grid must hold a
multiple of 64 tokens; the default 20x45x80 (72,000 tokens) is the 720p latent
grid with 20 frames.  The numbers describe these synthetic inputs only: the
pages' gap figures come from trained models.

Usage: python -m sparse_attention_diffusion_amd.selectors [--grid T Y X] [--heads H]
       [--density RHO] [--steps S] [--drift SIGMA]
"""
from __future__ import annotations

import argparse
import json
import sys


def _errors(o, ref):
    d = (o.float() - ref.float()).abs()
    return {"max_abs": round(d.max().item(), 5), "mean_abs": round(d.mean().item(), 6)}


def run(grid=(20, 45, 80), heads=8, density=0.2, steps=4, drift=0.02, seed=5, device="cuda:0"):
    import torch

    import sparse_attention_diffusion_amd as mcs
    from sparse_attention_diffusion_amd import workloads as W

    wl = W.Workload("selector_study", tuple(grid), heads, 128, "bf16", 64, (density,), seed, drift, steps)
    n = wl.n
    if n % 64:
        raise ValueError(f"the grid holds {n} tokens, not a multiple of 64")
    kk = wl.topk(density)
    kk = max(64, (kk // 64) * 64)  # whole blocks, so that both selectors keep exactly K keys
    dev = torch.device(device)
    q, k, v = W.make_qkv_torch(wl, dev)
    ident = torch.arange(n, dtype=torch.int32, device=dev).repeat(heads, 1).contiguous()

    anchor = mcs.mcs_anchor(q, k, v, kk, want_lse=True)
    o_dense, lse_dense = anchor["o_dense"], anchor["lse"]
    idx_block = mcs.mcs_block_select(q, k, kk)
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    mcs.mcs_block_select(q, k, kk, idx=idx_block)
    b.record()
    b.synchronize()
    sel = {"ours": (anchor["perm"], anchor["idx"]), "block": (ident, idx_block)}
    out = {"grid": list(grid), "tokens": n, "heads": heads, "head_dim": 128, "density": kk / n, "topk": kk,
           "drift_sigma": drift, "block_select_ms": round(a.elapsed_time(b), 3), "selectors": {}}
    resid = {}
    for name, (perm, idx) in sel.items():
        o_s = mcs.mcs_sparse_attn(q, k, v, perm, idx, kk)
        lse_s = mcs.mcs_sparse_lse(q, k, perm, idx, kk)
        cap = torch.exp(lse_s - lse_dense)
        resid[name] = mcs.mcs_residual(q, k, v, perm, idx, kk, o_dense)
        out["selectors"][name] = {"captured_mass_mean": round(cap.mean().item(), 5),
                                  "captured_mass_p10": round(torch.quantile(cap.flatten()[::97].float(), 0.1).item(), 5),
                                  "anchor_error": _errors(o_s, o_dense), "reuse": []}
    # the per-query oracle on one query per group, and the other selectors on the same queries
    sample_perm = torch.full_like(anchor["perm"], -1)
    sample_perm[:, ::64] = anchor["perm"][:, ::64]
    tok = anchor["perm"][:, ::64].long()
    idx_pq = mcs.mcs_select(q, k, sample_perm, kk, lse=lse_dense)
    sampled = {"queries_per_head": int(tok.shape[1])}
    runs = {"per_query": (sample_perm, idx_pq), "ours": sel["ours"], "block": sel["block"]}
    dense_rows = torch.gather(o_dense, 1, tok[..., None].expand(-1, -1, o_dense.shape[2]))
    for name, (perm, idx) in runs.items():
        lse_s = mcs.mcs_sparse_lse(q, k, perm, idx, kk)
        o_s = mcs.mcs_sparse_attn(q, k, v, perm, idx, kk)
        cap = torch.exp(torch.gather(lse_s, 1, tok) - torch.gather(lse_dense, 1, tok))
        rows = torch.gather(o_s, 1, tok[..., None].expand(-1, -1, o_s.shape[2]))
        sampled[name] = {"captured_mass_mean": round(cap.mean().item(), 5), "anchor_error": _errors(rows, dense_rows)}
    out["sampled_queries"] = sampled
    for t in range(1, steps + 1):
        qt, kt, vt = W.make_qkv_torch(wl, dev, step=t)
        o_t, _ = mcs.mcs_dense_attn(qt, kt, vt)
        for name, (perm, idx) in sel.items():
            plain = mcs.mcs_sparse_attn(qt, kt, vt, perm, idx, kk)
            with_r = mcs.mcs_reuse(qt, kt, vt, perm, idx, resid[name], kk)
            out["selectors"][name]["reuse"].append({"step": t, "no_residual": _errors(plain, o_t),
                                                    "residual": _errors(with_r, o_t)})
        del qt, kt, vt, o_t
    torch.cuda.synchronize()
    return out


def main(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("--grid", type=int, nargs=3, default=(20, 45, 80))
    ap.add_argument("--heads", type=int, default=8)
    ap.add_argument("--density", type=float, default=0.2)
    ap.add_argument("--steps", type=int, default=4)
    ap.add_argument("--drift", type=float, default=0.02)
    args = ap.parse_args(argv)
    res = run(tuple(args.grid), args.heads, args.density, args.steps, args.drift)
    print(json.dumps(res))
    print(f"[selectors] block selection of {res['tokens']} tokens x {res['heads']} heads: {res['block_select_ms']:.2f} ms",
          file=sys.stderr)
    sq = res["sampled_queries"]
    print(f"[selectors] one query per group ({sq['queries_per_head']} per head): captured mass per-query oracle "
          f"{sq['per_query']['captured_mass_mean']:.4f}, ours {sq['ours']['captured_mass_mean']:.4f}, block "
          f"{sq['block']['captured_mass_mean']:.4f}; mean-abs error {sq['per_query']['anchor_error']['mean_abs']:.3e} / "
          f"{sq['ours']['anchor_error']['mean_abs']:.3e} / {sq['block']['anchor_error']['mean_abs']:.3e}", file=sys.stderr)
    for name, r in res["selectors"].items():
        last = r["reuse"][-1] if r["reuse"] else None
        print(f"[selectors] {name:5s}: captured mass {r['captured_mass_mean']:.4f} (p10 {r['captured_mass_p10']:.4f}); "
              f"anchor mean-abs error {r['anchor_error']['mean_abs']:.2e}"
              + (f"; step {last['step']} mean-abs error {last['no_residual']['mean_abs']:.2e} without residual, "
                 f"{last['residual']['mean_abs']:.2e} with" if last else ""), file=sys.stderr)


if __name__ == "__main__":
    main()
