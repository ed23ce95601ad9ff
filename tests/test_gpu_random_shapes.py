"""Seeded random shapes through the C ABI against the fp64 oracle: token counts
from 1 to 2,500 (any remainder mod 64), K from 1 to N, head_dim 64 or 128,
fp32 or bf16, one to three heads.  Each case runs the anchor (grouping checked
node by node, selection up to mass ties, dense output and residual), the plain
and the pair-shared sparse kernels, and the logsumexp over kept keys."""
import numpy as np
import pytest
import torch

import sparse_attention_diffusion_amd as mcs
from oracle import ref
from sparse_attention_diffusion_amd import workloads as W
from tests.gpu_util import assert_close, check_index_row, host, to_dev

pytestmark = pytest.mark.gpu


def _case(seed):
    r = np.random.default_rng(1000 + seed)
    n = int(r.integers(1, 2501))
    k = int(r.integers(1, n + 1))
    d = int(r.choice([64, 128]))
    dtype = str(r.choice(["bf16", "f32"]))
    heads = int(r.integers(1, 4))
    return r, n, k, d, dtype, heads


@pytest.mark.parametrize("seed", range(48))
def test_random_shape_against_oracle(seed):
    r, n, k, d, dtype, heads = _case(seed)
    print(f"random shape seed={seed}: heads={heads} n={n} k={k} d={d} {dtype}", flush=True)
    # Q/K spread up to that of the other parity tests (logit std up to about 2).  The bf16
    # bound (2e-2 max-abs against fp64) is for attention as spread as the workloads'; with
    # near-one-hot rows |O| reaches the 4-8 binade, where bf16's half-ulp alone is 0.0156,
    # and the bf16 rounding of the probabilities adds about 2^-9 |v| on top.
    sd = 1.5 * r.uniform(0.5, 1.0)
    q = W.store(sd * r.standard_normal((heads, n, d)), dtype)
    kk = W.store(sd * r.standard_normal((heads, n, d)), dtype)
    v = W.store(r.standard_normal((heads, n, d)), dtype)
    tq, tk, tv = (to_dev(x, dtype) for x in (q, kk, v))
    out = mcs.mcs_anchor(tq, tk, tv, k, want_lse=True)
    o_sp = mcs.mcs_sparse_attn(tq, tk, tv, out["perm"], out["idx"], k)
    pidx, nc = mcs.mcs_pair_plan(out["idx"], n, k)
    o_pairs = mcs.mcs_sparse_attn_pairs(tq, tk, tv, out["perm"], pidx, nc, k)
    lse_s = mcs.mcs_sparse_lse(tq, tk, out["perm"], out["idx"], k)
    torch.cuda.synchronize()
    s = 1.0 / np.sqrt(d)
    mx, mn = (2e-2, 2e-3) if dtype == "bf16" else (1e-4, 1e-5)
    g = -(-n // 64)
    for h in range(heads):
        perm = host(out["perm"])[h]
        idx = host(out["idx"])[h]
        assert sorted(perm.tolist()) == list(range(n))
        rep = ref.pddp_verify(q[h], perm, 64)
        assert rep["bad"] == 0, rep
        lse = ref.row_lse(q[h], kk[h], s)
        assert_close(host(out["lse"])[h], lse, 2e-4, 3e-5, f"lse h{h}")
        mass = ref.group_mass(q[h], kk[h], lse, perm, 64, s)
        for gi in range(g):
            check_index_row(idx[gi], mass[gi], k, n)
        o_dense = ref.dense_attention(q[h], kk[h], v[h], s)
        o_ref = ref.sparse_attention(q[h], kk[h], v[h], perm, idx[:, :k], 64, s)
        assert_close(host(out["o_dense"])[h], o_dense, mx, mn, f"dense h{h}")
        assert_close(host(out["resid"])[h], o_dense - o_ref, mx, mn, f"residual h{h}")
        assert_close(host(o_sp)[h], o_ref, mx, mn, f"sparse h{h}")
        assert_close(host(o_pairs)[h], o_ref, mx, mn, f"pair-shared sparse h{h}")
        assert_close(host(lse_s)[h], ref.sparse_lse(q[h], kk[h], perm, idx[:, :k], 64, s), 2e-4, 3e-5,
                     f"sparse lse h{h}")
