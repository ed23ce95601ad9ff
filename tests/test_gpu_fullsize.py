"""Parity at the benchmark shape (75,600 tokens, 40 heads, D = 128, bf16,
density 0.2), in the launch configuration bench.py times, on sampled groups that
the fp64 oracle computes one by one."""
import numpy as np
import pytest
import torch

import sparse_attention_diffusion_amd as mcs
from oracle import ref
from sparse_attention_diffusion_amd import workloads as W
from tests.gpu_util import assert_close, check_index_row, host

pytestmark = pytest.mark.gpu


def test_wan14b_720p_sampled_parity():
    wl = W.WORKLOADS["wan14b_720p"]
    dev = torch.device("cuda:0")
    kk = wl.topk(0.2)
    q, k, v = W.make_qkv_torch(wl, dev)
    out = mcs.mcs_anchor(q, k, v, kk, heads_per_pass=8)
    o_sp = mcs.mcs_sparse_attn(q, k, v, out["perm"], out["idx"], kk)
    torch.cuda.synchronize()
    s = 1.0 / np.sqrt(wl.head_dim)
    rng = np.random.default_rng(0)
    for h in (0, 27):
        qh, khh, vh = (host(t[h]) for t in (q, k, v))
        perm = host(out["perm"][h])
        idx = host(out["idx"][h])
        assert sorted(perm.tolist()) == list(range(wl.n))
        groups = sorted(set(rng.choice(wl.groups, 3, replace=False).tolist()) | {wl.groups - 1})
        for g in groups:
            mem = perm[g * 64:(g + 1) * 64]
            lse = np.zeros(wl.n)
            lse[mem] = ref.row_lse(qh, khh, s, rows=mem)
            mass = ref.group_mass(qh, khh, lse, perm, 64, s, groups=[g])[0]
            check_index_row(idx[g], mass, kk, wl.n)
            want_s = ref.sparse_attention_group(qh, khh, vh, mem, idx[g][:kk].astype(np.int64), s)
            assert_close(host(o_sp[h])[mem], want_s, what=f"sparse h{h} g{g}")
            want_d = ref.dense_attention(qh, khh, vh, s, rows=mem)
            assert_close(host(out["o_dense"][h])[mem], want_d, what=f"dense h{h} g{g}")
            assert_close(host(out["resid"][h])[mem], want_d - want_s, what=f"resid h{h} g{g}")
    # grouping of two full heads, node by node
    for h in (5, 33):
        rep = ref.pddp_verify(host(q[h]), host(out["perm"][h]), 64)
        print(f"pddp verify head {h}: {rep}")
        assert rep["bad"] == 0


def test_hunyuan13b_720p_sampled_parity():
    # 118,800 tokens, 24 heads, density 0.15: grouping, selection and sparse
    # attention of the anchor, checked on sampled groups and two whole heads.
    wl = W.WORKLOADS["hunyuan13b_720p"]
    dev = torch.device("cuda:0")
    kk = wl.topk(0.15)
    q, k, v = W.make_qkv_torch(wl, dev)
    out = mcs.mcs_anchor(q, k, v, kk, heads_per_pass=8)
    torch.cuda.synchronize()
    s = 1.0 / np.sqrt(wl.head_dim)
    rng = np.random.default_rng(1)
    h = 17
    qh, khh, vh = (host(t[h]) for t in (q, k, v))
    perm = host(out["perm"][h])
    idx = host(out["idx"][h])
    assert sorted(perm.tolist()) == list(range(wl.n))
    for g in sorted(set(rng.choice(wl.groups, 2, replace=False).tolist()) | {wl.groups - 1}):
        mem = perm[g * 64:(g + 1) * 64]
        lse = np.zeros(wl.n)
        lse[mem] = ref.row_lse(qh, khh, s, rows=mem)
        mass = ref.group_mass(qh, khh, lse, perm, 64, s, groups=[g])[0]
        check_index_row(idx[g], mass, kk, wl.n)
        want_d = ref.dense_attention(qh, khh, vh, s, rows=mem)
        want_s = ref.sparse_attention_group(qh, khh, vh, mem, idx[g][:kk].astype(np.int64), s)
        assert_close(host(out["o_dense"][h])[mem], want_d, what=f"dense g{g}")
        assert_close(host(out["resid"][h])[mem], want_d - want_s, what=f"resid g{g}")
    for hv in (h, 3):
        rep = ref.pddp_verify(host(q[hv]), host(out["perm"][hv]), 64)
        print(f"pddp verify head {hv}: {rep}")
        assert rep["bad"] == 0
