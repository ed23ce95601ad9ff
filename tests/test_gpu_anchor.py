"""End-to-end anchor and reuse steps on the GPU against the fp64 oracle, and the
invariants of the method: sparse + residual = dense on the anchor, zero-drift
reuse = dense, bitwise determinism."""
import numpy as np
import pytest
import torch

import sparse_attention_diffusion_amd as mcs
from oracle import ref
from sparse_attention_diffusion_amd import workloads as W
from tests.gpu_util import assert_close, bf16_half_ulp, check_index_row, dev, host, to_dev

pytestmark = pytest.mark.gpu


def _run_anchor(wl, step=0):
    q, k, v = W.make_qkv(wl, step=step)
    qd, kd, vd = (to_dev(x, wl.dtype) for x in (q, k, v))
    out = mcs.mcs_anchor(qd, kd, vd, wl.topk(wl.densities[0]), want_lse=True)
    torch.cuda.synchronize()
    return (q, k, v), (qd, kd, vd), out


def test_tiny_anchor_and_reuse_against_full_oracle():
    wl = W.WORKLOADS["tiny"]
    (q, k, v), (qd, kd, vd), out = _run_anchor(wl)
    s = 1.0 / np.sqrt(wl.head_dim)
    kk = wl.topk(0.2)
    perm = host(out["perm"])[0]
    idx = host(out["idx"])[0]
    # grouping: node-local check of the GPU tree
    assert ref.pddp_verify(q[0], perm, 64)["bad"] == 0
    # selection on the GPU's groups
    lse = ref.row_lse(q[0], k[0], s)
    mass = ref.group_mass(q[0], k[0], lse, perm, 64, s)
    for g in range(wl.groups):
        check_index_row(idx[g], mass[g], kk, wl.n)
    # dense output, logsumexp, residual on the GPU's groups and indices
    o_dense = ref.dense_attention(q[0], k[0], v[0], s)
    mx, mn = assert_close(host(out["o_dense"])[0], o_dense, 1e-4, 1e-5, "o_dense")
    assert_close(host(out["lse"])[0], lse, 1e-4, 1e-5, "lse")
    o_sparse = ref.sparse_attention(q[0], k[0], v[0], perm, idx[:, :kk], 64, s)
    mx_r, mn_r = assert_close(host(out["resid"])[0], o_dense - o_sparse, 1e-4, 1e-5, "resid")
    # reuse step on drifted inputs
    q1, k1, v1 = W.make_qkv(wl, step=1)
    o1 = mcs.mcs_reuse(to_dev(q1, "f32"), to_dev(k1, "f32"), to_dev(v1, "f32"), out["perm"], out["idx"],
                       out["resid"], kk)
    torch.cuda.synchronize()
    want1 = ref.reuse(q1[0], k1[0], v1[0], perm, idx[:, :kk], host(out["resid"])[0], 64, s)
    mx1, mn1 = assert_close(host(o1)[0], want1, 1e-4, 1e-5, "reuse")
    dense1 = ref.dense_attention(q1[0], k1[0], v1[0], s)
    print(f"tiny fp32: o_dense max {mx:.1e}/mean {mn:.1e}; resid max {mx_r:.1e}; reuse max {mx1:.1e}/mean {mn1:.1e}; "
          f"reuse vs dense mean-abs {np.abs(host(o1)[0] - dense1).mean():.2e}")


def test_anchor_invariants_bf16():
    wl = W.Workload("t", (6, 10, 17), 3, 128, "bf16", 64, (0.2,), 7, 0.0, 0)
    (q, k, v), (qd, kd, vd), out = _run_anchor(wl)
    kk = wl.topk(0.2)
    # sparse + residual = dense (the residual is stored in bf16)
    o_s = mcs.mcs_sparse_attn(qd, kd, vd, out["perm"], out["idx"], kk)
    torch.cuda.synchronize()
    # R = bf16(O_dense - O_S) and O_S is rounded to bf16 too, so the sum may differ
    # from O_dense by at most the two roundings (plus fp32 noise).
    o_s_h, r_h, od_h = host(o_s), host(out["resid"]), host(out["o_dense"])
    err = np.abs(o_s_h + r_h - od_h)
    bound = bf16_half_ulp(o_s_h) + bf16_half_ulp(r_h) + 1e-5
    assert (err <= bound).all(), f"O_S + R vs O_dense: worst excess {(err - bound).max():.3e}"
    # zero drift: reuse reproduces the anchor's dense output up to the same roundings
    o_r = mcs.mcs_reuse(qd, kd, vd, out["perm"], out["idx"], out["resid"], kk)
    torch.cuda.synchronize()
    o_r_h = host(o_r)
    err = np.abs(o_r_h - od_h)
    bound = bf16_half_ulp(o_r_h) + bf16_half_ulp(r_h) + 1e-5
    assert (err <= bound).all(), f"zero-drift reuse vs dense: worst excess {(err - bound).max():.3e}"
    # determinism of the whole anchor
    again = mcs.mcs_anchor(qd, kd, vd, kk, want_lse=True)
    torch.cuda.synchronize()
    for key in ("perm", "idx", "resid", "o_dense", "lse"):
        assert torch.equal(out[key], again[key]), key


def test_wan13b_480p_anchor_sampled_against_oracle():
    wl = W.WORKLOADS["wan13b_480p"]
    heads = [0, 5, 11]
    q, k, v = W.make_qkv(wl, heads=heads)
    qd, kd, vd = (to_dev(x, "bf16") for x in (q, k, v))
    kk = wl.topk(0.2)
    out = mcs.mcs_anchor(qd, kd, vd, kk, heads_per_pass=1)
    torch.cuda.synchronize()
    s = 1.0 / np.sqrt(wl.head_dim)
    r = np.random.default_rng(0)
    perm_all, idx_all = host(out["perm"]), host(out["idx"])
    for hi in range(len(heads)):
        perm, idx = perm_all[hi], idx_all[hi]
        assert sorted(perm.tolist()) == list(range(wl.n))
        if hi == 0:
            rep = ref.pddp_verify(q[hi], perm, 64)
            print(f"pddp verify head {heads[hi]}: {rep}")
            assert rep["bad"] == 0
        groups = sorted(set(r.choice(wl.groups, 6, replace=False).tolist()) | {wl.groups - 1})
        rows = np.concatenate([perm[g * 64:(g + 1) * 64] for g in groups])
        lse = ref.row_lse(q[hi], k[hi], s)
        mass = ref.group_mass(q[hi], k[hi], lse, perm, 64, s, groups=groups)
        for gi, g in enumerate(groups):
            check_index_row(idx[g], mass[gi], kk, wl.n)
        o_dense = ref.dense_attention(q[hi], k[hi], v[hi], s, rows=rows)
        assert_close(host(out["o_dense"])[hi][rows], o_dense, what="o_dense sampled")
        o_sp = ref.sparse_attention(q[hi], k[hi], v[hi], perm, {g: idx[g][:kk] for g in groups}, 64, s, groups=groups)
        assert_close(host(out["resid"])[hi][rows], o_dense - o_sp[rows], what="resid sampled")


def test_anchor_with_grouping_beside_dense_equals_serial_anchor():
    """A workspace holding both the grouping and the selection regions lets the
    anchor group on a side stream while dense attention runs; one of
    max(group, select) bytes runs the steps in turn.  Both give the same bits,
    also when anchors follow each other with no host synchronisation between."""
    wl = W.Workload("t", (7, 11, 19), 5, 128, "bf16", 64, (0.2,), 11, 0.0, 0)
    q, k, v = W.make_qkv(wl)
    qd, kd, vd = (to_dev(x, wl.dtype) for x in (q, k, v))
    kk = wl.topk(0.2)
    d = mcs.make_dims(qd, topk=kk)
    n_group = mcs.mcs_workspace_bytes(d, mcs.MCS_OP_GROUP)
    n_select = mcs.mcs_workspace_bytes(d, mcs.MCS_OP_SELECT)
    n_anchor = mcs.mcs_workspace_bytes(d, mcs.MCS_OP_ANCHOR)
    assert n_anchor >= n_group + n_select
    ws_serial = torch.empty(max(n_group, n_select), dtype=torch.uint8, device=qd.device)
    ws_side = torch.empty(n_anchor, dtype=torch.uint8, device=qd.device)
    serial = mcs.mcs_anchor(qd, kd, vd, kk, want_lse=True, ws=ws_serial)
    side = [mcs.mcs_anchor(qd, kd, vd, kk, want_lse=True, ws=ws_side) for _ in range(3)]
    torch.cuda.synchronize()
    assert ref.pddp_verify(q[0], host(serial["perm"])[0], 64)["bad"] == 0
    for out in side:
        for key in ("perm", "idx", "resid", "o_dense", "lse"):
            assert torch.equal(out[key], serial[key]), key
