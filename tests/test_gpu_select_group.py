"""GPU parity of PDDP grouping (node-local fp64 verifier) and of the two-pass
top-K selection (index sets against the oracle's fp64 masses on the same perm)."""
import numpy as np
import pytest
import torch

import sparse_attention_diffusion_amd as mcs
from oracle import ref
from sparse_attention_diffusion_amd import workloads as W
from tests.gpu_util import assert_close, check_index_row, check_index_row_window, dev, host, to_dev

pytestmark = pytest.mark.gpu


def _grid_qk(grid, heads, d, dtype, seed):
    wl = W.Workload("t", grid, heads, d, dtype, 64, (0.2,), seed, 0.0, 0)
    return W.make_qkv(wl)


def _group_sizes_ok(perm, n):
    assert sorted(perm.tolist()) == list(range(n))


@pytest.mark.parametrize("grid,heads,d,dtype", [((8, 8, 16), 1, 64, "f32"), ((5, 9, 13), 3, 128, "bf16"),
                                                  ((3, 7, 11), 2, 64, "bf16"), ((4, 16, 20), 2, 128, "f32"),
                                                  # several statistics blocks per node at the top levels
                                                  ((16, 16, 33), 1, 128, "bf16"), ((12, 16, 25), 1, 64, "bf16")])
def test_pddp_passes_node_local_verifier(grid, heads, d, dtype):
    q, _, _ = _grid_qk(grid, heads, d, dtype, seed=1)
    n = q.shape[1]
    perm = host(mcs.mcs_group(to_dev(q, dtype)))
    torch.cuda.synchronize()
    for h in range(heads):
        _group_sizes_ok(perm[h], n)
        rep = ref.pddp_verify(q[h], perm[h], 64)
        assert rep["bad"] == 0, rep
        print(f"head {h}: {rep}")


def _tree_differences_explained(q, gpu, orc, c):
    """Walk the split tree root first.  Where a node holds the same members on both
    sides, its split must agree except for members the verifier records as
    near-ties at that node; only below such a node may member sets differ (those
    subtrees are checked node by node by the verifier alone).  Returns the number of
    nodes whose split differs."""
    rep = ref.pddp_verify(q, gpu, c)
    assert rep["bad"] == 0, rep
    ties = {}
    for s, m, t in rep["ties"]:
        ties.setdefault((s, m), set()).add(t)
    n = len(gpu)
    may_differ = set()
    split_diffs = 0
    stack = [(0, n)]
    while stack:
        s, m = stack.pop()
        same = set(gpu[s:s + m].tolist()) == set(orc[s:s + m].tolist())
        assert same or (s, m) in may_differ, f"node ({s}, {m}) differs with no near-tie above it"
        if m <= c:
            continue
        cut = ref.split_rank(m, c)
        kids = [(s, cut), (s + cut, m - cut)]
        if not same:
            may_differ.update(kids)
        else:
            diff = set(gpu[s:s + cut].tolist()) ^ set(orc[s:s + cut].tolist())
            unexplained = diff - ties.get((s, m), set())
            assert not unexplained, f"node ({s}, {m}): members {sorted(unexplained)[:8]} split differently"
            if diff:
                split_diffs += 1
                may_differ.update(kids)
        stack.extend(kids)
    return split_diffs


def test_tiny_full_pipeline_against_independent_oracle_run():
    # The 1,024-token workload end to end against the oracle's own run of every
    # stage (c1 grouping ... c8 reuse).  Grouping: every group the GPU forms differs
    # from the oracle's only below a recorded near-tie.  Then selection, dense and
    # sparse attention, residual and reuse run on the oracle's own perm (supplied
    # inputs), so every later stage is compared with the oracle's full run.
    wl = W.WORKLOADS["tiny"]
    q, k, v = W.make_qkv(wl)
    q1, k1, v1 = W.make_qkv(wl, step=1)
    kk = wl.topk(0.2)
    s = 1.0 / np.sqrt(wl.head_dim)
    full = ref.anchor(q[0], k[0], v[0], 64, kk, s)
    gpu_perm = host(mcs.mcs_group(to_dev(q, "f32")))[0]
    torch.cuda.synchronize()
    diffs = _tree_differences_explained(q[0], gpu_perm, full["perm"], 64)
    same = sum(sorted(gpu_perm[i:i + 64].tolist()) == sorted(full["perm"][i:i + 64].tolist())
               for i in range(0, wl.n, 64))
    print(f"tiny: {same}/16 groups identical to the oracle run; {diffs} splits differ by near-ties")

    tq, tk, tv = (to_dev(x, "f32") for x in (q, k, v))
    perm = torch.from_numpy(full["perm"].astype(np.int32))[None].to(dev())
    idx_o = np.full((1, wl.groups, mcs.kpad_for(kk)), -1, np.int32)
    idx_o[0, :, :kk] = full["idx"]
    idx_o = torch.from_numpy(idx_o).to(dev())
    idx_gpu = mcs.mcs_select(tq, tk, perm, kk)                                    # c2-c4 (pass 1 in the kernel)
    o_dense, lse = mcs.mcs_dense_attn(tq, tk, tv, want_lse=True)                  # c5 (+ c2 statistics)
    o_sparse = mcs.mcs_sparse_attn(tq, tk, tv, perm, idx_o, kk)                   # c6
    resid = mcs.mcs_residual(tq, tk, tv, perm, idx_o, kk, o_dense)                # c7
    o_reuse = mcs.mcs_reuse(to_dev(q1, "f32"), to_dev(k1, "f32"), to_dev(v1, "f32"), perm, idx_o, resid, kk)  # c8
    torch.cuda.synchronize()
    mass = ref.group_mass(q[0], k[0], full["lse"], full["perm"], 64, s)
    differing = 0
    for g in range(wl.groups):
        differing += check_index_row(host(idx_gpu)[0, g], mass[g], kk, wl.n)
    exact = sum((host(idx_gpu)[0, g, :kk] == full["idx"][g]).all() for g in range(wl.groups))
    assert_close(host(lse)[0], full["lse"], 1e-4, 1e-5, "lse")
    assert_close(host(o_dense)[0], full["o_dense"], 1e-4, 1e-5, "dense")
    assert_close(host(o_sparse)[0], full["o_sparse"], 1e-4, 1e-5, "sparse")
    assert_close(host(resid)[0], full["resid"], 1e-4, 1e-5, "residual")
    want1 = ref.reuse(q1[0], k1[0], v1[0], full["perm"], full["idx"], full["resid"], 64, s)
    mx, mn = assert_close(host(o_reuse)[0], want1, 1e-4, 1e-5, "reuse")
    print(f"tiny on the oracle's perm: {exact}/16 index rows identical ({differing} keys within the tie window); "
          f"reuse max-abs {mx:.1e}, mean-abs {mn:.1e}")


def test_pddp_identical_queries_split_by_token_id():
    q = np.tile(np.random.default_rng(0).standard_normal((1, 1, 128)), (2, 300, 1)).astype(np.float32)
    q = W.store(q, "bf16")
    perm = host(mcs.mcs_group(to_dev(q, "bf16")))
    assert (perm == np.arange(300)).all()


def test_pddp_is_deterministic_and_handles_single_group():
    q, _, _ = _grid_qk((4, 8, 8), 2, 128, "bf16", seed=3)
    a = mcs.mcs_group(to_dev(q, "bf16"))
    b = mcs.mcs_group(to_dev(q, "bf16"))
    torch.cuda.synchronize()
    assert torch.equal(a, b)
    small = to_dev(q[:, :50], "bf16")
    assert (host(mcs.mcs_group(small)) == np.arange(50)).all()


@pytest.mark.parametrize("grid,heads,d,dtype,rho", [((8, 8, 16), 1, 64, "f32", 0.2), ((5, 9, 13), 2, 128, "bf16", 0.2),
                                                      ((3, 7, 11), 2, 64, "bf16", 0.5), ((6, 10, 12), 1, 128, "bf16", 0.05)])
@pytest.mark.parametrize("pass1", ["kernel", "supplied_lse"])
def test_select_matches_oracle_on_supplied_perm(grid, heads, d, dtype, rho, pass1):
    q, k, _ = _grid_qk(grid, heads, d, dtype, seed=2)
    n = q.shape[1]
    kk = max(1, int(np.floor(rho * n + 0.5)))
    s = 1.0 / np.sqrt(d)
    r = np.random.default_rng(5)
    perm = np.stack([r.permutation(n) for _ in range(heads)]).astype(np.int32)
    lse_np = np.stack([ref.row_lse(q[h], k[h], s) for h in range(heads)])
    lse = torch.from_numpy(lse_np.astype(np.float32)).to(dev()) if pass1 == "supplied_lse" else None
    idx = host(mcs.mcs_select(to_dev(q, dtype), to_dev(k, dtype), torch.from_numpy(perm).to(dev()), kk, lse=lse,
                              heads_per_pass=1))
    torch.cuda.synchronize()
    g = -(-n // 64)
    ties = 0
    for h in range(heads):
        mass = ref.group_mass(q[h], k[h], lse_np[h], perm[h], 64, s)
        for gi in range(g):
            ties += check_index_row(idx[h, gi], mass[gi], kk, n)
    print(f"index entries differing within the tie window: {ties}")


@pytest.mark.parametrize("d", [128, 64])
@pytest.mark.parametrize("n", [1, 17, 32, 33, 100, 600])
def test_select_pass1_short_key_lists(d, n):
    # Selection with pass 1 run by the library on one to 19 32-key steps: fewer steps
    # than the pass-1 ring holds, a ragged last step, and blocks of eight groups
    # with idle waves.
    h = 2
    r = np.random.default_rng(7 * n + d)
    q = W.store(1.5 * r.standard_normal((h, n, d)), "bf16")
    k = W.store(1.5 * r.standard_normal((h, n, d)), "bf16")
    kk = max(1, n // 5)
    s = 1.0 / np.sqrt(d)
    perm = np.stack([r.permutation(n) for _ in range(h)]).astype(np.int32)
    idx = host(mcs.mcs_select(to_dev(q, "bf16"), to_dev(k, "bf16"), torch.from_numpy(perm).to(dev()), kk))
    torch.cuda.synchronize()
    for hh in range(h):
        mass = ref.group_mass(q[hh], k[hh], ref.row_lse(q[hh], k[hh], s), perm[hh], 64, s)
        for gi in range(-(-n // 64)):
            check_index_row(idx[hh, gi], mass[gi], kk, n)


def test_select_group_of_equal_logits_ties_to_lowest_ids():
    n, d = 300, 64
    q = np.zeros((1, n, d), np.float32)
    k = W.store(np.random.default_rng(1).standard_normal((1, n, d)), "f32")
    perm = np.random.default_rng(2).permutation(n).astype(np.int32)[None]
    idx = host(mcs.mcs_select(to_dev(q, "f32"), to_dev(k, "f32"), torch.from_numpy(perm).to(dev()), 37))
    assert (idx[:, :, :37] == np.arange(37)).all()
    assert (idx[:, :, 37:] == -1).all()


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("kk", [100, 3000])
def test_select_more_equal_masses_than_the_candidate_list_holds(dtype, kk):
    # Q = 0: every key of a group gets the same mass |g| / N, computed the same way,
    # so 5,000 entries share the threshold value: more than the top-K's 2,048-entry
    # candidate list.  The threshold resolves to that value and the first K ids are
    # kept, also when K itself is past the list's size.
    n, d = 5000, 128
    q = np.zeros((2, n, d), np.float32)
    k = W.store(np.random.default_rng(3).standard_normal((2, n, d)), dtype)
    perm = np.stack([np.random.default_rng(4 + h).permutation(n) for h in range(2)]).astype(np.int32)
    qd, kd = to_dev(q, dtype), to_dev(k, dtype)
    pd = torch.from_numpy(perm).to(dev())
    for idx in (mcs.mcs_select(qd, kd, pd, kk), mcs.mcs_select_noalloc(qd, kd, pd, kk)):
        idx = host(idx)
        assert (idx[:, :, :kk] == np.arange(kk)).all()
        assert (idx[:, :, kk:] == -1).all()


def _hist_bins(mass):
    # the selection histogram's bins: exponent and top six mantissa bits of the
    # fp32 mass over the 32 binades [2^-27, 2^5), values outside in the end bins
    key = np.asarray(mass, np.float32).view(np.uint32).astype(np.int64) >> 17
    return np.clip(key - (100 << 6), 0, 2047)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_select_refines_a_crowded_threshold_bin(dtype):
    # Small logits: the masses of a group lie within about 2% of each other, so
    # thousands of the 6,000 keys share the threshold's histogram bin (1/64 of a
    # binade) and the top-K narrows the threshold with passes over the row before
    # it can list the candidates.  Index sets against the oracle's masses.
    n, d, kk = 6000, 64, 1500
    r = np.random.default_rng(11)
    u = r.standard_normal(d)
    u /= np.linalg.norm(u)
    q = W.store(np.tile(0.02 * u, (1, n, 1)) + 1e-4 * r.standard_normal((1, n, d)), dtype)
    k = W.store(r.standard_normal((1, n, d)), dtype)
    perm = r.permutation(n).astype(np.int32)[None]
    s = 1.0 / np.sqrt(d)
    idx = host(mcs.mcs_select(to_dev(q, dtype), to_dev(k, dtype), torch.from_numpy(perm).to(dev()), kk))
    lse = ref.row_lse(q[0], k[0], s)
    mass = ref.group_mass(q[0], k[0], lse, perm[0], 64, s)
    bins = _hist_bins(mass[0])
    tau = np.sort(mass[0])[::-1][kk - 1]
    crowd = int((bins == _hist_bins(tau)).sum())
    ties = sum(check_index_row(idx[0, g], mass[g], kk, n) for g in range(mass.shape[0]))
    print(f"{dtype}: {crowd} of group 0's {n} masses share the threshold's bin; {ties} keys within the tie window")
    assert crowd > 2048  # the construction does crowd the bin past the candidate list


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_select_threshold_in_the_top_end_bin(dtype):
    # One key takes nearly all of every query's weight, so its group mass is close
    # to 64: above the histogram's window, where every mass of 32 or more shares the
    # last bin.  With K = 1 the threshold lies in that bin and the top-K narrows it
    # from the top value bits with passes over the row.
    n, d = 3000, 64
    r = np.random.default_rng(21)
    u = r.standard_normal(d)
    u /= np.linalg.norm(u)
    q = W.store((np.tile(4.0 * u, (n, 1)) + 0.05 * r.standard_normal((n, d)))[None], dtype)
    k = 0.3 * r.standard_normal((n, d))
    k[0] = 100.0 * u
    k = W.store(k[None], dtype)
    perm = r.permutation(n).astype(np.int32)[None]
    s = 1.0 / np.sqrt(d)
    idx = host(mcs.mcs_select(to_dev(q, dtype), to_dev(k, dtype), torch.from_numpy(perm).to(dev()), 1))
    lse = ref.row_lse(q[0], k[0], s)
    mass = ref.group_mass(q[0], k[0], lse, perm[0], 64, s)
    assert (_hist_bins(mass.max(axis=1)) == 2047).all()  # every group's threshold is in the last bin
    for g in range(mass.shape[0]):
        check_index_row(idx[0, g], mass[g], 1, n)
    assert (idx[0, :, 0] == 0).all()


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_select_threshold_in_the_bottom_end_bin(dtype):
    # The first 100 keys take nearly all of the weight; every other key's group mass
    # is about 8e-14, below the histogram's window (2^-27), where those masses share
    # the first bin.  With K = 500 the threshold lies among them and the top-K
    # narrows it from the top value bits.  The small masses are exp() of logits about
    # 30 below each row's largest, so fp32 rounding of the row offsets moves them by
    # a few 1e-6 relative: ties within 1e-4 of the threshold are accepted.
    n, d, kk = 3000, 64, 500
    r = np.random.default_rng(22)
    u = r.standard_normal(d)
    u /= np.linalg.norm(u)
    q = W.store((np.tile(4.0 * u, (n, 1)) + 0.05 * r.standard_normal((n, d)))[None], dtype)
    k = 0.5 * r.standard_normal((n, d))
    k[:100] += 60.0 * u
    k = W.store(k[None], dtype)
    perm = r.permutation(n).astype(np.int32)[None]
    s = 1.0 / np.sqrt(d)
    idx = host(mcs.mcs_select(to_dev(q, dtype), to_dev(k, dtype), torch.from_numpy(perm).to(dev()), kk))
    lse = ref.row_lse(q[0], k[0], s)
    mass = ref.group_mass(q[0], k[0], lse, perm[0], 64, s)
    taus = np.sort(mass, axis=1)[:, ::-1][:, kk - 1]
    assert (_hist_bins(taus) == 0).all()  # every group's threshold is in the first bin
    ties = sum(check_index_row_window(idx[0, g], mass[g], kk, n, 1e-4) for g in range(mass.shape[0]))
    print(f"{dtype}: thresholds {taus.min():.3e}..{taus.max():.3e}; {ties} keys within the tie window")


def test_select_full_density_keeps_everything():
    q, k, _ = _grid_qk((2, 5, 10), 1, 128, "bf16", seed=4)
    n = q.shape[1]
    perm = np.arange(n, dtype=np.int32)[None]
    idx = host(mcs.mcs_select(to_dev(q, "bf16"), to_dev(k, "bf16"), torch.from_numpy(perm).to(dev()), n))
    assert (idx[:, :, :n] == np.arange(n)).all()


@pytest.mark.parametrize("lse_given", [False, True])
def test_select_head_passes_give_the_same_lists(lse_given):
    """Heads are selected in passes of as many as the workspace holds (mass rows
    and their histograms, then the top-K of the pass).  Every pass size gives the
    same index lists, also with no host synchronisation between calls, and so
    does the entry point that allocates nothing.  The lists match the oracle."""
    wl = W.Workload("t", (5, 9, 23), 7, 128, "bf16", 64, (0.2,), 13, 0.0, 0)
    q, k, _ = W.make_qkv(wl)
    qd, kd = to_dev(q, "bf16"), to_dev(k, "bf16")
    kk = wl.topk(0.2)
    perm = mcs.mcs_group(qd)
    lse = mcs.mcs_dense_attn(qd, kd, to_dev(np.zeros_like(q), "bf16"), want_lse=True)[1] if lse_given else None
    outs = {hpp: mcs.mcs_select(qd, kd, perm, kk, lse=lse, heads_per_pass=hpp) for hpp in (1, 2, 3, 4, 6, 0)}
    again = mcs.mcs_select(qd, kd, perm, kk, lse=lse)
    noalloc = mcs.mcs_select_noalloc(qd, kd, perm, kk, lse=lse)
    torch.cuda.synchronize()
    for hpp, idx in outs.items():
        assert torch.equal(idx, outs[1]), f"heads_per_pass={hpp}"
    assert torch.equal(again, outs[1]) and torch.equal(noalloc, outs[1])
    s = 1.0 / np.sqrt(wl.head_dim)
    p, ih = host(perm), host(outs[1])
    for h in (0, wl.heads - 1):
        mass = ref.group_mass(q[h], k[h], ref.row_lse(q[h], k[h], s), p[h], 64, s)
        for g in range(wl.groups):
            check_index_row(ih[h, g], mass[g], kk, wl.n)
