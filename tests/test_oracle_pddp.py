"""Pins of the oracle's PDDP grouping (MC-Sparse summary page, grouping paragraph).

Each test checks the oracle against something other than itself: a hand-worked
fixture, a closed form, an independent eigendecomposition-based implementation,
or an invariant fixed by the split rule.
"""
import json
import os

import numpy as np
import pytest

from oracle import ref

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def groups_of(perm, c):
    return [sorted(perm[i:i + c].tolist()) for i in range(0, len(perm), c)]


def expected_sizes(n, c):
    g = -(-n // c)
    return [c] * (g - 1) + [n - c * (g - 1)]


@pytest.mark.parametrize("n,c,d", [(64, 8, 4), (100, 8, 3), (257, 16, 5), (33, 4, 2), (7, 8, 3), (1, 4, 2)])
def test_perm_is_bijection_with_exact_group_sizes(n, c, d):
    q = np.random.default_rng(n).standard_normal((n, d))
    perm = ref.pddp_perm(q, c)
    assert sorted(perm.tolist()) == list(range(n))
    sizes = [len(g) for g in groups_of(perm, c)]
    assert sizes == expected_sizes(n, c)  # all C except a final partial group


def test_golden_one_dimensional_examples():
    with open(os.path.join(GOLDEN, "pddp_d1_example.json")) as f:
        cases = json.load(f)["cases"]
    for case in cases:
        q = np.array(case["q"])[:, None]
        c = case["group"]
        got = ref.pddp_perm(q, c)
        assert groups_of(got, c) == groups_of(np.array(case["perm"]), c)


def test_one_dimension_is_sorted_chunks():
    # D = 1: the principal direction is +1 (start vector is +1 and cov > 0), so
    # the depth-first leaves are the values in ascending order, ties by id.
    rng = np.random.default_rng(5)
    x = rng.integers(0, 40, size=200).astype(np.float64)  # many ties
    perm = ref.pddp_perm(x[:, None], 8)
    want = np.lexsort((np.arange(200), x))
    assert groups_of(perm, 8) == groups_of(want, 8)


@pytest.mark.parametrize("sign", [1.0, -1.0])
def test_collinear_points_give_consecutive_chunks(sign):
    # q = t*u + mu (+ tiny noise): every node's principal axis is +-u, so each
    # group is a run of consecutive t-ranks.  Start vector is ones/sqrt(D), so
    # the direction is the one with positive sum, which fixes the order.
    rng = np.random.default_rng(11)
    d, n, c = 6, 96, 8
    u = rng.standard_normal(d)
    u = u / np.linalg.norm(u)
    u = u if u.sum() > 0 else -u
    t = rng.permutation(n).astype(np.float64)
    q = sign * t[:, None] * u[None, :] + rng.standard_normal(d) + 1e-9 * rng.standard_normal((n, d))
    perm = ref.pddp_perm(q, c)
    ranks = np.argsort(np.argsort(sign * t))  # rank along +u
    got = [sorted(ranks[g].tolist()) for g in groups_of(perm, c)]
    assert got == [list(range(i, i + c)) for i in range(0, n, c)]


def test_identical_queries_split_by_token_id():
    # all projections are zero (|w| = 0 stops the power steps) -> ties broken by id
    q = np.tile(np.array([[0.3, -1.2, 2.0]]), (50, 1))
    perm = ref.pddp_perm(q, 4)
    assert perm.tolist() == list(range(50))


def test_two_far_clusters_separate_at_root():
    rng = np.random.default_rng(3)
    c = 8
    a = rng.standard_normal((64, 4)) + np.array([50.0, 0, 0, 0])
    b = rng.standard_normal((64, 4)) - np.array([50.0, 0, 0, 0])
    q = np.concatenate([a, b])
    ids = rng.permutation(128)
    q = q[ids]  # interleave token ids
    in_a = ids < 64
    perm = ref.pddp_perm(q, c)
    left = perm[:64]
    assert in_a[left].all() or (~in_a[left]).all()


def _eigh_pddp(q, c):
    """Independent PDDP: exact leading eigenvector (numpy.linalg.eigh) and a
    Python sort on (projection, id).  The eigenvector sign is the one with a
    non-negative component along ones, which is where power steps from the
    all-ones start converge."""
    leaves = []

    def rec(members):
        n = len(members)
        if n <= c:
            leaves.append(members)
            return
        x = q[members]
        xc = x - x.mean(axis=0)
        w, vecs = np.linalg.eigh(xc.T @ xc)
        v = vecs[:, -1]
        if v.sum() < 0:
            v = -v
        p = xc @ v
        order = sorted(range(n), key=lambda i: (p[i], members[i]))
        g = -(-n // c)
        cut = (g // 2) * c
        rec([members[i] for i in order[:cut]])
        rec([members[i] for i in order[cut:]])

    rec(list(range(q.shape[0])))
    return np.array([t for leaf in leaves for t in leaf])


def _well_separated(q, c):
    """True when every node of the oracle tree has a clear eigengap (so 32 power
    steps converge) and no projection tie at the cut."""
    perm = ref.pddp_perm(q, c)
    for s, m in ref.pddp_tree_nodes(q.shape[0], c):
        x = q[perm[s:s + m]]
        xc = x - x.mean(axis=0)
        w, vecs = np.linalg.eigh(xc.T @ xc)
        if w[-1] <= 0 or (len(w) > 1 and w[-2] / w[-1] > 0.5) or abs(vecs[:, -1].sum()) < 1e-3:
            return False
        p = np.sort(xc @ vecs[:, -1])
        cut = ref.split_rank(m, c)
        if p[cut] - p[cut - 1] < 1e-6:
            return False
    return True


def test_matches_eigh_brute_force_on_tiny_inputs():
    checked = 0
    for seed in range(400):
        rng = np.random.default_rng(seed)
        n = int(rng.integers(5, 25))
        d = int(rng.integers(1, 5))
        c = int(rng.choice([2, 4]))
        scales = np.array([8.0, 2.0, 0.5, 0.125])[:d]
        q = rng.standard_normal((n, d)) * scales
        if not _well_separated(q, c):
            continue
        got = ref.pddp_perm(q, c)
        want = _eigh_pddp(q, c)
        assert groups_of(got, c) == groups_of(want, c), seed
        checked += 1
    assert checked >= 100


def test_tree_nodes_match_emitted_groups():
    n, c = 1000, 16
    nodes = ref.pddp_tree_nodes(n, c)
    assert nodes[0] == (0, n)
    for s, m in nodes:
        assert s % c == 0  # every node starts on a group boundary
        assert m > c
    # 62 full groups and one partial: a binary tree with 63 leaves has 62 internal nodes
    assert len(nodes) == -(-n // c) - 1


def test_verifier_accepts_oracle_tree_and_rejects_a_wrong_split():
    rng = np.random.default_rng(9)
    q = rng.standard_normal((256, 8)) * np.linspace(3, 0.5, 8)
    c = 16
    perm = ref.pddp_perm(q, c)
    rep = ref.pddp_verify(q, perm, c)
    assert rep["bad"] == 0 and rep["nodes"] == 15
    # swap the queries at the two ends of the root projection: far from the cut
    p, _ = ref.node_projection(q)
    lo, hi = int(np.argmin(p)), int(np.argmax(p))
    bad = perm.copy()
    i, j = int(np.where(bad == lo)[0][0]), int(np.where(bad == hi)[0][0])
    bad[i], bad[j] = bad[j], bad[i]
    assert ref.pddp_verify(q, bad, c)["bad"] > 0
    # a non-permutation is rejected outright
    dup = perm.copy()
    dup[0] = dup[1]
    assert ref.pddp_verify(q, dup, c)["bad"] > 0


def test_power_direction_matches_eigh_on_a_gapped_matrix():
    rng = np.random.default_rng(2)
    a = rng.standard_normal((20, 5)) * np.array([5, 2, 1, 0.5, 0.1])
    cov = a.T @ a
    v = ref.principal_direction(cov)
    w, vecs = np.linalg.eigh(cov)
    top = vecs[:, -1] * np.sign(vecs[:, -1].sum())
    assert np.allclose(v, top, atol=1e-9)
    assert np.allclose(ref.principal_direction(np.zeros((5, 5))), np.full(5, 1 / np.sqrt(5)))


# Hand-worked tie window of the node-local verifier.  One dimension, C = 2, eight
# tokens.  With D = 1 the covariance is a positive scalar, so the direction stays
# +1 and a node's projections are its values minus the node mean.  Sorted root
# order: t3 (0), t6 (1), t1 (3), t5 (7.5 - e) | t2 (7.5 + e), t0 (10), t4 (14),
# t7 (20); the cut point p* is the midpoint of t5 and t2, i.e. 7.5 before
# centring, and the window is 1e-5 * (20 - 0) = 2e-4.  Correct perm, depth first:
# [t3 t6 | t1 t5 | t2 t0 | t4 t7].
def _verify_case(e, top=20.0):
    x = np.array([10.0, 3.0, 7.5 + e, 0.0, 14.0, 7.5 - e, 1.0, top])
    return x[:, None]


@pytest.mark.parametrize("e,top,perm,want", [
    # correct grouping: nothing to report
    (5e-5, 20.0, [3, 6, 1, 5, 2, 0, 4, 7], dict(nodes=3, mismatched=0, tolerated=0, bad=0)),
    # t5 and t2 swapped across the root cut, both e = 5e-5 from p*: inside the window
    # (the children {t3 t6 t1 t2} and {t5 t0 t4 t7} then split correctly)
    (5e-5, 20.0, [3, 6, 1, 2, 5, 0, 4, 7], dict(nodes=3, mismatched=2, tolerated=2, bad=0)),
    # the same swap with e = 3e-4: outside the 2e-4 window
    (3e-4, 20.0, [3, 6, 1, 2, 5, 0, 4, 7], dict(nodes=3, mismatched=2, tolerated=0, bad=2)),
    # ... but inside once the node's range grows tenfold (window 2e-3): the window is
    # relative to the node's projection range
    (3e-4, 200.0, [3, 6, 1, 2, 5, 0, 4, 7], dict(nodes=3, mismatched=2, tolerated=2, bad=0)),
    # t5 (e from p*) swapped with t0 (2.5 from p*): one tolerated, one bad
    (5e-5, 20.0, [3, 6, 1, 0, 5, 2, 4, 7], dict(nodes=3, mismatched=2, tolerated=1, bad=1)),
    # root right, left child wrong: t1 (3) and t6 (1) sit 1 from that node's cut point 2
    (5e-5, 20.0, [3, 1, 6, 5, 2, 0, 4, 7], dict(nodes=3, mismatched=2, tolerated=0, bad=2)),
])
def test_verifier_tie_window_hand_worked(e, top, perm, want):
    rep = ref.pddp_verify(_verify_case(e, top), np.array(perm), 2)
    assert {k: rep[k] for k in want} == want, rep
    assert len(rep["ties"]) == rep["tolerated"]
    assert all(s == 0 and m == 8 for s, m, _ in rep["ties"])  # every tie here is at the root


def test_verifier_reports_which_tokens_are_near_ties():
    rep = ref.pddp_verify(_verify_case(5e-5), np.array([3, 6, 1, 0, 5, 2, 4, 7]), 2)
    assert rep["ties"] == [(0, 8, 5)]  # t5 tolerated; t0, 2.5 from the cut, is not
    # a near-tie at a child node (slot range 4..7): with t4 moved from 14 to
    # 10 + 4e-5, the right child {t2 t0 t4 t7} = {7.5+e, 10, 10+4e-5, 20} cuts
    # between t0 and t4, each 2e-5 from the midpoint, inside the window
    # 1e-5 * (20 - 7.5 - e); t0 and t4 are swapped there
    x = _verify_case(5e-5)
    x[4, 0] = 10.0 + 4e-5
    rep = ref.pddp_verify(x, np.array([3, 6, 1, 5, 2, 4, 0, 7]), 2)
    assert rep["bad"] == 0 and sorted(rep["ties"]) == [(4, 4, 0), (4, 4, 4)], rep
