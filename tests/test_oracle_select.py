"""Pins of the oracle's two-pass selection (MC-Sparse summary page, selection paragraph):
row logsumexp, summed group mass and the per-group top-K."""
import itertools

import numpy as np
import pytest
from scipy.special import logsumexp

from oracle import ref


def _rand(n, d, seed):
    r = np.random.default_rng(seed)
    return r.standard_normal((n, d)), r.standard_normal((n, d))


def test_lse_matches_scipy_and_normalises():
    q, k = _rand(77, 16, 0)
    s = 0.25
    lse = ref.row_lse(q, k, s)
    z = s * q @ k.T
    assert np.allclose(lse, logsumexp(z, axis=1), rtol=0, atol=1e-12)
    assert np.allclose(np.exp(z - lse[:, None]).sum(axis=1), 1.0, atol=1e-12)


def test_lse_of_zero_queries_is_log_n():
    _, k = _rand(50, 8, 1)
    lse = ref.row_lse(np.zeros((10, 8)), k, 0.3)
    assert np.allclose(lse, np.log(50.0), atol=1e-14)


def test_lse_of_large_logits_is_stable():
    q = np.full((2, 4), 100.0)
    k = np.full((3, 4), 100.0)
    lse = ref.row_lse(q, k, 1.0)  # all logits 40000
    assert np.allclose(lse, 40000.0 + np.log(3.0))


def test_group_mass_sums_to_group_size():
    q, k = _rand(70, 8, 2)
    perm = np.random.default_rng(3).permutation(70)
    lse = ref.row_lse(q, k, 0.4)
    mass = ref.group_mass(q, k, lse, perm, 16, 0.4)
    assert mass.shape == (5, 70)
    assert np.allclose(mass.sum(axis=1), [16, 16, 16, 16, 6], atol=1e-12)
    assert (mass >= 0).all()


def test_group_mass_uses_supplied_groups():
    # mass of group g equals the column sums of the softmax rows of exactly its members
    q, k = _rand(24, 4, 4)
    perm = np.random.default_rng(5).permutation(24)
    z = 0.7 * q @ k.T
    p = np.exp(z - logsumexp(z, axis=1, keepdims=True))
    mass = ref.group_mass(q, k, ref.row_lse(q, k, 0.7), perm, 8, 0.7)
    for g in range(3):
        assert np.allclose(mass[g], p[perm[8 * g:8 * g + 8]].sum(axis=0), atol=1e-12)


def test_group_of_one_selects_that_querys_largest_logits():
    q, k = _rand(40, 8, 6)
    perm = np.arange(40)
    idx = ref.select(q, k, perm, 1, 7, 0.5)
    z = q @ k.T
    for i in range(40):
        assert idx[i].tolist() == sorted(np.argsort(-z[i], kind="stable")[:7].tolist())


def test_equal_logits_tie_to_lowest_ids():
    q = np.zeros((32, 4))
    _, k = _rand(32, 4, 7)
    perm = np.random.default_rng(8).permutation(32)
    lse = ref.row_lse(q, k, 1.0)
    mass = ref.group_mass(q, k, lse, perm, 8, 1.0)
    assert np.allclose(mass, 8 / 32, atol=1e-15)
    idx = ref.select(q, k, perm, 8, 5, 1.0)
    assert (idx == np.arange(5)).all()


def _brute_topk(mass, k):
    """The unique K-subset S with (m_j, -j) > (m_i, -i) for all j in S, i not in S."""
    n = len(mass)
    found = []
    for sub in itertools.combinations(range(n), k):
        s = set(sub)
        ok = all((mass[j], -j) > (mass[i], -i) for j in s for i in range(n) if i not in s)
        if ok:
            found.append(list(sub))
    assert len(found) == 1
    return found[0]


@pytest.mark.parametrize("seed", range(30))
def test_topk_matches_subset_brute_force(seed):
    r = np.random.default_rng(seed)
    n = int(r.integers(1, 11))
    k = int(r.integers(1, n + 1))
    mass = r.integers(0, 4, size=n).astype(np.float64)  # plenty of ties
    assert ref.topk_from_mass(mass, k).tolist() == _brute_topk(mass, k)


def test_topk_of_all_keys_is_everything_sorted():
    mass = np.random.default_rng(0).random(33)
    assert ref.topk_from_mass(mass, 33).tolist() == list(range(33))
    out = ref.topk_from_mass(mass, 10)
    assert (np.diff(out) > 0).all()
