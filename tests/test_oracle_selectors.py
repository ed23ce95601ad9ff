"""Pins of the oracle's matched-density selectors: vanilla block sparsity
(mean-pooled block scores), the block-mass oracle, the per-query oracle, the
captured-mass measure and the logsumexp over kept keys."""
import itertools

import numpy as np
import pytest
from scipy.special import logsumexp

from oracle import ref


def _inputs(n, d, seed, sharp=1.0):
    """Locally correlated Q/K (neighbouring ids share features) plus noise."""
    r = np.random.default_rng(seed)
    pos = np.arange(n)[:, None] / n
    w = r.normal(size=(1, d)) * 6.0
    b = r.uniform(0, 2 * np.pi, size=(1, d))
    f = np.sqrt(2) * np.cos(pos @ w + b)
    q = sharp * f + 0.5 * r.normal(size=(n, d))
    k = f + 0.5 * r.normal(size=(n, d))
    v = r.normal(size=(n, d))
    return q, k, v


def test_block_means_hand_example():
    x = np.array([[1, 2], [3, 4], [5, 6], [7, 8]], float)
    assert ref.block_means(x, 2).tolist() == [[2, 3], [6, 7]]
    with pytest.raises(ValueError):
        ref.block_means(np.zeros((5, 2)), 2)


def test_bsa_hand_example():
    # block means: q -> [1, -1], k -> [1, -3]; scores [[1, -3], [-1, 3]]
    q = np.array([[1.0], [1.0], [-1.0], [-1.0]])
    k = np.array([[0.0], [2.0], [-2.0], [-4.0]])
    assert ref.bsa_scores(q, k, 2, 1.0).tolist() == [[1.0, -3.0], [-1.0, 3.0]]
    assert ref.bsa_select(q, k, 2, 1, 1.0).tolist() == [[0, 1], [2, 3]]


@pytest.mark.parametrize("seed", [0, 1])
def test_blocks_of_one_token_reduce_to_the_per_query_oracle(seed):
    q, k, _ = _inputs(48, 8, seed)
    scale = 1 / np.sqrt(8)
    want = ref.private_select(q, k, 7, scale)
    assert np.array_equal(ref.bsa_select(q, k, 1, 7, scale), want)
    assert np.array_equal(ref.block_oracle_select(q, k, 1, 7, scale), want)


def test_block_mass_rows_sum_to_block_size():
    q, k, _ = _inputs(64, 8, 3)
    b = ref.block_mass(q, k, 8, 1 / np.sqrt(8))
    assert b.shape == (8, 8)
    assert np.allclose(b.sum(axis=1), 8.0, rtol=0, atol=1e-12)


@pytest.mark.parametrize("kb", [1, 2, 3])
def test_block_oracle_is_the_best_block_set_by_brute_force(kb):
    q, k, _ = _inputs(48, 6, 10 + kb)
    c, scale = 8, 1 / np.sqrt(6)
    b = ref.block_mass(q, k, c, scale)
    got = ref.block_oracle_select(q, k, c, kb, scale)
    for row in range(b.shape[0]):
        best = max(itertools.combinations(range(b.shape[1]), kb), key=lambda s: b[row, list(s)].sum())
        assert got[row].tolist() == ref._expand_blocks(sorted(best), c).tolist()


@pytest.mark.parametrize("seed,kb", [(0, 1), (1, 2), (2, 3)])
def test_captured_mass_rises_from_blocks_to_groups_to_queries(seed, kb):
    """Each selector maximises the captured mass over a larger family of key sets
    of the same size, so per query block: BSA <= block oracle <= shared set <=
    per-query sets (the last also per query)."""
    n, d, c = 96, 8, 16
    q, k, _ = _inputs(n, d, seed)
    scale = 1 / np.sqrt(d)
    kk = kb * c
    lse = ref.row_lse(q, k, scale)
    ident = np.arange(n)
    per_block = lambda idx: ref.captured_mass(q, k, ref.keys_per_query(ident, idx, c), scale, lse)
    m_bsa = per_block(ref.bsa_select(q, k, c, kb, scale))
    m_blk = per_block(ref.block_oracle_select(q, k, c, kb, scale, lse))
    m_shared = per_block(ref.select(q, k, ident, c, kk, scale, lse=lse))
    m_priv = ref.captured_mass(q, k, list(ref.private_select(q, k, kk, scale)), scale, lse)
    sums = [m.reshape(-1, c).sum(axis=1) for m in (m_bsa, m_blk, m_shared, m_priv)]
    eps = 1e-12
    for lo, hi in zip(sums, sums[1:]):
        assert (lo <= hi + eps).all()
    assert (m_shared <= m_priv + eps).all()
    assert (m_priv <= 1 + eps).all()
    assert sums[-1].sum() > sums[0].sum()  # the chain is not flat on local inputs


def test_full_budget_captures_everything():
    n, d, c = 64, 4, 16
    q, k, _ = _inputs(n, d, 7)
    scale = 0.5
    lse = ref.row_lse(q, k, scale)
    ident = np.arange(n)
    for idx in (ref.bsa_select(q, k, c, n // c, scale), ref.block_oracle_select(q, k, c, n // c, scale)):
        assert idx.tolist() == [list(range(n))] * (n // c)
        assert np.allclose(ref.captured_mass(q, k, ref.keys_per_query(ident, idx, c), scale, lse), 1.0)


def test_sparse_lse_against_captured_mass_and_scipy():
    n, d, c, kk = 80, 8, 16, 20
    q, k, _ = _inputs(n, d, 5)
    scale = 1 / np.sqrt(d)
    r = np.random.default_rng(4)
    perm = r.permutation(n)
    idx = np.stack([np.sort(r.choice(n, kk, replace=False)) for _ in range(n // c)])
    lse = ref.row_lse(q, k, scale)
    sl = ref.sparse_lse(q, k, perm, idx, c, scale)
    mass = ref.captured_mass(q, k, ref.keys_per_query(perm, idx, c), scale, lse)
    assert np.allclose(np.exp(sl - lse), mass, rtol=1e-12, atol=0)
    z = scale * q @ k.T
    i = int(perm[17])  # member of group 1
    assert np.isclose(sl[i], logsumexp(z[i, idx[1]]), rtol=1e-13)
    full = ref.sparse_lse(q, k, perm, np.tile(np.arange(n), (n // c, 1)), c, scale)
    assert np.allclose(full, lse, rtol=1e-13)


def test_private_attention_with_all_keys_is_dense():
    q, k, v = _inputs(40, 6, 9)
    scale = 0.4
    keys = [np.arange(40)] * 40
    assert np.allclose(ref.private_attention(q, k, v, keys, scale), ref.dense_attention(q, k, v, scale), atol=1e-12)


def test_block_mass_by_double_loop():
    from scipy.special import softmax
    q, k, _ = _inputs(24, 4, 12)
    c, scale = 6, 0.7
    p = softmax(scale * q @ k.T, axis=1)
    want = np.array([[sum(p[i, t] for i in range(b * c, b * c + c) for t in range(j * c, j * c + c))
                      for j in range(4)] for b in range(4)])
    assert np.allclose(ref.block_mass(q, k, c, scale), want, rtol=1e-12, atol=0)
