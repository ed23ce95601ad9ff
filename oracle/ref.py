"""Plain fp64 reference of each stage of the MC-Sparse hot path (one head at a time).

TEST INFRASTRUCTURE: imported only by tests, the smoke check and the benchmark's
CPU-baseline leg.  Inputs are the stored values (fp32 / bf16-exact float32)
upcast to float64; every computation below is float64 numpy.

Citations refer to the MC-Sparse summary page (agihunt.info, arXiv 2610.06801)
by paragraph, as listed in ``oracle/__init__.py``.

Conventions (readings where the page is silent):

* Logits are z_ij = scale * q_i . k_j with scale = 1/sqrt(D); Q/K are stored
  unscaled.
* perm[s] is the token held by slot s; group g is slots [g*C, min((g+1)*C, N)).
  G = ceil(N / C); when C does not divide N the last group is partial.
* idx rows list each group's kept key ids in ascending order.
"""
from __future__ import annotations

import numpy as np

POWER_ITERS = 32


def _f64(x):
    return np.asarray(x, dtype=np.float64)


# ---------------------------------------------------------------------------
# PDDP grouping (grouping paragraph)
# ---------------------------------------------------------------------------

def principal_direction(cov, iters=POWER_ITERS):
    """Leading direction of a PSD matrix by a fixed number of power steps.

    Start v = 1/sqrt(D) * ones; repeat `iters` times: w = cov @ v; stop early
    only if |w| == 0; v = w / |w|.  A fixed step count is the reading taken for
    "project onto the principal direction" (the page does not say how the
    direction is found; power iteration is the method's stated choice).
    """
    d = cov.shape[0]
    v = np.full(d, 1.0 / np.sqrt(d))
    for _ in range(iters):
        w = cov @ v
        nw = np.sqrt(np.dot(w, w))
        if nw == 0.0:
            break
        v = w / nw
    return v


def split_rank(n, group):
    """Number of queries sent to the left child of a node of n queries.

    The node holds g = ceil(n / C) groups; the left child takes floor(g/2) full
    groups.  With n a multiple of C and g even this is the exact median; otherwise
    it is the reading that keeps every group at exactly C except one partial
    group, which always ends up last in depth-first order.
    """
    g = -(-n // group)
    return (g // 2) * group


def node_projection(x, iters=POWER_ITERS):
    """Centred projections p_i = (x_i - mean) . v of one node's queries."""
    mu = x.mean(axis=0)
    xc = x - mu
    cov = xc.T @ xc
    v = principal_direction(cov, iters)
    return xc @ v, v


def pddp_perm(q, group, iters=POWER_ITERS):
    """PDDP grouping of one head's queries (grouping paragraph).

    Recursively: centre the node, take its principal direction, project, order
    the node by (projection, token id) and cut it after split_rank(n) queries;
    stop when a node holds at most one group.  Leaves are emitted in depth-first,
    left-first order; their concatenation is perm (slot -> token).
    """
    q = _f64(q)
    n = q.shape[0]
    leaves = []
    stack = [np.arange(n, dtype=np.int64)]
    while stack:
        members = stack.pop()
        m = members.shape[0]
        if m <= group:
            leaves.append(members)
            continue
        p, _ = node_projection(q[members], iters)
        order = np.lexsort((members, p))  # by p, then token id
        cut = split_rank(m, group)
        # push right first so that the left child is emitted first
        stack.append(members[order[cut:]])
        stack.append(members[order[:cut]])
    return np.concatenate(leaves)


def pddp_tree_nodes(n, group):
    """Internal nodes of the split tree as (start_slot, size) pairs, root first.

    Sizes depend only on n and C, so the tree shape is fixed before any data is
    seen; a node covers a contiguous slot range of perm.
    """
    out = []
    stack = [(0, n)]
    while stack:
        s, m = stack.pop()
        if m <= group:
            continue
        out.append((s, m))
        cut = split_rank(m, group)
        stack.append((s + cut, m - cut))
        stack.append((s, cut))
    return out


def pddp_verify(q, perm, group, iters=POWER_ITERS, rel_tol=1e-5):
    """Node-local check of a grouping produced elsewhere (e.g. on the GPU).

    For every internal node of the tree (a contiguous slot range of `perm`),
    recompute the node's centred projection in fp64 on the members that `perm`
    puts there and check that the left range holds the split_rank smallest
    (projection, token id) members.  A member may sit on the other side only when
    its projection lies within rel_tol * (max p - min p) of the cut point
    (midpoint of the two order statistics around the cut).

    Returns dict(nodes, mismatched, tolerated, bad, ties) - `bad` counts
    mismatches outside the tolerance window (a correct grouping has bad == 0);
    `ties` lists the tolerated ones as (node start slot, node size, token).
    """
    q = _f64(q)
    perm = np.asarray(perm, dtype=np.int64)
    n = q.shape[0]
    res = dict(nodes=0, mismatched=0, tolerated=0, bad=0, ties=[])
    if sorted(perm.tolist()) != list(range(n)):
        res["bad"] = n
        return res
    for s, m in pddp_tree_nodes(n, group):
        members = perm[s:s + m]
        p, _ = node_projection(q[members], iters)
        order = np.lexsort((members, p))
        cut = split_rank(m, group)
        want_left = set(members[order[:cut]].tolist())
        got_left = members[:cut]
        wrong = [t for t in got_left.tolist() if t not in want_left]
        res["nodes"] += 1
        if not wrong:
            continue
        sp = p[order]
        pstar = 0.5 * (sp[cut - 1] + sp[cut])
        width = rel_tol * max(sp[-1] - sp[0], np.finfo(np.float64).tiny)
        pos = {t: i for i, t in enumerate(members.tolist())}
        got_right = members[cut:]
        wrong_r = [t for t in got_right.tolist() if t in want_left]
        for t in wrong + wrong_r:
            res["mismatched"] += 1
            if abs(p[pos[t]] - pstar) <= width:
                res["tolerated"] += 1
                res["ties"].append((int(s), int(m), int(t)))
            else:
                res["bad"] += 1
    return res


# ---------------------------------------------------------------------------
# Two-pass selection (selection paragraph)
# ---------------------------------------------------------------------------

def logits(q, k, scale, rows=None):
    q = _f64(q)
    if rows is not None:
        q = q[rows]
    return scale * (q @ _f64(k).T)


def row_lse(q, k, scale, rows=None, block=2048):
    """Pass 1: natural-log logsumexp of each query's logits over all keys.

    L_i = m_i + log sum_j exp(z_ij - m_i), m_i = max_j z_ij.
    """
    q = _f64(q)
    rows = np.arange(q.shape[0]) if rows is None else np.asarray(rows)
    out = np.empty(rows.shape[0])
    for b in range(0, rows.shape[0], block):
        z = logits(q, k, scale, rows[b:b + block])
        m = z.max(axis=1, keepdims=True)
        out[b:b + block] = (m + np.log(np.exp(z - m).sum(axis=1, keepdims=True)))[:, 0]
    return out


def group_members(perm, group, g):
    return np.asarray(perm[g * group:(g + 1) * group], dtype=np.int64)


def group_mass(q, k, lse, perm, group, scale, groups=None):
    """Pass 2: summed softmax weight of every key over each group's queries.

    M_g[j] = sum_{i in group g} exp(z_ij - L_i), with groups taken from the
    supplied perm.  Returns (len(groups), N).
    """
    n = _f64(k).shape[0]
    gcount = -(-len(perm) // group)
    groups = range(gcount) if groups is None else groups
    lse = _f64(lse)
    out = []
    for g in groups:
        mem = group_members(perm, group, g)
        z = logits(q, k, scale, mem)
        out.append(np.exp(z - lse[mem][:, None]).sum(axis=0))
    return np.stack(out) if out else np.zeros((0, n))


def topk_from_mass(mass_row, topk):
    """Keys of largest mass, ties to the lower key id, returned ascending."""
    mass_row = _f64(mass_row)
    ids = np.arange(mass_row.shape[0])
    order = np.lexsort((ids, -mass_row))
    return np.sort(order[:topk])


def select(q, k, perm, group, topk, scale, lse=None, groups=None):
    """Both passes plus the per-group top-K: (len(groups), K) ascending key ids."""
    if lse is None:
        lse = row_lse(q, k, scale)
    mass = group_mass(q, k, lse, perm, group, scale, groups)
    return np.stack([topk_from_mass(r, topk) for r in mass]) if len(mass) else np.zeros((0, topk), np.int64)


# ---------------------------------------------------------------------------
# Attention (limitations paragraph: dense on anchors; grouping paragraph: gather)
# ---------------------------------------------------------------------------

def dense_attention(q, k, v, scale, rows=None, block=1024):
    """O_i = sum_j softmax_j(z_ij) v_j for the requested query rows (all by default)."""
    q = _f64(q)
    v = _f64(v)
    rows = np.arange(q.shape[0]) if rows is None else np.asarray(rows)
    out = np.empty((rows.shape[0], v.shape[1]))
    for b in range(0, rows.shape[0], block):
        z = logits(q, k, scale, rows[b:b + block])
        z = z - z.max(axis=1, keepdims=True)
        w = np.exp(z)
        out[b:b + block] = (w @ v) / w.sum(axis=1, keepdims=True)
    return out


def sparse_attention_group(q, k, v, members, keys, scale):
    """Softmax attention of the given queries restricted to the given keys.

    The softmax is renormalised over the kept keys only (gap paragraph: the
    dropped tail still has weight; that difference is what the residual holds).
    """
    z = logits(q, _f64(k)[keys], scale, members)
    z = z - z.max(axis=1, keepdims=True)
    w = np.exp(z)
    return (w @ _f64(v)[keys]) / w.sum(axis=1, keepdims=True)


def sparse_attention(q, k, v, perm, idx, group, scale, groups=None):
    """Gather-sparse attention, (N, D) in token order.

    idx[g] lists group g's kept keys (indexable by group id).  Only the requested
    groups are computed; rows of other groups are NaN.
    """
    q = _f64(q)
    n = q.shape[0]
    out = np.full((n, _f64(v).shape[1]), np.nan)
    gcount = -(-n // group)
    groups = range(gcount) if groups is None else groups
    for g in groups:
        mem = group_members(perm, group, g)
        out[mem] = sparse_attention_group(q, k, v, mem, np.asarray(idx[g], dtype=np.int64), scale)
    return out


# ---------------------------------------------------------------------------
# Anchor / reuse with the dense-minus-sparse residual (residual paragraph)
# ---------------------------------------------------------------------------

def anchor(q, k, v, group, topk, scale, iters=POWER_ITERS):
    """Full anchor step of one head.

    perm = PDDP(Q); lse = pass 1; idx = top-K of pass 2; O_dense = dense
    attention; O_sparse = gather-sparse attention; R = O_dense - O_sparse.
    The anchor's output is O_dense.
    """
    perm = pddp_perm(q, group, iters)
    lse = row_lse(q, k, scale)
    idx = select(q, k, perm, group, topk, scale, lse=lse)
    o_dense = dense_attention(q, k, v, scale)
    o_sparse = sparse_attention(q, k, v, perm, idx, group, scale)
    return dict(perm=perm, lse=lse, idx=idx, o_dense=o_dense, o_sparse=o_sparse,
                resid=o_dense - o_sparse)


def reuse(q, k, v, perm, idx, resid, group, scale, groups=None):
    """Reuse step: fresh sparse attention on the current Q/K/V with the cached
    groups and indices, plus the cached residual (no regrouping, no reselection)."""
    o = sparse_attention(q, k, v, perm, idx, group, scale, groups)
    return o + _f64(resid)


# ---------------------------------------------------------------------------
# Compact kept-key sets of the meta-cache (residual paragraph: cached indices
# move to host memory; their size sets the host-link traffic)
# ---------------------------------------------------------------------------

def idx_to_bits(idx_rows, n, topk):
    """Kept-key lists -> bitmaps: row r of the result has ceil(n/32) uint32
    words; bit b of word w is set when key 32*w + b is among the first `topk`
    entries of idx_rows[r] (entries outside [0, n) are ignored)."""
    idx_rows = np.asarray(idx_rows)
    words = (n + 31) // 32
    out = np.zeros(idx_rows.shape[:-1] + (words,), dtype=np.uint32)
    flat_idx = idx_rows.reshape(-1, idx_rows.shape[-1])
    flat_out = out.reshape(-1, words)
    for r in range(flat_idx.shape[0]):
        for key in flat_idx[r, :topk]:
            key = int(key)
            if 0 <= key < n:
                flat_out[r, key // 32] |= np.uint32(1 << (key % 32))
    return out


def bits_to_idx(bits_rows, n, topk, kpad):
    """Bitmaps -> kept-key lists: the keys of the set bits below n in ascending
    order, at most `topk` of them, then -1 up to kpad."""
    bits_rows = np.asarray(bits_rows, dtype=np.uint32)
    words = bits_rows.shape[-1]
    out = np.full(bits_rows.shape[:-1] + (kpad,), -1, dtype=np.int32)
    flat_bits = bits_rows.reshape(-1, words)
    flat_out = out.reshape(-1, kpad)
    for r in range(flat_bits.shape[0]):
        keys = [32 * w + b for w in range(words) for b in range(32)
                if (int(flat_bits[r, w]) >> b) & 1 and 32 * w + b < n]
        keys = keys[:topk]
        flat_out[r, :len(keys)] = keys
    return out


# ---------------------------------------------------------------------------
# Matched-density selectors (block-sparsity and matched-density-oracle
# paragraphs): vanilla block sparsity scores C-token blocks of Q and K by their
# mean-pooled vectors and keeps whole key blocks; the oracles keep, within the
# same budget of keys, as much true attention mass as their structure allows:
# whole key blocks per query block, one key set per query group, one key set
# per query.  Blocks are runs of C consecutive token ids (N a multiple of C).
# ---------------------------------------------------------------------------

def block_means(x, c):
    """Mean of each run of c consecutive rows: (N / c, D)."""
    x = _f64(x)
    n, d = x.shape
    if n % c:
        raise ValueError("block grid needs N to be a multiple of C")
    return x.reshape(n // c, c, d).mean(axis=1)


def bsa_scores(q, k, c, scale):
    """Block score of query block b and key block j: scale * mean(q_b) . mean(k_j)."""
    return scale * (block_means(q, c) @ block_means(k, c).T)


def _expand_blocks(blocks, c):
    return (np.asarray(blocks, np.int64)[:, None] * c + np.arange(c)[None, :]).reshape(-1)


def bsa_select(q, k, c, kb, scale):
    """Vanilla block sparsity: for each query block, the kb key blocks of highest
    mean-pooled score (ties to the lower block id), expanded to their keys in
    ascending order: (N / c, kb * c)."""
    s = bsa_scores(q, k, c, scale)
    return np.stack([_expand_blocks(topk_from_mass(row, kb), c) for row in s])


def block_mass(q, k, c, scale, lse=None):
    """True attention mass between blocks: B[b][j] = sum over queries i of block b
    and keys t of block j of softmax_t(z_it)."""
    n = _f64(q).shape[0]
    if lse is None:
        lse = row_lse(q, k, scale)
    m = group_mass(q, k, lse, np.arange(n), c, scale)  # (N / c, N): groups are the query blocks
    return m.reshape(m.shape[0], n // c, c).sum(axis=2)


def block_oracle_select(q, k, c, kb, scale, lse=None):
    """Block oracle: per query block, the kb key blocks of largest true mass
    (ties to the lower block id), expanded: (N / c, kb * c)."""
    b = block_mass(q, k, c, scale, lse)
    return np.stack([_expand_blocks(topk_from_mass(row, kb), c) for row in b])


def private_select(q, k, topk, scale, rows=None):
    """Per-query oracle: each query's own top-K keys by logit (equivalently by
    softmax weight), ties to the lower key id, ascending: (rows, K)."""
    z = logits(q, k, scale, rows)
    return np.stack([topk_from_mass(r, topk) for r in z])


def sparse_lse(q, k, perm, idx, group, scale, groups=None):
    """Natural-log logsumexp of each query's logits over its group's kept keys,
    in token order (rows of groups not computed are NaN)."""
    q = _f64(q)
    n = q.shape[0]
    out = np.full(n, np.nan)
    gcount = -(-n // group)
    for g in (range(gcount) if groups is None else groups):
        mem = group_members(perm, group, g)
        z = logits(q, _f64(k)[np.asarray(idx[g], np.int64)], scale, mem)
        m = z.max(axis=1, keepdims=True)
        out[mem] = (m + np.log(np.exp(z - m).sum(axis=1, keepdims=True)))[:, 0]
    return out


def captured_mass(q, k, keys_of_query, scale, lse=None):
    """Per query: the dense softmax weight that falls on its kept keys,
    sum over kept t of exp(z_it - L_i).  keys_of_query[i] lists query i's keys."""
    if lse is None:
        lse = row_lse(q, k, scale)
    z = logits(q, k, scale)
    return np.array([np.exp(z[i, np.asarray(keys, np.int64)] - lse[i]).sum()
                     for i, keys in enumerate(keys_of_query)])


def keys_per_query(perm, idx, group):
    """Expand per-group key sets to per-query key sets (token order)."""
    n = len(perm)
    out = [None] * n
    for g in range(-(-n // group)):
        for i in group_members(perm, group, g):
            out[int(i)] = np.asarray(idx[g], np.int64)
    return out


def private_attention(q, k, v, keys_of_query, scale):
    """Each query attends over its own kept keys only (renormalised softmax)."""
    return np.stack([sparse_attention_group(q, k, v, np.array([i]), np.asarray(keys, np.int64), scale)[0]
                     for i, keys in enumerate(keys_of_query)])
