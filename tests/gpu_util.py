"""Helpers of the GPU parity tests: device transfer, oracle comparisons and the
tolerances of the hot path (bf16 outputs against fp64: max-abs 2e-2,
mean-abs 2e-3; index sets exact up to mass ties within 1e-6 relative)."""
import numpy as np
import torch

from oracle import ref

MAX_ABS = 2e-2
MEAN_ABS = 2e-3
TIE_REL = 1e-6


def dev():
    return torch.device("cuda:0")


def to_dev(x, dtype):
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    return t.to(device=dev(), dtype=torch.float32 if dtype == "f32" else torch.bfloat16).contiguous()


def host(t):
    return t.detach().to("cpu", torch.float32).numpy().astype(np.float64) if t.is_floating_point() \
        else t.detach().cpu().numpy()


def assert_close(got, want, max_abs=MAX_ABS, mean_abs=MEAN_ABS, what=""):
    got = np.asarray(got, np.float64)
    want = np.asarray(want, np.float64)
    assert got.shape == want.shape, (what, got.shape, want.shape)
    assert np.isfinite(got).all(), f"{what}: non-finite output"
    err = np.abs(got - want)
    mx, mn = float(err.max()), float(err.mean())
    assert mx <= max_abs and mn <= mean_abs, f"{what}: max-abs {mx:.3e} (<= {max_abs}), mean-abs {mn:.3e} (<= {mean_abs})"
    return mx, mn


def bf16_half_ulp(x):
    """Half a bf16 unit in the last place at |x| (round-to-nearest error bound)."""
    a = np.maximum(np.abs(np.asarray(x, np.float64)), 2.0 ** -126)
    return 0.5 * np.exp2(np.floor(np.log2(a)) - 7)


def check_index_row(row, mass, k, n):
    """GPU idx row vs the oracle's fp64 masses of that group (ties within TIE_REL)."""
    row = np.asarray(row)
    kept, pad = row[:k], row[k:]
    assert (pad == -1).all(), "padding must be -1"
    assert ((kept >= 0) & (kept < n)).all(), "index out of range"
    assert (np.diff(kept) > 0).all(), "indices must be strictly ascending"
    want = ref.topk_from_mass(mass, k)
    tau = np.sort(mass)[::-1][k - 1]
    diff = np.setxor1d(kept, want)
    bad = [j for j in diff if abs(mass[j] - tau) > TIE_REL * tau]
    assert not bad, f"{len(bad)} keys differ beyond ties (tau={tau:.6e}): {bad[:8]}"
    return len(diff)


def random_groups(n, k, heads, seed, c=64):
    """Random perm and ascending random key sets (oracle-side inputs for the sparse kernel)."""
    r = np.random.default_rng(seed)
    g = -(-n // c)
    kpad = ((k + 31) // 32) * 32
    perm = np.stack([r.permutation(n) for _ in range(heads)]).astype(np.int32)
    idx = np.full((heads, g, kpad), -1, np.int32)
    for h in range(heads):
        for gi in range(g):
            idx[h, gi, :k] = np.sort(r.choice(n, k, replace=False))
    return perm, idx


# Error bound of a bf16 attention output against fp64, per element.  The kernel
# multiplies V by the probabilities rounded to bf16 (relative error <= 2^-8 each)
# and divides by the sum of those same rounded values, so the weights it applies
# are w~_j = w_j (1 + e_j) / (1 + sum_k w_k e_k), |e_j| <= 2^-8, and
#   O~ - O = sum_j w_j (e_j - e) (v_j - O) / (1 + e),  |e_j - e| <= 2^-7,
# i.e. |O~ - O| <= 2^-7 (1 + 2^-7) sum_j w_j |v_j - O| per output dimension.  The
# fp32 accumulation adds a few 2^-24 relative, and the single rounding of the
# result to bf16 adds half a bf16 ulp of the result.
P_ROUND = 2.0 ** -7 * (1.0 + 2.0 ** -7)


def attention_spread(q, k, v, rows, keys, scale, block=64):
    """fp64 (O, spread) of the given query rows over `keys` (an index array shared by
    all rows): spread[i, d] = sum_j w_ij |v_jd - O_id|."""
    q = np.asarray(q, np.float64)
    kk = np.asarray(k, np.float64)[keys]
    vv = np.asarray(v, np.float64)[keys]
    rows = np.asarray(rows)
    o = np.empty((len(rows), vv.shape[1]))
    sp = np.empty_like(o)
    for b in range(0, len(rows), block):
        z = scale * (q[rows[b:b + block]] @ kk.T)
        w = np.exp(z - z.max(axis=1, keepdims=True))
        w /= w.sum(axis=1, keepdims=True)
        ob = w @ vv
        o[b:b + block] = ob
        sp[b:b + block] = np.einsum("ij,ijd->id", w, np.abs(vv[None, :, :] - ob[:, None, :]))
    return o, sp


def bf16_attention_bound(o, spread, slack=1e-5):
    """Per-element bound on |bf16 kernel output - fp64 O| (see P_ROUND)."""
    dev_ = P_ROUND * spread + slack * (1.0 + np.abs(o))
    return dev_ + bf16_half_ulp(np.abs(o) + dev_)


def assert_within(got, want, bound, what=""):
    err = np.abs(np.asarray(got, np.float64) - want)
    over = err > bound
    assert np.isfinite(got).all(), f"{what}: non-finite output"
    assert not over.any(), (f"{what}: {int(over.sum())} elements above the derived bound; worst "
                            f"err {float(err[over].max()):.3e} vs bound {float(bound[over][np.argmax(err[over])]):.3e}")
    return float(err.max())


def check_index_row_window(row, mass, k, n, rel):
    """check_index_row with a wider relative tie window `rel` (for logits large enough
    that their fp32 rounding moves exp() by more than 1e-6 relative)."""
    row = np.asarray(row)
    kept, pad = row[:k], row[k:]
    assert (pad == -1).all() and ((kept >= 0) & (kept < n)).all() and (np.diff(kept) > 0).all()
    want = ref.topk_from_mass(mass, k)
    tau = np.sort(mass)[::-1][k - 1]
    diff = np.setxor1d(kept, want)
    bad = [j for j in diff if abs(mass[j] - tau) > rel * tau]
    assert not bad, f"{len(bad)} keys differ beyond ties (tau={tau:.6e}, rel={rel:.2e}): {bad[:8]}"
    return len(diff)
