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
