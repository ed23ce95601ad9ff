"""The Python binding checks every tensor argument before any library call: the C
ABI gets bare pointers and cannot tell an int64 perm, an undersized output or a
key list of the wrong width from a good one.  Runs on the CPU: every case here
must raise ValueError before anything reaches the GPU."""
import pytest
import torch

import sparse_attention_diffusion_amd as mcs

H, N, D, K = 2, 100, 64, 20
G = -(-N // 64)
KPAD = 32


def qkv(dtype=torch.bfloat16):
    return tuple(torch.zeros((H, N, D), dtype=dtype) for _ in range(3))


def perm(dtype=torch.int32, shape=(H, N)):
    return torch.zeros(shape, dtype=dtype)


def idx(dtype=torch.int32, shape=(H, G, KPAD)):
    return torch.full(shape, -1, dtype=dtype)


def raises(fn, match):
    with pytest.raises(ValueError, match=match):
        fn()


def test_sparse_attention_rejects_bad_perm_idx_and_outputs():
    q, k, v = qkv()
    raises(lambda: mcs.mcs_sparse_attn(q, k, v, perm(torch.int64), idx(), K), "perm must be torch.int32")
    raises(lambda: mcs.mcs_sparse_attn(q, k, v, perm(shape=(H, N - 1)), idx(), K), "perm must have shape")
    raises(lambda: mcs.mcs_sparse_attn(q, k, v, perm(), idx(torch.int64), K), "idx must be torch.int32")
    raises(lambda: mcs.mcs_sparse_attn(q, k, v, perm(), idx(shape=(H, G + 1, KPAD)), K), "idx must have shape")
    raises(lambda: mcs.mcs_sparse_attn(q, k, v, perm(), idx(shape=(H, G, 16)), K), "kpad 16")
    raises(lambda: mcs.mcs_sparse_attn(q, k, v, perm(), idx(shape=(H, G, 40)), K), "multiple of 32")
    raises(lambda: mcs.mcs_sparse_attn(q, k, v, perm(), idx(), K, o=torch.zeros((H, N, D))), "o must be")
    raises(lambda: mcs.mcs_sparse_attn(q, k, v, perm(), idx(), K, o=torch.zeros((H, N, D // 2), dtype=q.dtype)),
           "o must have shape")
    raises(lambda: mcs.mcs_sparse_attn(q, k, v, perm(), idx(), K, resid_add=torch.zeros((H, N, D))), "share")
    raises(lambda: mcs.mcs_sparse_attn(q, k, v.float(), perm(), idx(), K), "share")
    # a well-formed call stops at the device check on a CPU tensor
    raises(lambda: mcs.mcs_sparse_attn(q, k, v, perm(), idx(), K), "GPU device")


def test_reuse_and_sparse_lse_and_pairs_check_their_tensors():
    q, k, v = qkv()
    r = torch.zeros_like(q)
    raises(lambda: mcs.mcs_reuse(q, k, v, perm(), idx(), None, K), "resid is required")
    raises(lambda: mcs.mcs_reuse(q, k, v, perm(torch.int64), idx(), r, K), "perm must be")
    raises(lambda: mcs.mcs_reuse(q, k, v, perm(), idx(shape=(1, G, KPAD)), r, K), "idx must have shape")
    raises(lambda: mcs.mcs_sparse_lse(q, k, perm(), idx(), K, lse=torch.zeros((H, N), dtype=torch.float64)),
           "lse must be torch.float32")
    raises(lambda: mcs.mcs_sparse_lse(q, k, perm(), idx(), K, lse=torch.zeros((H, N + 1))), "lse must have")
    nc = torch.zeros((H, mcs.pairs_of(N)), dtype=torch.int32)
    raises(lambda: mcs.mcs_sparse_attn_pairs(q, k, v, perm(), idx(), nc.long(), K), "ncommon must be")
    raises(lambda: mcs.mcs_sparse_attn_pairs(q, k, v, perm(), idx(shape=(H, G, 64)), nc[:, :0], K), "ncommon")
    raises(lambda: mcs.mcs_sparse_attn_pairs(q, k, v, perm(), idx(torch.int16), nc, K), "pidx must be")


def test_select_checks_idx_width_lse_and_perm():
    q, k, _ = qkv()
    raises(lambda: mcs.mcs_select(q, k, perm(torch.int64), K), "perm must be")
    raises(lambda: mcs.mcs_select(q, k, perm(), K, idx=idx(shape=(H, G, 16))), "kpad 16")
    raises(lambda: mcs.mcs_select(q, k, perm(), K, lse=torch.zeros((H, N), dtype=torch.bfloat16)), "lse must be")
    raises(lambda: mcs.mcs_select(q, k, perm(), K), "GPU device")
    # a caller-supplied list of another (valid) width is accepted up to the device check
    raises(lambda: mcs.mcs_select(q, k, perm(), K, idx=idx(shape=(H, G, 64))), "GPU device")


def test_anchor_checks_every_output():
    q, k, v = qkv()

    def out(**kw):
        o = dict(perm=perm(), idx=idx(), resid=torch.zeros_like(q), o_dense=torch.zeros_like(q), lse=None)
        o.update(kw)
        return o

    raises(lambda: mcs.mcs_anchor(q, k, v, K, out=out(perm=perm(torch.int64))), "perm must be")
    raises(lambda: mcs.mcs_anchor(q, k, v, K, out=out(idx=idx(shape=(H, G, 16)))), "kpad 16")
    raises(lambda: mcs.mcs_anchor(q, k, v, K, out=out(resid=torch.zeros((H, N, D)))), "resid")
    raises(lambda: mcs.mcs_anchor(q, k, v, K, out=out(o_dense=None)), "o_dense")
    raises(lambda: mcs.mcs_anchor(q, k, v, K, out=out(lse=torch.zeros((H, N), dtype=torch.float64))), "lse")
    raises(lambda: mcs.mcs_anchor(q, k, v, K, out=out()), "GPU device")


def test_dense_group_and_bitmaps_check_their_tensors():
    q, k, v = qkv()
    raises(lambda: mcs.mcs_dense_attn(q, k, v, o=torch.zeros((H, N, D))), "o must be")
    raises(lambda: mcs.mcs_dense_attn(q, k, v), "GPU device")
    raises(lambda: mcs.mcs_group(q, perm=perm(torch.int64)), "perm must be")
    raises(lambda: mcs.mcs_group(q), "GPU device")
    raises(lambda: mcs.mcs_idx_to_bits(idx(shape=(H, G, 16)), N, K), "kpad 16")
    raises(lambda: mcs.mcs_idx_to_bits(idx(), N, K, bits=torch.zeros((H, G, 3), dtype=torch.int32)), "shape")
    raises(lambda: mcs.mcs_bits_to_idx(torch.zeros((H, G, 4), dtype=torch.int32), N, K,
                                       idx=idx(shape=(H, G, 16))), "kpad 16")
    raises(lambda: mcs.mcs_pair_plan(idx(torch.int64), N, K), "int32")


def test_copy_kind_must_match_the_devices():
    a = torch.zeros(16, dtype=torch.int32)
    b = torch.zeros(16, dtype=torch.int32)
    raises(lambda: mcs.mcs_copy_async(a, b, mcs.MCS_COPY_H2D), "does not match")
    raises(lambda: mcs.mcs_copy_async(a, b, 7), "unknown copy kind")
    raises(lambda: mcs.mcs_copy_async(a[:8], b, mcs.MCS_COPY_D2D), "sizes differ")
