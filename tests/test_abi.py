"""The C-ABI library on the host: it loads, exports every entry point that
include/mcs.h declares, and rejects bad arguments with the documented codes
before anything is enqueued (no GPU needed, no compute is launched)."""
import ctypes
import os
import re

import pytest

from sparse_attention_diffusion_amd import _abi

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared():
    with open(os.path.join(ROOT, "include", "mcs.h")) as f:
        text = f.read()
    return sorted(set(re.findall(r"^\s*(?:int|int32_t|const char\*)\s+(mcs_\w+)\s*\(", text, re.M)))


@pytest.fixture(scope="module")
def lib():
    # MCS_ABI_TEST_LIB: run these checks against another build of the library (the
    # AddressSanitizer build, test_abi_asan.py)
    other = os.environ.get("MCS_ABI_TEST_LIB")
    if other:
        _abi.LIB_PATH = other
        _abi._lib = None
    elif not os.path.exists(_abi.LIB_PATH):
        from sparse_attention_diffusion_amd import build
        build.build()
    return _abi.load()


def _dims(**kw):
    d = dict(heads=2, n=1000, head_dim=128, group=64, topk=200, kpad=224, dtype=_abi.MCS_BF16,
             power_iters=32, scale=0.088)
    d.update(kw)
    return _abi.McsDims(**d)


FAKE = ctypes.c_void_p(1 << 20)  # never dereferenced: every call below fails validation first


def test_exports_every_declared_symbol(lib):
    names = _declared()
    assert set(names) == set(_abi.EXPORTED), names
    for n in names:
        assert hasattr(lib, n)
    assert lib.mcs_abi_version() == _abi.ABI_VERSION


def test_workspace_sizes_are_consistent(lib):
    out = ctypes.c_size_t()
    d = _dims()
    sizes = {}
    for op in (_abi.MCS_OP_GROUP, _abi.MCS_OP_SELECT, _abi.MCS_OP_ANCHOR):
        for hpp in (1, 0):
            assert lib.mcs_workspace_bytes(ctypes.byref(d), op, hpp, ctypes.byref(out)) == 0
            sizes[(op, hpp)] = out.value
    g = -(-1000 // 64)
    assert sizes[(_abi.MCS_OP_SELECT, 0)] - sizes[(_abi.MCS_OP_SELECT, 1)] >= g * 1000 * 4
    # the anchor keeps the grouping's workspace beside the selection's
    assert sizes[(_abi.MCS_OP_ANCHOR, 0)] >= sizes[(_abi.MCS_OP_GROUP, 0)] + sizes[(_abi.MCS_OP_SELECT, 0)]
    assert lib.mcs_workspace_bytes(ctypes.byref(d), 99, 0, ctypes.byref(out)) == _abi.MCS_EINVAL
    assert lib.mcs_workspace_bytes(None, 1, 0, ctypes.byref(out)) == _abi.MCS_EINVAL


@pytest.mark.parametrize("kw,code", [
    (dict(group=32), _abi.MCS_EUNSUPPORTED),
    (dict(head_dim=96), _abi.MCS_EUNSUPPORTED),
    (dict(dtype=7), _abi.MCS_EUNSUPPORTED),
    (dict(heads=0), _abi.MCS_EINVAL),
    (dict(n=0), _abi.MCS_EINVAL),
    (dict(topk=0), _abi.MCS_EINVAL),
    (dict(topk=1001), _abi.MCS_EINVAL),
    (dict(kpad=200), _abi.MCS_EINVAL),
    (dict(kpad=230), _abi.MCS_EINVAL),
    (dict(scale=0.0), _abi.MCS_EINVAL),
    (dict(scale=float("inf")), _abi.MCS_EINVAL),
    (dict(n=1 << 24, head_dim=128, dtype=_abi.MCS_F32, topk=1, kpad=32), _abi.MCS_EINVAL),
])
def test_sparse_attn_rejects_bad_dims(lib, kw, code):
    d = _dims(**kw)
    rc = lib.mcs_sparse_attn(ctypes.byref(d), FAKE, FAKE, FAKE, FAKE, FAKE, None, FAKE, None)
    assert rc == code, lib.mcs_last_error()
    assert lib.mcs_last_error()


def test_null_and_misaligned_pointers(lib):
    d = _dims()
    assert lib.mcs_dense_attn(ctypes.byref(d), None, FAKE, FAKE, FAKE, None, None) == _abi.MCS_EINVAL
    assert b"q" in lib.mcs_last_error()
    odd = ctypes.c_void_p((1 << 20) + 2)
    assert lib.mcs_dense_attn(ctypes.byref(d), FAKE, odd, FAKE, FAKE, None, None) == _abi.MCS_EINVAL
    assert b"aligned" in lib.mcs_last_error()
    assert lib.mcs_reuse(ctypes.byref(d), FAKE, FAKE, FAKE, FAKE, FAKE, None, FAKE, None) == _abi.MCS_EINVAL


def test_workspace_too_small(lib):
    d = _dims()
    need = ctypes.c_size_t()
    lib.mcs_workspace_bytes(ctypes.byref(d), _abi.MCS_OP_GROUP, 0, ctypes.byref(need))
    ws = ctypes.c_void_p(1 << 24)
    assert lib.mcs_group(ctypes.byref(d), FAKE, FAKE, ws, need.value - 1, None) == _abi.MCS_EWORKSPACE
    assert lib.mcs_select(ctypes.byref(d), FAKE, FAKE, FAKE, None, FAKE, ws, 1024, None) == _abi.MCS_EWORKSPACE
    assert lib.mcs_anchor(ctypes.byref(d), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, ws, 1024,
                          None) == _abi.MCS_EWORKSPACE
    bad_iters = _dims(power_iters=0)
    assert lib.mcs_group(ctypes.byref(bad_iters), FAKE, FAKE, ws, need.value, None) == _abi.MCS_EINVAL


def test_copy_rejects_bad_kind(lib):
    assert lib.mcs_copy_async(FAKE, FAKE, 16, 9, None, None) == _abi.MCS_EINVAL
    assert lib.mcs_copy_async(None, FAKE, 16, _abi.MCS_COPY_H2D, None, None) == _abi.MCS_EINVAL


def test_python_binding_raises_on_missing_library(monkeypatch, tmp_path):
    monkeypatch.setattr(_abi, "_lib", None)
    monkeypatch.setattr(_abi, "LIB_PATH", str(tmp_path / "missing.so"))
    with pytest.raises(_abi.McsError):
        _abi.load()


def test_key_bitmaps_reject_bad_args(lib):
    big = _dims(n=(1 << 20) + 1, topk=1, kpad=32)
    assert lib.mcs_idx_to_bits(ctypes.byref(big), FAKE, FAKE, None) == _abi.MCS_EUNSUPPORTED
    assert lib.mcs_bits_to_idx(ctypes.byref(big), FAKE, FAKE, None) == _abi.MCS_EUNSUPPORTED
    d = _dims()
    assert lib.mcs_idx_to_bits(ctypes.byref(d), None, FAKE, None) == _abi.MCS_EINVAL
    assert lib.mcs_bits_to_idx(ctypes.byref(d), FAKE, ctypes.c_void_p((1 << 20) + 2), None) == _abi.MCS_EINVAL
    assert b"aligned" in lib.mcs_last_error()
    assert lib.mcs_idx_to_bits(ctypes.byref(_dims(topk=0)), FAKE, FAKE, None) == _abi.MCS_EINVAL


def test_pair_entry_points_reject_bad_args(lib):
    big = _dims(n=(1 << 19) + 1, head_dim=64, topk=1, kpad=32)
    assert lib.mcs_pair_plan(ctypes.byref(big), FAKE, FAKE, FAKE, None) == _abi.MCS_EUNSUPPORTED
    d = _dims()
    assert lib.mcs_pair_plan(ctypes.byref(d), FAKE, FAKE, None, None) == _abi.MCS_EINVAL
    assert lib.mcs_pair_plan(ctypes.byref(d), FAKE, ctypes.c_void_p((1 << 20) + 4), FAKE, None) == _abi.MCS_EINVAL
    assert b"aligned" in lib.mcs_last_error()
    assert lib.mcs_pair_plan(ctypes.byref(_dims(kpad=200)), FAKE, FAKE, FAKE, None) == _abi.MCS_EINVAL
    args = [FAKE] * 6 + [None, FAKE, None]  # q k v perm pidx ncommon, resid, o, stream
    assert lib.mcs_sparse_attn_pairs(ctypes.byref(_dims(group=32)), *args) == _abi.MCS_EUNSUPPORTED
    assert lib.mcs_sparse_attn_pairs(ctypes.byref(_dims(topk=1001)), *args) == _abi.MCS_EINVAL
    no_counts = [FAKE] * 5 + [None, None, FAKE, None]
    assert lib.mcs_sparse_attn_pairs(ctypes.byref(d), *no_counts) == _abi.MCS_EINVAL
    assert b"ncommon" in lib.mcs_last_error()


def test_block_select_and_sparse_lse_reject_bad_args(lib):
    d = _dims(n=1024, topk=256, kpad=256)
    ws = ctypes.c_size_t(0)
    assert lib.mcs_workspace_bytes(ctypes.byref(d), _abi.MCS_OP_BLOCK_SELECT, 0, ctypes.byref(ws)) == _abi.MCS_OK
    assert ws.value >= 2 * 2 * 16 * 128 * 4
    big = ctypes.c_size_t(1 << 30)
    assert lib.mcs_block_select(ctypes.byref(_dims(n=1000, topk=192, kpad=192)), FAKE, FAKE, FAKE, FAKE, big,
                                None) == _abi.MCS_EUNSUPPORTED
    assert lib.mcs_block_select(ctypes.byref(_dims(n=1024, topk=200, kpad=224)), FAKE, FAKE, FAKE, FAKE, big,
                                None) == _abi.MCS_EINVAL
    assert b"block" in lib.mcs_last_error()
    assert lib.mcs_block_select(ctypes.byref(d), FAKE, FAKE, FAKE, FAKE, ctypes.c_size_t(16), None) \
        == _abi.MCS_EWORKSPACE
    assert lib.mcs_sparse_lse(ctypes.byref(d), FAKE, FAKE, FAKE, FAKE, None, None) == _abi.MCS_EINVAL
    assert b"lse" in lib.mcs_last_error()


def test_residual_rejects_bad_args(lib):
    d = _dims()
    other = ctypes.c_void_p(1 << 21)
    args = lambda od, r: [FAKE, FAKE, FAKE, FAKE, FAKE, od, r, None]  # q k v perm idx o_dense resid stream
    assert lib.mcs_residual(ctypes.byref(d), *args(FAKE, FAKE)) == _abi.MCS_EINVAL
    assert b"alias" in lib.mcs_last_error()
    assert lib.mcs_residual(ctypes.byref(d), *args(None, other)) == _abi.MCS_EINVAL
    assert b"o_dense" in lib.mcs_last_error()
    assert lib.mcs_residual(ctypes.byref(_dims(topk=0)), *args(FAKE, other)) == _abi.MCS_EINVAL
    assert lib.mcs_residual(ctypes.byref(_dims(head_dim=80)), *args(FAKE, other)) == _abi.MCS_EUNSUPPORTED


def test_select_noalloc_checks_sizes_before_any_hip_call(lib):
    # 50,000 tokens: one head of mass rows is 782 x 50,000 x 4 bytes > the 128 MiB scratch
    big = _dims(heads=1, n=50000, head_dim=64, topk=100, kpad=128)
    assert lib.mcs_select_noalloc(ctypes.byref(big), FAKE, FAKE, FAKE, None, FAKE, None) == _abi.MCS_EUNSUPPORTED
    assert b"scratch" in lib.mcs_last_error()
    assert lib.mcs_select_noalloc(ctypes.byref(_dims()), FAKE, FAKE, None, None, FAKE, None) == _abi.MCS_EINVAL
    assert lib.mcs_select_noalloc(ctypes.byref(_dims(topk=0)), FAKE, FAKE, FAKE, None, FAKE, None) == _abi.MCS_EINVAL
