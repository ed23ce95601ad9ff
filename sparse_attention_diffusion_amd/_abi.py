"""ctypes declarations of include/mcs.h (argument marshalling only)."""
from __future__ import annotations

import ctypes
import os

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libmcs.so")

MCS_OK, MCS_EINVAL, MCS_EUNSUPPORTED, MCS_EWORKSPACE, MCS_EHIP = 0, -1, -2, -3, -4
MCS_F32, MCS_BF16 = 0, 1
MCS_OP_GROUP, MCS_OP_SELECT, MCS_OP_ANCHOR, MCS_OP_BLOCK_SELECT = 1, 2, 3, 4
MCS_COPY_H2D, MCS_COPY_D2H, MCS_COPY_D2D = 1, 2, 3
ABI_VERSION = 1

EXPORTED = ("mcs_abi_version", "mcs_last_error", "mcs_workspace_bytes", "mcs_group", "mcs_select", "mcs_select_noalloc",
            "mcs_dense_attn", "mcs_sparse_attn", "mcs_anchor", "mcs_residual", "mcs_reuse", "mcs_idx_to_bits", "mcs_bits_to_idx",
            "mcs_pair_plan", "mcs_sparse_attn_pairs", "mcs_block_select", "mcs_sparse_lse", "mcs_copy_async")
BITS_MAX_N = 1 << 20
PAIRS_MAX_N = 1 << 19
SCRATCH_BYTES = 128 << 20


class McsDims(ctypes.Structure):
    _fields_ = [("heads", ctypes.c_int32), ("n", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("group", ctypes.c_int32), ("topk", ctypes.c_int32), ("kpad", ctypes.c_int32),
                ("dtype", ctypes.c_int32), ("power_iters", ctypes.c_int32), ("scale", ctypes.c_float)]


class McsError(RuntimeError):
    def __init__(self, code, msg):
        super().__init__(f"mcs error {code}: {msg}")
        self.code = code


_lib = None


def load():
    """Load libmcs.so from the package directory; raise if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise McsError(MCS_EHIP, f"{LIB_PATH} is missing: build it with "
                                 "`python -m sparse_attention_diffusion_amd.build`")
    lib = ctypes.CDLL(LIB_PATH)
    P, S, I32, St = ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int32, ctypes.c_void_p
    D = ctypes.POINTER(McsDims)
    sig = {
        "mcs_abi_version": (I32, []),
        "mcs_last_error": (ctypes.c_char_p, []),
        "mcs_workspace_bytes": (ctypes.c_int, [D, I32, I32, ctypes.POINTER(ctypes.c_size_t)]),
        "mcs_group": (ctypes.c_int, [D, P, P, P, S, St]),
        "mcs_select": (ctypes.c_int, [D, P, P, P, P, P, P, S, St]),
        "mcs_select_noalloc": (ctypes.c_int, [D, P, P, P, P, P, St]),
        "mcs_dense_attn": (ctypes.c_int, [D, P, P, P, P, P, St]),
        "mcs_sparse_attn": (ctypes.c_int, [D, P, P, P, P, P, P, P, St]),
        "mcs_anchor": (ctypes.c_int, [D, P, P, P, P, P, P, P, P, P, S, St]),
        "mcs_residual": (ctypes.c_int, [D, P, P, P, P, P, P, P, St]),
        "mcs_reuse": (ctypes.c_int, [D, P, P, P, P, P, P, P, St]),
        "mcs_idx_to_bits": (ctypes.c_int, [D, P, P, St]),
        "mcs_bits_to_idx": (ctypes.c_int, [D, P, P, St]),
        "mcs_pair_plan": (ctypes.c_int, [D, P, P, P, St]),
        "mcs_block_select": (ctypes.c_int, [D, P, P, P, P, S, St]),
        "mcs_sparse_lse": (ctypes.c_int, [D, P, P, P, P, P, St]),
        "mcs_sparse_attn_pairs": (ctypes.c_int, [D, P, P, P, P, P, P, P, P, St]),
        "mcs_copy_async": (ctypes.c_int, [P, P, S, I32, St, P]),
    }
    for name, (res, args) in sig.items():
        f = getattr(lib, name)
        f.restype = res
        f.argtypes = args
    if lib.mcs_abi_version() != ABI_VERSION:
        raise McsError(MCS_EHIP, "libmcs.so ABI version mismatch")
    _lib = lib
    return lib


def check(rc):
    if rc != MCS_OK:
        raise McsError(rc, load().mcs_last_error().decode())
    return rc
