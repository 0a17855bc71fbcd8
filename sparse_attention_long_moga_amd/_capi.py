"""ctypes declarations of the C ABI in include/moga.h (libmoga.so)."""
from __future__ import annotations

import ctypes
import os

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libmoga.so")

MOGA_OK, MOGA_ERR_ARG, MOGA_ERR_UNSUPPORTED, MOGA_ERR_WORKSPACE, MOGA_ERR_HIP = range(5)
MOGA_F32, MOGA_BF16 = 0, 1
STATUS_NAMES = {0: "MOGA_OK", 1: "MOGA_ERR_ARG", 2: "MOGA_ERR_UNSUPPORTED",
                3: "MOGA_ERR_WORKSPACE", 4: "MOGA_ERR_HIP"}

EXPORTS = ["moga_last_error", "moga_workspace_bytes", "moga_group_attn_workspace_bytes",
           "moga_route", "moga_permute", "moga_group_attn", "stga_group_attn",
           "moga_balance_loss", "moga_forward", "moga_forward_fused",
           "moga_backward_workspace_bytes", "moga_backward", "moga_group_attn_noalloc",
           "moga_hybrid_backward_workspace_bytes", "moga_hybrid_backward"]


class MogaDims(ctypes.Structure):
    _fields_ = [("n_tokens", ctypes.c_int64), ("d_model", ctypes.c_int32),
                ("n_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("n_groups", ctypes.c_int32), ("softmax_scale", ctypes.c_float),
                ("alpha", ctypes.c_double)]


class StgaLayout(ctypes.Structure):
    _fields_ = [("frames", ctypes.c_int32), ("height", ctypes.c_int32),
                ("width", ctypes.c_int32), ("n_shots", ctypes.c_int32),
                ("shot_start", ctypes.POINTER(ctypes.c_int32)), ("win_h", ctypes.c_int32),
                ("win_w", ctypes.c_int32), ("t_group", ctypes.c_int32),
                ("aug_frames", ctypes.c_int32)]


class MogaInputs(ctypes.Structure):
    _fields_ = [("x", ctypes.c_void_p), ("x_dtype", ctypes.c_int), ("w", ctypes.c_void_p),
                ("q", ctypes.c_void_p), ("k", ctypes.c_void_p), ("v", ctypes.c_void_p),
                ("pin", ctypes.c_void_p)]


class MogaOutputs(ctypes.Structure):
    _fields_ = [("out", ctypes.c_void_p), ("loss", ctypes.c_void_p),
                ("group_id", ctypes.c_void_p), ("p_sel", ctypes.c_void_p),
                ("cu_seqlens", ctypes.c_void_p), ("perm", ctypes.c_void_p),
                ("counts", ctypes.c_void_p), ("prob_sum", ctypes.c_void_p),
                ("lse", ctypes.c_void_p), ("o_branches", ctypes.c_void_p)]


class MogaSaved(ctypes.Structure):
    _fields_ = [("group_id", ctypes.c_void_p), ("p_sel", ctypes.c_void_p),
                ("counts", ctypes.c_void_p), ("cu_seqlens", ctypes.c_void_p),
                ("perm", ctypes.c_void_p), ("out", ctypes.c_void_p), ("lse", ctypes.c_void_p)]


class MogaGrads(ctypes.Structure):
    _fields_ = [("dq", ctypes.c_void_p), ("dk", ctypes.c_void_p), ("dv", ctypes.c_void_p),
                ("dx", ctypes.c_void_p), ("dw", ctypes.c_void_p), ("dp", ctypes.c_void_p)]


_lib = None


def load(path: str = LIB_PATH):
    """Load libmoga.so and declare every entry point.  Raises if it is missing."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is not built; run __graft_entry__.build() "
                           "(python -m sparse_attention_long_moga_amd.build)")
    # torch ships its own HIP runtime under the same soname; loading torch first makes the
    # library bind to that one instead of pulling a second runtime into the process
    import torch  # noqa: F401
    lib = ctypes.CDLL(path)
    vp, sz, st, i32, i64 = (ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int, ctypes.c_int32,
                            ctypes.c_int64)
    pdims, pstga = ctypes.POINTER(MogaDims), ctypes.POINTER(StgaLayout)
    lib.moga_last_error.argtypes = []
    lib.moga_last_error.restype = ctypes.c_char_p
    lib.moga_workspace_bytes.argtypes = [pdims, pstga]
    lib.moga_workspace_bytes.restype = sz
    lib.moga_group_attn_workspace_bytes.argtypes = [pdims, i32, i64]
    lib.moga_group_attn_workspace_bytes.restype = sz
    lib.moga_route.argtypes = [vp, ctypes.c_int, vp, vp, pdims, vp, vp, vp, vp, vp, sz, vp]
    lib.moga_route.restype = st
    lib.moga_permute.argtypes = [ctypes.c_int, vp, pdims, vp, vp, ctypes.POINTER(vp),
                                 ctypes.POINTER(vp), ctypes.c_int, vp, vp, vp, sz, vp]
    lib.moga_permute.restype = st
    lib.moga_group_attn.argtypes = [vp, vp, vp, i64, i64, i32, vp, vp, vp, pdims, vp, vp, sz, vp]
    lib.moga_group_attn.restype = st
    lib.moga_group_attn_noalloc.argtypes = [vp, vp, vp, i64, i64, i32, vp, vp, vp, pdims, vp, vp]
    lib.moga_group_attn_noalloc.restype = st
    lib.stga_group_attn.argtypes = [vp, vp, vp, pdims, pstga, vp, vp, vp, sz, vp]
    lib.stga_group_attn.restype = st
    lib.moga_balance_loss.argtypes = [vp, vp, pdims, vp, vp, vp, vp]
    lib.moga_balance_loss.restype = st
    lib.moga_forward.argtypes = [ctypes.POINTER(MogaInputs), pdims, pstga,
                                 ctypes.POINTER(MogaOutputs), vp, sz, vp]
    lib.moga_forward.restype = st
    lib.moga_forward_fused.argtypes = lib.moga_forward.argtypes
    lib.moga_forward_fused.restype = st
    lib.moga_backward_workspace_bytes.argtypes = [pdims]
    lib.moga_backward_workspace_bytes.restype = sz
    lib.moga_backward.argtypes = [ctypes.POINTER(MogaInputs), ctypes.POINTER(MogaSaved), vp,
                                  ctypes.c_double, pdims, ctypes.POINTER(MogaGrads), vp, sz, vp]
    lib.moga_backward.restype = st
    lib.moga_hybrid_backward_workspace_bytes.argtypes = [pdims, pstga]
    lib.moga_hybrid_backward_workspace_bytes.restype = sz
    lib.moga_hybrid_backward.argtypes = [ctypes.POINTER(MogaInputs), ctypes.POINTER(MogaSaved),
                                         pstga, vp, ctypes.c_double, pdims,
                                         ctypes.POINTER(MogaGrads), vp, sz, vp]
    lib.moga_hybrid_backward.restype = st
    _lib = lib
    return lib


class MogaError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{STATUS_NAMES.get(status, status)}: {message}")
        self.status = status


def check(status: int):
    if status != MOGA_OK:
        raise MogaError(status, load().moga_last_error().decode(errors="replace"))
