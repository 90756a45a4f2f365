"""ctypes view of libditattn.so (the C ABI in include/dit_attn.h).

Loading fails loudly when the library has not been built: there is no other
implementation to fall back to.
"""
from __future__ import annotations

import ctypes
import os

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "lib", "libditattn.so")

DIT_OK = 0
DIT_ERR_INVALID = -1
DIT_ERR_UNSUPPORTED = -2
DIT_ERR_HIP = -3
DIT_BF16 = 0
DIT_F32 = 1
DIT_SCHED_AUTO = 0
DIT_SCHED_PER_QTILE = 1
DIT_SCHED_BALANCED = 2
DIT_SCHED_DYNAMIC = 3

EXPORTED = (
    "dit_attn_workspace_size",
    "dit_attn_fwd",
    "dit_attn_fwd_noalloc",
    "dit_lse_merge",
    "dit_rope_split_tables",
    "dit_pad_tokens",
    "dit_pad_tokens_rope",
    "dit_unpad_tokens",
    "dit_plan_padding",
    "dit_last_error",
)


class AttnDesc(ctypes.Structure):
    """Mirror of dit_attn_desc (field order and C types must match)."""
    _fields_ = [
        ("B", ctypes.c_int32), ("H", ctypes.c_int32), ("d", ctypes.c_int32),
        ("s_q", ctypes.c_int32), ("s_kv", ctypes.c_int32),
        ("q_valid", ctypes.c_int32), ("kv_valid", ctypes.c_int32),
        ("o_dtype", ctypes.c_int32),
        ("q", ctypes.c_void_p), ("k", ctypes.c_void_p), ("v", ctypes.c_void_p),
        ("o", ctypes.c_void_p),
        ("lse", ctypes.c_void_p),
        ("q_stride", ctypes.c_int64 * 3), ("k_stride", ctypes.c_int64 * 3),
        ("v_stride", ctypes.c_int64 * 3), ("o_stride", ctypes.c_int64 * 3),
        ("sm_scale", ctypes.c_float),
        ("cos_q", ctypes.c_void_p), ("sin_q", ctypes.c_void_p),
        ("cos_k", ctypes.c_void_p), ("sin_k", ctypes.c_void_p),
        ("workspace", ctypes.c_void_p),
        ("workspace_bytes", ctypes.c_size_t),
        ("schedule", ctypes.c_int32),
        ("q_norm_w", ctypes.c_void_p), ("k_norm_w", ctypes.c_void_p),
        ("norm_eps", ctypes.c_float),
        ("q_seg_len", ctypes.c_int32), ("kv_seg_len", ctypes.c_int32),
        ("fixed_m", ctypes.c_int32),
        ("ws_counters_zero", ctypes.c_int32),
    ]


class DitError(RuntimeError):
    pass


_lib = None


def lib() -> ctypes.CDLL:
    """Load the library once. Raises if it is missing."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"{LIB_PATH} is missing: build it with `python -m long_sequence_attention_amd.build` "
            "(there is no non-HIP implementation)")
    L = ctypes.CDLL(LIB_PATH)
    vp, i32, i64, f32 = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_float
    L.dit_attn_workspace_size.argtypes = [ctypes.POINTER(AttnDesc), ctypes.POINTER(ctypes.c_size_t)]
    L.dit_attn_fwd.argtypes = [ctypes.POINTER(AttnDesc), vp]
    L.dit_attn_fwd_noalloc.argtypes = [ctypes.POINTER(AttnDesc), vp]
    L.dit_lse_merge.argtypes = [i32, ctypes.POINTER(vp), ctypes.POINTER(vp), i32, i32, i32, i32, i32, i32,
                                vp, i32, vp, vp]
    L.dit_rope_split_tables.argtypes = [vp, i32, i32, ctypes.POINTER(ctypes.c_int32), i32, f32, vp, vp, vp]
    L.dit_pad_tokens.argtypes = [vp, vp, i32, i32, i32, i64, vp]
    L.dit_unpad_tokens.argtypes = [vp, vp, i32, i32, i32, i64, vp]
    L.dit_pad_tokens_rope.argtypes = [vp, vp, i32, i32, i32, i32, i32, i32, i32, vp, vp, vp]
    L.dit_plan_padding.argtypes = [i32, i32, ctypes.POINTER(ctypes.c_int)]
    L.dit_last_error.argtypes = []
    L.dit_last_error.restype = ctypes.c_char_p
    for name in EXPORTED[:-1]:
        getattr(L, name).restype = ctypes.c_int
    _lib = L
    return L


def check(rc: int, what: str) -> None:
    """Map a dit_status to a Python exception (ValueError / NotImplementedError / RuntimeError)."""
    if rc == DIT_OK:
        return
    msg = lib().dit_last_error().decode(errors="replace")
    if rc == DIT_ERR_INVALID:
        raise ValueError(f"{what}: {msg}")
    if rc == DIT_ERR_UNSUPPORTED:
        raise NotImplementedError(f"{what}: {msg}")
    raise DitError(f"{what} failed ({rc}): {msg}")
