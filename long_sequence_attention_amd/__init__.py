"""Python binding of the MI355X DiT self-attention library (libditattn.so).

Argument marshalling only: every step of the path runs in the HIP kernels
behind the C ABI (include/dit_attn.h). torch supplies device memory and the
current stream. Function names follow the C entry points without the `dit_`
prefix.
"""
from __future__ import annotations

import contextlib
import ctypes
import math

import torch

from . import _native as N
from ._native import DitError  # noqa: F401

__all__ = ["attn_fwd", "attn_fwd_noalloc", "lse_merge", "rope_split_tables", "pad_tokens", "pad_tokens_rope", "unpad_tokens",
           "plan_padding", "library_path", "attn_workspace_size", "NOALLOC_SCRATCH_BYTES"]

NOALLOC_SCRATCH_BYTES = 128 << 20   # DIT_NOALLOC_SCRATCH_BYTES


def library_path() -> str:
    N.lib()
    return N.LIB_PATH


def _on_device(dev: torch.device):
    """Make dev current for the library call (it launches on the current
    device); a no-op when it already is."""
    if dev.index is None or torch.cuda.current_device() == dev.index:
        return contextlib.nullcontext()
    return torch.cuda.device(dev)


def _stream(dev: torch.device) -> ctypes.c_void_p:
    return ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _need_cuda(name, t, dtype=None):
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise ValueError(f"{name} must be a CUDA (HIP) tensor")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")


def _same_device(dev, **tensors):
    for name, t in tensors.items():
        if t is not None and t.device != dev:
            raise ValueError(f"{name} is on {t.device}, expected {dev}")


def _check_out(name, t, shape, dtypes, dev):
    """A caller-provided output: on dev, one of dtypes, exactly shape, dense."""
    _need_cuda(name, t)
    if t.dtype not in dtypes or tuple(t.shape) != tuple(shape) or not t.is_contiguous() or t.device != dev:
        raise ValueError(f"{name} must be a dense {' or '.join(str(x) for x in dtypes)} tensor of shape "
                         f"{tuple(shape)} on {dev}; got {t.dtype} {tuple(t.shape)} on {t.device}")


def _strides4(name, t):
    if t.dim() != 4:
        raise ValueError(f"{name} must be 4-D [B, H, S, d] (any layout with d contiguous)")
    if t.stride(-1) != 1:
        raise NotImplementedError(f"{name}: the head dimension must be contiguous")
    return (t.stride(0), t.stride(1), t.stride(2))


def plan_padding(s_valid: int, multiple: int) -> int:
    out = ctypes.c_int()
    N.check(N.lib().dit_plan_padding(int(s_valid), int(multiple), ctypes.byref(out)), "plan_padding")
    return out.value


def _attn_desc(q, k, v, o, lse, q_valid, kv_valid, rope_q, rope_k, sm_scale, schedule=0,
               q_norm=None, k_norm=None, norm_eps=1e-6, q_seg_len=0, kv_seg_len=0, fixed_m=None,
               ws_counters_zero=False):
    B, H, s_q, d = q.shape
    desc = N.AttnDesc()
    desc.B, desc.H, desc.d = B, H, d
    desc.s_q, desc.s_kv = s_q, k.shape[2]
    desc.q_valid, desc.kv_valid = q_valid, kv_valid
    desc.o_dtype = N.DIT_F32 if o.dtype == torch.float32 else N.DIT_BF16
    desc.q, desc.k, desc.v, desc.o = q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr()
    desc.lse = lse.data_ptr() if lse is not None else None
    for field, t, name in (("q_stride", q, "q"), ("k_stride", k, "k"), ("v_stride", v, "v"), ("o_stride", o, "out")):
        getattr(desc, field)[:] = _strides4(name, t)
    desc.sm_scale = float(sm_scale)
    if rope_q is not None:
        desc.cos_q, desc.sin_q = rope_q[0].data_ptr(), rope_q[1].data_ptr()
    if rope_k is not None:
        desc.cos_k, desc.sin_k = rope_k[0].data_ptr(), rope_k[1].data_ptr()
    desc.schedule = int(schedule)
    if q_norm is not None:
        desc.q_norm_w = q_norm.data_ptr()
    if k_norm is not None:
        desc.k_norm_w = k_norm.data_ptr()
    desc.norm_eps = float(norm_eps)
    desc.q_seg_len, desc.kv_seg_len = int(q_seg_len), int(kv_seg_len)
    desc.fixed_m = 0 if fixed_m is None else (1 if fixed_m else 2)
    desc.ws_counters_zero = 1 if ws_counters_zero else 0
    return desc


def attn_workspace_size(q, k, v, *, q_valid=None, kv_valid=None, rope_q=None, rope_k=None, schedule=0,
                        q_norm=None, k_norm=None, q_seg_len=0, kv_seg_len=0, fixed_m=None) -> int:
    """Workspace bytes attn_fwd needs (dit_attn_workspace_size) on q's device."""
    q_valid = (q_seg_len or q.shape[2]) if q_valid is None else int(q_valid)
    kv_valid = (kv_seg_len or k.shape[2]) if kv_valid is None else int(kv_valid)
    desc = _attn_desc(q, k, v, q, None, q_valid, kv_valid, rope_q, rope_k, 0.0, schedule, q_norm, k_norm,
                      q_seg_len=q_seg_len, kv_seg_len=kv_seg_len, fixed_m=fixed_m)
    need = ctypes.c_size_t()
    with _on_device(q.device):
        N.check(N.lib().dit_attn_workspace_size(ctypes.byref(desc), ctypes.byref(need)), "attn_workspace_size")
    return need.value


def attn_fwd(q, k, v, *, q_valid=None, kv_valid=None, rope_q=None, rope_k=None, sm_scale=0.0,
             out=None, out_dtype=torch.bfloat16, lse=None, return_lse=True, workspace=None, schedule=0,
             q_norm=None, k_norm=None, norm_eps=1e-6, q_seg_len=0, kv_seg_len=0, fixed_m=None,
             ws_counters_zero=False, _noalloc=False):
    """Attention forward (dit_attn_fwd).

    q: [B, H, s_q, d], k/v: [B, H, s_kv, d] bf16 device tensors, any strides
    with d contiguous (e.g. a permuted [B, S, H, d] buffer). Rows >= q_valid /
    kv_valid are tail pads. rope_q / rope_k: (cos, sin) fp32 [S, d/2] tables
    or None. schedule: 0 auto, 1 one workgroup per query tile, 2 balanced
    (split key ranges, Stream-K style), 3 dynamic (one workgroup per query
    tile, tiles taken at run time from per-XCD queues; auto from four query
    tiles per compute unit).
    q_norm / k_norm: fp32 [d] RMSNorm weights (per-head q/k RMS normalisation
    before RoPE, epsilon norm_eps) or None. q_seg_len / kv_seg_len > 0: the
    rows form segments of that length, each padded at its own tail, and
    q_valid / kv_valid count the real rows of each segment. fixed_m: True =
    the fixed-m softmax (a-priori row-max bound where it is tight enough),
    False = the online softmax, None = AUTO (fixed-m for at least 32768 real
    keys per head; dit_attn_desc.fixed_m).
    ws_counters_zero: the caller's `workspace` comes unchanged from an earlier
    completed call with the same arguments, so its schedule counters are
    already zero and the call skips clearing them.
    Returns (O, LSE) with O [B, H, s_q, d] in out_dtype (or `out`) and LSE
    fp32 [B, H, s_q] (natural log), or O alone if return_lse=False.
    """
    for name, t in (("q", q), ("k", k), ("v", v)):
        _need_cuda(name, t, torch.bfloat16)
    _same_device(q.device, k=k, v=v, out=out, lse=lse, workspace=workspace, q_norm=q_norm, k_norm=k_norm,
                 cos_q=None if rope_q is None else rope_q[0], sin_q=None if rope_q is None else rope_q[1],
                 cos_k=None if rope_k is None else rope_k[0], sin_k=None if rope_k is None else rope_k[1])
    B, H, s_q, d = q.shape
    if k.shape[:2] != (B, H) or v.shape != k.shape or k.shape[3] != d:
        raise ValueError(f"shape mismatch: q {tuple(q.shape)}, k {tuple(k.shape)}, v {tuple(v.shape)}")
    q_valid = (q_seg_len or s_q) if q_valid is None else int(q_valid)
    kv_valid = (kv_seg_len or k.shape[2]) if kv_valid is None else int(kv_valid)
    for name, tab, rows in (("rope_q", rope_q, s_q), ("rope_k", rope_k, k.shape[2])):
        if tab is not None:
            for t in tab:
                _need_cuda(name, t, torch.float32)
                if t.shape != (rows, d // 2) or not t.is_contiguous():
                    raise ValueError(f"{name} tables must be contiguous fp32 [{rows}, {d // 2}]")
    if out is None:
        out = torch.empty((B, H, s_q, d), dtype=out_dtype, device=q.device)
    else:
        _need_cuda("out", out)
        if out.dtype not in (torch.bfloat16, torch.float32) or out.shape != (B, H, s_q, d):
            raise ValueError("out must be bf16 or fp32 [B, H, s_q, d]")
    if lse is None and return_lse:
        lse = torch.empty((B, H, s_q), dtype=torch.float32, device=q.device)
    if lse is not None:
        _need_cuda("lse", lse, torch.float32)
        if lse.shape != (B, H, s_q) or not lse.is_contiguous():
            raise ValueError("lse must be contiguous fp32 [B, H, s_q]")
    for name, wt in (("q_norm", q_norm), ("k_norm", k_norm)):
        if wt is not None:
            _need_cuda(name, wt, torch.float32)
            if wt.shape != (d,) or not wt.is_contiguous():
                raise ValueError(f"{name} must be a contiguous fp32 [{d}] tensor")
    if ws_counters_zero and workspace is None:
        raise ValueError("ws_counters_zero needs the caller's workspace")
    desc = _attn_desc(q, k, v, out, lse, q_valid, kv_valid, rope_q, rope_k, sm_scale, schedule, q_norm, k_norm,
                      norm_eps, q_seg_len, kv_seg_len, fixed_m, ws_counters_zero)
    with _on_device(q.device):
        if _noalloc:
            N.check(N.lib().dit_attn_fwd_noalloc(ctypes.byref(desc), _stream(q.device)), "attn_fwd_noalloc")
            return (out, lse) if return_lse else out
        if workspace is None:   # ask the library how much it needs and allocate that
            need = ctypes.c_size_t()
            N.check(N.lib().dit_attn_workspace_size(ctypes.byref(desc), ctypes.byref(need)), "attn_fwd")
            if need.value:
                workspace = torch.empty(need.value, dtype=torch.uint8, device=q.device)
        if workspace is not None:   # the library checks its size against the call
            _need_cuda("workspace", workspace)
            if not workspace.is_contiguous():
                raise ValueError("workspace must be a dense tensor")
            desc.workspace = workspace.data_ptr()
            desc.workspace_bytes = workspace.numel() * workspace.element_size()
        N.check(N.lib().dit_attn_fwd(ctypes.byref(desc), _stream(q.device)), "attn_fwd")
    return (out, lse) if return_lse else out


def attn_fwd_noalloc(q, k, v, *, q_valid=None, kv_valid=None, rope_q=None, rope_k=None, sm_scale=0.0,
                     out=None, out_dtype=torch.bfloat16, lse=None, return_lse=True, schedule=0,
                     q_norm=None, k_norm=None, norm_eps=1e-6, q_seg_len=0, kv_seg_len=0, fixed_m=None):
    """dit_attn_fwd_noalloc: attn_fwd with the library's static device scratch
    (NOALLOC_SCRATCH_BYTES per GPU) as the workspace; the library allocates
    nothing (pass `out` and `lse` to allocate nothing here either). Calls on
    one GPU share the scratch and must not overlap."""
    return attn_fwd(q, k, v, q_valid=q_valid, kv_valid=kv_valid, rope_q=rope_q, rope_k=rope_k, sm_scale=sm_scale,
                    out=out, out_dtype=out_dtype, lse=lse, return_lse=return_lse, schedule=schedule, q_norm=q_norm,
                    k_norm=k_norm, norm_eps=norm_eps, q_seg_len=q_seg_len, kv_seg_len=kv_seg_len, fixed_m=fixed_m,
                    _noalloc=True)


def lse_merge(o_parts, lse_parts, *, q_valid=None, out_dtype=torch.bfloat16, out=None, lse_out=None,
              return_lse=True):
    """Merge partial (O, LSE) results over key shards (dit_lse_merge).

    o_parts: list of dense [B, H, S, d] bf16/fp32 tensors (one dtype);
    lse_parts: list of dense fp32 [B, H, S].
    """
    n = len(o_parts)
    if n != len(lse_parts) or n == 0:
        raise ValueError("need matching, non-empty lists of O and LSE parts")
    B, H, S, d = o_parts[0].shape
    pdt = o_parts[0].dtype
    for o, l in zip(o_parts, lse_parts):
        _need_cuda("o_part", o)
        _need_cuda("lse_part", l, torch.float32)
        if o.dtype != pdt or o.shape != (B, H, S, d) or not o.is_contiguous():
            raise ValueError("O parts must share dtype and be dense [B, H, S, d]")
        if l.shape != (B, H, S) or not l.is_contiguous():
            raise ValueError("LSE parts must be dense fp32 [B, H, S]")
    q_valid = S if q_valid is None else int(q_valid)
    dev = o_parts[0].device
    _same_device(dev, **{f"o_part{i}": o for i, o in enumerate(o_parts)},
                 **{f"lse_part{i}": l for i, l in enumerate(lse_parts)})
    if out is None:
        out = torch.empty((B, H, S, d), dtype=out_dtype, device=dev)
    else:
        _check_out("out", out, (B, H, S, d), (torch.bfloat16, torch.float32), dev)
    if lse_out is None and return_lse:
        lse_out = torch.empty((B, H, S), dtype=torch.float32, device=dev)
    elif lse_out is not None:
        _check_out("lse_out", lse_out, (B, H, S), (torch.float32,), dev)
    optr = (ctypes.c_void_p * n)(*[o.data_ptr() for o in o_parts])
    lptr = (ctypes.c_void_p * n)(*[l.data_ptr() for l in lse_parts])
    with _on_device(dev):
        rc = N.lib().dit_lse_merge(n, optr, lptr, N.DIT_F32 if pdt == torch.float32 else N.DIT_BF16,
                                   B, H, S, d, q_valid, _ptr(out),
                                   N.DIT_F32 if out.dtype == torch.float32 else N.DIT_BF16,
                                   _ptr(lse_out), _stream(dev))
    N.check(rc, "lse_merge")
    return (out, lse_out) if return_lse else out


def rope_split_tables(pos, axis_channels, d: int, theta: float = 10000.0):
    """cos, sin fp32 [S, d/2] from int32 positions [S, n_axes] (dit_rope_split_tables)."""
    _need_cuda("pos", pos, torch.int32)
    if pos.dim() == 1:
        pos = pos[:, None]
    pos = pos.contiguous()
    S, n_axes = pos.shape
    chans = (ctypes.c_int32 * len(axis_channels))(*[int(c) for c in axis_channels])
    if len(axis_channels) != n_axes:
        raise ValueError("one channel count per position column")
    cos = torch.empty((S, d // 2), dtype=torch.float32, device=pos.device)
    sin = torch.empty_like(cos)
    with _on_device(pos.device):
        N.check(N.lib().dit_rope_split_tables(_ptr(pos), S, n_axes, chans, int(d), float(theta), _ptr(cos),
                                              _ptr(sin), _stream(pos.device)), "rope_split_tables")
    return cos, sin


def pad_tokens(x, s_pad: int, out=None):
    """[B, s_valid, ...] -> [B, s_pad, ...] with zero tail rows (dit_pad_tokens)."""
    _need_cuda("x", x)
    if not x.is_contiguous():
        raise ValueError("x must be contiguous")
    B, s_valid = x.shape[:2]
    row_bytes = x.element_size() * math.prod(x.shape[2:])
    if out is None:
        out = torch.empty((B, s_pad) + tuple(x.shape[2:]), dtype=x.dtype, device=x.device)
    else:
        _check_out("out", out, (B, int(s_pad)) + tuple(x.shape[2:]), (x.dtype,), x.device)
    with _on_device(x.device):
        N.check(N.lib().dit_pad_tokens(_ptr(x), _ptr(out), B, s_valid, int(s_pad), row_bytes, _stream(x.device)),
                "pad_tokens")
    return out


def pad_tokens_rope(x, s_pad: int, cos, sin, n_rot: int = 2, out=None):
    """Fused token rows [B, s_valid, T, H, d] (bf16, dense) -> [B, s_pad, T, H, d]
    with zero tail rows, the head vectors of the first n_rot tensors of every
    real row rotated (split halves) with row s of cos / sin (fp32 [>= s_valid,
    d/2]) on the way (dit_pad_tokens_rope)."""
    _need_cuda("x", x, torch.bfloat16)
    if not x.is_contiguous() or x.dim() != 5:
        raise ValueError("x must be a dense [B, s_valid, T, H, d] tensor")
    B, s_valid, T, H, d = x.shape
    _need_cuda("cos", cos, torch.float32)
    _need_cuda("sin", sin, torch.float32)
    _same_device(x.device, cos=cos, sin=sin)
    for name, t in (("cos", cos), ("sin", sin)):
        if t.dim() != 2 or t.shape[0] < s_valid or t.shape[1] != d // 2 or not t.is_contiguous():
            raise ValueError(f"{name} must be a dense fp32 [>= {s_valid}, {d // 2}] tensor")
    if out is None:
        out = torch.empty((B, int(s_pad), T, H, d), dtype=x.dtype, device=x.device)
    else:
        _check_out("out", out, (B, int(s_pad), T, H, d), (x.dtype,), x.device)
    with _on_device(x.device):
        N.check(N.lib().dit_pad_tokens_rope(_ptr(x), _ptr(out), B, s_valid, int(s_pad), T, H, d, int(n_rot),
                                            _ptr(cos), _ptr(sin), _stream(x.device)), "pad_tokens_rope")
    return out


def unpad_tokens(x, s_valid: int, out=None):
    """[B, s_pad, ...] -> [B, s_valid, ...] (dit_unpad_tokens)."""
    _need_cuda("x", x)
    if not x.is_contiguous():
        raise ValueError("x must be contiguous")
    B, s_pad = x.shape[:2]
    row_bytes = x.element_size() * math.prod(x.shape[2:])
    if out is None:
        out = torch.empty((B, int(s_valid)) + tuple(x.shape[2:]), dtype=x.dtype, device=x.device)
    else:
        _check_out("out", out, (B, int(s_valid)) + tuple(x.shape[2:]), (x.dtype,), x.device)
    with _on_device(x.device):
        N.check(N.lib().dit_unpad_tokens(_ptr(x), _ptr(out), B, s_pad, int(s_valid), row_bytes, _stream(x.device)),
                "unpad_tokens")
    return out
