"""The C-ABI library loads, exports every entry point include/dit_attn.h
declares, and rejects bad arguments before any HIP call (so these run on a
machine without a GPU)."""
import ctypes
import json
import os
import re

import pytest

from helpers import ensure_built

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def L():
    return ensure_built()


def header_functions():
    with open(os.path.join(ROOT, "include", "dit_attn.h")) as fh:
        text = fh.read()
    return sorted(set(re.findall(r"DIT_API\s+[\w\s\*]+?\b(dit_\w+)\s*\(", text)))


def test_header_declares_the_boundary():
    names = header_functions()
    for want in ("dit_attn_fwd", "dit_lse_merge", "dit_rope_split_tables", "dit_pad_tokens", "dit_pad_tokens_rope",
                 "dit_unpad_tokens"):
        assert want in names


def test_library_exports_every_declared_symbol(L):
    from long_sequence_attention_amd import _native as N
    for name in header_functions():
        assert hasattr(L, name), name
    assert set(header_functions()) == set(N.EXPORTED)


def test_plan_padding_matches_the_pages(L):
    with open(os.path.join(ROOT, "tests", "golden", "padding_plans.json")) as fh:
        cases = json.load(fh)["cases"]
    out = ctypes.c_int()
    for c in cases:
        assert L.dit_plan_padding(c["s_valid"], c["multiple"], ctypes.byref(out)) == 0
        assert out.value == c["s_pad"], c["cite"]
    assert L.dit_plan_padding(10, 0, ctypes.byref(out)) == -1
    assert b"multiple" in L.dit_last_error()


def _desc(**kw):
    from long_sequence_attention_amd._native import AttnDesc
    d = AttnDesc()
    d.B, d.H, d.d, d.s_q, d.s_kv, d.q_valid, d.kv_valid = 1, 2, 128, 256, 256, 256, 256
    fake = 0x10000000  # never dereferenced: validation fails first
    d.q = d.k = d.v = d.o = fake
    for k, v in kw.items():
        setattr(d, k, v)
    return d


@pytest.mark.parametrize("kw,code,msg", [
    (dict(d=96), -2, b"d in {64, 128}"),
    (dict(d=63), -1, b"even"),
    (dict(q_valid=300), -1, b"q_valid"),
    (dict(kv_valid=-1), -1, b"kv_valid"),
    (dict(B=0), -1, b"B and H"),
    (dict(q=None), -1, b"q and o"),
    (dict(k=None), -1, b"k and v"),
    (dict(o_dtype=7), -1, b"o_dtype"),
    (dict(sm_scale=-1.0), -1, b"sm_scale"),
    (dict(sm_scale=float("nan")), -1, b"sm_scale"),
    (dict(cos_q=0x20000000), -1, b"cos_q and sin_q"),
    (dict(sin_k=0x20000000), -1, b"cos_k and sin_k"),
    (dict(q=0x10000008), -2, b"16-byte aligned"),
    (dict(q_norm_w=0x20000000, norm_eps=-1.0), -1, b"norm_eps"),
    (dict(k_norm_w=0x20000000, norm_eps=float("inf")), -1, b"norm_eps"),
    (dict(k_norm_w=0x20000004, norm_eps=1e-6), -2, b"16-byte aligned"),
    (dict(kv_seg_len=100), -1, b"multiple of kv_seg_len"),
    (dict(q_seg_len=96), -1, b"multiple of q_seg_len"),
    (dict(kv_seg_len=128, kv_valid=129), -1, b"kv_valid"),
    (dict(q_seg_len=128, q_valid=200), -1, b"q_valid"),
    (dict(kv_seg_len=32, kv_valid=32), -2, b"key tile"),
    (dict(kv_seg_len=-1), -1, b"segment lengths"),
    (dict(fixed_m=3), -1, b"fixed_m"),
    (dict(ws_counters_zero=3), -1, b"ws_counters_zero"),
    (dict(schedule=4), -1, b"schedule"),
    (dict(schedule=-1), -1, b"schedule"),
])
def test_attn_fwd_rejects_bad_arguments_before_any_hip_call(L, kw, code, msg):
    d = _desc(**kw)
    assert L.dit_attn_fwd(ctypes.byref(d), None) == code
    assert msg in L.dit_last_error()
    # the allocation-free entry point validates the same way, before any HIP call
    assert L.dit_attn_fwd_noalloc(ctypes.byref(d), None) == code
    assert msg in L.dit_last_error()


def test_attn_fwd_rejects_bad_strides_and_missing_workspace(L):
    d = _desc()
    d.q_stride[:] = (256 * 2 * 128, 128, 132)
    assert L.dit_attn_fwd(ctypes.byref(d), None) == -2
    assert b"multiples of 8" in L.dit_last_error()
    d = _desc(cos_k=0x20000000, sin_k=0x20000000)
    assert L.dit_attn_fwd(ctypes.byref(d), None) == -1
    assert b"workspace" in L.dit_last_error()
    size = ctypes.c_size_t()
    assert L.dit_attn_workspace_size(ctypes.byref(d), ctypes.byref(size)) == 0
    assert size.value == 1 * 2 * 256 * 128 * 2
    d = _desc()
    assert L.dit_attn_workspace_size(ctypes.byref(d), ctypes.byref(size)) == 0 and size.value == 0
    # norm weights alone also need the prepared copy (Q after K, 256-byte aligned)
    d = _desc(q_norm_w=0x20000000, k_norm_w=0x20000000, norm_eps=1e-6)
    assert L.dit_attn_workspace_size(ctypes.byref(d), ctypes.byref(size)) == 0
    assert size.value == 2 * (1 * 2 * 256 * 128 * 2)
    assert L.dit_attn_fwd(ctypes.byref(d), None) == -1 and b"workspace" in L.dit_last_error()
    assert L.dit_attn_fwd(None, None) == -1


def test_merge_tables_pad_reject_bad_arguments(L):
    vp = ctypes.c_void_p
    parts = (vp * 2)(0x10000000, 0x10000000)
    assert L.dit_lse_merge(0, parts, parts, 1, 1, 1, 8, 128, 8, vp(0x10000000), 0, None, None) == -1
    assert L.dit_lse_merge(17, parts, parts, 1, 1, 1, 8, 128, 8, vp(0x10000000), 0, None, None) == -1
    assert L.dit_lse_merge(2, parts, parts, 1, 1, 1, 8, 96, 8, vp(0x10000000), 0, None, None) == -2
    assert L.dit_lse_merge(2, parts, parts, 1, 1, 1, 8, 128, 9, vp(0x10000000), 0, None, None) == -1
    chans = (ctypes.c_int32 * 3)(44, 42, 40)
    assert L.dit_rope_split_tables(vp(0x10000000), 10, 3, chans, 128, 10000.0, vp(0x1000), vp(0x1000), None) == -1
    assert b"sum to 126" in L.dit_last_error()
    chans = (ctypes.c_int32 * 3)(44, 43, 41)
    assert L.dit_rope_split_tables(vp(0x10000000), 10, 3, chans, 128, 10000.0, vp(0x1000), vp(0x1000), None) == -1
    assert L.dit_pad_tokens(vp(0x1000), vp(0x2000), 1, 10, 5, 256, None) == -1
    assert L.dit_unpad_tokens(vp(0x1000), vp(0x1000), 1, 10, 5, 256, None) == -1
    assert L.dit_pad_tokens(vp(0x1000), vp(0x2000), 1, 10, 16, 0, None) == -1
    # fused pad + rotation: shape, d, alias, tables, alignment and size checks
    t = vp(0x30000000)
    rope = L.dit_pad_tokens_rope
    assert rope(vp(0x1000), vp(0x2000), 1, 10, 5, 3, 2, 128, 2, t, t, None) == -1
    assert rope(vp(0x1000), vp(0x2000), 1, 10, 16, 3, 2, 128, 4, t, t, None) == -1
    assert b"n_rot" in L.dit_last_error()
    assert rope(vp(0x1000), vp(0x2000), 1, 10, 16, 0, 2, 128, 0, t, t, None) == -1
    assert rope(vp(0x1000), vp(0x2000), 1, 10, 16, 3, 2, 96, 2, t, t, None) == -2
    assert rope(vp(0x1000), vp(0x1000), 1, 10, 16, 3, 2, 128, 2, t, t, None) == -1
    assert b"alias" in L.dit_last_error()
    assert rope(vp(0x1000), vp(0x2000), 1, 10, 16, 3, 2, 128, 2, None, t, None) == -1
    assert b"cos_t" in L.dit_last_error()
    assert rope(vp(0x1008), vp(0x2000), 1, 10, 16, 3, 2, 128, 2, t, t, None) == -1
    assert b"16-byte" in L.dit_last_error()
    assert rope(vp(0x1000), vp(0x2000), 70000, 10, 16, 3, 2, 128, 2, t, t, None) == -2
    assert rope(vp(0x1000), vp(0x2000), 1, 10, 1 << 24, 3, 24, 128, 2, t, t, None) == -2
    assert b"2^31" in L.dit_last_error()
    assert rope(None, None, 1, 0, 0, 3, 2, 128, 2, None, None, None) == 0   # nothing to do, no launch
