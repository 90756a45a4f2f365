"""dit_attn_fwd_noalloc (the allocation-free entry point) through the C ABI:
its O and LSE equal dit_attn_fwd's on the same inputs, bit for bit, on two
calls in a row (Wan 480p with RoPE, whose workspace holds the rotated Q / K,
then the smaller 300-token d = 64 case), under the schedules whose
workspace also holds counters and partial results (the split and the
dynamic placement, which must find their counters cleared in the reused
scratch), and a call whose workspace exceeds the static scratch is refused
before any launch."""
import ctypes

import numpy as np
import pytest

import workloads as W
from helpers import ensure_built, raw_bits, to_dev_bf16

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def ops():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    ensure_built()
    import long_sequence_attention_amd as ops
    return ops


def _run_both(ops, name, schedule=0):
    """The same call through dit_attn_fwd (caller workspace) and through
    dit_attn_fwd_noalloc (ctypes, raw C ABI); returns both (O, LSE)."""
    import torch
    from long_sequence_attention_amd import _native as N
    w = W.WORKLOADS[name]
    print(f"\n>>> no-alloc vs dit_attn_fwd: {name} schedule={schedule} B={w.B} H={w.H} d={w.d} "
          f"S={w.s_valid}->{w.s_pad}", flush=True)
    dev = torch.device("cuda:0")
    q, k, v = (to_dev_bf16(x) for x in W.make_qkv(w))
    tabs = ops.rope_split_tables(torch.from_numpy(W.positions(w)).to(dev), w.axes, w.d, w.theta)
    o_ref, l_ref = ops.attn_fwd(q, k, v, q_valid=w.s_valid, kv_valid=w.s_valid, rope_q=tabs, rope_k=tabs,
                                schedule=schedule)
    # outputs prefilled with NaN: every row must be written
    o = torch.full_like(o_ref, float("nan"))
    l = torch.full_like(l_ref, float("nan"))
    desc = ops._attn_desc(q, k, v, o, l, w.s_valid, w.s_valid, tabs, tabs, 0.0, schedule)
    rc = N.lib().dit_attn_fwd_noalloc(ctypes.byref(desc), ops._stream(dev))
    N.check(rc, "dit_attn_fwd_noalloc")
    torch.cuda.synchronize()
    return (o_ref, l_ref), (o, l)


def test_noalloc_equals_attn_fwd_on_two_calls_second_smaller(ops):
    for name in ("wan480", "tiny"):
        (o_ref, l_ref), (o, l) = _run_both(ops, name)
        assert np.array_equal(raw_bits(o), raw_bits(o_ref)), name
        assert np.array_equal(raw_bits(l), raw_bits(l_ref)), name


@pytest.mark.parametrize("schedule", [2, 3])
def test_noalloc_equals_attn_fwd_with_schedule_counters(ops, schedule):
    for name in ("wan480", "tiny"):
        (o_ref, l_ref), (o, l) = _run_both(ops, name, schedule)
        assert np.array_equal(raw_bits(o), raw_bits(o_ref)), (name, schedule)
        assert np.array_equal(raw_bits(l), raw_bits(l_ref)), (name, schedule)


def test_noalloc_refuses_a_workspace_beyond_the_scratch(ops):
    """The Wan 720p call needs 388 MB of rotated Q / K: refused on the host,
    before any launch, with the sizes named."""
    import torch
    from long_sequence_attention_amd import _native as N
    dev = torch.device("cuda:0")
    w = W.WORKLOADS["wan720"]
    q = torch.zeros((w.B, w.H, w.s_pad, w.d), dtype=torch.bfloat16, device=dev)
    cos = torch.ones((w.s_pad, w.d // 2), dtype=torch.float32, device=dev)
    sin = torch.zeros_like(cos)
    need = ops.attn_workspace_size(q, q, q, q_valid=w.s_valid, kv_valid=w.s_valid, rope_q=(cos, sin),
                                   rope_k=(cos, sin))
    assert need > ops.NOALLOC_SCRATCH_BYTES
    desc = ops._attn_desc(q, q, q, q, None, w.s_valid, w.s_valid, (cos, sin), (cos, sin), 0.0)
    assert N.lib().dit_attn_fwd_noalloc(ctypes.byref(desc), ops._stream(dev)) == N.DIT_ERR_UNSUPPORTED
    assert b"static scratch" in N.lib().dit_last_error()
