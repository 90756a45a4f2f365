"""Benchmark of the DiT self-attention hot path on one MI355X.

One step = one pass of the whole path over one batch of synthetic tokens:
  RoPE tables from positions -> tail pad of Q, K, V tokens ([B, S, H, d]) ->
  attention forward (K rotation pre-pass + the fused attention kernel, Q RoPE
  fused, pad keys masked) -> unpad of O.
Inputs are resident in HBM before timing starts. Throughput is counted over
valid tokens: FLOP = 4 * B * H * S_valid^2 * d per step.

Prints ONE JSON line. Usage: python bench.py [--steps K] [--warmup W] [--gpus 1]
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2516.6  # 256 CU x 2.4 GHz x 4096 dense bf16 FLOP/clk/CU (MI355X published dense peak)
PEAK_HBM_GBS = 8000.0
METRIC = "attn fwd TFLOP/s at Wan S=4736,H=10,d=128 bf16; % of bf16 MFMA peak"


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="wan480")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--kernel-iters", type=int, default=50)
    return ap.parse_args()


def cpu_baseline(w, q, k, v):
    """The fp64 oracle as it stands, timed on this host over the whole
    workload (all heads, all rows: ~10 s on 8 cores)."""
    import oracle
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        threads = len(os.sched_getaffinity(0))
    pos = __import__("workloads").positions(w)
    t0 = time.perf_counter()
    oracle.dit_path(q, k, v, pos, pos, w.axes, w.theta, w.s_valid, w.s_valid)
    dt = time.perf_counter() - t0
    return {"value": w.valid_flop / dt / 1e12, "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
            "sample": f"full {w.name} workload (B={w.B}, H={w.H}, all {w.s_valid} valid query rows), "
                      f"NumPy float64, {dt:.2f} s wall"}


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "this build runs on one GPU only; --gpus must be 1 "
                          "(the path shards by head across GPUs; see DESIGN.md)"}))
        sys.exit(2)
    import numpy as np
    import torch
    import workloads as W
    import long_sequence_attention_amd as ops

    ops.library_path()  # fails loudly if the HIP library is not built
    w = W.WORKLOADS[args.workload]
    dev = torch.device("cuda:0")
    B, H, d, Sv, Sp = w.B, w.H, w.d, w.s_valid, w.s_pad

    q, k, v = W.make_qkv(w)
    # token-major inputs [B, S_valid, H, d] (what an all-to-all hands over)
    def tok(x):
        t = torch.from_numpy(np.ascontiguousarray(x[:, :, :Sv].transpose(0, 2, 1, 3)).view(np.int16))
        return t.view(torch.bfloat16).to(dev)
    q_tok, k_tok, v_tok = tok(q), tok(k), tok(v)
    pos = torch.from_numpy(W.positions(w)).to(dev)
    qp = torch.empty((B, Sp, H, d), dtype=torch.bfloat16, device=dev)
    kp, vp, op = torch.empty_like(qp), torch.empty_like(qp), torch.empty_like(qp)
    o_tok = torch.empty_like(q_tok)
    lse = torch.empty((B, H, Sp), dtype=torch.float32, device=dev)
    cos = torch.empty((Sp, d // 2), dtype=torch.float32, device=dev)
    sin = torch.empty_like(cos)
    L = ops._native.lib()
    import ctypes
    chans = (ctypes.c_int32 * len(w.axes))(*w.axes)

    qv, kv_, vv = qp.transpose(1, 2), kp.transpose(1, 2), vp.transpose(1, 2)
    ws = torch.empty(ops.attn_workspace_size(qv, kv_, vv, q_valid=Sv, kv_valid=Sv, rope_q=(cos, sin), rope_k=(cos, sin)),
                     dtype=torch.uint8, device=dev)

    def step():
        s = ops._stream(dev)
        ops._native.check(L.dit_rope_split_tables(ctypes.c_void_p(pos.data_ptr()), Sp, len(w.axes), chans, d,
                                                  float(w.theta), ctypes.c_void_p(cos.data_ptr()),
                                                  ctypes.c_void_p(sin.data_ptr()), s), "tables")
        ops.pad_tokens(q_tok, Sp, out=qp)
        ops.pad_tokens(k_tok, Sp, out=kp)
        ops.pad_tokens(v_tok, Sp, out=vp)
        ops.attn_fwd(qp.transpose(1, 2), kp.transpose(1, 2), vp.transpose(1, 2), q_valid=Sv, kv_valid=Sv,
                     rope_q=(cos, sin), rope_k=(cos, sin), out=op.transpose(1, 2), lse=lse, workspace=ws)
        ops.unpad_tokens(op, Sv, out=o_tok)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record()
    for _ in range(args.steps):
        step()
    e1.record()
    torch.cuda.synchronize()
    ms_step = e0.elapsed_time(e1) / args.steps

    # Dominant kernel alone: one attention-kernel launch per call (K already
    # rotated, so dit_attn_fwd launches only the fused attention kernel).
    k_rot = torch.empty((B, H, Sp, d), dtype=torch.bfloat16, device=dev)
    ops.attn_fwd(qp.transpose(1, 2), kp.transpose(1, 2), vp.transpose(1, 2), q_valid=Sv, kv_valid=Sv,
                 rope_q=(cos, sin), rope_k=(cos, sin), out=op.transpose(1, 2), lse=lse, workspace=ws)
    torch.cuda.synchronize()
    k_rot.view(-1).copy_(ws[: B * H * Sp * d * 2].view(torch.bfloat16)[: B * H * Sp * d])

    def attn_only():
        ops.attn_fwd(qp.transpose(1, 2), k_rot, vp.transpose(1, 2), q_valid=Sv, kv_valid=Sv,
                     rope_q=(cos, sin), rope_k=None, out=op.transpose(1, 2), lse=lse)

    def time_loop(fn, n):
        for _ in range(3):
            fn()
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(n):
            fn()
        b.record()
        torch.cuda.synchronize()
        return a.elapsed_time(b) / n * 1e3  # us

    n = args.kernel_iters
    us_attn = time_loop(attn_only, n)
    us_pad = time_loop(lambda: ops.pad_tokens(q_tok, Sp, out=qp), n)
    us_unpad = time_loop(lambda: ops.unpad_tokens(op, Sv, out=o_tok), n)
    us_attn_call = time_loop(lambda: ops.attn_fwd(qp.transpose(1, 2), kp.transpose(1, 2), vp.transpose(1, 2),
                                                  q_valid=Sv, kv_valid=Sv, rope_q=(cos, sin), rope_k=(cos, sin),
                                                  out=op.transpose(1, 2), lse=lse, workspace=ws), n)
    flop = w.valid_flop
    achieved = flop / (us_attn * 1e-6) / 1e12
    pad_bytes = (Sv + Sp) * H * d * 2 * B

    out = {
        "metric": METRIC,
        "value": flop / (ms_step * 1e-3) / 1e12,
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": f"{w.name}: {w.description}", "B": B, "H": H, "d": d, "s_valid": Sv, "s_pad": Sp,
                   "flop_per_step": flop, "step": "tables + pad(Q,K,V) + attn_fwd(K-rope pre-pass + fused kernel) + unpad(O)"},
        "roofline": {"bound": "mfma", "achieved": achieved, "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": achieved / PEAK_BF16_TFLOPS, "traffic": None,
                     "kernel": "attn_fwd_kernel<128>", "kernel_us": us_attn},
        "kernels_us": {"attn_fwd_kernel": us_attn, "dit_attn_fwd_call(prepass+kernel)": us_attn_call,
                       "pad_tokens(one tensor)": us_pad, "unpad_tokens": us_unpad,
                       "pad_GBps": pad_bytes / (us_pad * 1e-6) / 1e9},
        "pct_of_peak_step": flop / (ms_step * 1e-3) / 1e12 / PEAK_BF16_TFLOPS * 100,
    }
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(w, q, k, v)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
