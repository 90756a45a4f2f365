"""Benchmark of the DiT self-attention hot path on one MI355X.

One step = one pass of the whole path over one batch of synthetic tokens:
  RoPE tables from positions -> tail pad of the fused QKV tokens
  ([B, S, 3, H, d], one call) -> attention forward on the strided Q, K, V
  views (Q / K rotation pre-pass + the attention kernel, pad keys masked)
  -> unpad of O.
Inputs are resident in HBM before timing starts. Throughput is counted over
valid tokens: FLOP = 4 * B * H * S_valid^2 * d per step.

Prints ONE JSON line:
  python bench.py [--steps K] [--warmup W] [--gpus 1] [--no-cpu-baseline] [--no-configs]

Shader clock of the attention kernel's key loop per config (clock-probe build):
  python bench.py --clock-probe

Counter collection (HBM traffic of the attention kernel, calibrated against a
plain copy of known size), run under rocprofv3 once per counter:
  python bench.py --pmc-target              # launches only the measured kernels
  python bench.py --traffic-summary FETCH_DIR WRITE_DIR   # writes the profiles/ record
"""
from __future__ import annotations

import argparse
import glob
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2516.6  # 256 CU x 2.4 GHz x 4096 dense bf16 FLOP/clk/CU (MI355X published dense peak)
PEAK_HBM_GBS = 8000.0
METRIC = "attn fwd TFLOP/s at Wan S=4736,H=10,d=128 bf16; % of bf16 MFMA peak"
TRAFFIC_RECORD = os.path.join(ROOT, "profiles", "attn_fwd_wan480_traffic.json")
COPY_CAL_BYTES = 256 << 20  # calibration copy: 256 MiB read + 256 MiB written
KERNEL_SOURCES = ("long_sequence_attention_amd/csrc/attn_fwd.hip", "long_sequence_attention_amd/csrc/common.h")


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    # the clocks settle only after a few hundred ms of sustained load
    ap.add_argument("--steps", type=int, default=500)
    ap.add_argument("--warmup", type=int, default=2000)
    ap.add_argument("--workload", default="wan480")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-configs", action="store_true", help="skip the per-config kernel table")
    ap.add_argument("--kernel-iters", type=int, default=200)
    ap.add_argument("--pmc-target", action="store_true")
    ap.add_argument("--pmc-variant", default="percall", choices=("percall", "split", "seg", "fixed_m"))
    ap.add_argument("--traffic-summary", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"))
    ap.add_argument("--clock-probe", action="store_true",
                    help="shader clock of the attention kernel's key loop per config (clock-probe build)")
    ap.add_argument("--hbm-passes", action="store_true",
                    help="time the HBM-bound passes (pad, unpad, LSE merge, tables) on Wan 720p-sized buffers")
    return ap.parse_args()


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


# ---------------------------------------------------------------- helpers
def sclk_levels():
    """Shader-clock DPM levels of each amdgpu card in sysfs (MHz); `current`
    holds the level(s) the driver marks active. None where sysfs hides them."""
    import re
    out = []
    for f in sorted(glob.glob("/sys/class/drm/card*/device/pp_dpm_sclk"))[:16]:
        try:
            with open(f) as fh:
                txt = fh.read()
        except OSError:
            continue
        lv = re.findall(r"(\d+)\s*[Mm][Hh]z(\s*\*)?", txt)
        out.append({"card": f.split("/")[4], "levels_mhz": [int(a) for a, _ in lv],
                    "current_mhz": [int(a) for a, star in lv if star.strip()]})
    return out or None


def device_info(torch, sclk_busy, sclk_kernel=None):
    p = torch.cuda.get_device_properties(0)
    return {"name": p.name, "arch": getattr(p, "gcnArchName", None), "compute_units": p.multi_processor_count,
            "sclk_during_timed_steps": sclk_busy, "sclk_during_kernel_loop": sclk_kernel,
            "sclk_after": sclk_levels(),
            "torch": torch.__version__, "hip": getattr(torch.version, "hip", None)}


def dev_tensors(w, np, torch, dev, inputs=None):
    import workloads as W
    q, k, v = inputs[w.name] if inputs and w.name in inputs else W.make_qkv(w)
    tod = lambda x: torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).view(torch.bfloat16).to(dev)
    return (q, k, v), (tod(q), tod(k), tod(v))


def time_us(torch, fn, n, warm=3, warm_s=0.0, clock=None):
    """Average microseconds per call of fn over n back-to-back calls, HIP
    events on torch's current stream (the stream every dit_* call uses),
    after `warm` calls and at least warm_s seconds of calls. With a list
    `clock`, the sysfs shader-clock levels read while the timed calls are
    still queued are appended to it."""
    for _ in range(warm):
        fn()
    torch.cuda.synchronize()
    t_end = time.perf_counter() + warm_s
    while time.perf_counter() < t_end:
        for _ in range(20):
            fn()
        torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(n):
        fn()
    b.record()
    if clock is not None:
        clock.append(sclk_levels())
    torch.cuda.synchronize()
    return a.elapsed_time(b) / n * 1e3


def host_submit_us(torch, fn, n):
    """Host microseconds per call to enqueue fn (no synchronisation inside
    the n calls): when this is near the per-call time, the host, not the
    GPU, sets the pace of back-to-back calls."""
    fn()
    torch.cuda.synchronize()
    t = time.perf_counter()
    for _ in range(n):
        fn()
    dt = time.perf_counter() - t
    torch.cuda.synchronize()
    return dt / n * 1e6


def graph_us(torch, fn, outs, calls=20, replays=20):
    """Average microseconds per call when `calls` calls of fn are replayed
    from one captured graph (torch.cuda.CUDAGraph): the device time per call
    without the host's per-call cost. Every replay checked below writes
    `outs` again; the replays, each after an eager call and a
    synchronisation, must give the eager result's bits, else None."""
    fn()
    torch.cuda.synchronize()
    ref = [t.clone() for t in outs]
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fn()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for _ in range(calls):
            fn()
    for _ in range(3):
        fn()
        torch.cuda.synchronize()
        for t in outs:
            t.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        for t, r in zip(outs, ref):
            iv = torch.int16 if t.element_size() == 2 else torch.int32
            if not torch.equal(t.view(iv), r.view(iv)):
                return None
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(replays):
        g.replay()
    b.record()
    torch.cuda.synchronize()
    del g
    return a.elapsed_time(b) / (replays * calls) * 1e3


CONFIGS = ("tiny", "flux", "wan480", "hunyuan", "wan720")
SETTLE_S = 1.0              # minimum seconds of warm-up steps before the timed ones
ORACLE_ROW_BLOCK = 1024     # query rows per oracle task
MAX_POOL = 16               # the host share of one GPU on the box


def pool_size():
    return max(1, min(len(os.sched_getaffinity(0)), MAX_POOL))


BLAS_ENV = ("OMP_NUM_THREADS", "OPENBLAS_NUM_THREADS", "MKL_NUM_THREADS")


def _worker_init():
    """Each worker runs the oracle on one BLAS thread (the pool spreads the
    work over the cores); the environment set by spawn_pool covers the BLAS
    library loaded later, the limit here one already loaded."""
    import numpy  # noqa: F401  (loads BLAS, so the limit below applies to it)
    try:
        from threadpoolctl import threadpool_limits
        threadpool_limits(1)
    except Exception:
        pass


def spawn_pool(n):
    """A pool of n spawned worker processes, each limited to one BLAS thread."""
    import multiprocessing as mp
    saved = {k: os.environ.get(k) for k in BLAS_ENV}
    os.environ.update({k: "1" for k in BLAS_ENV})
    try:
        return mp.get_context("spawn").Pool(n, initializer=_worker_init)
    finally:
        for k, val in saved.items():
            if val is None:
                os.environ.pop(k, None)
            else:
                os.environ[k] = val


def _gen_head(task):
    """Seeded synthetic inputs of one head (all batches): bf16 bits [B, S, d] x 3."""
    import numpy as np
    import workloads as W
    name, h = task
    w = W.WORKLOADS[name]
    return name, h, [np.stack([W.make_head(w, t, b, h) for b in range(w.B)]) for t in "qkv"]


def make_inputs(names, pool):
    """Q, K, V bf16 bit arrays [B, H, S, d] of every named workload, generated
    head by head in the pool (the same bits as workloads.make_qkv)."""
    import numpy as np
    import workloads as W
    out = {}
    for name in names:
        w = W.WORKLOADS[name]
        out[name] = [np.empty((w.B, w.H, w.s_pad if t == "q" else w.k_pad, w.d), dtype=np.uint16) for t in "qkv"]
    for name, h, arrs in pool.imap_unordered(_gen_head, [(n, h) for n in names for h in range(W.WORKLOADS[n].H)]):
        for dst, a in zip(out[name], arrs):
            dst[:, h] = a
    return {n: tuple(v) for n, v in out.items()}


def _oracle_task(task):
    """The fp64 oracle (RoPE tables, RoPE, masked attention, LSE) on the
    given query rows of one head; returns its wall time and, when asked,
    the result."""
    import oracle
    import workloads as W
    name, h, rows, q, k, v, keep = task
    w = W.WORKLOADS[name]
    pos = W.positions(w)
    t0 = time.perf_counter()
    O, L = oracle.dit_path(q, k, v, pos, pos, w.axes, w.theta, w.s_valid, w.s_valid, rows=rows)
    dt = time.perf_counter() - t0
    return name, h, rows, dt, (O, L) if keep else None


def oracle_rows(w):
    """Query rows the oracle times per head: every valid row, or 2048 seeded
    sampled rows per head for the 720p shard."""
    import numpy as np
    import workloads as W
    if w.n_key_shards > 1:
        return [W.sample_rows(w, h) for h in range(w.H)], "2048 seeded sampled valid query rows per head"
    return [np.arange(w.s_valid)] * w.H, "all valid query rows"


def cpu_baseline_all(inputs, pool, keep=("wan480",)):
    """The fp64 oracle as it stands, timed on this host's cores for every
    config: one task per (head, block of up to 1024 query rows), spread over
    a process pool of one single-threaded worker per core; wall time per
    config measured around the whole pool map (inputs shipped to the workers
    included). Returns the per-config figures and the full results of the
    configs in `keep`."""
    import numpy as np
    import workloads as W
    per, results = {}, {}
    for name in CONFIGS:
        w = W.WORKLOADS[name]
        q, k, v = inputs[name]
        rows_per_head, what = oracle_rows(w)
        tasks = []
        for h in range(w.H):
            rh = rows_per_head[h]
            for r0 in range(0, len(rh), ORACLE_ROW_BLOCK):
                tasks.append((name, h, rh[r0:r0 + ORACLE_ROW_BLOCK], q[:, h:h + 1], k[:, h:h + 1], v[:, h:h + 1],
                              name in keep))
        n_rows = sum(len(r) for r in rows_per_head)
        flop = 4.0 * w.B * n_rows * w.k_valid * w.d
        t0 = time.perf_counter()
        outs = list(pool.imap_unordered(_oracle_task, tasks))
        wall = time.perf_counter() - t0
        ent = {"wall_s": wall, "task_s_sum": sum(o[3] for o in outs), "tasks": len(tasks), "rows": what,
               "query_rows_computed": n_rows, "flop_computed": flop, "gflops": flop / wall / 1e9}
        if n_rows < w.H * w.B * w.s_valid:
            ent["full_workload_s_extrapolated"] = wall * w.valid_flop / flop
            ent["note"] = "full_workload_s_extrapolated scales the sampled wall time to all valid rows (not measured)"
        per[name] = ent
        if name in keep:
            if n_rows == w.H * w.B * w.s_valid:   # every valid row: full arrays, pad rows 0 / -inf
                O = np.zeros((w.B, w.H, w.s_pad, w.d))
                L = np.full((w.B, w.H, w.s_pad), -np.inf)
                for _, h, rows, _, (Ob, Lb) in outs:
                    O[:, h, rows] = Ob[:, 0]
                    L[:, h, rows] = Lb[:, 0]
                results[name] = (O, L)
            else:                                # sampled rows: {head: (rows, O, LSE)}
                per_head = {}
                for _, h, rows, _, (Ob, Lb) in outs:
                    per_head.setdefault(h, []).append((rows, Ob[:, 0], Lb[:, 0]))
                results[name] = {h: (np.concatenate([r for r, _, _ in v]), np.concatenate([o for _, o, _ in v], axis=1),
                                     np.concatenate([l for _, _, l in v], axis=1)) for h, v in per_head.items()}
    return per, results


def cpu_baseline_line(per, workers):
    w3 = per["wan480"]
    return {"value": w3["gflops"] / 1e3, "unit": "TFLOP/s", "cores": workers, "kind": "oracle",
            "sample": (f"full wan480 workload (B=1, H=10, all 4680 valid query rows: RoPE tables, RoPE, masked "
                       f"attention, LSE), NumPy float64, {w3['tasks']} tasks of <= {ORACLE_ROW_BLOCK} query rows "
                       f"over {workers} single-threaded worker processes: {w3['wall_s']:.2f} s wall; every config "
                       f"in per_config (720p on 2048 sampled rows per head)"),
            "affinity_cores": len(os.sched_getaffinity(0)), "workers": workers, "blas_threads_per_worker": 1,
            "per_config": per}


def parity_of_step(np, o_tok, lse, ref, s_valid):
    """The last timed step's O ([B, S_valid, H, d]) and LSE against the
    oracle's result on the same inputs, with the acceptance bar."""
    O_ref, L_ref = ref
    og = o_tok.float().cpu().numpy().astype(np.float64).transpose(0, 2, 1, 3)
    lg = lse[:, :, :s_valid].cpu().numpy().astype(np.float64)
    do = np.abs(og - O_ref[:, :, :s_valid])
    dl = np.abs(lg - L_ref[:, :, :s_valid])
    res = {"o_max_abs": float(do.max()), "o_mean_abs": float(do.mean()), "lse_max_abs": float(dl.max()),
           "bar": {"o_max_abs": 1.5e-2, "o_mean_abs": 2e-3, "lse_max_abs": 5e-3}}
    res["pass"] = bool(res["o_max_abs"] <= 1.5e-2 and res["o_mean_abs"] <= 2e-3 and res["lse_max_abs"] <= 5e-3)
    return res


def config_parity(np, o, lse, ref, w):
    """A config's GPU output (O [B, H, S, d], LSE [B, H, S] device tensors)
    against the oracle's result on the same inputs, with the acceptance bar:
    every valid row, or the oracle's sampled rows per head."""
    bar = {"o_max_abs": 1.5e-2, "o_mean_abs": 2e-3, "lse_max_abs": 5e-3}
    if isinstance(ref, tuple):
        O_ref, L_ref = ref
        sv = w.s_valid
        og = o[:, :, :sv].float().cpu().numpy().astype(np.float64)
        lg = lse[:, :, :sv].cpu().numpy().astype(np.float64)
        do, dl = np.abs(og - O_ref[:, :, :sv]), np.abs(lg - L_ref[:, :, :sv])
        rows = "every valid row"
    else:
        dos, dls = [], []
        for h, (r, Oh, Lh) in ref.items():
            ri = np.asarray(r)
            og = o[:, h, ri].float().cpu().numpy().astype(np.float64)
            lg = lse[:, h, ri].cpu().numpy().astype(np.float64)
            dos.append(np.abs(og - Oh))
            dls.append(np.abs(lg - Lh))
        do, dl = np.concatenate(dos, axis=1), np.concatenate(dls, axis=1)
        rows = f"{do.shape[1] // len(ref)} sampled rows per head"
    res = {"o_max_abs": float(do.max()), "o_mean_abs": float(do.mean()), "lse_max_abs": float(dl.max()),
           "rows": rows}
    res["pass"] = bool(all(res[k] <= bar[k] for k in bar))
    return res


def read_traffic():
    """HBM bytes per launch of the attention kernel from the committed counter
    record, or None when the kernel source changed since it was taken."""
    try:
        with open(TRAFFIC_RECORD) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None, "no counter record"
    if rec.get("kernel_source_sha256_16") != kernel_source_hash():
        return None, "kernel changed since the counters were taken"
    return rec["hbm_bytes_per_launch"], rec.get("command", "")


# ------------------------------------------------------- counter workflow
def pmc_target(args):
    """Launch one kernel variant a few times on its workload, plus the
    calibration copy (for the traffic record); nothing else runs on the GPU.
    --pmc-variant picks the variant:
      percall  attn_fwd_kernel<128, false>, one workgroup per q-tile (the
               step's kernel; Q and K unrotated, no pre-pass)
      split    attn_fwd_kernel<128, true>, the split (BALANCED) schedule
      seg      attn_fwd_seg_kernel<128>: the ring layout, two segments of
               2340 real keys each padded to 2368 (Q likewise)
      fixed_m  the fixed-m statistics kernels and the FIXED loop (forced)"""
    import numpy as np
    import torch
    import workloads as W
    import long_sequence_attention_amd as ops
    ops.library_path()
    w = W.WORKLOADS[args.workload]
    dev = torch.device("cuda:0")
    _, (qd, kd, vd) = dev_tensors(w, np, torch, dev)
    kw = dict(q_valid=w.s_valid, kv_valid=w.k_valid, rope_q=None, rope_k=None, fixed_m=False)
    if args.pmc_variant == "split":
        kw["schedule"] = 2
    elif args.pmc_variant == "fixed_m":
        kw["fixed_m"] = True
    elif args.pmc_variant == "seg":
        per, L = w.s_valid // 2, 2368
        qs, ks, vs = (torch.zeros((w.B, w.H, 2 * L, w.d), dtype=torch.bfloat16, device=dev) for _ in range(3))
        for src, dst in ((qd, qs), (kd, ks), (vd, vs)):
            for i in range(2):
                dst[:, :, i * L:i * L + per] = src[:, :, i * per:(i + 1) * per]
        qd, kd, vd = qs, ks, vs
        kw.update(q_valid=per, kv_valid=per, q_seg_len=L, kv_seg_len=L)
    elif args.pmc_variant != "percall":
        raise SystemExit(f"unknown --pmc-variant {args.pmc_variant}")
    o = torch.empty_like(qd)
    lse = torch.empty(qd.shape[:3], dtype=torch.float32, device=dev)
    ws = torch.empty(max(256, ops.attn_workspace_size(qd, kd, vd, **kw)), dtype=torch.uint8, device=dev)
    for i in range(5):   # the first call clears the schedule counters, the rest launch the attention kernel alone
        ops.attn_fwd(qd, kd, vd, out=o, lse=lse, workspace=ws, ws_counters_zero=i > 0, **kw)
    src = torch.empty(COPY_CAL_BYTES, dtype=torch.uint8, device=dev)
    src.fill_(1)
    dst = torch.empty_like(src)
    rows = COPY_CAL_BYTES // 4096
    for _ in range(5):  # a plain copy: pad with s_pad == s_valid
        ops.pad_tokens(src.view(1, rows, 4096), rows, out=dst.view(1, rows, 4096))
    torch.cuda.synchronize()
    print("pmc target done", flush=True)


def hbm_passes(args):
    """The HBM-bound passes on Wan 720p-sized buffers (larger than the 256 MB
    MALL, so the figures are HBM rates): pad and unpad of one token-major
    tensor [1, S, 10, 128] bf16, the pad of the fused Q/K/V rows with Q and K
    rotated, the 4-part fp32 -> bf16 LSE merge, and the RoPE tables. Prints one JSON line of average µs and GB/s per pass (HIP
    events over 20 back-to-back calls after 5 warm-up calls); run under
    rocprofv3 --kernel-trace for the per-kernel durations."""
    import torch
    import workloads as W
    import long_sequence_attention_amd as ops
    ops.library_path()
    w = W.WORKLOADS["wan720"]
    dev = torch.device("cuda:0")
    Sv, Sp, H, d = w.s_valid, w.s_pad, w.H, w.d
    x = torch.randn((1, Sv, H, d), device=dev).to(torch.bfloat16)
    xp = torch.empty((1, Sp, H, d), dtype=torch.bfloat16, device=dev)
    xu = torch.empty_like(x)
    parts_o = [torch.randn((1, H, Sp, d), device=dev) for _ in range(4)]
    parts_l = [torch.randn((1, H, Sp), device=dev) for _ in range(4)]
    om = torch.empty((1, H, Sp, d), dtype=torch.bfloat16, device=dev)
    lm = torch.empty((1, H, Sp), dtype=torch.float32, device=dev)
    pos = torch.from_numpy(W.positions(w)).to(dev)
    row = H * d * 2
    # a full attention call on token-major random inputs, for the Q / K
    # rotation pre-pass's duration in a kernel trace (its bytes: Q and K rows
    # read and written, plus the fp32 tables once per row and group of four heads)
    cos, sin = ops.rope_split_tables(pos, w.axes, d, w.theta)
    qa, ka, va = (torch.randn((1, Sp, H, d), device=dev).to(torch.bfloat16).transpose(1, 2) for _ in range(3))
    oa = torch.empty((1, Sp, H, d), dtype=torch.bfloat16, device=dev).transpose(1, 2)
    ws = torch.empty(ops.attn_workspace_size(qa, ka, va, q_valid=Sv, kv_valid=Sv, rope_q=(cos, sin), rope_k=(cos, sin)),
                     dtype=torch.uint8, device=dev)
    groups = -(-H // 4)
    prepass_bytes = (Sp + Sv) * row * 2 + (Sp + Sv) * groups * d * 4
    # the fused Q/K/V pad with Q and K rotated on the way: rows read and
    # written, plus the fp32 tables once per real row
    qkv = torch.randn((1, Sv, 3, H, d), device=dev).to(torch.bfloat16)
    qkvp = torch.empty((1, Sp, 3, H, d), dtype=torch.bfloat16, device=dev)
    res = {}
    for name, fn, nbytes in (
            ("pad_tokens", lambda: ops.pad_tokens(x, Sp, out=xp), (Sv + Sp) * row),
            ("pad_tokens_rope(fused QKV, Q/K rotated)", lambda: ops.pad_tokens_rope(qkv, Sp, cos, sin, n_rot=2, out=qkvp),
             (Sv + Sp) * 3 * row + Sv * d * 4),
            ("unpad_tokens", lambda: ops.unpad_tokens(xp, Sv, out=xu), 2 * Sv * row),
            ("lse_merge_4xf32_to_bf16", lambda: ops.lse_merge(parts_o, parts_l, q_valid=Sv, out=om, lse_out=lm),
             4 * H * Sp * (d * 4 + 4) + H * Sp * (d * 2 + 4)),
            ("rope_split_tables", lambda: ops.rope_split_tables(pos, w.axes, d, w.theta), Sp * d // 2 * 8),
            ("attn_fwd_call(pre-pass + attention kernel)", lambda: ops.attn_fwd(
                qa, ka, va, q_valid=Sv, kv_valid=Sv, rope_q=(cos, sin), rope_k=(cos, sin), out=oa, workspace=ws),
             None)):
        us = time_us(torch, fn, 20 if nbytes else 3, warm=5 if nbytes else 1)
        res[name] = {"us": us, "bytes": nbytes, "GBps": nbytes / us / 1e3} if nbytes else {"us": us}
    res["prepass_algorithmic_bytes"] = prepass_bytes
    print(json.dumps({"hbm_passes_wan720": res}), flush=True)


def clock_probe(args):
    """Shader clock of the attention kernel's key loop, per config, from the
    clock-probe build of the library (libditattn_clockprobe.so: the first
    thread of each workgroup stamps the shader-clock counter and the 100 MHz
    counter when its key loop starts and ends). The kernel alone runs on
    each workload's Q, K, V for 1 s, then 3 rounds of 20 calls; the stamps
    of each round's last call give, per workgroup, the loop's cycles and its
    real time, hence the clock and the cycles per MFMA (each SIMD runs two
    waves of 32 MFMAs per key tile). Prints one JSON line."""
    import ctypes
    import numpy as np
    import torch
    import workloads as W
    from long_sequence_attention_amd import _native as N, build as Bld
    N.LIB_PATH = Bld.LIB_CLOCK_PROBE
    import long_sequence_attention_amd as ops
    L = N.lib()
    L.dit_clock_probe_read.argtypes = [ctypes.c_void_p]
    L.dit_clock_probe_read.restype = ctypes.c_int
    dev = torch.device("cuda:0")
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    res = {"library": os.path.basename(Bld.LIB_CLOCK_PROBE), "compute_units": cus}
    for name, sched in (("wan480", 1), ("flux", 1), ("hunyuan", 1), ("wan720", 1), ("wan480", 2)):
        w = W.WORKLOADS[name]
        _, (qd, kd, vd) = dev_tensors(w, np, torch, dev)
        o = torch.empty_like(qd)
        lse = torch.empty((w.B, w.H, w.s_pad), dtype=torch.float32, device=dev)
        ws = torch.empty(max(256, ops.attn_workspace_size(qd, kd, vd, q_valid=w.s_valid, kv_valid=w.k_valid,
                                                          schedule=sched, fixed_m=False)),
                         dtype=torch.uint8, device=dev)
        fn = lambda: ops.attn_fwd(qd, kd, vd, q_valid=w.s_valid, kv_valid=w.k_valid, out=o, lse=lse,
                                  schedule=sched, fixed_m=False, workspace=ws)
        time_us(torch, fn, 1, warm_s=1.0)
        nwg = w.B * w.H * (-(-w.s_pad // 256))
        if sched == 2:   # the split grid: one workgroup per CU at most
            nwg = min(cus, nwg * (-(-w.k_valid // 64)))
        nk = -(-w.k_valid // 64)
        buf = np.zeros(4096 * 8, dtype=np.uint64)
        rounds = []
        for _ in range(3):
            n_calls = 20 if w.valid_flop < 1e12 else 2
            call_us = time_us(torch, fn, n_calls, warm=0)   # the round's calls, back to back
            if L.dit_clock_probe_read(buf.ctypes.data) != 0:
                raise RuntimeError("dit_clock_probe_read failed")
            b = buf[:min(nwg, 4096) * 8].reshape(-1, 8).astype(np.float64)
            cyc, real = b[:, 2] - b[:, 0], b[:, 3] - b[:, 1]
            mhz = cyc / real * 100.0
            tiles = np.maximum(b[:, 6], 1)   # key tiles of the stamped loop
            ent = {"workgroups": int(len(b)), "key_tiles": nk, "loop_us_median": float(np.median(real) / 100),
                   "loop_cycles_median": float(np.median(cyc)), "mhz_median": float(np.median(mhz)),
                   "mhz_min": float(mhz.min()), "mhz_max": float(mhz.max()),
                   "cycles_per_mfma_median": float(np.median(cyc / (tiles * 64)))}
            if sched == 2:
                ent["stamped_tiles_min_max"] = [int(b[:, 6].min()), int(b[:, 6].max())]
            # the last call's launch: workgroup entry (word 4) to loop start,
            # loop end to stores complete (word 5), and the span from the
            # first entry to the last exit against the per-call time
            if sched == 2:   # no entry / exit stamps under the split schedule
                rounds.append(ent)
                continue
            entry, exit_ = b[:, 4], b[:, 5]
            ent.update({"call_us": call_us, "span_us": float((exit_.max() - entry.min()) / 100),
                        "entry_spread_us": float((entry.max() - entry.min()) / 100),
                        "prologue_us_median": float(np.median(b[:, 1] - entry) / 100),
                        "epilogue_us_median": float(np.median(exit_ - b[:, 3]) / 100)})
            ent["outside_workgroups_us"] = call_us - ent["span_us"]
            # workgroup i runs on XCD i % 8 (round-robin dispatch): per-XCD
            # medians of the clock and of the loop's cycles and time
            xcd = np.arange(len(b)) % 8
            ent["per_xcd"] = [{"workgroups": int((xcd == x).sum()), "mhz": float(np.median(mhz[xcd == x])),
                               "loop_cycles": float(np.median(cyc[xcd == x])),
                               "loop_us": float(np.median(real[xcd == x]) / 100),
                               "loop_us_max": float(real[xcd == x].max() / 100)} for x in range(8) if (xcd == x).any()]
            if nwg > cus:   # workgroups of the first wave (every CU busy) against the rest
                first = b[:, 1] < np.sort(b[:, 3])[0]
                ent["mhz_median_first_wave"] = float(np.median(mhz[first]))
                ent["mhz_median_later"] = float(np.median(mhz[~first])) if (~first).any() else None
                ent["first_wave_workgroups"] = int(first.sum())
            rounds.append(ent)
        res[name if sched == 1 else name + "_split"] = rounds
        del qd, kd, vd, o
        torch.cuda.empty_cache()
    print(json.dumps({"clock_probe": res}), flush=True)


def traffic_summary(args):
    import csv

    def per_dispatch(d, counter):
        vals = {}
        for f in glob.glob(os.path.join(d, "*counter_collection.csv")):
            for r in csv.DictReader(open(f)):
                if r["Counter_Name"] != counter:
                    continue
                kind = "attn" if "attn_fwd_kernel" in r["Kernel_Name"] else (
                    "copy" if "row_copy_kernel" in r["Kernel_Name"] else None)
                if kind is None:
                    continue
                key = (kind, r["Dispatch_Id"])
                vals[key] = vals.get(key, 0.0) + float(r["Counter_Value"])
        out = {}
        for (kind, _), v in vals.items():
            out.setdefault(kind, []).append(v)
        return {k: sorted(v)[len(v) // 2] for k, v in out.items()}  # median over dispatches, KiB

    fetch = per_dispatch(args.traffic_summary[0], "FETCH_SIZE")
    write = per_dispatch(args.traffic_summary[1], "WRITE_SIZE")
    f_fac = COPY_CAL_BYTES / (fetch["copy"] * 1024.0)
    w_fac = COPY_CAL_BYTES / (write["copy"] * 1024.0)
    rec = {
        "kernel": "attn_fwd_kernel<128, false> (wan480, Q and K pre-rotated)",
        "kernel_source_sha256_16": kernel_source_hash(),
        "fetch_kib_per_launch_raw": fetch["attn"], "write_kib_per_launch_raw": write["attn"],
        "copy_fetch_kib_raw": fetch["copy"], "copy_write_kib_raw": write["copy"],
        "copy_bytes_each_way": COPY_CAL_BYTES,
        "fetch_scale": f_fac, "write_scale": w_fac,
        "hbm_fetch_bytes_per_launch": fetch["attn"] * 1024.0 * f_fac,
        "hbm_write_bytes_per_launch": write["attn"] * 1024.0 * w_fac,
        "hbm_bytes_per_launch": fetch["attn"] * 1024.0 * f_fac + write["attn"] * 1024.0 * w_fac,
        "command": "rocprofv3 --pmc FETCH_SIZE (then WRITE_SIZE) --output-format csv -- python3 bench.py --pmc-target",
    }
    os.makedirs(os.path.dirname(TRAFFIC_RECORD), exist_ok=True)
    with open(TRAFFIC_RECORD, "w") as f:
        json.dump(rec, f, indent=1)
    print(json.dumps(rec))


# -------------------------------------------------------------- the bench
def config_table(np, torch, ops, W, dev, n_iter, inputs=None, refs=None):
    """Attention throughput on every config (dit_attn_fwd call = Q / K
    rotation pre-pass + attention kernel, or the kernel alone for the
    cross-attention config, which has no RoPE; the Wan 720p config also as 4 key shards plus
    dit_lse_merge)."""
    res = {}
    for name in ("tiny", "flux", "wan480", "hunyuan", "wan720", "xattn480"):
        w = W.WORKLOADS[name]
        _, (qd, kd, vd) = dev_tensors(w, np, torch, dev, inputs)
        cos, sin = ops.rope_split_tables(torch.from_numpy(W.positions(w)).to(dev), w.axes, w.d, w.theta)
        tabs = (cos, sin) if w.rope else None
        o = torch.empty_like(qd)
        lse = torch.empty((w.B, w.H, w.s_pad), dtype=torch.float32, device=dev)
        ws = torch.empty(max(ops.attn_workspace_size(qd, kd, vd, q_valid=w.s_valid, kv_valid=w.k_valid,
                                                     rope_q=tabs, rope_k=tabs), 256),
                         dtype=torch.uint8, device=dev)
        n = max(3, n_iter if w.valid_flop < 1e12 else 3)
        # 0.3 s of calls first: the shader clock settles under sustained load
        us = time_us(torch, lambda: ops.attn_fwd(qd, kd, vd, q_valid=w.s_valid, kv_valid=w.k_valid,
                                                 rope_q=tabs, rope_k=tabs, out=o, lse=lse,
                                                 workspace=ws), n, warm_s=0.3)
        ent = {"us": us, "tflops": w.valid_flop / us / 1e6, "pct_peak": w.valid_flop / us / 1e6 / PEAK_BF16_TFLOPS * 100}
        if name in ("tiny", "wan480", "xattn480"):   # how much of the call time is the host's
            call = lambda: ops.attn_fwd(qd, kd, vd, q_valid=w.s_valid, kv_valid=w.k_valid, rope_q=tabs, rope_k=tabs,
                                        out=o, lse=lse, workspace=ws)
            ent["host_submit_us"] = host_submit_us(torch, call, n)
            gus = graph_us(torch, call, (o, lse))
            ent["graph_us"] = gus
            if gus:
                ent["graph_pct_peak"] = w.valid_flop / gus / 1e6 / PEAK_BF16_TFLOPS * 100
        if refs and name in refs:   # the timed call's output against the oracle (same inputs, same run)
            torch.cuda.synchronize()
            ent["parity_vs_oracle"] = config_parity(np, o, lse, refs[name], w)
        if w.rope and w.valid_flop < 1e12:   # the kernel alone, on the Q / K the pre-pass left in the workspace
            n_el = w.B * w.H * w.s_pad * w.d
            k_rot = ws[: n_el * 2].view(torch.bfloat16).view(w.B, w.H, w.s_pad, w.d).clone()
            q_rot = ws[n_el * 2: n_el * 4].view(torch.bfloat16).view(w.B, w.H, w.s_pad, w.d).clone()
            wsk = torch.empty(max(256, ops.attn_workspace_size(q_rot, k_rot, vd, q_valid=w.s_valid,
                                                               kv_valid=w.k_valid)), dtype=torch.uint8, device=dev)
            ops.attn_fwd(q_rot, k_rot, vd, q_valid=w.s_valid, kv_valid=w.k_valid, out=o, lse=lse, workspace=wsk)
            kus = time_us(torch, lambda: ops.attn_fwd(q_rot, k_rot, vd, q_valid=w.s_valid, kv_valid=w.k_valid,
                                                      out=o, lse=lse, workspace=wsk, ws_counters_zero=True),
                          n, warm_s=0.3)
            ent.update({"kernel_us": kus, "kernel_pct_peak": w.valid_flop / kus / 1e6 / PEAK_BF16_TFLOPS * 100,
                        "prepass_us": us - kus})
            if name in ("wan480", "hunyuan"):   # the kept variants of the kernel alone, warm
                for tag, extra in (("kernel_split_us", dict(schedule=2)), ("kernel_fixed_m_us", dict(fixed_m=True))):
                    wsv = torch.empty(max(256, ops.attn_workspace_size(q_rot, k_rot, vd, q_valid=w.s_valid,
                                                                       kv_valid=w.k_valid, **extra)),
                                      dtype=torch.uint8, device=dev)
                    ent[tag] = time_us(torch, lambda: ops.attn_fwd(q_rot, k_rot, vd, q_valid=w.s_valid,
                                                                   kv_valid=w.k_valid, out=o, lse=lse,
                                                                   workspace=wsv, **extra), n, warm_s=0.3)
                    del wsv
            del k_rot, q_rot
        if name in ("flux", "wan480", "hunyuan", "wan720"):   # the placement forced each way (AUTO:
            for tag, sc in (("per_qtile_us", 1), ("dynamic_us", 3)):   # dynamic from 4 waves of q-tiles)
                wsd = torch.empty(max(ops.attn_workspace_size(qd, kd, vd, q_valid=w.s_valid, kv_valid=w.k_valid,
                                                              rope_q=tabs, rope_k=tabs, schedule=sc), 256),
                                  dtype=torch.uint8, device=dev)
                ent[tag] = time_us(torch, lambda: ops.attn_fwd(
                    qd, kd, vd, q_valid=w.s_valid, kv_valid=w.k_valid, rope_q=tabs, rope_k=tabs, out=o, lse=lse,
                    workspace=wsd, schedule=sc), n, warm_s=0.3)
                del wsd
        if name in ("wan480", "hunyuan", "wan720"):   # the softmax forced each way (AUTO: fixed-m from 32768 keys)
            for tag, fm in (("fixed_m_us", True), ("online_us", False)):
                wsf = torch.empty(max(ops.attn_workspace_size(qd, kd, vd, q_valid=w.s_valid, kv_valid=w.k_valid,
                                                              rope_q=tabs, rope_k=tabs, fixed_m=fm), 256),
                                  dtype=torch.uint8, device=dev)
                ent[tag] = time_us(torch, lambda: ops.attn_fwd(
                    qd, kd, vd, q_valid=w.s_valid, kv_valid=w.k_valid, rope_q=tabs, rope_k=tabs, out=o, lse=lse,
                    workspace=wsf, fixed_m=fm), n)
                del wsf
        if name == "wan480":   # the same call with the per-head q/k RMSNorm fused into the pre-pass
            wn = torch.ones(w.d, dtype=torch.float32, device=dev)
            wsn = torch.empty(max(ops.attn_workspace_size(qd, kd, vd, q_valid=w.s_valid, kv_valid=w.k_valid,
                                                          rope_q=tabs, rope_k=tabs, q_norm=wn, k_norm=wn), 256),
                              dtype=torch.uint8, device=dev)
            ent["with_qk_rmsnorm_us"] = time_us(torch, lambda: ops.attn_fwd(
                qd, kd, vd, q_valid=w.s_valid, kv_valid=w.k_valid, rope_q=tabs, rope_k=tabs, out=o, lse=lse,
                workspace=wsn, q_norm=wn, k_norm=wn), n)
        if name == "wan480":   # the ring layout: two segments of 2340 real rows, each padded to 2368
            per, L = w.s_valid // 2, 2368
            qs, ks, vs = (torch.zeros((w.B, w.H, 2 * L, w.d), dtype=torch.bfloat16, device=dev) for _ in range(3))
            for src, dst in ((qd, qs), (kd, ks), (vd, vs)):
                for i in range(2):
                    dst[:, :, i * L:i * L + per] = src[:, :, i * per:(i + 1) * per]
            cs2, sn2 = (torch.zeros((2 * L, w.d // 2), dtype=torch.float32, device=dev) for _ in range(2))
            for i in range(2):
                cs2[i * L:i * L + per] = cos[i * per:(i + 1) * per]
                sn2[i * L:i * L + per] = sin[i * per:(i + 1) * per]
            os2 = torch.empty_like(qs)
            ls2 = torch.empty((w.B, w.H, 2 * L), dtype=torch.float32, device=dev)
            wss = torch.empty(max(ops.attn_workspace_size(qs, ks, vs, q_valid=per, kv_valid=per, q_seg_len=L,
                                                          kv_seg_len=L, rope_q=(cs2, sn2), rope_k=(cs2, sn2)), 256),
                              dtype=torch.uint8, device=dev)
            ent["ring_2_segments_us"] = time_us(torch, lambda: ops.attn_fwd(
                qs, ks, vs, q_valid=per, kv_valid=per, q_seg_len=L, kv_seg_len=L, rope_q=(cs2, sn2),
                rope_k=(cs2, sn2), out=os2, lse=ls2, workspace=wss), n)
            del qs, ks, vs, os2, wss
        if w.kv_valid:   # short-KV: report the HBM side too (Q, K, V, O, LSE once each)
            nbytes = w.B * w.H * (2 * w.s_pad * w.d * 2 + 2 * w.k_pad * w.d * 2 + w.s_pad * 4)
            ent.update({"hbm_bytes": nbytes, "hbm_GBps": nbytes / us / 1e3})
        if w.n_key_shards > 1:
            shards = W.key_shards(w)
            po = [torch.empty((w.B, w.H, w.s_pad, w.d), dtype=torch.float32, device=dev) for _ in shards]
            pl = [torch.empty((w.B, w.H, w.s_pad), dtype=torch.float32, device=dev) for _ in shards]
            tabs = [(cos[s0:s0 + L].contiguous(), sin[s0:s0 + L].contiguous()) for (s0, L, _) in shards]
            wss = [torch.empty(max(ops.attn_workspace_size(qd, kd[:, :, s0:s0 + L], vd[:, :, s0:s0 + L],
                                                           kv_valid=kvv, rope_q=(cos, sin), rope_k=tabs[i]), 256),
                               dtype=torch.uint8, device=dev) for i, (s0, L, kvv) in enumerate(shards)]
            om = torch.empty_like(qd)

            def sharded():
                for i, (s0, L, kvv) in enumerate(shards):
                    ops.attn_fwd(qd, kd[:, :, s0:s0 + L], vd[:, :, s0:s0 + L], q_valid=w.s_valid, kv_valid=kvv,
                                 rope_q=(cos, sin), rope_k=tabs[i], out=po[i], lse=pl[i], workspace=wss[i])
                ops.lse_merge(po, pl, q_valid=w.s_valid, out=om, lse_out=lse)

            us_m = time_us(torch, lambda: ops.lse_merge(po, pl, q_valid=w.s_valid, out=om, lse_out=lse), 10)
            us_s = time_us(torch, sharded, 3, warm=1)
            merge_bytes = len(shards) * (w.B * w.H * w.s_pad * (w.d * 4 + 4)) + w.B * w.H * w.s_pad * (w.d * 2 + 4)
            ent.update({"sharded_4_plus_merge_us": us_s, "sharded_tflops": w.valid_flop / us_s / 1e6,
                        "lse_merge_us": us_m, "lse_merge_GBps": merge_bytes / us_m / 1e3})
            del po, pl, wss, om
        res[name] = ent
        del qd, kd, vd, o, ws
        torch.cuda.empty_cache()
    return res


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "the benchmark runs on one GPU; --gpus must be 1 "
                          "(across GPUs the path would shard by head: each GPU runs this kernel on its head share)"}))
        sys.exit(2)
    if args.traffic_summary:
        traffic_summary(args)
        return
    if args.pmc_target:
        pmc_target(args)
        return
    if args.hbm_passes:
        hbm_passes(args)
        return
    if args.clock_probe:
        clock_probe(args)
        return
    import ctypes
    import numpy as np
    import workloads as W

    w = W.WORKLOADS[args.workload]
    # Host work first, before anything touches the GPU: the seeded inputs of
    # every config (and, unless skipped, the oracle timed on them) in a pool
    # of spawned single-threaded workers, one per core.
    names = [args.workload]
    if not args.no_configs:
        names += [n for n in CONFIGS + ("xattn480",) if n not in names]
    cpu_per, refs, workers = None, {}, pool_size()
    if args.no_cpu_baseline:
        inputs = {n: W.make_qkv(W.WORKLOADS[n]) for n in names}
    else:
        names += [n for n in CONFIGS if n not in names]
        with spawn_pool(workers) as pool:
            inputs = make_inputs(names, pool)
            cpu_per, refs = cpu_baseline_all(inputs, pool, keep=CONFIGS)

    import torch
    import long_sequence_attention_amd as ops

    ops.library_path()  # fails loudly if the HIP library is not built
    dev = torch.device("cuda:0")
    B, H, d, Sv, Sp = w.B, w.H, w.d, w.s_valid, w.s_pad

    q, k, v = inputs[args.workload]

    # token-major fused QKV [B, S_valid, 3, H, d]: what one all-to-all of the
    # stacked Q, K, V hands over (sequence shard -> head shard)
    def tok(x):
        t = torch.from_numpy(np.ascontiguousarray(x[:, :, :Sv].transpose(0, 2, 1, 3)).view(np.int16))
        return t.view(torch.bfloat16)
    qkv_tok = torch.stack([tok(q), tok(k), tok(v)], dim=2).to(dev)
    q_tok = qkv_tok[:, :, 0].contiguous()   # one tensor's worth, for the single-tensor pad figure
    pos = torch.from_numpy(W.positions(w)).to(dev)
    qkvp = torch.empty((B, Sp, 3, H, d), dtype=torch.bfloat16, device=dev)
    qp = torch.empty((B, Sp, H, d), dtype=torch.bfloat16, device=dev)
    op = torch.empty_like(qp)
    o_tok = torch.empty_like(q_tok)
    lse = torch.empty((B, H, Sp), dtype=torch.float32, device=dev)
    cos = torch.empty((Sp, d // 2), dtype=torch.float32, device=dev)
    sin = torch.empty_like(cos)
    L = ops._native.lib()
    chans = (ctypes.c_int32 * len(w.axes))(*w.axes)
    qv, kv_, vv = (qkvp[:, :, i].transpose(1, 2) for i in range(3))   # [B, H, S_pad, d] views
    ws = torch.empty(ops.attn_workspace_size(qv, kv_, vv, q_valid=Sv, kv_valid=Sv, rope_q=(cos, sin), rope_k=(cos, sin)),
                     dtype=torch.uint8, device=dev)
    # the step's padded buffer: Q and K rotated by the pad itself
    qkvr = torch.empty_like(qkvp)
    qr_v, kr_v, vr_v = (qkvr[:, :, i].transpose(1, 2) for i in range(3))
    ws_step = torch.empty(max(256, ops.attn_workspace_size(qr_v, kr_v, vr_v, q_valid=Sv, kv_valid=Sv)),
                          dtype=torch.uint8, device=dev)

    def step():
        s = ops._stream(dev)
        ops._native.check(L.dit_rope_split_tables(ctypes.c_void_p(pos.data_ptr()), Sp, len(w.axes), chans, d,
                                                  float(w.theta), ctypes.c_void_p(cos.data_ptr()),
                                                  ctypes.c_void_p(sin.data_ptr()), s), "tables")
        ops.pad_tokens_rope(qkv_tok, Sp, cos, sin, n_rot=2, out=qkvr)
        ops.attn_fwd(qr_v, kr_v, vr_v, q_valid=Sv, kv_valid=Sv, out=op.transpose(1, 2), lse=lse, workspace=ws_step)
        ops.unpad_tokens(op, Sv, out=o_tok)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    # whatever --warmup says, at least SETTLE_S seconds of steps: the shader
    # clock settles only after some hundreds of ms of sustained load
    t_end = time.perf_counter() + SETTLE_S
    while time.perf_counter() < t_end:
        for _ in range(50):
            step()
        torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(args.steps):
        step()
    e1.record()
    sclk_busy = sclk_levels()   # read while the queued steps still run
    torch.cuda.synchronize()
    ms_step = e0.elapsed_time(e1) / args.steps

    # Dominant kernel alone: with Q and K already rotated (the copies the
    # pre-pass left in the workspace: K first, then Q), dit_attn_fwd launches
    # exactly one kernel (the attention kernel) per call.
    ops.pad_tokens(qkv_tok, Sp, out=qkvp)
    ops.attn_fwd(qv, kv_, vv, q_valid=Sv, kv_valid=Sv, rope_q=(cos, sin), rope_k=(cos, sin), out=op.transpose(1, 2),
                 lse=lse, workspace=ws)
    torch.cuda.synchronize()
    n_el = B * H * Sp * d
    k_rot = ws[: n_el * 2].view(torch.bfloat16).view(B, H, Sp, d).clone()
    q_rot = ws[n_el * 2: n_el * 4].view(torch.bfloat16).view(B, H, Sp, d).clone()

    # the kernel-only call's own workspace (schedule partials): after one
    # clearing call its arrival counters stay zero, so the timed calls pass
    # ws_counters_zero and each launches the attention kernel alone
    ws_k = torch.empty(max(256, ops.attn_workspace_size(q_rot, k_rot, vv, q_valid=Sv, kv_valid=Sv)),
                       dtype=torch.uint8, device=dev)
    ops.attn_fwd(q_rot, k_rot, vv, q_valid=Sv, kv_valid=Sv, out=op.transpose(1, 2), lse=lse, workspace=ws_k)

    def attn_only():
        ops.attn_fwd(q_rot, k_rot, vv, q_valid=Sv, kv_valid=Sv, rope_q=None, rope_k=None,
                     out=op.transpose(1, 2), lse=lse, workspace=ws_k, ws_counters_zero=True)

    n = args.kernel_iters
    sclk_kernel = []
    us_attn = time_us(torch, attn_only, n, warm_s=1.0, clock=sclk_kernel)
    # the full call (pre-pass + kernel) on the step's strided views, right
    # after the kernel loop and with its own settling time, so both see the
    # clock of sustained load (the short passes below let it drift)
    us_call = time_us(torch, lambda: ops.attn_fwd(qv, kv_, vv, q_valid=Sv, kv_valid=Sv, rope_q=(cos, sin),
                                                  rope_k=(cos, sin), out=op.transpose(1, 2), lse=lse,
                                                  workspace=ws), n, warm_s=0.5)
    us_tables = time_us(torch, lambda: ops._native.check(L.dit_rope_split_tables(
        ctypes.c_void_p(pos.data_ptr()), Sp, len(w.axes), chans, d, float(w.theta), ctypes.c_void_p(cos.data_ptr()),
        ctypes.c_void_p(sin.data_ptr()), ops._stream(dev)), "tables"), n)
    us_pad = time_us(torch, lambda: ops.pad_tokens(q_tok, Sp, out=qp), n)
    us_pad_qkv = time_us(torch, lambda: ops.pad_tokens(qkv_tok, Sp, out=qkvp), n)
    us_pad_rope = time_us(torch, lambda: ops.pad_tokens_rope(qkv_tok, Sp, cos, sin, n_rot=2, out=qkvr), n)
    us_unpad = time_us(torch, lambda: ops.unpad_tokens(op, Sv, out=o_tok), n)
    flop = w.valid_flop
    achieved = flop / (us_attn * 1e-6) / 1e12
    pad_bytes = (Sv + Sp) * H * d * 2 * B
    traffic, traffic_src = read_traffic()

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
                   "flop_per_step": flop,
                   "step": "tables + pad of the fused QKV [B,S,3,H,d] with the Q/K RoPE applied on the way "
                           "(dit_pad_tokens_rope) + attn_fwd(attention kernel on the strided Q/K/V views) + unpad(O)"},
        "roofline": {"bound": "mfma", "achieved": achieved, "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": achieved / PEAK_BF16_TFLOPS, "traffic": traffic,
                     "traffic_unit": "HBM bytes per launch", "traffic_source": traffic_src,
                     "algorithmic_flop_per_launch": flop, "kernel": "attn_fwd_kernel<128, false>",
                     "kernel_us": us_attn},
        "kernels_us": {"attn_fwd_kernel": us_attn, "dit_attn_fwd_call(Q/K pre-pass + kernel)": us_call,
                       "rope_tables": us_tables, "pad_tokens(one tensor)": us_pad,
                       "pad_tokens(fused QKV)": us_pad_qkv, "pad_tokens_rope(fused QKV, Q/K rotated)": us_pad_rope,
                       "unpad_tokens": us_unpad,
                       "pad_GBps": pad_bytes / (us_pad * 1e-6) / 1e9,
                       "pad_qkv_GBps": 3 * pad_bytes / (us_pad_qkv * 1e-6) / 1e9,
                       "unpad_GBps": 2 * Sv * H * d * 2 * B / (us_unpad * 1e-6) / 1e9},
        "pct_of_peak_step": flop / (ms_step * 1e-3) / 1e12 / PEAK_BF16_TFLOPS * 100,
        # the dit_attn_fwd call (Q/K RoPE pre-pass + attention kernel) and the
        # attention kernel alone, against the bf16 dense peak
        "call_tflops": flop / (us_call * 1e-6) / 1e12,
        "call_pct_of_peak": flop / (us_call * 1e-6) / 1e12 / PEAK_BF16_TFLOPS * 100,
        "kernel_pct_of_peak": achieved / PEAK_BF16_TFLOPS * 100,
        "device": device_info(torch, sclk_busy, sclk_kernel[0] if sclk_kernel else None),
    }
    del k_rot
    if not args.no_configs:
        out["configs_attn_fwd"] = config_table(np, torch, ops, W, dev, n, inputs, refs)
    if cpu_per is not None:
        out["cpu_baseline"] = cpu_baseline_line(cpu_per, workers)
        step()   # the step's own output (the timings above reuse op / lse / o_tok)
        torch.cuda.synchronize()
        out["step_parity_vs_oracle"] = parity_of_step(np, o_tok, lse, refs[args.workload], Sv)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
