"""Builds the HIP library libditattn.so for gfx950, in-tree.

    python -m long_sequence_attention_amd.build [--verbose]

The library is a plain C ABI (include/dit_attn.h); the Python binding loads
it with ctypes. Every call compiles from scratch (a few seconds per file).
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIBDIR = os.path.join(PKG, "lib")
LIB = os.path.join(LIBDIR, "libditattn.so")
# the same sources with a wait and a barrier after every DMA issue and LDS
# read phase of the attention kernel (results must equal LIB's bit for bit)
LIB_DEBUG_SYNC = os.path.join(LIBDIR, "libditattn_debugsync.so")
# the same sources with shader-clock stamps around each workgroup's key loop
# (bench.py --clock-probe reads them)
LIB_CLOCK_PROBE = os.path.join(LIBDIR, "libditattn_clockprobe.so")
SOURCES = ["api.hip", "attn_fwd.hip", "elementwise.hip", "fixed_m.hip"]

HIPCC_FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-shared",
    "-Wall",
    "-Wno-unused-result",
    # keep the compiler from forming packed fp32 VALU ops
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-fvisibility=hidden",
]


def source_hash() -> str:
    """sha256 (16 hex digits) of every library source and header: written
    next to the library at build time, so a library older than its sources
    can be told apart."""
    import hashlib
    h = hashlib.sha256()
    for d in (CSRC, os.path.join(ROOT, "include")):
        for name in sorted(os.listdir(d)):
            if name.endswith((".hip", ".h", ".hpp", ".cpp")):
                h.update(name.encode())
                with open(os.path.join(d, name), "rb") as f:
                    h.update(f.read())
    return h.hexdigest()[:16]


HASH_FILE = LIB + ".srchash"


def is_current() -> bool:
    """Both libraries exist and were built from the sources as they are now."""
    try:
        with open(HASH_FILE) as f:
            recorded = f.read().strip()
    except OSError:
        return False
    return all(os.path.exists(x) for x in (LIB, LIB_DEBUG_SYNC, LIB_CLOCK_PROBE)) and recorded == source_hash()


def hipcc() -> str:
    for cand in (shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found: the HIP library cannot be built")


def _command(out, extra_flags):
    return [hipcc(), *HIPCC_FLAGS, *(extra_flags or []), "-I", os.path.join(ROOT, "include"), "-I", CSRC,
            *[os.path.join(CSRC, s) for s in SOURCES], "-o", out]


def build(verbose: bool = False, extra_flags=None, debug_sync: bool = True) -> str:
    """Compile LIB (and, unless debug_sync is False, LIB_DEBUG_SYNC and
    LIB_CLOCK_PROBE alongside it in parallel compiler processes); returns
    LIB's path."""
    os.makedirs(LIBDIR, exist_ok=True)
    jobs = [(LIB, list(extra_flags or []))]
    if debug_sync:
        jobs.append((LIB_DEBUG_SYNC, list(extra_flags or []) + ["-DDIT_DEBUG_SYNC=1"]))
        jobs.append((LIB_CLOCK_PROBE, list(extra_flags or []) + ["-DDIT_CLOCK_PROBE=1"]))
    procs = []
    for out, flags in jobs:
        cmd = _command(out + ".tmp", flags)
        if verbose:
            print(" ".join(cmd), flush=True)
        procs.append((out, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.PIPE, text=True)))
    noise = "is not a recognized feature for this target"
    failed = []
    for out, proc in procs:
        _, stderr = proc.communicate()
        err = "\n".join(l for l in (stderr or "").splitlines() if noise not in l)
        if proc.returncode != 0:
            failed.append(f"{os.path.basename(out)}: hipcc failed ({proc.returncode}):\n{err}")
            continue
        if verbose and err.strip():
            print(err, file=sys.stderr)
        os.replace(out + ".tmp", out)
    if failed:
        raise RuntimeError("\n".join(failed))
    if debug_sync and not extra_flags:
        with open(HASH_FILE, "w") as f:
            f.write(source_hash() + "\n")
    return LIB


if __name__ == "__main__":
    print(build(verbose="--verbose" in sys.argv))
