"""Seeded synthetic inputs for the DiT self-attention path.

This module is shared by the tests, the benchmark and the oracle checks. It
holds no arithmetic of the method itself (no RoPE, no attention, no merge):
only the workload shapes, integer token positions, seeded random draws, the
per-head RMS normalisation used to synthesise Q/K, and bf16 rounding of the
drawn values.

Workload shapes follow the token grids the pages describe:
  * Wan 2.1 480x832x9 -> a 3x30x52 latent grid, 4680 tokens, tail-padded to
    4736 (Difflet PR #153, "Wan padding + split RoPE" commit); 720p / 81
    frames -> 21x45x80 = 75,600 tokens (maxdiffusion PR #491, lane padding
    description).
  * HunyuanVideo 320x512x61 -> 10240 video + 226 text tokens = 10466, padded
    to 10496 (Difflet PR #153, HunyuanVideo single-stream SP commit).
  * FLUX.1-dev 1024^2 -> 4096 image tokens on a 64x64 grid + 512 text tokens
    (Difflet PR #153, FLUX SP commit).
The pages use real checkpoints and prompts; these synthetic N(0,1) draws of
the same shapes stand in for them.
"""
from __future__ import annotations

from dataclasses import dataclass
import numpy as np

__all__ = [
    "Workload", "WORKLOADS", "bf16_bits", "bf16_bits_to_f32", "finite_garbage_bits",
    "positions", "make_qkv", "sample_rows", "key_shards",
]


@dataclass(frozen=True)
class Workload:
    name: str
    B: int
    H: int
    d: int
    s_valid: int
    s_pad: int
    axes: tuple          # RoPE channels per axis (sum == d), in t,h,w order
    grid: tuple          # extents of the rotated token grid, same axis order
    n_text: int          # text tokens after the grid tokens, all at position 0
    qk_norm: bool        # per-head RMS normalisation of Q and K
    seed: int
    theta: float = 10000.0
    n_key_shards: int = 1
    description: str = ""
    # cross-attention: keys/values of their own length (0 = the query
    # tokens themselves), and whether RoPE applies at all
    kv_valid: int = 0
    kv_pad: int = 0
    rope: bool = True

    @property
    def n_axes(self) -> int:
        return len(self.axes)

    @property
    def k_valid(self) -> int:
        return self.kv_valid or self.s_valid

    @property
    def k_pad(self) -> int:
        return self.kv_pad or self.s_pad

    @property
    def valid_flop(self) -> float:
        """4*B*H*S_valid*K_valid*d: two dense contractions over valid tokens."""
        return 4.0 * self.B * self.H * self.s_valid * self.k_valid * self.d


WORKLOADS = {
    "tiny": Workload(
        "tiny", B=1, H=2, d=64, s_valid=300, s_pad=320, axes=(64,), grid=(300,),
        n_text=0, qk_norm=False, seed=0,
        description="B=1 H=2 d=64, 300 tokens padded to 320, 1-D RoPE on positions 0..299"),
    "flux": Workload(
        "flux", B=1, H=24, d=128, s_valid=4608, s_pad=4608, axes=(64, 64), grid=(64, 64),
        n_text=512, qk_norm=True, seed=1,
        description="FLUX-like joint attention: 64x64 image grid + 512 text tokens, H=24 d=128"),
    "wan480": Workload(
        "wan480", B=1, H=10, d=128, s_valid=4680, s_pad=4736, axes=(44, 42, 42),
        grid=(3, 30, 52), n_text=0, qk_norm=True, seed=2,
        description="Wan 480x832x9 Ulysses shard: 3x30x52 grid, 4680 tokens padded to 4736, H=10 d=128"),
    "hunyuan": Workload(
        "hunyuan", B=1, H=6, d=128, s_valid=10466, s_pad=10496, axes=(16, 56, 56),
        grid=(16, 20, 32), n_text=226, qk_norm=True, seed=3,
        description="HunyuanVideo-like shard: 16x20x32 video grid + 226 text, 10466 padded to 10496, H=6"),
    "wan720": Workload(
        "wan720", B=1, H=10, d=128, s_valid=75600, s_pad=75648, axes=(44, 42, 42),
        grid=(21, 45, 80), n_text=0, qk_norm=True, seed=4, n_key_shards=4,
        description="Wan 720p/81f shard: 21x45x80 grid, 75600 padded to 75648, H=10; 4 key shards"),
    "xattn480": Workload(
        "xattn480", B=1, H=10, d=128, s_valid=4680, s_pad=4736, axes=(44, 42, 42),
        grid=(3, 30, 52), n_text=0, qk_norm=True, seed=6, kv_valid=512, kv_pad=512, rope=False,
        description="Wan 480p short-KV cross-attention: 4680 video queries (padded to 4736) over 512 "
                    "text keys, H=10 d=128, no RoPE"),
}


# ---------------------------------------------------------------- bf16 rounding
def bf16_bits(x) -> np.ndarray:
    """Round float32 values to bfloat16 (round to nearest, ties to even).

    Returns the 16-bit patterns as uint16. NaN maps to a quiet NaN of the same
    sign; infinities and overflow behave as IEEE rounding prescribes.
    """
    f = np.ascontiguousarray(x, dtype=np.float32)
    u = f.view(np.uint32).astype(np.uint64)
    lsb = (u >> 16) & 1
    r = ((u + 0x7FFF + lsb) >> 16).astype(np.uint32).astype(np.uint16)
    nan = np.isnan(f)
    if nan.any():
        r = np.where(nan, ((u >> 16).astype(np.uint16) & 0x8000) | 0x7FC0, r).astype(np.uint16)
    return r


def bf16_bits_to_f32(bits) -> np.ndarray:
    """Exact widening of bf16 patterns (uint16) to float32."""
    b = np.ascontiguousarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32)


def finite_garbage_bits(rng: np.random.Generator, shape) -> np.ndarray:
    """Uniformly random bf16 bit patterns whose exponent field is never all
    ones, i.e. finite values of any magnitude (up to ~3.4e38) and sign."""
    bits = rng.integers(0, 1 << 16, size=shape, dtype=np.uint16)
    inf_nan = (bits & 0x7F80) == 0x7F80
    bits[inf_nan] &= np.uint16(0xBFFF)
    return bits


# ---------------------------------------------------------------- positions
def positions(w: Workload) -> np.ndarray:
    """Integer RoPE positions, int32 [s_pad, n_axes].

    Grid tokens take their grid coordinates, flattened with the first axis
    slowest and the last fastest. Text tokens (after the grid) and tail pads
    take position 0 on every axis, which is the identity rotation.
    """
    n_grid = int(np.prod(w.grid))
    assert n_grid + w.n_text == w.s_valid, (w.name, n_grid, w.n_text, w.s_valid)
    pos = np.zeros((w.s_pad, w.n_axes), dtype=np.int32)
    coords = np.indices(w.grid).reshape(w.n_axes, -1).T
    pos[:n_grid] = coords
    return pos


# ---------------------------------------------------------------- Q/K/V draws
def _rms_normalise(x: np.ndarray, eps: float = 1e-6) -> np.ndarray:
    x64 = x.astype(np.float64)
    return (x64 / np.sqrt(np.mean(x64 * x64, axis=-1, keepdims=True) + eps)).astype(np.float32)


def make_head(w: Workload, tensor: str, b: int, h: int, garbage_seed_offset: int = 1000) -> np.ndarray:
    """bf16 bits [s_pad, d] of one (tensor, batch, head).

    Valid rows are N(0,1) float32 draws from the stream seeded by
    (seed, tensor index, b, h), RMS-normalised per row for Q/K when the
    workload asks for it, then rounded to bf16. Pad rows are finite garbage
    from the stream seeded by (seed + garbage_seed_offset, tensor index, b, h).
    """
    ti = "qkv".index(tensor)
    valid, pad = (w.s_valid, w.s_pad) if tensor == "q" else (w.k_valid, w.k_pad)
    rng = np.random.default_rng([w.seed, ti, b, h])
    x = rng.standard_normal((valid, w.d), dtype=np.float32)
    if w.qk_norm and tensor in "qk":
        x = _rms_normalise(x)
    out = np.empty((pad, w.d), dtype=np.uint16)
    out[:valid] = bf16_bits(x)
    if pad > valid:
        g = np.random.default_rng([w.seed + garbage_seed_offset, ti, b, h])
        out[valid:] = finite_garbage_bits(g, (pad - valid, w.d))
    return out


def make_qkv(w: Workload, heads=None, garbage_seed_offset: int = 1000):
    """Q, K, V as bf16 bit arrays (uint16): Q [B, len(heads), s_pad, d], K and V
    [B, len(heads), k_pad, d]."""
    heads = list(range(w.H)) if heads is None else list(heads)
    res = []
    for t in "qkv":
        arr = np.empty((w.B, len(heads), w.s_pad if t == "q" else w.k_pad, w.d), dtype=np.uint16)
        for b in range(w.B):
            for j, h in enumerate(heads):
                arr[b, j] = make_head(w, t, b, h, garbage_seed_offset)
        res.append(arr)
    return tuple(res)


def sample_rows(w: Workload, h: int, n: int = 2048) -> np.ndarray:
    """Sorted query rows drawn without replacement from the valid rows, for
    workloads too large for the oracle to evaluate in full."""
    rng = np.random.default_rng(5000 + h)
    return np.sort(rng.choice(w.s_valid, size=min(n, w.s_valid), replace=False))


def key_shards(w: Workload, n: int | None = None):
    """Contiguous key shards of the padded length: list of (start, length,
    valid) with valid = number of real (non-pad) keys in that shard."""
    n = w.n_key_shards if n is None else n
    assert w.s_pad % n == 0
    L = w.s_pad // n
    out = []
    for i in range(n):
        s0 = i * L
        out.append((s0, L, int(max(0, min(w.s_valid - s0, L)))))
    return out
