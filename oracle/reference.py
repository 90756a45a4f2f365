"""fp64 reference implementation (test infrastructure only; see package doc).

Everything here works in float64 on the host and applies no intermediate
rounding. Inputs that arrive as bf16 bit patterns are widened exactly.
"""
from __future__ import annotations

import math
import numpy as np


# ------------------------------------------------------------------ inputs
def bf16_to_f64(bits) -> np.ndarray:
    """Exact widening of bf16 bit patterns (uint16) to float64."""
    b = np.asarray(bits, dtype=np.uint16)
    with np.errstate(invalid="ignore"):
        return (b.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


# ------------------------------------------------------------------ padding
def plan_padding(s_valid: int, multiple: int) -> int:
    """Smallest multiple of `multiple` that holds s_valid rows (tail padding,
    Difflet PR #153 Wan padding commit; maxdiffusion PR #491 lane padding)."""
    if multiple <= 0 or s_valid < 0:
        raise ValueError("multiple must be positive and s_valid non-negative")
    return ((s_valid + multiple - 1) // multiple) * multiple


def pad_tokens(x: np.ndarray, s_pad: int) -> np.ndarray:
    """[B, s_valid, ...] -> [B, s_pad, ...], pad rows at the tail set to zero."""
    B, s_valid = x.shape[:2]
    out = np.zeros((B, s_pad) + x.shape[2:], dtype=x.dtype)
    out[:, :s_valid] = x
    return out


def unpad_tokens(x: np.ndarray, s_valid: int) -> np.ndarray:
    """[B, s_pad, ...] -> [B, s_valid, ...]: drop the tail pad rows."""
    return np.array(x[:, :s_valid], copy=True)


# ------------------------------------------------------------------ RoPE
def rope_pair_frequencies(axis_channels, theta: float) -> np.ndarray:
    """Per-pair angular frequency, float64 [d/2], in pair-space order.

    Axis a with c_a channels owns c_a/2 consecutive pairs; pair j of that axis
    turns at theta^(-2j/c_a) radians per position step.
    """
    freqs = []
    for c in axis_channels:
        if c % 2:
            raise ValueError("each axis needs an even channel count")
        j = np.arange(c // 2, dtype=np.float64)
        freqs.append(np.power(float(theta), -2.0 * j / c))
    return np.concatenate(freqs)


def rope_tables(pos, axis_channels, theta: float):
    """cos and sin tables, float64 [S, d/2], from integer positions [S, n_axes].

    Column P_a + j (P_a = pair offset of axis a) holds the angle
    pos[s, a] * theta^(-2j/c_a).
    """
    pos = np.asarray(pos)
    if pos.ndim == 1:
        pos = pos[:, None]
    if pos.shape[1] != len(axis_channels):
        raise ValueError("positions need one column per axis")
    freqs = rope_pair_frequencies(axis_channels, theta)
    axis_of_pair = np.concatenate(
        [np.full(c // 2, a) for a, c in enumerate(axis_channels)])
    angle = pos[:, axis_of_pair].astype(np.float64) * freqs[None, :]
    return np.cos(angle), np.sin(angle)


def rope_split_halves(x: np.ndarray, cos: np.ndarray, sin: np.ndarray) -> np.ndarray:
    """Rotate-half RoPE on [..., S, d]: channel i pairs with i + d/2.

    x'_i       = x_i c_i - x_{i+d/2} s_i
    x'_{i+d/2} = x_{i+d/2} c_i + x_i s_i
    """
    d = x.shape[-1]
    h = d // 2
    x1 = x[..., :h]
    x2 = x[..., h:]
    return np.concatenate([x1 * cos - x2 * sin, x2 * cos + x1 * sin], axis=-1)


def rope_interleaved(x: np.ndarray, cos: np.ndarray, sin: np.ndarray) -> np.ndarray:
    """Pairwise RoPE on [..., S, d]: channels (2i, 2i+1) form pair i.

    y'_{2i}   = y_{2i} c_i - y_{2i+1} s_i
    y'_{2i+1} = y_{2i+1} c_i + y_{2i} s_i
    """
    out = np.empty_like(x)
    e = x[..., 0::2]
    o = x[..., 1::2]
    out[..., 0::2] = e * cos - o * sin
    out[..., 1::2] = o * cos + e * sin
    return out


def rms_norm(x: np.ndarray, weight, eps: float) -> np.ndarray:
    """Per-head RMS normalisation over the last axis (d), float64:

        y_c = x_c / sqrt(mean_c' x_c'^2 + eps) * w_c

    The q/k norm that precedes RoPE in the FLUX and Wan attention (Difflet
    PR #153: the FLUX split-RoPE commit permutes the per-head q/k RMSNorm
    weights together with the to_q / to_k channels, and the Wan split-RoPE
    commit does the same). `weight` is [d] in the same channel order as x.
    """
    x = np.asarray(x, dtype=np.float64)
    w = np.asarray(weight, dtype=np.float64)
    ms = np.mean(x * x, axis=-1, keepdims=True)
    return x / np.sqrt(ms + eps) * w


def interleaved_to_split_permutation(d: int) -> np.ndarray:
    """Channel order [0, 2, ..., d-2, 1, 3, ..., d-1]: x_split = x_inter[..., P]."""
    return np.concatenate([np.arange(0, d, 2), np.arange(1, d, 2)])


# ------------------------------------------------------------------ attention
def attention(q, k, v, q_valid: int, kv_valid: int, scale: float | None = None,
              rows=None, block: int = 512):
    """Masked softmax attention with its natural-log LSE, float64.

    q: [B, H, S_q, d]; k, v: [B, H, S_kv, d] (any real dtype, widened to f64).
    Only keys j < kv_valid take part. For each query row i < q_valid:
        s_ij  = scale * <q_i, k_j>
        LSE_i = m_i + ln sum_j exp(s_ij - m_i),  m_i = max_j s_ij
        O_i   = sum_j exp(s_ij - LSE_i) v_j
    Rows i >= q_valid, and every row when kv_valid == 0, give O = 0 and
    LSE = -inf. `rows` selects which query rows to evaluate (default: all);
    the outputs then have len(rows) in place of S_q.
    Returns (O [B, H, R, d], LSE [B, H, R]).
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    B, H, S_q, d = q.shape
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    rows = np.arange(S_q) if rows is None else np.asarray(rows)
    R = len(rows)
    O = np.zeros((B, H, R, d), dtype=np.float64)
    L = np.full((B, H, R), -np.inf, dtype=np.float64)
    live = np.nonzero(rows < q_valid)[0]
    if kv_valid == 0 or len(live) == 0:
        return O, L
    for b in range(B):
        for h in range(H):
            kk = k[b, h, :kv_valid]
            vv = v[b, h, :kv_valid]
            for s0 in range(0, len(live), block):
                sel = live[s0:s0 + block]
                s = scale * (q[b, h, rows[sel]] @ kk.T)
                m = s.max(axis=1, keepdims=True)
                e = np.exp(s - m)
                l = e.sum(axis=1)
                O[b, h, sel] = (e @ vv) / l[:, None]
                L[b, h, sel] = m[:, 0] + np.log(l)
    return O, L


def segment_valid_rows(S: int, seg_len: int, valid: int) -> np.ndarray:
    """Indices of the real rows of a sequence of S rows cut into segments of
    seg_len rows, each holding `valid` real rows followed by its own tail
    pad (maxdiffusion PR #491: with ring parallelism every segment carries
    its own tail padding)."""
    if seg_len <= 0 or S % seg_len:
        raise ValueError("S must be a positive multiple of seg_len")
    r = np.arange(S)
    return r[(r % seg_len) < valid]


def attention_segmented(q, k, v, q_seg_len: int, q_valid: int, kv_seg_len: int, kv_valid: int,
                        scale: float | None = None):
    """Attention over tail-padded segments, float64: query row i is real when
    i mod q_seg_len < q_valid, key j when j mod kv_seg_len < kv_valid; every
    real query attends to every real key of every segment (one softmax over
    their union). Pad query rows give O = 0 and LSE = -inf.

    Written as the plain definition: the real keys are gathered into one
    contiguous block and `attention` runs on it for the real query rows.
    """
    q = np.asarray(q, dtype=np.float64)
    B, H, S_q, d = q.shape
    qr = segment_valid_rows(S_q, q_seg_len, q_valid)
    kr = segment_valid_rows(np.asarray(k).shape[2], kv_seg_len, kv_valid)
    kc = np.asarray(k, dtype=np.float64)[:, :, kr]
    vc = np.asarray(v, dtype=np.float64)[:, :, kr]
    Oc, Lc = attention(q[:, :, qr], kc, vc, len(qr), len(kr), scale)
    O = np.zeros((B, H, S_q, d))
    L = np.full((B, H, S_q), -np.inf)
    O[:, :, qr] = Oc
    L[:, :, qr] = Lc
    return O, L


def fixed_m_bound(q, k, key_rows, scale: float | None = None) -> np.ndarray:
    """A-priori upper bound of each query row's largest score, float64:

        m_i = scale * (q_i . kbar + |q_i| * max_j |k_j - kbar|),
        kbar = mean of the real keys k_j (j in key_rows)

    since q_i . k_j = q_i . kbar + q_i . (k_j - kbar) <= q_i . kbar +
    |q_i| |k_j - kbar| (Cauchy-Schwarz). The fixed-m softmax uses it in place
    of the running maximum (maxdiffusion PR #491 builds it from norm
    reductions and the key mean over the real rows only, and sends a block
    whose bound is too loose to the online-softmax path). The pages do not
    print the formula; this is the plain reading. q: [B, H, S_q, d];
    k: [B, H, S_kv, d]; returns [B, H, S_q].
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)[:, :, np.asarray(key_rows)]
    d = q.shape[-1]
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    kbar = k.mean(axis=2, keepdims=True)                           # [B, H, 1, d]
    R = np.sqrt(((k - kbar) ** 2).sum(axis=-1)).max(axis=2)         # [B, H]
    qn = np.sqrt((q * q).sum(axis=-1))                              # [B, H, S_q]
    return scale * ((q @ np.swapaxes(kbar, -1, -2))[..., 0] + qn * R[..., None])


def attention_bruteforce(q, k, v, q_valid: int, kv_valid: int, scale: float | None = None):
    """The same definition as `attention`, in pure-Python loops (tiny sizes)."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    B, H, S_q, d = q.shape
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    O = np.zeros((B, H, S_q, d))
    L = np.full((B, H, S_q), -math.inf)
    for b in range(B):
        for h in range(H):
            for i in range(min(q_valid, S_q)):
                if kv_valid == 0:
                    continue
                scores = [scale * math.fsum(float(q[b, h, i, c]) * float(k[b, h, j, c]) for c in range(d))
                          for j in range(kv_valid)]
                mx = max(scores)
                w = [math.exp(s - mx) for s in scores]
                tot = math.fsum(w)
                for c in range(d):
                    O[b, h, i, c] = math.fsum(w[j] * float(v[b, h, j, c]) for j in range(kv_valid)) / tot
                L[b, h, i] = mx + math.log(tot)
    return O, L


def lse_merge(o_parts, lse_parts, q_valid: int | None = None):
    """Merge per-key-shard partial results into the single-pass result.

    For each row: M = max_k L_k, w_k = exp(L_k - M), L = M + ln sum_k w_k,
    O = sum_k w_k O_k / sum_k w_k. A row whose parts are all -inf (no keys)
    gives O = 0 and L = -inf. Rows >= q_valid (if given) give O = 0, L = -inf.
    o_parts: list of [..., S, d]; lse_parts: list of [..., S].
    """
    Os = np.stack([np.asarray(o, dtype=np.float64) for o in o_parts])
    Ls = np.stack([np.asarray(l, dtype=np.float64) for l in lse_parts])
    M = Ls.max(axis=0)
    empty = np.isneginf(M)
    Msafe = np.where(empty, 0.0, M)
    w = np.exp(Ls - Msafe[None])                 # exp(-inf) = 0 for empty parts
    wsum = w.sum(axis=0)
    wsafe = np.where(empty, 1.0, wsum)
    O = (w[..., None] * Os).sum(axis=0) / wsafe[..., None]
    L = np.where(empty, -np.inf, Msafe + np.log(wsafe))
    O = np.where(empty[..., None], 0.0, O)
    if q_valid is not None:
        S = O.shape[-2]
        pad = np.arange(S) >= q_valid
        O[..., pad, :] = 0.0
        L[..., pad] = -np.inf
    return O, L


# ------------------------------------------------------------------ whole path
def dit_path(q_bits, k_bits, v_bits, pos_q, pos_k, axis_channels, theta: float,
             q_valid: int, kv_valid: int, scale: float | None = None, rows=None):
    """RoPE (split halves) on Q and K, then masked attention with LSE.

    q_bits/k_bits/v_bits: bf16 patterns [B, H, S, d]; pos_q / pos_k: int
    positions [S, n_axes] for the query and key rows. Nothing is rounded
    between steps.
    """
    q = bf16_to_f64(q_bits)
    k = bf16_to_f64(k_bits)
    v = bf16_to_f64(v_bits)
    cq, sq = rope_tables(pos_q, axis_channels, theta)
    ck, sk = rope_tables(pos_k, axis_channels, theta)
    if rows is not None:
        qr = rope_split_halves(q[:, :, rows], cq[rows], sq[rows])
        O, L = attention(qr, rope_split_halves(k, ck, sk), v, q_valid=np.iinfo(np.int64).max,
                         kv_valid=kv_valid, scale=scale)
        live = np.asarray(rows) < q_valid
        O[:, :, ~live] = 0.0
        L[:, :, ~live] = -np.inf
        return O, L
    return attention(rope_split_halves(q, cq, sq), rope_split_halves(k, ck, sk), v,
                     q_valid=q_valid, kv_valid=kv_valid, scale=scale)
