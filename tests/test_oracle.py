"""Pins for the fp64 oracle: closed forms, invariants, library routines,
brute force, the pages' printed padding plans, and negative controls that
plant a plausible mistake in an oracle function and show a pin catches it.

All of these run on the CPU (no GPU marker).
"""
import json
import math
import os

import numpy as np
import pytest
import scipy.special
import torch

import oracle
from oracle import reference as R
import workloads as W

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def rng(seed=0):
    return np.random.default_rng(seed)


# ------------------------------------------------------------------ inputs
def test_bf16_rounding_matches_torch_on_every_pattern():
    # Every finite bf16 pattern survives f32 widening and re-rounding, and
    # torch's own RNE conversion agrees with the generator's on all of them.
    bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    f = W.bf16_bits_to_f32(bits)
    finite = np.isfinite(f)
    ours = W.bf16_bits(f[finite])
    assert np.array_equal(ours, bits[finite])
    t = torch.from_numpy(f[finite].copy()).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, t)


def test_bf16_rounding_matches_torch_on_random_and_tie_values():
    r = rng(1)
    x = np.concatenate([
        r.standard_normal(200000).astype(np.float32) * np.float32(10.0) ** r.integers(-30, 30, 200000).astype(np.float32),
        # exact ties: low 16 bits == 0x8000, both parities of the kept lsb
        (r.integers(0, 1 << 15, 50000, dtype=np.uint32) << 17 | 0x8000).view(np.float32),
        (r.integers(0, 1 << 15, 50000, dtype=np.uint32) << 17 | 0x18000).view(np.float32),
    ]).astype(np.float32)
    x = x[np.isfinite(x)]
    t = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(W.bf16_bits(x), t)


def test_oracle_widening_is_exact():
    bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    a = oracle.bf16_to_f64(bits)
    b = torch.from_numpy(bits.view(np.int16).copy()).view(torch.bfloat16).to(torch.float64).numpy()
    same = (a == b) | (np.isnan(a) & np.isnan(b))
    assert same.all()


def test_garbage_is_finite_and_uses_the_whole_range():
    g = W.finite_garbage_bits(rng(2), (4096, 64))
    f = W.bf16_bits_to_f32(g)
    assert np.isfinite(f).all()
    assert np.abs(f).max() > 1e30 and (f < 0).any() and (f > 0).any()


@pytest.mark.parametrize("name", list(W.WORKLOADS))
def test_workload_token_counts(name):
    w = W.WORKLOADS[name]
    assert int(np.prod(w.grid)) + w.n_text == w.s_valid
    assert sum(w.axes) == w.d and all(c % 2 == 0 for c in w.axes)
    assert w.s_pad >= w.s_valid and oracle.plan_padding(w.s_valid, 128 if w.d == 128 else 64) == w.s_pad
    pos = W.positions(w)
    assert pos.shape == (w.s_pad, len(w.axes))
    n_grid = int(np.prod(w.grid))
    assert (pos[n_grid:] == 0).all()
    assert tuple(pos[:n_grid].max(axis=0) + 1) == w.grid


def test_generator_is_deterministic_against_stored_hashes():
    import hashlib
    with open(os.path.join(GOLDEN, "input_hashes.json")) as fh:
        stored = json.load(fh)["hashes"]
    for key, want in stored.items():
        name, heads = key.split(":")
        w = W.WORKLOADS[name]
        hs = None if heads == "all" else [int(heads)]
        q, k, v = W.make_qkv(w, heads=hs)
        got = hashlib.sha256(q.tobytes() + k.tobytes() + v.tobytes()).hexdigest()
        assert got == want, key


# ------------------------------------------------------------------ padding
def test_padding_plans_printed_on_the_pages():
    with open(os.path.join(GOLDEN, "padding_plans.json")) as fh:
        cases = json.load(fh)["cases"]
    for c in cases:
        assert oracle.plan_padding(c["s_valid"], c["multiple"]) == c["s_pad"], c["cite"]


def test_pad_unpad_round_trip_and_zero_fill():
    x = rng(3).standard_normal((2, 37, 5, 8))
    p = oracle.pad_tokens(x, 48)
    assert p.shape == (2, 48, 5, 8)
    assert (p[:, 37:] == 0).all() and np.array_equal(p[:, :37], x)
    assert np.array_equal(oracle.unpad_tokens(p, 37), x)


# ------------------------------------------------------------------ RoPE
def test_rope_frequencies_closed_form():
    # theta = 16, axes of 4 and 8 channels:
    #   axis 0: 16^(-0/4), 16^(-2/4) = 1, 1/4
    #   axis 1: 16^(-2j/8) = 2^(-j): 1, 1/2, 1/4, 1/8
    f = oracle.rope_pair_frequencies((4, 8), 16.0)
    assert np.allclose(f, [1.0, 0.25, 1.0, 0.5, 0.25, 0.125], rtol=0, atol=1e-15)
    # the standard 1-D schedule at theta=10000, d=64: last pair 10000^(-62/64)
    f = oracle.rope_pair_frequencies((64,), 10000.0)
    assert f[0] == 1.0 and abs(f[31] - 10000.0 ** (-62 / 64)) < 1e-18


def test_rope_tables_closed_form_values():
    pos = np.array([[0, 0], [3, 5], [7, 2]])
    c, s = oracle.rope_tables(pos, (4, 8), 16.0)
    freqs = [1.0, 0.25, 1.0, 0.5, 0.25, 0.125]
    axis = [0, 0, 1, 1, 1, 1]
    for i in range(3):
        for j in range(6):
            ang = pos[i, axis[j]] * freqs[j]
            assert abs(c[i, j] - math.cos(ang)) < 1e-15
            assert abs(s[i, j] - math.sin(ang)) < 1e-15
    assert (c[0] == 1).all() and (s[0] == 0).all()


def test_rope_interleaved_is_complex_multiplication():
    r = rng(4)
    d, S = 16, 9
    y = r.standard_normal((S, d))
    pos = r.integers(0, 50, (S, 2))
    c, s = oracle.rope_tables(pos, (6, 10), 10000.0)
    ang = np.arctan2(s, c)
    z = (y[:, 0::2] + 1j * y[:, 1::2]) * np.exp(1j * ang)
    out = oracle.rope_interleaved(y, c, s)
    assert np.allclose(out[:, 0::2], z.real, atol=1e-13)
    assert np.allclose(out[:, 1::2], z.imag, atol=1e-13)


def test_split_halves_equals_interleaved_after_permutation():
    r = rng(5)
    for d in (8, 64, 128):
        x = r.standard_normal((3, 11, d))
        pos = r.integers(0, 100, (11, 1))
        c, s = oracle.rope_tables(pos, (d,), 10000.0)
        P = oracle.interleaved_to_split_permutation(d)
        a = oracle.rope_split_halves(x[..., P], c, s)
        b = oracle.rope_interleaved(x, c, s)[..., P]
        assert np.array_equal(a, b)


def test_rope_preserves_norm_and_position_zero_is_identity():
    r = rng(6)
    x = r.standard_normal((5, 20, 128)) * 3
    pos = r.integers(0, 80, (20, 3))
    c, s = oracle.rope_tables(pos, (44, 42, 42), 10000.0)
    y = oracle.rope_split_halves(x, c, s)
    assert np.allclose(np.linalg.norm(y, axis=-1), np.linalg.norm(x, axis=-1), rtol=1e-14)
    c0, s0 = oracle.rope_tables(np.zeros((20, 3), int), (44, 42, 42), 10000.0)
    assert np.array_equal(oracle.rope_split_halves(x, c0, s0), x)


def test_rope_relative_position_property():
    r = rng(7)
    axes = (44, 42, 42)
    q = r.standard_normal(128)
    k = r.standard_normal(128)
    p = np.array([[1, 4, 9]])
    pk = np.array([[2, 11, 3]])
    delta = np.array([[5, -3, 17]])

    def rot(x, pos):
        c, s = oracle.rope_tables(pos, axes, 10000.0)
        return oracle.rope_split_halves(x[None], c, s)[0]

    a = rot(q, p) @ rot(k, pk)
    b = rot(q, p + delta) @ rot(k, pk + delta)
    assert abs(a - b) < 1e-12 * (1 + abs(a))


# ------------------------------------------------------------------ q/k RMSNorm
def test_rms_norm_worked_example():
    # x = (3, 4): mean of squares 12.5, so y = x / sqrt(12.5); with eps = 0.5
    # the divisor is sqrt(13) (hand-computed values)
    y = oracle.rms_norm(np.array([3.0, 4.0]), np.ones(2), 0.0)
    assert np.allclose(y, [0.848528137423857, 1.131370849898476], rtol=0, atol=1e-15)
    y = oracle.rms_norm(np.array([3.0, 4.0]), np.array([2.0, -1.0]), 0.5)
    assert np.allclose(y, [2 * 0.8320502943378437, -1.1094003924504583], rtol=0, atol=1e-15)


def test_rms_norm_unit_rms_scale_invariance_and_zero():
    x = rng(20).standard_normal((3, 5, 128)) * 7.0
    y = oracle.rms_norm(x, np.ones(128), 0.0)
    assert np.allclose(np.mean(y * y, axis=-1), 1.0, rtol=0, atol=1e-13)
    assert np.allclose(oracle.rms_norm(0.01 * x, np.ones(128), 0.0), y, rtol=0, atol=1e-12)
    assert np.allclose(oracle.rms_norm(-x, np.ones(128), 0.0), -y, rtol=0, atol=0)
    z = oracle.rms_norm(np.zeros((2, 64)), np.ones(64), 1e-6)
    assert np.isfinite(z).all() and (z == 0).all()


def test_rms_norm_commutes_with_the_split_permutation():
    # permuting the weights together with the channels (the pages' split-RoPE
    # load step) leaves the normalised values permuted the same way
    r = rng(21)
    x, w = r.standard_normal((4, 128)), r.standard_normal(128)
    P = oracle.interleaved_to_split_permutation(128)
    assert np.allclose(oracle.rms_norm(x[:, P], w[P], 1e-6), oracle.rms_norm(x, w, 1e-6)[:, P], rtol=0, atol=1e-14)


def test_rms_norm_then_rope_keeps_unit_rms():
    r = rng(22)
    x = r.standard_normal((6, 64)) * 3.0
    cos, sin = oracle.rope_tables(np.arange(6)[:, None] * 5, (64,), 10000.0)
    y = oracle.rope_split_halves(oracle.rms_norm(x, np.ones(64), 0.0), cos, sin)
    assert np.allclose(np.mean(y * y, axis=-1), 1.0, rtol=0, atol=1e-13)


def test_negative_control_sum_instead_of_mean_fails_unit_rms():
    x = rng(23).standard_normal((2, 64))
    wrong = x / np.sqrt(np.sum(x * x, axis=-1, keepdims=True))
    assert not np.allclose(np.mean(wrong * wrong, axis=-1), 1.0, atol=1e-3)


# ------------------------------------------------------------------ attention
def rand_qkv(seed, B, H, Sq, Skv, d, scale=1.0):
    r = rng(seed)
    return (r.standard_normal((B, H, Sq, d)) * scale, r.standard_normal((B, H, Skv, d)),
            r.standard_normal((B, H, Skv, d)))


def test_softmax_weights_sum_to_one():
    q, k, v = rand_qkv(8, 1, 2, 33, 70, 64, scale=2.0)
    O, L = oracle.attention(q, k, v, q_valid=33, kv_valid=61)
    s = np.einsum("bhid,bhjd->bhij", q, k[:, :, :61]) / 8.0
    P = np.exp(s - L[..., None])
    assert np.allclose(P.sum(-1), 1.0, rtol=0, atol=1e-12)
    assert np.allclose(np.einsum("bhij,bhjd->bhid", P, v[:, :, :61]), O, atol=1e-12)


@pytest.mark.parametrize("kv_valid", [1, 7, 64, 300])
def test_zero_query_gives_mean_of_valid_values(kv_valid):
    _, k, v = rand_qkv(9, 1, 2, 5, 320, 64)
    q = np.zeros((1, 2, 5, 64))
    O, L = oracle.attention(q, k, v, q_valid=5, kv_valid=kv_valid)
    assert np.allclose(O, v[:, :, :kv_valid].mean(axis=2, keepdims=True), atol=1e-13)
    assert np.allclose(L, math.log(kv_valid), rtol=0, atol=1e-13)


def test_single_valid_key_gives_its_value_and_score():
    q, k, v = rand_qkv(10, 1, 1, 4, 16, 128)
    O, L = oracle.attention(q, k, v, q_valid=4, kv_valid=1)
    assert np.allclose(O, np.broadcast_to(v[:, :, :1], O.shape), atol=1e-14)
    assert np.allclose(L[0, 0], (q[0, 0] @ k[0, 0, 0]) / math.sqrt(128), atol=1e-13)


def test_two_key_worked_example():
    # q = a*e0, k0 = e0, k1 = -e0 -> s0 = a/sqrt(d), s1 = -s0
    d, a = 64, 3.0
    q = np.zeros((1, 1, 1, d)); q[..., 0] = a
    k = np.zeros((1, 1, 2, d)); k[0, 0, 0, 0] = 1; k[0, 0, 1, 0] = -1
    v = np.zeros((1, 1, 2, d)); v[0, 0, 0, :] = 1.0; v[0, 0, 1, :] = -2.0
    s0 = a / 8.0
    w0 = 1.0 / (1.0 + math.exp(-2 * s0))
    O, L = oracle.attention(q, k, v, 1, 2)
    assert np.allclose(O[0, 0, 0], w0 * 1.0 + (1 - w0) * -2.0, atol=1e-15)
    assert abs(L[0, 0, 0] - (s0 + math.log1p(math.exp(-2 * s0)))) < 1e-15


def test_lse_against_scipy_logsumexp():
    q, k, v = rand_qkv(11, 2, 3, 40, 90, 128, scale=4.0)
    O, L = oracle.attention(q, k, v, q_valid=40, kv_valid=77, scale=0.3)
    s = np.einsum("bhid,bhjd->bhij", q, k[:, :, :77]) * 0.3
    assert np.allclose(L, scipy.special.logsumexp(s, axis=-1), atol=1e-12)


def test_pad_rows_are_excluded_exactly():
    q, k, v = rand_qkv(12, 1, 2, 64, 64, 64)
    O1, L1 = oracle.attention(q, k, v, q_valid=50, kv_valid=45)
    g = W.bf16_bits_to_f32(W.finite_garbage_bits(rng(13), (1, 2, 19, 64))).astype(np.float64)
    k2, v2, q2 = k.copy(), v.copy(), q.copy()
    k2[:, :, 45:] = g; v2[:, :, 45:] = g[..., ::-1]; q2[:, :, 50:] = g[:, :, :14]
    O2, L2 = oracle.attention(q2, k2, v2, q_valid=50, kv_valid=45)
    assert np.array_equal(O1, O2) and np.array_equal(L1, L2)
    assert (O1[:, :, 50:] == 0).all() and np.isneginf(L1[:, :, 50:]).all()


def test_no_valid_keys_gives_zero_and_minus_inf():
    q, k, v = rand_qkv(14, 1, 1, 8, 8, 64)
    O, L = oracle.attention(q, k, v, q_valid=8, kv_valid=0)
    assert (O == 0).all() and np.isneginf(L).all()


@pytest.mark.parametrize("Sq,Skv,d,qv,kv", [(5, 9, 4, 5, 9), (16, 16, 8, 13, 11), (7, 3, 6, 7, 1), (12, 16, 16, 12, 16)])
def test_bruteforce_agrees(Sq, Skv, d, qv, kv):
    q, k, v = rand_qkv(15 + d, 1, 2, Sq, Skv, d, scale=1.5)
    O1, L1 = oracle.attention(q, k, v, qv, kv)
    O2, L2 = oracle.attention_bruteforce(q, k, v, qv, kv)
    assert np.allclose(O1, O2, rtol=0, atol=1e-12)
    fin = np.isfinite(L2)
    assert np.array_equal(np.isfinite(L1), fin)
    assert np.allclose(L1[fin], L2[fin], rtol=0, atol=1e-12)


def test_row_subset_matches_full_evaluation():
    q, k, v = rand_qkv(16, 1, 2, 100, 120, 64)
    rows = np.array([0, 3, 50, 98, 99])
    Of, Lf = oracle.attention(q, k, v, 97, 111)
    Or, Lr = oracle.attention(q, k, v, 97, 111, rows=rows)
    assert np.allclose(Or, Of[:, :, rows], rtol=0, atol=1e-14)
    assert np.array_equal(np.isneginf(Lr), np.isneginf(Lf[:, :, rows]))
    f = np.isfinite(Lr)
    assert np.allclose(Lr[f], Lf[:, :, rows][f], rtol=0, atol=1e-13)


# ------------------------------------------------------------------ segmented
def test_segment_rows_worked_example():
    # 3 segments of 4 rows, 3 real each: rows 3, 7, 11 are the tail pads
    assert oracle.segment_valid_rows(12, 4, 3).tolist() == [0, 1, 2, 4, 5, 6, 8, 9, 10]
    assert oracle.segment_valid_rows(12, 12, 12).tolist() == list(range(12))


def test_segmented_with_one_segment_is_plain_attention():
    r = rng(30)
    q, k, v = (r.standard_normal((1, 2, 40, 16)) for _ in range(3))
    O1, L1 = oracle.attention_segmented(q, k, v, 40, 37, 40, 33)
    O2, L2 = oracle.attention(q, k, v, 37, 33)
    assert np.array_equal(O1, O2) and np.array_equal(L1, L2)


def test_segmented_equals_merge_of_per_segment_attention():
    # one softmax over all real keys = lse_merge of each segment's own result
    r = rng(31)
    q = r.standard_normal((1, 2, 30, 16))
    k, v = r.standard_normal((1, 2, 48, 16)), r.standard_normal((1, 2, 48, 16))
    O, L = oracle.attention_segmented(q, k, v, 30, 30, 16, 13)
    parts = [oracle.attention(q, k[:, :, 16 * i:16 * (i + 1)], v[:, :, 16 * i:16 * (i + 1)], 30, 13)
             for i in range(3)]
    Om, Lm = oracle.lse_merge([p[0] for p in parts], [p[1] for p in parts])
    assert np.allclose(O, Om, rtol=0, atol=1e-12) and np.allclose(L, Lm, rtol=0, atol=1e-12)


def test_segmented_pads_and_segment_order_do_not_matter():
    r = rng(32)
    q = r.standard_normal((1, 1, 20, 8))
    k, v = r.standard_normal((1, 1, 30, 8)), r.standard_normal((1, 1, 30, 8))
    O, L = oracle.attention_segmented(q, k, v, 10, 7, 10, 6)
    pad = np.ones(30, bool)
    pad[oracle.segment_valid_rows(30, 10, 6)] = False
    k2, v2 = k.copy(), v.copy()
    k2[:, :, pad] = 1e30
    v2[:, :, pad] = -1e30
    O2, L2 = oracle.attention_segmented(q, k2, v2, 10, 7, 10, 6)
    assert np.array_equal(O, O2) and np.array_equal(L, L2)
    perm = np.r_[20:30, 0:10, 10:20]
    O3, L3 = oracle.attention_segmented(q, k[:, :, perm], v[:, :, perm], 10, 7, 10, 6)
    assert np.allclose(O, O3, rtol=0, atol=1e-12) and np.allclose(L, L3, rtol=0, atol=1e-12)
    qpad = ~np.isin(np.arange(20), oracle.segment_valid_rows(20, 10, 7))
    assert (O[:, :, qpad] == 0).all() and np.isneginf(L[:, :, qpad]).all()


# ------------------------------------------------------------------ fixed-m bound
def test_fixed_m_bound_bounds_every_score():
    r = rng(40)
    q = r.standard_normal((1, 3, 50, 32)) * 2.0
    k = r.standard_normal((1, 3, 70, 32)) + 1.5   # keys with a common mean
    rows = np.arange(61)
    m = oracle.fixed_m_bound(q, k, rows)
    s = np.einsum("bhqd,bhkd->bhqk", q, k[:, :, rows]) / math.sqrt(32)
    assert (m >= s.max(axis=-1) - 1e-12).all()


def test_fixed_m_bound_is_tight_for_identical_keys_and_shifts_with_the_mean():
    r = rng(41)
    q = r.standard_normal((1, 1, 8, 16))
    c = r.standard_normal(16)
    k = np.broadcast_to(c, (1, 1, 10, 16)).copy()
    m = oracle.fixed_m_bound(q, k, np.arange(10), scale=1.0)
    assert np.allclose(m, (q @ c)[..., :], rtol=0, atol=1e-12)     # R = 0: the bound is the score
    k2 = r.standard_normal((1, 1, 10, 16))
    mu = 3.0 * r.standard_normal(16)
    m1 = oracle.fixed_m_bound(q, k2, np.arange(10), scale=1.0)
    m2 = oracle.fixed_m_bound(q, k2 + mu, np.arange(10), scale=1.0)
    assert np.allclose(m2 - m1, q @ mu, rtol=0, atol=1e-12)          # a common key shift moves it by q.mu


def test_fixed_m_bound_ignores_pad_rows():
    r = rng(42)
    q = r.standard_normal((1, 2, 5, 8))
    k = r.standard_normal((1, 2, 20, 8))
    rows = oracle.segment_valid_rows(20, 10, 7)
    m = oracle.fixed_m_bound(q, k, rows)
    k2 = k.copy()
    k2[:, :, [7, 8, 9, 17, 18, 19]] = 1e6
    assert np.array_equal(oracle.fixed_m_bound(q, k2, rows), m)


# ------------------------------------------------------------------ merge
def _shards(q, k, v, cuts, q_valid, total_valid):
    parts = []
    for a, b in zip(cuts[:-1], cuts[1:]):
        kv_valid = max(0, min(total_valid - a, b - a))
        parts.append(oracle.attention(q, k[:, :, a:b], v[:, :, a:b], q_valid, kv_valid))
    return parts


@pytest.mark.parametrize("cuts", [[0, 64, 128], [0, 10, 10, 77, 128], [0, 128], [0, 100, 120, 128]])
def test_merge_of_key_shards_equals_single_pass(cuts):
    q, k, v = rand_qkv(17, 1, 2, 40, 128, 64, scale=2.0)
    O, L = oracle.attention(q, k, v, 37, 110)
    parts = _shards(q, k, v, cuts, 37, 110)
    Om, Lm = oracle.lse_merge([p[0] for p in parts], [p[1] for p in parts], q_valid=37)
    assert np.allclose(Om, O, rtol=0, atol=1e-12)
    assert np.array_equal(np.isneginf(Lm), np.isneginf(L))
    f = np.isfinite(L)
    assert np.allclose(Lm[f], L[f], rtol=1e-13, atol=0)


def test_merge_lse_is_logaddexp():
    r = rng(18)
    L1, L2 = r.standard_normal((3, 7)) * 5, r.standard_normal((3, 7)) * 5
    O1, O2 = r.standard_normal((3, 7, 4)), r.standard_normal((3, 7, 4))
    O, L = oracle.lse_merge([O1, O2], [L1, L2])
    assert np.allclose(L, np.logaddexp(L1, L2), atol=1e-13)
    w1 = scipy.special.expit(L1 - L2)
    assert np.allclose(O, w1[..., None] * O1 + (1 - w1)[..., None] * O2, atol=1e-13)


def test_merge_all_empty_and_identity():
    O1 = rng(19).standard_normal((2, 5, 4))
    L1 = rng(20).standard_normal((2, 5))
    O, L = oracle.lse_merge([O1], [L1])
    assert np.allclose(O, O1, atol=1e-15) and np.allclose(L, L1, atol=1e-15)
    ninf = np.full((2, 5), -np.inf)
    O, L = oracle.lse_merge([O1, O1], [ninf, ninf])
    assert (O == 0).all() and np.isneginf(L).all()


# ------------------------------------------------------------------ whole path
def test_dit_path_tiny_rows_and_properties():
    w = W.WORKLOADS["tiny"]
    q, k, v = W.make_qkv(w)
    pos = W.positions(w)
    O, L = oracle.dit_path(q, k, v, pos, pos, w.axes, w.theta, w.s_valid, w.s_valid)
    rows = np.array([0, 17, 299, 300, 319])
    Or, Lr = oracle.dit_path(q, k, v, pos, pos, w.axes, w.theta, w.s_valid, w.s_valid, rows=rows)
    assert np.allclose(Or, O[:, :, rows], atol=1e-14)
    assert np.array_equal(np.isneginf(Lr), np.isneginf(L[:, :, rows]))
    assert (O[:, :, 300:] == 0).all() and np.isneginf(L[:, :, 300:]).all()
    # LSE of N(0,1)-ish scores over 300 keys sits near ln(300) + 1/2
    assert abs(np.mean(L[:, :, :300]) - (math.log(300) + 0.5)) < 0.3


def _distinct_positions(seed, S_q, S_kv, n_axes):
    r = rng(seed)
    return (r.integers(0, 50, (S_q, n_axes)).astype(np.int64), r.integers(0, 50, (S_kv, n_axes)).astype(np.int64))


def _bits(seed, shape):
    return W.bf16_bits(rng(seed).standard_normal(shape).astype(np.float32))


def test_dit_path_common_position_shift_changes_nothing():
    """Query and key positions differ (pos_q != pos_k); shifting BOTH sets by
    the same per-axis offset leaves every score, so O and LSE, unchanged:
    RoPE scores depend on position differences only (the relative-position
    reason the pages give for the rotation)."""
    axes, d = (8, 12, 12), 32
    q, k, v = _bits(60, (1, 2, 9, d)), _bits(61, (1, 2, 13, d)), _bits(62, (1, 2, 13, d))
    pq, pk = _distinct_positions(63, 9, 13, 3)
    O1, L1 = oracle.dit_path(q, k, v, pq, pk, axes, 100.0, 9, 11)
    delta = np.array([[17, -5, 300]])
    O2, L2 = oracle.dit_path(q, k, v, pq + delta, pk + delta, axes, 100.0, 9, 11)
    assert np.allclose(O1, O2, rtol=0, atol=1e-12) and np.allclose(L1, L2, rtol=0, atol=1e-12)
    # shifting only the keys does change the result (the pin is not vacuous)
    O3, _ = oracle.dit_path(q, k, v, pq, pk + delta, axes, 100.0, 9, 11)
    assert not np.allclose(O1, O3, atol=1e-6)


def test_dit_path_zero_key_positions_rotate_the_queries_only():
    """Key positions all 0 (the identity rotation) with pos_q != 0: the path
    equals attention of the rotated queries over the unrotated keys."""
    axes, d = (64,), 64
    q, k, v = _bits(64, (1, 1, 7, d)), _bits(65, (1, 1, 10, d)), _bits(66, (1, 1, 10, d))
    pq, _ = _distinct_positions(67, 7, 10, 1)
    pk0 = np.zeros((10, 1), dtype=np.int64)
    O, L = oracle.dit_path(q, k, v, pq, pk0, axes, 10000.0, 7, 10)
    c, s = oracle.rope_tables(pq, axes, 10000.0)
    O2, L2 = oracle.attention(oracle.rope_split_halves(oracle.bf16_to_f64(q), c, s), oracle.bf16_to_f64(k),
                              oracle.bf16_to_f64(v), 7, 10)
    assert np.allclose(O, O2, rtol=0, atol=1e-13) and np.allclose(L, L2, rtol=0, atol=1e-13)


def test_dit_path_scores_match_complex_relative_angles():
    """Independent route to the whole path with distinct positions: with
    z = x_i + i x_{i+d/2} per channel pair, the split-halves rotation
    multiplies z by e^{i w p}, so the score is
        scale * Re(sum_i z_q,i conj(z_k,i) e^{i w_i (p_q - p_k)}),
    evaluated here in numpy complex arithmetic; LSE from scipy's logsumexp
    and O from the softmax weights. Swapping the query and key tables flips
    the relative angle and fails this pin."""
    axes, d, theta = (16, 8, 8), 32, 500.0
    Sq, Skv, kv_valid = 6, 11, 9
    q, k, v = _bits(68, (1, 1, Sq, d)), _bits(69, (1, 1, Skv, d)), _bits(70, (1, 1, Skv, d))
    pq, pk = _distinct_positions(71, Sq, Skv, 3)
    O, L = oracle.dit_path(q, k, v, pq, pk, axes, theta, Sq, kv_valid)
    qf, kf, vf = (oracle.bf16_to_f64(x)[0, 0] for x in (q, k, v))
    h = d // 2
    zq = qf[:, :h] + 1j * qf[:, h:]
    zk = kf[:kv_valid, :h] + 1j * kf[:kv_valid, h:]
    # per-pair frequencies written out: axis a with c_a channels, pair j turns at theta^(-2j/c_a)
    w = np.concatenate([theta ** (-2.0 * np.arange(c // 2) / c) for c in axes])
    ax = np.concatenate([np.full(c // 2, a) for a, c in enumerate(axes)])
    dp = pq[:, None, ax] - pk[None, :kv_valid, ax]                       # [Sq, kv, h]
    s = np.real((zq[:, None, :] * np.conj(zk)[None, :, :] * np.exp(1j * w * dp)).sum(-1)) / math.sqrt(d)
    L_ref = scipy.special.logsumexp(s, axis=1)
    O_ref = np.exp(s - L_ref[:, None]) @ vf[:kv_valid]
    assert np.allclose(L[0, 0], L_ref, rtol=0, atol=1e-12)
    assert np.allclose(O[0, 0], O_ref, rtol=0, atol=1e-12)
    # negative control: the tables swapped between Q and K (relative angle negated)
    s_sw = np.real((zq[:, None, :] * np.conj(zk)[None, :, :] * np.exp(-1j * w * dp)).sum(-1)) / math.sqrt(d)
    assert not np.allclose(L_ref, scipy.special.logsumexp(s_sw, axis=1), atol=1e-6)


# ------------------------------------------------------------------ negative controls
def test_negative_control_missing_mask_breaks_pad_invariance():
    q, k, v = rand_qkv(21, 1, 1, 16, 32, 64)
    g = W.bf16_bits_to_f32(W.finite_garbage_bits(rng(22), (1, 1, 8, 64))).astype(np.float64)
    k2 = k.copy(); k2[:, :, 24:] = np.clip(g, -1e3, 1e3)
    no_mask = lambda q_, k_, v_: oracle.attention(q_, k_, v_, 16, 32)  # plants: pads not dropped
    assert not np.allclose(no_mask(q, k, v)[0], no_mask(q, k2, v)[0])


def test_negative_control_log2_lse_fails_closed_form():
    _, k, v = rand_qkv(23, 1, 1, 3, 50, 64)
    q = np.zeros((1, 1, 3, 64))
    O, L = oracle.attention(q, k, v, 3, 50)
    planted = L / math.log(2.0)        # plants: LSE reported in base 2
    assert np.allclose(L, math.log(50))
    assert not np.allclose(planted, math.log(50))


def test_negative_control_missing_permutation_breaks_equivalence():
    x = rng(24).standard_normal((4, 64))
    c, s = oracle.rope_tables(rng(25).integers(1, 90, (4, 1)), (64,), 10000.0)
    assert not np.allclose(oracle.rope_split_halves(x, c, s), oracle.rope_interleaved(x, c, s))


def test_negative_control_transposed_operand_fails_bruteforce():
    q, k, v = rand_qkv(26, 1, 1, 6, 6, 6)
    O2, _ = oracle.attention_bruteforce(q, k, v, 6, 6)
    planted, _ = oracle.attention(k, q, v, 6, 6)   # plants: Q and K swapped (S^T)
    assert not np.allclose(planted, O2, atol=1e-6)


def test_negative_control_sign_flip_fails_complex_pin():
    y = rng(27).standard_normal((5, 16))
    c, s = oracle.rope_tables(rng(28).integers(1, 40, (5, 1)), (16,), 10000.0)
    planted = oracle.rope_interleaved(y, c, -s)      # plants: rotation sign flipped
    z = (y[:, 0::2] + 1j * y[:, 1::2]) * (c + 1j * s)
    assert not np.allclose(planted[:, 0::2], z.real)
