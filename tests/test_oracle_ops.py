"""Pins for the CPU oracle's per-operation functions.

Each test ties an oracle function to something other than itself: a closed
form, an invariant, a library routine (numpy, torch, scipy) computing the same
definition, or a brute-force special case.  Each names the plausible mistake it
would catch.
"""
import math

import numpy as np
import pytest
import scipy.special
import torch
import torch.nn.functional as F

import oracle

RNG = np.random.default_rng(1234)


# ----------------------------------------------------------------------------- bf16

def test_bf16_decode_exact_values():
    assert oracle.bf16_to_f64(0x3F80) == 1.0
    assert oracle.bf16_to_f64(0xC000) == -2.0
    assert oracle.bf16_to_f64(0x0001) == 2.0 ** -133
    assert math.isinf(oracle.bf16_to_f64(0x7F80))
    assert oracle.bf16_to_f64(0x7F7F) == (2 - 2 ** -7) * 2.0 ** 127


@pytest.mark.parametrize("value,bits", [
    (1.0, 0x3F80),
    (1 + 2 ** -8, 0x3F80),             # exact tie -> even (down)
    (1 + 3 * 2 ** -8, 0x3F82),         # exact tie -> even (up)
    (1 + 2 ** -8 + 2 ** -40, 0x3F81),  # just above the tie: one rounding, not two
    (-(1 + 2 ** -8 + 2 ** -40), 0xBF81),
    (2.0 ** -133, 0x0001),             # smallest subnormal
    (0.5 * 2.0 ** -133, 0x0000),       # tie between 0 and the smallest -> even
    (0.75 * 2.0 ** -133, 0x0001),
    (1.5 * 2.0 ** -133, 0x0002),       # tie -> even
    ((2 - 2 ** -7) * 2.0 ** 127, 0x7F7F),
    ((2 - 2 ** -8) * 2.0 ** 127, 0x7F80),  # halfway to 2^128 -> even -> overflow
    (0.0, 0x0000),
    (-0.0, 0x8000),
])
def test_bf16_round_nearest_even(value, bits):
    assert int(oracle.f64_to_bf16(value)) == bits


def test_bf16_round_matches_torch_on_fp32_values():
    # For values that are exactly fp32, torch's fp32 -> bf16 cast is one
    # round-to-nearest-even step: the oracle must agree bit for bit.
    x32 = (RNG.standard_normal(4000) * np.exp(RNG.uniform(-20, 20, 4000))).astype(np.float32)
    want = torch.from_numpy(x32).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = oracle.f64_to_bf16(x32.astype(np.float64))
    np.testing.assert_array_equal(got, want)


# ----------------------------------------------------------------------------- RMSNorm

def test_rmsnorm_unit_rms_before_gain():
    # Closed form: with m = mean(x^2), y/g has mean square m / (m + eps).
    for n in (64, 256, 2560):
        x = RNG.standard_normal(n) * RNG.uniform(0.01, 10)
        g = oracle.f64_to_bf16(1 + 0.1 * RNG.standard_normal(n))
        eps = 1e-6
        y = oracle.rmsnorm(x, g, eps)
        m = np.mean(x * x)
        ms = np.mean((y / oracle.bf16_to_f64(g)) ** 2)
        assert abs(ms - m / (m + eps)) < 1e-12


def test_rmsnorm_matches_torch_rms_norm():
    x = RNG.standard_normal((5, 128))
    g = oracle.f64_to_bf16(1 + 0.1 * RNG.standard_normal(128))
    want = F.rms_norm(torch.from_numpy(x), (128,), torch.from_numpy(oracle.bf16_to_f64(g)),
                      eps=1e-6).numpy()
    np.testing.assert_allclose(oracle.rmsnorm(x, g, 1e-6), want, rtol=1e-13, atol=1e-14)


def test_rmsnorm_scale_invariance():
    x = RNG.standard_normal(256)
    g = oracle.f64_to_bf16(np.ones(256))
    y1 = oracle.rmsnorm(x, g, 0.0)
    y2 = oracle.rmsnorm(37.5 * x, g, 0.0)
    np.testing.assert_allclose(y1, y2, rtol=1e-13)


# ----------------------------------------------------------------------------- linear

def test_linear_matches_numpy_matmul():
    w = oracle.f64_to_bf16(0.02 * RNG.standard_normal((96, 320)))
    x = RNG.standard_normal((3, 320))
    want = x @ oracle.bf16_to_f64(w).T          # [B, K] x [K, N]: W is [out, in]
    np.testing.assert_allclose(oracle.linear(x, w), want, rtol=1e-12, atol=1e-14)


def test_linear_orientation():
    # One hot input picks column k of W ([out, in] layout): a transposed
    # operand would pick a row instead.
    w = oracle.f64_to_bf16(RNG.standard_normal((8, 5)))
    x = np.zeros((1, 5))
    x[0, 3] = 1.0
    np.testing.assert_array_equal(oracle.linear(x, w)[0], oracle.bf16_to_f64(w)[:, 3])


# ----------------------------------------------------------------------------- RoPE

def test_rope_position_zero_is_identity():
    v = RNG.standard_normal((4, 128))
    np.testing.assert_array_equal(oracle.rope_neox(v, 0), v)


def test_rope_first_pair_angle_is_position():
    # Pair i = 0 has inverse frequency theta^0 = 1, so its angle is pos radians,
    # and NeoX pairs element 0 with element D/2 (not element 1).
    D = 128
    for pos in (1, 2, 7, 8191):
        e0 = np.zeros(D); e0[0] = 1.0
        r = oracle.rope_neox(e0, pos)
        want = np.zeros(D); want[0] = math.cos(pos); want[D // 2] = math.sin(pos)
        np.testing.assert_allclose(r, want, atol=1e-15)
        eh = np.zeros(D); eh[D // 2] = 1.0    # rotate_half(x) = cat(-x2, x1)
        r = oracle.rope_neox(eh, pos)
        want = np.zeros(D); want[0] = -math.sin(pos); want[D // 2] = math.cos(pos)
        np.testing.assert_allclose(r, want, atol=1e-15)


def test_rope_quarter_pair_frequency():
    # Pair i = D/4 has inverse frequency theta^(-1/2) = 1e-3 for theta = 1e6:
    # at pos 1000 its angle is exactly 1 rad.
    D = 128
    e = np.zeros(D); e[32] = 1.0
    r = oracle.rope_neox(e, 1000, 1e6)
    assert abs(r[32] - math.cos(1.0)) < 1e-12 and abs(r[96] - math.sin(1.0)) < 1e-12


def test_rope_norm_preservation_and_composition():
    D = 64
    v = RNG.standard_normal(D)
    r = oracle.rope_neox(v, 123)
    for i in range(D // 2):
        assert abs(math.hypot(r[i], r[i + D // 2]) - math.hypot(v[i], v[i + D // 2])) < 1e-12
    np.testing.assert_allclose(oracle.rope_neox(oracle.rope_neox(v, 40), 83),
                               oracle.rope_neox(v, 123), atol=1e-12)


def test_rope_relative_position_identity():
    D = 128
    q, k = RNG.standard_normal(D), RNG.standard_normal(D)
    for m, n, t in ((5, 2, 11), (100, 900, 3000), (0, 7, 8000)):
        a = oracle.rope_neox(q, m) @ oracle.rope_neox(k, n)
        b = oracle.rope_neox(q, m + t) @ oracle.rope_neox(k, n + t)
        assert abs(a - b) < 1e-9


# ----------------------------------------------------------------------------- attention

def _pool_from_contiguous(K, V, perm):
    """K, V: [Hkv, ctx, D] bf16 bits -> (pool [1][P][2][Hkv][16][D], table row)."""
    Hkv, ctx, D = K.shape
    npg = -(-ctx // 16)
    P = len(perm)
    pool = np.full((1, P, 2, Hkv, 16, D), 0x7FC0, dtype=np.uint16)   # NaN everywhere else
    row = np.asarray(perm[:npg], dtype=np.int32)
    for t in range(ctx):
        pool[0, row[t // 16], 0, :, t % 16] = K[:, t]
        pool[0, row[t // 16], 1, :, t % 16] = V[:, t]
    return pool, row


@pytest.mark.parametrize("Hq,Hkv,D,ctx", [(4, 2, 64, 1), (4, 2, 64, 37), (8, 2, 128, 64),
                                          (32, 8, 128, 100), (4, 4, 64, 50)])
def test_attention_matches_torch_sdpa(Hq, Hkv, D, ctx):
    K = oracle.f64_to_bf16(RNG.standard_normal((Hkv, ctx, D)))
    V = oracle.f64_to_bf16(RNG.standard_normal((Hkv, ctx, D)))
    q = RNG.standard_normal((Hq, D))
    npg = -(-ctx // 16)
    perm = RNG.permutation(npg + 3)
    pool, row = _pool_from_contiguous(K, V, perm)
    got = oracle.attention(q, pool, 0, row, ctx, Hkv)
    # library: scaled dot-product attention, query heads grouped onto KV heads
    # in contiguous groups (head h -> KV head h // (Hq/Hkv)), scale 1/sqrt(D)
    qt = torch.from_numpy(q)[None, :, None, :]
    kt = torch.from_numpy(oracle.bf16_to_f64(K))[None]
    vt = torch.from_numpy(oracle.bf16_to_f64(V))[None]
    want = F.scaled_dot_product_attention(qt, kt, vt, enable_gqa=True)[0, :, 0].numpy()
    np.testing.assert_allclose(got, want, rtol=1e-10, atol=1e-12)


def test_attention_single_token_returns_value():
    K = oracle.f64_to_bf16(RNG.standard_normal((2, 1, 64)))
    V = oracle.f64_to_bf16(RNG.standard_normal((2, 1, 64)))
    pool, row = _pool_from_contiguous(K, V, [3, 0, 1, 2])
    o = oracle.attention(RNG.standard_normal((4, 64)), pool, 0, row, 1, 2)
    vv = oracle.bf16_to_f64(V)
    np.testing.assert_array_equal(o, np.stack([vv[0, 0], vv[0, 0], vv[1, 0], vv[1, 0]]))


def test_attention_identical_keys_average_values():
    ctx = 45
    k1 = oracle.f64_to_bf16(RNG.standard_normal((2, 1, 64)))
    K = np.repeat(k1, ctx, axis=1)
    V = oracle.f64_to_bf16(RNG.standard_normal((2, ctx, 64)))
    pool, row = _pool_from_contiguous(K, V, RNG.permutation(5))
    o = oracle.attention(RNG.standard_normal((4, 64)), pool, 0, row, ctx, 2)
    mean_v = oracle.bf16_to_f64(V).mean(axis=1)
    np.testing.assert_allclose(o, np.repeat(mean_v, 2, axis=0), rtol=1e-12, atol=1e-14)


def test_attention_paged_equals_contiguous_bitwise():
    ctx = 83
    K = oracle.f64_to_bf16(RNG.standard_normal((2, ctx, 64)))
    V = oracle.f64_to_bf16(RNG.standard_normal((2, ctx, 64)))
    q = RNG.standard_normal((4, 64))
    pool_a, row_a = _pool_from_contiguous(K, V, np.arange(8))
    pool_b, row_b = _pool_from_contiguous(K, V, RNG.permutation(8))
    np.testing.assert_array_equal(oracle.attention(q, pool_a, 0, row_a, ctx, 2),
                                  oracle.attention(q, pool_b, 0, row_b, ctx, 2))


def test_attention_reads_only_its_context():
    # Slots past ctx and pages past the last one hold NaN: any read of them
    # would poison the output.
    ctx = 20
    K = oracle.f64_to_bf16(RNG.standard_normal((2, 32, 64)))
    V = oracle.f64_to_bf16(RNG.standard_normal((2, 32, 64)))
    K[:, ctx:] = 0x7FC0
    V[:, ctx:] = 0x7FC0
    pool, row = _pool_from_contiguous(K, V, [2, 0, 1])
    o = oracle.attention(RNG.standard_normal((4, 64)), pool, 0, row, ctx, 2)
    assert np.isfinite(o).all()


def test_split_lse_combine_identity():
    # The split-KV combine used by the GPU path: partials (o_s, m_s, l_s) over
    # disjoint token ranges merge to the single-pass softmax:
    #   LSE_s = m_s + ln l_s,  o = sum_s exp(LSE_s - LSE) o_s,  LSE = ln sum exp LSE_s.
    # Checked against the oracle's single pass over the whole context.
    ctx, D = 70, 64
    K = oracle.f64_to_bf16(RNG.standard_normal((1, ctx, D)))
    V = oracle.f64_to_bf16(RNG.standard_normal((1, ctx, D)))
    q = RNG.standard_normal((1, D))
    pool, row = _pool_from_contiguous(K, V, RNG.permutation(6))
    full = oracle.attention(q, pool, 0, row, ctx, 1)[0]
    s = (oracle.bf16_to_f64(K[0]) @ q[0]) / math.sqrt(D)
    vv = oracle.bf16_to_f64(V[0])
    for cuts in ([0, 70], [0, 16, 70], [0, 5, 33, 34, 70], list(range(0, 71, 7)) + [70]):
        parts = []
        for a, b in zip(cuts[:-1], cuts[1:]):
            if a == b:
                continue
            m = s[a:b].max()
            p = np.exp(s[a:b] - m)
            parts.append((p @ vv[a:b] / p.sum(), m + math.log(p.sum())))
        lse = scipy.special.logsumexp([p[1] for p in parts])
        o = sum(math.exp(p[1] - lse) * p[0] for p in parts)
        np.testing.assert_allclose(o, full, rtol=1e-12, atol=1e-13)


# ----------------------------------------------------------------------------- SwiGLU, argmax

def test_silu_closed_forms():
    z = np.linspace(-30, 30, 241)
    np.testing.assert_allclose(oracle.silu(z), z * scipy.special.expit(z), rtol=1e-14,
                               atol=1e-300)
    assert oracle.silu(0.0) == 0.0
    assert abs(oracle.silu(40.0) - 40.0) < 1e-12
    assert abs(oracle.silu(-40.0)) < 1e-15


def test_argmax_ties_lowest_index_and_nan():
    v = RNG.standard_normal(1000)
    assert oracle.argmax(v) == int(np.argmax(v))
    v[[17, 400, 999]] = v.max() + 1.0
    assert oracle.argmax(v) == 17
    v[3] = np.nan
    assert oracle.argmax(v) == -1
