"""Pins of the oracle's numeric primitives against definitions, closed forms,
library routines and invariants (CPU only)."""
import math

import numpy as np
import pytest
import torch

from oracle import numerics as nx


# ----------------------------------------------------------------------------- bf16
def test_round_bf16_matches_torch_bitwise():
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.standard_normal(200000) * s for s in (1e-3, 1.0, 1e3)]).astype(np.float32)
    ref = torch.from_numpy(x).to(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(nx.round_bf16(x), ref)


def test_round_bf16_ties_to_even():
    # 1 + 2^-8 lies halfway between 1 and 1 + 2^-7: even mantissa (1.0) wins.
    assert nx.round_bf16(1.0 + 2.0 ** -8) == 1.0
    # 1 + 3 * 2^-8 lies halfway between 1 + 2^-7 (odd) and 1 + 2^-6 (even).
    assert nx.round_bf16(1.0 + 3 * 2.0 ** -8) == 1.0 + 2.0 ** -6
    assert nx.round_bf16(-(1.0 + 2.0 ** -8)) == -1.0


def test_bf16_bits_to_float():
    assert nx.bf16_bits_to_float(np.array([0x3F80, 0xC000, 0x0000], dtype=np.uint16)).tolist() == [1.0, -2.0, 0.0]


# ----------------------------------------------------------------------------- e4m3
def test_e4m3_decode_known_values():
    # OCP e4m3fn: 0x38 = 1.0, 0x7E = 448 (largest finite), 0x01 = 2^-9 (smallest subnormal),
    # 0x08 = 2^-6 (smallest normal), 0x7F = NaN, 0xB8 = -1.
    v = nx.e4m3_decode([0x38, 0x7E, 0x01, 0x08, 0xB8, 0x77])
    assert v.tolist() == [1.0, 448.0, 2.0 ** -9, 2.0 ** -6, -1.0, 240.0]
    assert math.isnan(nx.e4m3_decode([0x7F])[0]) and math.isnan(nx.e4m3_decode([0xFF])[0])


def test_e4m3_exhaustive_round_trip():
    codes = np.arange(256)
    vals = nx.e4m3_decode(codes)
    finite = ~np.isnan(vals)
    assert finite.sum() == 254
    assert np.array_equal(nx.e4m3_encode(vals[finite]), codes[finite].astype(np.uint8))
    assert np.array_equal(nx.e4m3_round(vals[finite]), vals[finite])


def test_e4m3_midpoints_round_to_even_code():
    vals = nx.e4m3_decode(np.arange(127))  # non-negative finite codes, ascending
    assert np.all(np.diff(vals) > 0)
    mids = (vals[:-1] + vals[1:]) / 2
    enc = nx.e4m3_encode(mids).astype(int)
    lo = np.arange(126)
    expect = np.where(lo % 2 == 0, lo, lo + 1)
    assert np.array_equal(enc, expect)
    # just off the midpoint goes to the nearer neighbour
    eps = 1e-6 * (vals[1:] - vals[:-1])
    assert np.array_equal(nx.e4m3_encode(mids - eps).astype(int), lo)
    assert np.array_equal(nx.e4m3_encode(mids + eps).astype(int), lo + 1)


def test_e4m3_saturation():
    x = np.array([448.0, 449.0, 464.0, 480.0, 1e9, np.inf, -1e9, -464.0])
    assert nx.e4m3_round(x).tolist() == [448.0, 448.0, 448.0, 448.0, 448.0, 448.0, -448.0, -448.0]


def test_e4m3_matches_torch_in_range():
    rng = np.random.default_rng(1)
    x = np.concatenate([rng.standard_normal(100000) * s for s in (0.003, 0.3, 30, 300)])
    x = np.clip(x, -448, 448).astype(np.float32)
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(nx.e4m3_encode(x.astype(np.float64)), ref)


def test_e4m3_round_trip_error_bounds():
    rng = np.random.default_rng(2)
    x = rng.uniform(-448, 448, 200000)
    x = np.concatenate([x, rng.uniform(-2.0 ** -6, 2.0 ** -6, 20000)])
    r = nx.e4m3_round(x)
    normal = np.abs(x) >= 2.0 ** -6
    assert np.all(np.abs(r[normal] - x[normal]) <= 2.0 ** -4 * np.abs(x[normal]))
    assert np.all(np.abs(r[~normal] - x[~normal]) <= 2.0 ** -10)


def test_weight_quantisation_row_max_is_448():
    rng = np.random.default_rng(3)
    w = (rng.standard_normal((64, 300)) * 0.02).astype(np.float32)
    w[5] = 0.0
    q, s = nx.quantize_weight_rows(w)
    assert s[5] == np.float32(1.0) and np.all(q[5] == 0)
    rows = [i for i in range(64) if i != 5]
    assert np.all(np.max(np.abs(q[rows]), axis=1) == 448.0)
    deq = q * s[:, None].astype(np.float64)
    # relative bound 2^-4 for normal codes, absolute 2^-10 * s for subnormal codes
    big = np.abs(q) >= 2.0 ** -6
    err = np.abs(deq - w)
    assert np.all(err[big] <= 2.0 ** -4 * np.abs(w[big]) + 1e-12)
    assert np.all(err[~big] <= 2.0 ** -10 * np.broadcast_to(s[:, None], w.shape)[~big] + 1e-12)


def test_quantize_static_float32_decision():
    # 3 * 2^-4 / 2^-4 = 3 exactly; a value whose float32 quotient lands on a midpoint rounds to even.
    s = np.float32(0.5)
    assert nx.quantize_static(np.array([8.5]), s)[0] == 16.0  # 17 -> tie between 16 and 18 -> 16
    assert nx.quantize_static(np.array([9.5]), s)[0] == 20.0  # 19 -> tie between 18 and 20 -> 20
    assert nx.quantize_static(np.array([1e6]), s)[0] == 448.0


# ----------------------------------------------------------------------------- rmsnorm
def test_rmsnorm_closed_form_and_scale_invariance():
    rng = np.random.default_rng(4)
    x = rng.standard_normal((5, 256))
    g = 1 + 0.1 * rng.standard_normal(256)
    eps = 1e-6
    y = nx.rmsnorm(x, g, eps)
    ms = np.mean(x * x, axis=-1)
    assert np.allclose(np.sqrt(np.mean((y / g) ** 2, axis=-1)), np.sqrt(ms / (ms + eps)), rtol=1e-13)
    assert np.allclose(nx.rmsnorm(3.7 * x, g, 0.0), nx.rmsnorm(x, g, 0.0), rtol=1e-13)
    # direction: y / g is parallel to x
    assert np.allclose((y / g) * np.sqrt(ms + eps)[:, None], x, rtol=1e-12)


def test_rmsnorm_matches_torch():
    rng = np.random.default_rng(5)
    x = rng.standard_normal((3, 64))
    g = 1 + 0.1 * rng.standard_normal(64)
    ref = torch.nn.functional.rms_norm(torch.from_numpy(x), (64,), torch.from_numpy(g), eps=1e-6).numpy()
    assert np.allclose(nx.rmsnorm(x, g, 1e-6), ref, rtol=1e-12, atol=1e-14)


# ----------------------------------------------------------------------------- rope
def test_rope_hd2_closed_form():
    # hd = 2: one pair with inverse frequency theta^0 = 1, so the angle is the position itself.
    x = np.array([[[0.3, -1.2]]])
    for p in (0, 1, 5, 1000):
        y = nx.rope(x, np.array([p]), 1e6)[0, 0]
        c, s = math.cos(p), math.sin(p)
        assert np.allclose(y, [0.3 * c + 1.2 * s, -1.2 * c + 0.3 * s], rtol=0, atol=1e-14)


def test_rope_hd4_pairs_and_frequencies():
    # hd = 4, theta = 1e6: pairs (0, 2) at frequency 1 and (1, 3) at 1e6^(-1/2) = 1e-3.
    x = np.array([[[1.0, 2.0, 3.0, 4.0]]])
    p = 7
    y = nx.rope(x, np.array([p]), 1e6)[0, 0]
    a0, a1 = p * 1.0, p * 1e-3
    expect = [1 * math.cos(a0) - 3 * math.sin(a0), 2 * math.cos(a1) - 4 * math.sin(a1),
              3 * math.cos(a0) + 1 * math.sin(a0), 4 * math.cos(a1) + 2 * math.sin(a1)]
    assert np.allclose(y, expect, rtol=0, atol=1e-13)


def test_rope_invariants():
    rng = np.random.default_rng(6)
    hd = 128
    q = rng.standard_normal((1, 1, hd))
    k = rng.standard_normal((1, 1, hd))
    assert np.allclose(nx.rope(q, np.array([0]), 1e6), q, rtol=0, atol=0)
    for p in (1, 17, 4095):
        assert np.isclose(np.linalg.norm(nx.rope(q, np.array([p]), 1e6)), np.linalg.norm(q), rtol=1e-13)
    dots = []
    for m, n in ((10, 3), (107, 100), (4000, 3993)):
        dots.append(float(np.sum(nx.rope(q, np.array([m]), 1e6) * nx.rope(k, np.array([n]), 1e6))))
    assert np.allclose(dots, dots[0], rtol=1e-9)


def test_rope_complex_form():
    # Independent formulation: pair (x_i, x_{i+h}) as x_i + 1j * x_{i+h}, multiplied by exp(1j * phi_i).
    rng = np.random.default_rng(7)
    hd = 64
    x = rng.standard_normal((3, 2, hd))
    pos = np.array([0, 9, 1234])
    z = x[..., : hd // 2] + 1j * x[..., hd // 2:]
    inv = 1e6 ** (-np.arange(hd // 2) * 2.0 / hd)
    zr = z * np.exp(1j * pos[:, None, None] * inv[None, None, :])
    ref = np.concatenate([zr.real, zr.imag], axis=-1)
    assert np.allclose(nx.rope(x, pos, 1e6), ref, rtol=0, atol=1e-12)


# ----------------------------------------------------------------------------- attention
def test_attention_special_cases():
    rng = np.random.default_rng(8)
    q = rng.standard_normal(64)
    K1, V1 = rng.standard_normal((1, 64)), rng.standard_normal((1, 64))
    assert np.allclose(nx.attention_one(q, K1, V1), V1[0], rtol=0, atol=1e-15)
    K = np.repeat(rng.standard_normal((1, 64)), 9, axis=0)
    V = rng.standard_normal((9, 64))
    assert np.allclose(nx.attention_one(q, K, V), V.mean(axis=0), rtol=1e-13)


def test_attention_hand_example():
    # q = (1, 0), keys e1, e2: scores (1/sqrt2, 0); weights (e^a, 1)/(e^a + 1) with a = 1/sqrt2.
    q = np.array([1.0, 0.0])
    K = np.eye(2)
    V = np.array([[2.0, 0.0], [0.0, 4.0]])
    a = 1 / math.sqrt(2)
    w0 = math.exp(a) / (math.exp(a) + 1)
    assert np.allclose(nx.attention_one(q, K, V), [2 * w0, 4 * (1 - w0)], rtol=1e-14)


@pytest.mark.parametrize("splits", [1, 2, 7, 64])
def test_split_combine_equals_one_pass(splits):
    rng = np.random.default_rng(9)
    q = rng.standard_normal(128) * 3
    K = rng.standard_normal((300, 128))
    V = rng.standard_normal((300, 128))
    assert np.allclose(nx.attention_split_combine(q, K, V, splits), nx.attention_one(q, K, V), rtol=1e-12, atol=1e-14)


def test_attention_matches_torch_sdpa():
    rng = np.random.default_rng(10)
    q = rng.standard_normal(64)
    K = rng.standard_normal((37, 64))
    V = rng.standard_normal((37, 64))
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q)[None, None, None], torch.from_numpy(K)[None, None], torch.from_numpy(V)[None, None])
    assert np.allclose(nx.attention_one(q, K, V), ref[0, 0, 0].numpy(), rtol=1e-12, atol=1e-14)


def test_silu_values():
    assert nx.silu(np.array([0.0]))[0] == 0.0
    assert np.isclose(nx.silu(np.array([1.0]))[0], 1 / (1 + math.exp(-1)), rtol=1e-15)
    x = np.linspace(-8, 8, 101)
    assert np.allclose(nx.silu(x), torch.nn.functional.silu(torch.from_numpy(x)).numpy(), rtol=1e-13)
