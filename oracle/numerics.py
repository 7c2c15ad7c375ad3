"""Scalar building blocks of the oracle: rounding to the storage formats and the
per-vector primitives of the backbone, written from their definitions.

TEST INFRASTRUCTURE ONLY: nothing in the product path may import this package.

Sources (pages of the reference text):
* FlashRT "Higgs Audio v3 TTS-4B" page, summary: Qwen3-4B backbone with RoPE
  theta 1e6, SwiGLU, GQA 32q/8kv, head_dim 128.
* same page, section 5 ("What runs under the hood"): the per-frame chain
  RMSNorm (+ FP8 quant) -> GEMV qkv -> q/k-norm + RoPE -> attention ->
  quant -> o_proj (+ residual) -> RMSNorm -> gate/up -> SiLU*mul -> quant ->
  down (+ residual) -> final RMSNorm + quant -> fused head.
* same page, section 8: FP8 is per-tensor static for activations with scale
  amax/448, i.e. the OCP e4m3 format whose largest finite value is 448.

Readings taken where the pages are silent: RMSNorm multiplies by the gain
(x / sqrt(mean(x^2) + eps) * g); RoPE is the rotate-half form over pairs
(i, i + hd/2) with inverse frequency theta^(-2i/hd), applied after the q/k
norm; FP8 rounding is round-to-nearest-even with saturation to +-448.
"""
from __future__ import annotations

import numpy as np

E4M3_MAX = 448.0


# --------------------------------------------------------------------------- bf16
def round_bf16(x) -> np.ndarray:
    """Round to the nearest bfloat16 value, ties to even (8 significant bits).

    Written from the definition: with x = m * 2**e and 0.5 <= |m| < 1, the
    bfloat16 neighbours are multiples of 2**(e-8); ``np.rint`` rounds half to
    even.  Values here are O(1); the bfloat16 subnormal and overflow ranges
    are rejected rather than handled.
    """
    x = np.asarray(x, dtype=np.float64)
    m, e = np.frexp(x)
    y = np.ldexp(np.rint(np.ldexp(m, 8)), e - 8)
    nz = x != 0
    if np.any(np.abs(x[nz]) < 2.0 ** -126) or np.any(np.abs(x) > 3.0e38):
        raise ValueError("round_bf16: value outside the normal bfloat16 range")
    return y


def bf16_bits_to_float(bits) -> np.ndarray:
    """Exact value of bfloat16 bit patterns (the upper half of a float32)."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return b.view(np.float32).astype(np.float64)


# --------------------------------------------------------------------------- e4m3
def e4m3_decode(codes) -> np.ndarray:
    """Value of OCP e4m3fn codes: 1 sign, 4 exponent bits (bias 7), 3 mantissa bits.

    Exponent field 0 holds subnormals m * 2**-9; S.1111.111 is NaN; there is no
    infinity, so the largest finite value is 1.75 * 2**8 = 448.
    """
    c = np.asarray(codes, dtype=np.int64) & 0xFF
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = c & 0x7
    val = np.where(e == 0, m * 2.0 ** -9, (1.0 + m / 8.0) * np.exp2(e.astype(np.float64) - 7.0))
    val = np.where((e == 15) & (m == 7), np.nan, val)
    return sign * val


def e4m3_round(x) -> np.ndarray:
    """Round to the nearest e4m3fn value, ties to even, saturating to +-448.

    Normal range (|x| >= 2**-6): 4 significant bits, so with x = m * 2**e the
    neighbours are multiples of 2**(e-4).  Subnormal range: multiples of 2**-9.
    A result beyond 448 saturates to 448 (same as clamping first, since 448 is
    itself representable).
    """
    x = np.asarray(x, dtype=np.float64)
    m, e = np.frexp(x)
    normal = np.ldexp(np.rint(np.ldexp(m, 4)), e - 4)
    sub = np.rint(x * 2.0 ** 9) * 2.0 ** -9
    y = np.where(np.abs(x) >= 2.0 ** -6, normal, sub)
    return np.clip(y, -E4M3_MAX, E4M3_MAX)


def e4m3_encode(x) -> np.ndarray:
    """Code (uint8) of ``e4m3_round(x)``; NaN inputs map to the NaN code 0x7F (sign kept)."""
    x = np.asarray(x, dtype=np.float64)
    r = e4m3_round(np.nan_to_num(x, nan=0.0))
    a = np.abs(r)
    m, e = np.frexp(a)
    # normal: a = (1 + mant/8) * 2**(E-7) with E = e - 1 + 7
    E = np.where(a >= 2.0 ** -6, e - 1 + 7, 0)
    mant = np.where(a >= 2.0 ** -6, np.rint((np.ldexp(m, 1) - 1.0) * 8.0), np.rint(a * 2.0 ** 9))
    code = (E.astype(np.int64) << 3) | mant.astype(np.int64)
    code = np.where(np.signbit(r), code | 0x80, code)
    code = np.where(np.isnan(x), np.where(np.signbit(x), 0xFF, 0x7F), code)
    return code.astype(np.uint8)


def quantize_static(x, scale) -> np.ndarray:
    """e4m3 value of x / scale, taken in float32 (the precision the kernels use).

    The division and the rounding decide a code, so both are done on float32
    operands: fp32(x) / fp32(scale) correctly rounded in float32, then RNE to e4m3.
    """
    q = np.asarray(x, dtype=np.float64).astype(np.float32) / np.float32(scale)
    return e4m3_round(q.astype(np.float64))


def weight_scales(w) -> np.ndarray:
    """Per-output-row FP8 weight scales: float32(max_k |W[n,k]|) / 448 in float32; 1 for an all-zero row."""
    amax = np.max(np.abs(np.asarray(w, dtype=np.float32)), axis=-1)
    s = amax / np.float32(E4M3_MAX)
    return np.where(amax > 0, s, np.float32(1.0)).astype(np.float32)


def quantize_weight_rows(w):
    """(codes as float values, per-row scales): W ~= q * s[:, None] with q on the e4m3 grid."""
    w32 = np.asarray(w, dtype=np.float32)
    s = weight_scales(w32)
    q = e4m3_round((w32 / s[:, None]).astype(np.float64))
    return q, s


def act_scale(amax: float) -> np.float32:
    """Static activation scale amax / 448 (float32); 1 when amax is 0."""
    a = np.float32(amax)
    return np.float32(a / np.float32(E4M3_MAX)) if a > 0 else np.float32(1.0)


# --------------------------------------------------------------------------- primitives
def rmsnorm(x, g, eps: float) -> np.ndarray:
    """x / sqrt(mean(x**2) + eps) * g over the last axis."""
    x = np.asarray(x, dtype=np.float64)
    ms = np.mean(x * x, axis=-1, keepdims=True)
    return x / np.sqrt(ms + eps) * np.asarray(g, dtype=np.float64)


def rope_angles(positions, head_dim: int, theta: float) -> np.ndarray:
    """phi[p, i] = p * theta**(-2i/hd) for i < hd/2, in float64."""
    i = np.arange(head_dim // 2, dtype=np.float64)
    inv_freq = theta ** (-2.0 * i / head_dim)
    return np.asarray(positions, dtype=np.float64)[:, None] * inv_freq[None, :]


def rope(x, positions, theta: float) -> np.ndarray:
    """Rotate-half RoPE: (x_i, x_{i+h}) -> (x_i cos - x_{i+h} sin, x_{i+h} cos + x_i sin).

    ``x`` is [T, n_heads, hd]; ``positions`` is [T].
    """
    x = np.asarray(x, dtype=np.float64)
    hd = x.shape[-1]
    half = hd // 2
    phi = rope_angles(positions, hd, theta)[:, None, :]
    c, s = np.cos(phi), np.sin(phi)
    a, b = x[..., :half], x[..., half:]
    return np.concatenate([a * c - b * s, b * c + a * s], axis=-1)


def silu(x) -> np.ndarray:
    x = np.asarray(x, dtype=np.float64)
    return x / (1.0 + np.exp(-x))


def softmax(s, axis=-1) -> np.ndarray:
    s = np.asarray(s, dtype=np.float64)
    m = np.max(s, axis=axis, keepdims=True)
    e = np.exp(s - m)
    return e / np.sum(e, axis=axis, keepdims=True)


def attention_one(q, K, V) -> np.ndarray:
    """softmax(q . K^T / sqrt(hd)) . V for one query vector over L keys (float64)."""
    q = np.asarray(q, dtype=np.float64)
    scores = (np.asarray(K, dtype=np.float64) @ q) / np.sqrt(q.shape[-1])
    return softmax(scores) @ np.asarray(V, dtype=np.float64)


def attention_split_combine(q, K, V, n_splits: int) -> np.ndarray:
    """The same attention as ``attention_one`` computed as split-K partials
    (running max m, sum l, unnormalised o per key chunk) merged with the
    log-sum-exp rule.  Used only to pin that the split form is the plain softmax."""
    q = np.asarray(q, dtype=np.float64)
    L = K.shape[0]
    bounds = np.linspace(0, L, n_splits + 1).astype(int)
    parts = []
    for a, b in zip(bounds[:-1], bounds[1:]):
        if b <= a:
            continue
        s = (np.asarray(K[a:b], np.float64) @ q) / np.sqrt(q.shape[-1])
        m = s.max()
        p = np.exp(s - m)
        parts.append((m, p.sum(), p @ np.asarray(V[a:b], np.float64)))
    M = max(p[0] for p in parts)
    num = sum(np.exp(m - M) * o for m, _, o in parts)
    den = sum(np.exp(m - M) * l for m, l, _ in parts)
    return num / den
