"""Seeded synthetic inputs for the codebook-TTS decode path.

This module is the only code that the CPU oracle and the GPU path share, and it
holds none of the method's arithmetic: it draws random numbers, shapes them into
named tensors and token lists, and rounds the draws to the storage dtype.  The
model shape is the one the FlashRT "Higgs Audio v3 TTS-4B" page gives for its
backbone (summary paragraph: 36 layers, hidden 2560, GQA 32 q / 8 kv heads,
head_dim 128, SwiGLU, RoPE theta 1e6, an 8-codebook x 1026 head); FFN width,
norm eps and text vocabulary follow the Qwen3-4B shape.  No trained weights
exist here, so every tensor is a seeded draw:

* matrices and embeddings: 0.02 * N(0, 1);
* RMSNorm gains: 1 + 0.1 * N(0, 1) (a gain near 1 keeps activations O(1), and
  the jitter makes a dropped or misplaced gain a large, visible error).

Every tensor is split into fixed chunks of ``CHUNK`` elements; chunk ``c`` of
tensor ``i`` is drawn from ``PCG64(SeedSequence(seed, spawn_key=(i, c)))``, so
the values do not depend on how many threads fill them.
"""
from __future__ import annotations

import dataclasses
import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

CHUNK = 1 << 22


@dataclasses.dataclass(frozen=True)
class ModelShape:
    """Backbone and head dimensions."""

    n_layers: int
    hidden: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    ffn: int
    text_vocab: int
    n_codebooks: int = 8
    codebook_size: int = 1026
    bos_id: int = 1024
    eos_id: int = 1025
    rope_theta: float = 1.0e6
    rms_eps: float = 1.0e-6

    @property
    def q_dim(self) -> int:
        return self.n_q_heads * self.head_dim

    @property
    def kv_dim(self) -> int:
        return self.n_kv_heads * self.head_dim

    def with_layers(self, n: int) -> "ModelShape":
        return dataclasses.replace(self, n_layers=n)


# The small case: 2 layers, hidden 256, GQA 4q/2kv, head_dim 64, FFN 768, text vocab 1024.
TINY = ModelShape(n_layers=2, hidden=256, n_q_heads=4, n_kv_heads=2, head_dim=64, ffn=768, text_vocab=1024)
# The Qwen3-4B-shaped backbone with the 8 x 1026 acoustic head.
QWEN3_4B = ModelShape(n_layers=36, hidden=2560, n_q_heads=32, n_kv_heads=8, head_dim=128, ffn=9728,
                      text_vocab=151936)

# Per-layer tensor names, in the order the weight list carries them.
LAYER_TENSORS = ("g_attn", "wq", "wk", "wv", "g_q", "g_k", "wo", "g_mlp", "wg", "wu", "wd")
GAIN_TENSORS = frozenset({"g_attn", "g_q", "g_k", "g_mlp", "g_final"})


def tensor_specs(shape: ModelShape):
    """Ordered list of (name, dims) for every weight tensor of ``shape``.

    Order: text embedding, audio embedding, then 11 tensors per layer
    (``LAYER_TENSORS``), then the final norm gain and the fused head.
    """
    d, hd, F = shape.hidden, shape.head_dim, shape.ffn
    specs = [("e_text", (shape.text_vocab, d)),
             ("e_aud", (shape.n_codebooks, shape.codebook_size, d))]
    for layer in range(shape.n_layers):
        dims = {"g_attn": (d,), "wq": (shape.q_dim, d), "wk": (shape.kv_dim, d), "wv": (shape.kv_dim, d),
                "g_q": (hd,), "g_k": (hd,), "wo": (d, shape.q_dim), "g_mlp": (d,),
                "wg": (F, d), "wu": (F, d), "wd": (d, F)}
        for name in LAYER_TENSORS:
            specs.append((f"layers.{layer}.{name}", dims[name]))
    specs.append(("g_final", (d,)))
    specs.append(("w_head", (shape.n_codebooks * shape.codebook_size, d)))
    return specs


def _n_threads() -> int:
    env = os.environ.get("OMP_NUM_THREADS")
    n = int(env) if env and env.isdigit() else (os.cpu_count() or 1)
    return max(1, min(n, 16))


def standard_normal(seed: int, index: int, n: int, threads: int | None = None) -> np.ndarray:
    """float32 N(0,1) draws for tensor ``index``: chunk c from spawn_key (index, c)."""
    out = np.empty(n, dtype=np.float32)
    n_chunks = (n + CHUNK - 1) // CHUNK

    def fill(c: int) -> None:
        lo, hi = c * CHUNK, min(n, (c + 1) * CHUNK)
        gen = np.random.Generator(np.random.PCG64(np.random.SeedSequence(seed, spawn_key=(index, c))))
        gen.standard_normal(out=out[lo:hi], dtype=np.float32)

    if n_chunks <= 1:
        for c in range(n_chunks):
            fill(c)
    else:
        with ThreadPoolExecutor(threads or _n_threads()) as ex:
            list(ex.map(fill, range(n_chunks)))
    return out


def to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (round to nearest even) and return the raw uint16 bits.

    Uses torch's CPU conversion, which is independent of both the oracle's own
    bfloat16 encoder and the GPU kernels.
    """
    import torch

    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """Exact widening of bfloat16 bit patterns to float32."""
    return (bits.astype(np.uint32) << 16).view(np.float32)


def draw_tensor(seed: int, index: int, name: str, dims, dtype: str) -> np.ndarray:
    """One weight tensor. ``dtype`` 'f32' gives float32 values, 'bf16' gives uint16 bit patterns."""
    n = int(np.prod(dims))
    z = standard_normal(seed, index, n)
    base = name.rsplit(".", 1)[-1]
    if base in GAIN_TENSORS:
        z *= np.float32(0.1)
        z += np.float32(1.0)
    else:
        z *= np.float32(0.02)
    z = z.reshape(dims)
    if dtype == "f32":
        return z
    if dtype == "bf16":
        return to_bf16_bits(z)
    raise ValueError(f"unknown dtype {dtype}")


def make_weights(shape: ModelShape, seed: int, dtype: str, names=None) -> dict:
    """All weight tensors of ``shape`` as numpy arrays keyed by name (see ``tensor_specs``).

    ``names`` optionally restricts which tensors are drawn (the others are
    skipped, and the draws of the ones kept do not change).
    """
    out = {}
    for index, (name, dims) in enumerate(tensor_specs(shape)):
        if names is not None and name not in names:
            continue
        out[name] = draw_tensor(seed, index, name, dims, dtype)
    return out


def token_ids(seed: int, n: int, vocab: int) -> np.ndarray:
    """``n`` uniform text-token ids in [0, vocab) as int32."""
    gen = np.random.Generator(np.random.PCG64(seed))
    return gen.integers(0, vocab, size=n, dtype=np.int64).astype(np.int32)


def normal_vector(seed: int, shape) -> np.ndarray:
    """float32 N(0, 1) array of the given shape (hidden-state and KV pre-fill inputs)."""
    gen = np.random.Generator(np.random.PCG64(seed))
    return gen.standard_normal(size=shape, dtype=np.float32)


def code_frames(seed: int, n_frames: int, n_codebooks: int = 8, n_codes: int = 1024) -> np.ndarray:
    """Uniform acoustic codes in [0, n_codes) of shape [n_frames, n_codebooks] (teacher-forcing input)."""
    gen = np.random.Generator(np.random.PCG64(seed))
    return gen.integers(0, n_codes, size=(n_frames, n_codebooks), dtype=np.int64).astype(np.int32)


def e4m3_code_matrix(seed: int, rows: int, cols: int, max_exp_field: int, big_every: int = 0,
                     big_exp_field: int = 9) -> np.ndarray:
    """uint8 e4m3 codes [rows][cols] drawn field by field: a uniform sign bit, an exponent
    field uniform in 0..max_exp_field and a uniform 3-bit mantissa (never the NaN code).
    With big_every > 0, about one entry in big_every gets exponent field big_exp_field
    instead (a few large products among many small ones: the operands of the GEMM
    accumulation checks)."""
    gen = np.random.Generator(np.random.PCG64(seed))
    sign = gen.integers(0, 2, size=(rows, cols), dtype=np.int64)
    exp = gen.integers(0, max_exp_field + 1, size=(rows, cols), dtype=np.int64)
    man = gen.integers(0, 8, size=(rows, cols), dtype=np.int64)
    if big_every > 0:
        exp = np.where(gen.integers(0, big_every, size=(rows, cols)) == 0, big_exp_field, exp)
    return ((sign << 7) | (exp << 3) | man).astype(np.uint8)


# Seeds of the synthetic workloads.
SEEDS = {
    "tiny_weights": 1001, "tiny_prompt": 2001, "calib_prompt": 3001,
    "layer_weights": 1002, "layer_h": 2002, "layer_kv": 2003,
    "full_weights": 1003, "full_prompt": 2004,
    "prefill_13": 2005, "prefill_128": 2006, "prefill_512": 2007,
    "preamble": 2064, "suffix_base": 2101, "long_prompt": 2409,
    "gemm_a": 4001, "gemm_w": 4002, "gemm_scales": 4003,
}
