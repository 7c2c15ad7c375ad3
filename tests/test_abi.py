"""The C-ABI library loads, exports every entry point include/hta.h declares,
and its host-only helpers agree with the oracle (no GPU needed)."""
import os
import re
import subprocess

import numpy as np
import pytest

import synthetic as S
from autoregressive_codebook_tts_amd import hta
from oracle.delay import delay_frames, undelay

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def declared_functions():
    text = open(os.path.join(ROOT, "include", "hta.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(hta_[a-z_]+)\s*\(", text)))


def test_library_exports_every_declared_symbol():
    names = declared_functions()
    assert len(names) >= 15
    out = subprocess.run(["nm", "-D", "--defined-only", hta.LIB_PATH], capture_output=True, text=True, check=True).stdout
    exported = set(re.findall(r"\bT (hta_[a-z_]+)", out))
    missing = [n for n in names if n not in exported]
    assert not missing, missing
    lib = hta.lib()
    for n in names:
        assert getattr(lib, n) is not None


def test_library_targets_gfx950_only():
    out = subprocess.run(["strings", hta.LIB_PATH], capture_output=True, text=True, check=True).stdout
    assert "gfx950" in out
    assert hta.lib().hta_version().decode().endswith("gfx950")


def test_workspace_bytes():
    cfg = hta.make_config(S.QWEN3_4B, hta.HTA_BF16, 4096, 512)
    n_bf16 = hta.workspace_bytes(cfg)
    cfg8 = hta.make_config(S.QWEN3_4B, hta.HTA_FP8_E4M3, 4096, 512)
    n_fp8 = hta.workspace_bytes(cfg8)
    # projections alone: 3.633e9 params x 2 bytes (bf16) or 1 byte (fp8)
    assert 7.27e9 < n_bf16 < 12e9 and 3.63e9 < n_fp8 < n_bf16
    assert n_bf16 - n_fp8 >= 3.633e9 * 1.0 - 1e6
    bad = hta.make_config(S.QWEN3_4B, hta.HTA_BF16, 4096, 512)
    bad.head_dim = 96
    assert hta.workspace_bytes(bad) == 0


@pytest.mark.parametrize("n", [0, 1, 3, 25])
def test_undelay_matches_oracle(n):
    rng = np.random.default_rng(n)
    frames = rng.integers(0, 1024, size=(n, 8))
    steps = delay_frames(frames)
    assert np.array_equal(hta.undelay(steps), frames)
    # a run capped before EOC: T - 7 frames come back
    capped = steps[: max(n, 8)]
    if capped[:, 0].tolist().count(1025) == 0:
        assert np.array_equal(hta.undelay(capped), undelay(capped, None))


def test_abi_weight_order_matches_generator():
    names = [n for n, _ in S.tensor_specs(S.TINY)]
    assert names == hta.abi_tensor_names(S.TINY.n_layers)


def _cfg(**kw):
    cfg = hta.make_config(S.QWEN3_4B, kw.pop("precision", hta.HTA_FP8_E4M3), kw.pop("max_seq", 4096),
                          kw.pop("max_prefill", 512), kw.pop("n_streams", 1))
    for k, v in kw.items():
        setattr(cfg, k, v)
    return cfg


@pytest.mark.parametrize("field,value", [
    ("head_dim", 96),          # head_dim must be 64 or 128
    ("n_q_heads", 24),         # GQA group 3
    ("n_kv_heads", 5),         # not a divisor of the query heads
    ("hidden", 2560 + 64),     # not a multiple of 128
    ("ffn", 9728 + 64),
    ("n_codebooks", 0),
    ("n_codebooks", 17),
    ("codebook_size", 1),
    ("bos_id", 1026),          # outside the codebook
    ("eos_id", -1),
    ("precision", 7),
    ("n_streams", 129),
    ("n_streams", -1),
    ("max_prefill", 0),
    ("max_prefill", 5000),     # above max_seq
    ("hidden", 6144),          # above the GEMV prologue budget
])
def test_workspace_bytes_rejects_unsupported_shapes(field, value):
    """hta_workspace_bytes (host only) applies hta_create's shape rules: 0 for a shape the
    kernels do not take."""
    assert hta.workspace_bytes(_cfg()) > 0
    assert hta.workspace_bytes(_cfg(**{field: value})) == 0


def test_workspace_bytes_of_batched_contexts():
    """Streams beyond max_prefill are refused; each stream adds its own KV cache (36 layers
    x 2 x 8 kv heads x max_seq x 128 x 2 bytes) and device state."""
    one = hta.workspace_bytes(_cfg(max_seq=1024, max_prefill=128))
    assert hta.workspace_bytes(_cfg(max_seq=1024, max_prefill=16, n_streams=32)) == 0
    kv = 36 * 2 * 8 * 1024 * 128 * 2
    prev = one
    for m in (2, 16, 128):
        n = hta.workspace_bytes(_cfg(max_seq=1024, max_prefill=128, n_streams=m))
        assert n >= one + (m - 1) * kv
        assert n > prev
        prev = n
