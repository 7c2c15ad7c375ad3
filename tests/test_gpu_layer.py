"""One decoder layer at the Qwen3-4B shape (hidden 2560, 32q/8kv heads, head_dim
128, FFN 9728) on the GPU against the CPU oracle: a single M = 1 decode step
at KV length 512, 2048 and 4096 with N(0,1) cache contents and a N(0,1) input
hidden state, in BF16 and FP8."""
import dataclasses

import numpy as np
import pytest
import torch

import synthetic as S
from gpu_common import gpu_context, rel_l2
from oracle import numerics as nx
from oracle.model import OracleModel

pytestmark = pytest.mark.gpu

# the layer never reads the text embedding, so the vocabulary is kept small; the
# per-tensor seeding makes the layer's draws independent of it
SH = dataclasses.replace(S.QWEN3_4B, n_layers=1, text_vocab=1024)


@pytest.fixture(scope="module")
def layer_weights():
    return S.make_weights(SH, S.SEEDS["layer_weights"], "bf16")


def _inputs(L):
    h = S.normal_vector(S.SEEDS["layer_h"], (SH.hidden,))
    kv = S.normal_vector(S.SEEDS["layer_kv"], (2, SH.n_kv_heads, L - 1, SH.head_dim))
    return h, S.to_bf16_bits(kv[0]), S.to_bf16_bits(kv[1])


def _oracle(w, precision, mode, L, h, kb, vb, scales=None):
    m = OracleModel(SH, w, precision, mode, act_scales=scales, max_seq=L + 1, layers_only=True)
    m.set_kv(0, nx.bf16_bits_to_float(kb).transpose(1, 0, 2), nx.bf16_bits_to_float(vb).transpose(1, 0, 2))
    m.record = np.zeros(5)
    out = m.layer_step(0, h)
    return out, m


def _gpu(w, precision, L, h, kb, vb, scales=None):
    ctx = gpu_context(SH, w, precision, max_seq=4096, max_prefill=16, act_scales=scales)
    ht = torch.from_numpy(h.astype(np.float32)).cuda()
    ctx.layer_step(0, L, torch.from_numpy(kb.view(np.int16)).cuda(), torch.from_numpy(vb.view(np.int16)).cuda(), ht)
    torch.cuda.synchronize()
    k_new, v_new = ctx.tap_kv(0, L)
    ctx.close()
    return ht.cpu().numpy().astype(np.float64), k_new[:, L - 1], v_new[:, L - 1]


@pytest.mark.parametrize("L", [512, 2048, 4096])
def test_layer_bf16(layer_weights, L):
    h, kb, vb = _inputs(L)
    ref_s, ms = _oracle(layer_weights, "bf16", "S", L, h, kb, vb)
    ref_e, _ = _oracle(layer_weights, "bf16", "E", L, h, kb, vb)
    out, k_new, v_new = _gpu(layer_weights, "bf16", L, h, kb, vb)
    d_s = rel_l2(out - h, ref_s - h)
    d_e = rel_l2(out - h, ref_e - h)
    print(f"layer bf16 L={L}: update rel vs storage-faithful {d_s:.3e}, vs exact {d_e:.3e}, output rel vs exact "
          f"{rel_l2(out, ref_e):.3e}")
    assert d_s <= 2e-3
    assert rel_l2(out, ref_e) <= 2e-2
    # the new key/value landed in slot L-1 as the oracle's bf16 values (up to rounding flips)
    k_ref = ms.k_cache[0, L - 1]
    k_gpu = nx.bf16_bits_to_float(k_new)
    assert np.mean(k_gpu == k_ref) > 0.99 and rel_l2(k_gpu, k_ref) < 1e-2


@pytest.mark.parametrize("L", [512, 2048, 4096])
def test_layer_fp8(layer_weights, L):
    h, kb, vb = _inputs(L)
    ref_e, me = _oracle(layer_weights, "fp8", "E", L, h, kb, vb)
    scales = np.array([nx.act_scale(a) for a in me.record], dtype=np.float32)
    scales[4] = 1.0
    ref_s, _ = _oracle(layer_weights, "fp8", "S", L, h, kb, vb, scales=scales)
    out, _, _ = _gpu(layer_weights, "fp8", L, h, kb, vb, scales=scales)
    d_s = rel_l2(out - h, ref_s - h)
    q = rel_l2(ref_s - h, ref_e - h)
    print(f"layer fp8 L={L}: update rel vs fp8 oracle {d_s:.3e}; fp8 oracle vs exact {q:.3e}; "
          f"gpu vs exact {rel_l2(out - h, ref_e - h):.3e}")
    assert d_s <= 6e-2
