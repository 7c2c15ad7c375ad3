"""GPU sampling head (hta_set_sampling) against the sampling oracle, on the tiny backbone.

Each frame's draw is checked on the GPU's own fp32 logits of that frame: the oracle
(float64 weights and cumulative sums, the published Philox4x32-10) must pick the same id,
except where u times the total lies within 2e-6 of the total of a cumulative boundary:
there the fp32 sums of the kernel may fall on either side, and either neighbour of that
boundary is accepted (and counted).  2e-6 bounds the kernel's fp32 error relative to the
total: a lane's sequential sum of at most 17 weights, six scan additions, the exponentials
and the product u * total, each within 2^-24 relative.  With about a thousand boundaries a
random target falls in that band with probability near 0.4 %.  The delay rule's forced
codes must be exact."""
import numpy as np
import pytest

import synthetic as S
from autoregressive_codebook_tts_amd import hta
from gpu_common import SAMPLE_BAND, gpu_context, sampled_run, tiny_weights
from oracle.model import calibrate

pytestmark = pytest.mark.gpu
SH = S.TINY


@pytest.fixture(scope="module")
def w():
    return tiny_weights()


@pytest.fixture(scope="module")
def prompt():
    return S.token_ids(S.SEEDS["tiny_prompt"], 8, SH.text_vocab)


@pytest.fixture(scope="module")
def scales(w):
    return calibrate(SH, w, S.token_ids(S.SEEDS["calib_prompt"], 16, SH.text_vocab), 16)[0]


@pytest.mark.parametrize("precision,T", [("bf16", 1.0), ("bf16", 0.7), ("fp8", 1.0), ("fp8", 1.6)])
def test_sampled_draws_match_oracle(w, prompt, scales, precision, T):
    ctx = gpu_context(SH, w, precision, act_scales=scales if precision == "fp8" else None)
    try:
        seed = 0x0123456789ABCDEF
        ctx.set_sampling(T, seed)
        ctx.prefill(prompt)
        codes, n_draws, n_band = sampled_run(ctx, SH, 24, T, seed)
        print(f"sampling {precision} T={T}: {n_draws} draws checked, {n_band} within {SAMPLE_BAND} of a boundary "
              f"(a neighbour accepted); distinct codes drawn {len(np.unique(codes[:, 1:]))}")
        assert n_draws >= 100  # 24 x 8 draws less the BOS forced on the lagging codebooks (and any EOS)
        assert n_band <= max(3, n_draws // 30)
    finally:
        ctx.close()


def test_fixed_seed_repeats_and_other_seed_differs(w, prompt):
    ctx = gpu_context(SH, w, "bf16")
    try:
        runs = []
        for seed in (1234, 1234, 1235):
            ctx.reset(0)
            ctx.set_sampling(1.0, seed)
            ctx.prefill(prompt)
            runs.append(ctx.decode_frames(16)[0])
        assert np.array_equal(runs[0], runs[1])
        assert not np.array_equal(runs[0], runs[2])
    finally:
        ctx.close()


def test_temperature_zero_and_tiny_temperature_give_the_argmax(w, prompt):
    ref = gpu_context(SH, w, "bf16")
    ctx = gpu_context(SH, w, "bf16")
    try:
        ref.prefill(prompt)
        greedy = ref.decode_frames(12)[0]
        ctx.set_sampling(0.0, 99)
        ctx.prefill(prompt)
        assert np.array_equal(ctx.decode_frames(12)[0], greedy)
        # at T = 1e-4 every weight but the largest logit's underflows (random logits have no
        # near-ties at that scale): the draw is the argmax
        ctx.reset(0)
        ctx.set_sampling(1e-4, 99)
        ctx.prefill(prompt)
        assert np.array_equal(ctx.decode_frames(12)[0], greedy)
    finally:
        ref.close()
        ctx.close()


def test_set_sampling_rejects_bad_temperatures(w):
    with gpu_context(SH, w, "bf16") as ctx:
        for bad in (-1.0, float("nan"), float("inf")):
            with pytest.raises(hta.HtaError) as e:
                ctx.set_sampling(bad, 1)
            assert e.value.code == hta.HTA_E_ARG
