"""hta_decode_frames_noalloc against hta_decode_frames through the C ABI.

Two twin contexts per shape hold the same weights and prompt; one decodes with the
ordinary entry point (exchange words in its workspace), the other with the allocation-free
one (exchange words in the library's static per-GPU array).  The frame kernel is the same
and its reductions run in a fixed order, so codes, the final residual, the logits and the
decode state must be bit-identical.  The allocation-free calls run back to back: first a
Qwen3-4B-wide two-layer context (1.2 MiB of exchange words), then the tiny shape with fewer
frames, whose smaller footprint sits inside what the first call left behind; then the wide
context again, which must continue its utterance unharmed by the tiny call's tags."""
import dataclasses

import numpy as np
import pytest

import synthetic as S
from autoregressive_codebook_tts_amd import hta
from gpu_common import gpu_context

pytestmark = pytest.mark.gpu

WIDE = dataclasses.replace(S.QWEN3_4B, n_layers=2, text_vocab=1024)


def _pair(shape, seed, precision, act_scales=None):
    w = S.make_weights(shape, seed, "f32")
    ref = gpu_context(shape, w, precision, act_scales=act_scales)
    dut = gpu_context(shape, w, precision, act_scales=act_scales)
    return ref, dut


def _same(ref, dut, codes_ref, codes_dut, what):
    assert np.array_equal(codes_ref, codes_dut), f"{what}: codes differ"
    for tap in ("tap_hidden", "tap_logits"):
        a, b = getattr(ref, tap)(), getattr(dut, tap)()
        assert np.array_equal(a.view(np.uint32), b.view(np.uint32)), f"{what}: {tap} differs"
    sr, sd = ref.tap_state(), dut.tap_state()
    assert sr.keys() == sd.keys() and all(np.array_equal(sr[k], sd[k]) for k in sr), f"{what}: decode state differs"


def test_noalloc_matches_decode_frames_on_consecutive_calls():
    prompt_w = S.token_ids(S.SEEDS["tiny_prompt"], 12, WIDE.text_vocab)
    prompt_t = S.token_ids(S.SEEDS["tiny_prompt"], 8, S.TINY.text_vocab)
    wide_ref, wide_dut = _pair(WIDE, S.SEEDS["tiny_weights"] + 1, "bf16")
    # FP8 tiny context with scales from a BF16 calibration run on the GPU
    w_t = S.make_weights(S.TINY, S.SEEDS["tiny_weights"], "f32")
    with gpu_context(S.TINY, w_t, "bf16") as cal:
        scales = cal.calibrate(S.token_ids(S.SEEDS["calib_prompt"], 16, S.TINY.text_vocab), 8)
    tiny_ref = gpu_context(S.TINY, w_t, "fp8", act_scales=scales)
    tiny_dut = gpu_context(S.TINY, w_t, "fp8", act_scales=scales)
    try:
        for c in (wide_ref, wide_dut):
            c.prefill(prompt_w)
        for c in (tiny_ref, tiny_dut):
            c.prefill(prompt_t)
        # ordinary entry point first (graph replay), for every reference
        ref_w1, _ = wide_ref.decode_frames(6)
        print(f"[no-alloc] wide reference: 6 frames, first codes {ref_w1[0].tolist()}", flush=True)
        ref_t, _ = tiny_ref.decode_frames(3)
        # the allocation-free calls back to back: wide (6 frames), then tiny (3 frames)
        out_w1 = np.full((6, WIDE.n_codebooks), -1, np.int32)
        got_w1, _ = wide_dut.decode_frames_noalloc(6, out=out_w1)
        assert got_w1 is out_w1
        got_t, _ = tiny_dut.decode_frames_noalloc(3)
        _same(wide_ref, wide_dut, ref_w1, got_w1, "wide, first call")
        _same(tiny_ref, tiny_dut, ref_t, got_t, "tiny, second call")
        # the wide utterance goes on through the array the tiny call used last
        ref_w2, _ = wide_ref.decode_frames(2)
        got_w2, _ = wide_dut.decode_frames_noalloc(2)
        _same(wide_ref, wide_dut, ref_w2, got_w2, "wide, third call")
        # and the ordinary entry point still continues where the allocation-free one stopped
        ref_w3, _ = wide_ref.decode_frames(1)
        got_w3, _ = wide_dut.decode_frames(1)
        _same(wide_ref, wide_dut, ref_w3, got_w3, "wide, ordinary call after the allocation-free ones")
        print(f"[no-alloc] wide 6+2+1 and tiny 3 frames bit-identical to hta_decode_frames", flush=True)
    finally:
        for c in (wide_ref, wide_dut, tiny_ref, tiny_dut):
            c.close()


def test_noalloc_argument_errors():
    w_t = S.make_weights(S.TINY, S.SEEDS["tiny_weights"], "f32")
    with gpu_context(S.TINY, w_t, "bf16", max_seq=16, max_prefill=16) as c:
        with pytest.raises(ValueError):
            c.decode_frames_noalloc(2, out=np.zeros((3, S.TINY.n_codebooks), np.int32))
        out = np.zeros((1, S.TINY.n_codebooks), np.int32)
        rc = hta.lib().hta_decode_frames_noalloc(c.ctx, 0, hta._ptr(out), None)
        assert rc == hta.HTA_E_ARG
        with pytest.raises(hta.HtaError) as e:
            c.decode_frames_noalloc(17)
        assert e.value.code == hta.HTA_E_CAPACITY
