"""Batched multi-stream decode (n_streams > 1) on the tiny backbone: every stream of a
batch against its own oracle, stream isolation, and the calls a batched context refuses.

Each stream is teacher-forced by its own oracle run (the codes of the oracle mode named
first) and compared at every step: BF16 hidden state within 5e-3 of the bf16
storage-faithful oracle and within the end-to-end tolerance of the exact model, FP8 within
the FP8 tolerance of the FP8 storage-faithful oracle, logits cosine >= 0.999, and every
argmax whose oracle margin is robust equal.  The BF16 gate against the storage-faithful
oracle is the single-stream path's 2e-3 widened for the GEMMs' accumulation order: one
rounding decision at a bf16 boundary taken the other way moves the 256-wide hidden state
by about 1e-3 of its norm, and the MFMA GEMMs sum in another order than the single-stream
GEMV, so a few such decisions per 12-step run are expected."""
import numpy as np
import pytest

import synthetic as S
from autoregressive_codebook_tts_amd import hta
from gpu_common import COS_MIN, HIDDEN_TOL, cosines, gpu_context, id_agreement, rel_l2, tiny_weights
from oracle.model import OracleModel, calibrate

pytestmark = pytest.mark.gpu
SH = S.TINY


@pytest.fixture(scope="module")
def w():
    return tiny_weights()


@pytest.fixture(scope="module")
def scales(w):
    return calibrate(SH, w, S.token_ids(S.SEEDS["calib_prompt"], 16, SH.text_vocab), 16)[0]


def _prompts(lengths, seed0=7000):
    return [S.token_ids(seed0 + i, n, SH.text_vocab) for i, n in enumerate(lengths)]


def _batched_teacher_forced(w, prompts, precision, act_scales, n_frames, modes, check=None):
    """recs[i] for stream check[i] (default: every stream); the other streams decode freely."""
    M = len(prompts)
    check = list(range(M)) if check is None else list(check)
    ctx = gpu_context(SH, w, precision, max_seq=128, max_prefill=max(16, M), act_scales=act_scales, n_streams=M)
    oracles = {m: {mo: OracleModel(SH, w, precision, mo, act_scales=act_scales if mo == "S" else None, max_seq=128)
                   for mo in modes} for m in check}
    try:
        for m, p in enumerate(prompts):
            ctx.select_stream(m)
            ctx.prefill(p)
            for o in oracles.get(m, {}).values():
                o.prefill(p)
        recs = {m: [] for m in check}
        for f in range(n_frames):
            codes, _ = ctx.decode_frame()
            assert codes.shape == (M, SH.n_codebooks)
            for m in check:
                ctx.select_stream(m)
                rec = {"t": f, "gpu": {"codes": codes[m], "hidden": ctx.tap_hidden().astype(np.float64),
                                       "logits": ctx.tap_logits().astype(np.float64)}}
                st = ctx.tap_state()
                assert st["len"] == len(prompts[m]) + f + 1 and st["t"] == f + 1
                for mo, o in oracles[m].items():
                    c_, d_ = o.decode_frame()
                    rec[mo] = {"codes": c_, "done": d_, "hidden": o.last_hidden.copy(), "logits": o.last_logits.copy()}
                forced = rec[modes[0]]["codes"]
                for o in oracles[m].values():
                    o.force_codes(forced)
                ctx.force_codes(forced)
                recs[m].append(rec)
        return [recs[m] for m in check]
    finally:
        ctx.close()


def test_batched_bf16_streams_match_their_oracles(w):
    prompts = _prompts([5, 8, 11])
    recs = _batched_teacher_forced(w, prompts, "bf16", None, 12, ("E", "S"))
    for m, rs in enumerate(recs):
        rel_e = max(rel_l2(r["gpu"]["hidden"], r["E"]["hidden"]) for r in rs)
        rel_s = max(rel_l2(r["gpu"]["hidden"], r["S"]["hidden"]) for r in rs)
        cos = min(cosines(r["gpu"]["logits"], r["E"]["logits"]).min() for r in rs)
        n, bad = id_agreement(SH, rs, "E")
        print(f"batched bf16 stream {m} (P={len(prompts[m])}): hidden rel {rel_e:.3e} vs exact, {rel_s:.3e} vs bf16 "
              f"oracle; logits cos {cos:.6f}; {n} robust ids, {len(bad)} mismatches")
        assert rel_e <= HIDDEN_TOL["bf16"] and rel_s <= 5e-3 and cos >= COS_MIN
        assert n > 30 and not bad


def test_batched_fp8_streams_match_their_oracles(w, scales):
    prompts = _prompts([9, 4, 13])
    recs = _batched_teacher_forced(w, prompts, "fp8", scales, 12, ("S", "E"))
    for m, rs in enumerate(recs):
        rel_s = max(rel_l2(r["gpu"]["hidden"], r["S"]["hidden"]) for r in rs)
        cos_s = min(cosines(r["gpu"]["logits"], r["S"]["logits"]).min() for r in rs)
        n, bad = id_agreement(SH, rs, "S")
        print(f"batched fp8 stream {m} (P={len(prompts[m])}): hidden rel {rel_s:.3e} vs fp8 oracle (cos {cos_s:.6f}); "
              f"{n} robust ids, {len(bad)} mismatches")
        assert rel_s <= HIDDEN_TOL["fp8"] and cos_s >= COS_MIN
        assert n > 30 and not bad


@pytest.mark.parametrize("precision,M,check", [("fp8", 70, (0, 35, 69)), ("bf16", 40, (0, 39))])
def test_batched_many_streams_match_their_oracles(w, scales, precision, M, check):
    """Batches past one 32-row GEMM tile (40 streams: two row tiles of the skinny GEMM; 70:
    the LDS-tiled GEMM) and down to one key split per stream: the checked streams against
    their own oracles, to the gates of the three-stream tests."""
    lengths = [4 + (7 * m) % 12 for m in range(M)]
    prompts = _prompts(lengths, seed0=7100)
    modes = ("S", "E") if precision == "fp8" else ("E", "S")
    recs = _batched_teacher_forced(w, prompts, precision, scales if precision == "fp8" else None, 8, modes, check)
    for m, rs in zip(check, recs):
        if precision == "fp8":
            rel = max(rel_l2(r["gpu"]["hidden"], r["S"]["hidden"]) for r in rs)
            cos = min(cosines(r["gpu"]["logits"], r["S"]["logits"]).min() for r in rs)
            n, bad = id_agreement(SH, rs, "S")
            ok = rel <= HIDDEN_TOL["fp8"]
        else:
            rel = max(rel_l2(r["gpu"]["hidden"], r["S"]["hidden"]) for r in rs)
            cos = min(cosines(r["gpu"]["logits"], r["E"]["logits"]).min() for r in rs)
            n, bad = id_agreement(SH, rs, "E")
            ok = rel <= 5e-3 and max(rel_l2(r["gpu"]["hidden"], r["E"]["hidden"]) for r in rs) <= HIDDEN_TOL["bf16"]
        print(f"batched {precision} M={M} stream {m} (P={lengths[m]}): hidden rel {rel:.3e} vs the storage-faithful "
              f"oracle; logits cos {cos:.6f}; {n} robust ids, {len(bad)} mismatches")
        assert ok and cos >= COS_MIN
        assert n > 15 and not bad


def test_batched_streams_are_isolated(w):
    """A stream's codes and final residual are bit-identical whatever the other streams
    hold: the GEMM rows, the attention and the head choice of one stream never read another's."""
    base = _prompts([6, 9, 7, 10])
    other = list(base)
    other[2] = S.token_ids(9999, 12, SH.text_vocab)
    runs = []
    for prompts in (base, other):
        with gpu_context(SH, w, "bf16", max_seq=64, max_prefill=16, n_streams=4) as ctx:
            for m, p in enumerate(prompts):
                ctx.select_stream(m)
                ctx.prefill(p)
            codes, _ = ctx.decode_frames(10)
            hid = []
            for m in range(4):
                ctx.select_stream(m)
                hid.append(ctx.tap_hidden().copy())
            runs.append((codes, hid))
    for m in (0, 1, 3):
        assert np.array_equal(runs[0][0][:, m], runs[1][0][:, m]), f"stream {m} codes changed"
        assert np.array_equal(runs[0][1][m].view(np.uint32), runs[1][1][m].view(np.uint32))
    assert not np.array_equal(runs[0][0][:, 2], runs[1][0][:, 2])


def test_batched_context_refuses_single_stream_calls(w):
    with gpu_context(SH, w, "bf16", max_seq=32, max_prefill=16, n_streams=2) as ctx:
        with pytest.raises(hta.HtaError) as e:
            ctx.select_stream(2)
        assert e.value.code == hta.HTA_E_ARG
        for call in (lambda: ctx.set_sampling(1.0, 1), lambda: ctx.decode_frames_noalloc(1),
                     lambda: ctx.set_option(hta.OPT_TAPS, 1),
                     lambda: ctx.calibrate(S.token_ids(1, 4, SH.text_vocab), 2)):
            with pytest.raises(hta.HtaError) as e:
                call()
            assert e.value.code == hta.HTA_E_UNSUPPORTED
        # every stream's KV capacity is checked
        ctx.select_stream(1)
        ctx.prefill(S.token_ids(5, 16, SH.text_vocab))
        ctx.prefill(S.token_ids(6, 14, SH.text_vocab))
        with pytest.raises(hta.HtaError) as e:
            ctx.decode_frames(3)
        assert e.value.code == hta.HTA_E_CAPACITY
