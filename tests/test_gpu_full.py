"""GPU parity of the full 36-layer Qwen3-4B-shaped backbone (hidden 2560, 32q/8kv
heads, head_dim 128, FFN 9728, text vocabulary 151936, 8 x 1026 head) against
the CPU oracle, in the launch configuration that the benchmark times (one
persistent kernel per decode frame; batched prefill).

Two kinds of comparison:

* Site-anchored (sharp, decode frames): with the taps on, every rounding point of
  every one of the 36 layers is checked on its own.  The oracle recomputes each
  layer from the GPU's input residual and KV cache, with every GEMV fed the GPU's
  own rounded input (the bf16 values or e4m3 codes the frame kernel multiplied
  with); each of the four GEMV inputs, the head input and the K/V row the GPU
  rounded must then equal the oracle's rounding of the same values, except for
  counted flips of values lying within a stated band of a rounding boundary, and
  the layer output must match to fp32 accumulation (rel 1e-5).  The head is
  checked the same way, and its logits re-anchored on the GPU's final residual
  give cosine >= 0.999 and greedy ids equal wherever the oracle's top-2 margin
  exceeds 1e-2.
* Re-anchored (prefill): layers 0, 18 and 35 of a prefill recomputed by the
  oracle from the GPU's input rows and KV: BF16 update rel <= 2^-8 (one bf16
  ulp), FP8 <= 6e-2; the K/V written agree with the oracle's bf16 values.
* End to end (teacher forced, against the exact oracle): these random
  N(0, 0.02) weights amplify every rounding about fifteenfold over 36 layers,
  so the oracle's own storage-faithful run lands 1.9 % (BF16) and 35 % (FP8)
  from the exact model.  The gate is therefore that the GPU is no further
  from the exact model than the oracle's own run of the same precision
  (x 1.25), and for BF16 decode also logits cosine 0.999 and equal robust ids.

Also: FP8 calibration against the oracle's own calibration, prefill at
P = 13, 128, 512, prefix reuse (a 64-token preamble kept once, 8 suffixes of
16 tokens, bit-identical to cold prefills), and an FP8 frame at KV length 4096
after a chunked 4095-token prefill.  The oracle runs with float32 weight
storage (float32 BLAS products, float64 everything else)."""
import time

import numpy as np
import pytest

import synthetic as S
from autoregressive_codebook_tts_amd import hta
from gpu_common import (COS_MIN, FLIP_LOG, HEAD_BAND, HIDDEN_TOL, MARGIN, allowed_mask, bf16_values,
                        check_layer_sites, check_site, cosines, gpu_context, kv_rows as _kv_rows, rel_l2, sampled_run,
                        top2_margin)
from oracle import numerics as nx
from oracle.model import OracleModel, calibrate

pytestmark = [pytest.mark.gpu, pytest.mark.slow]
SH = S.QWEN3_4B
F32 = np.float32
MAX_SEQ = 4096
MAX_PREFILL = 512
# One re-anchored layer against the storage-faithful oracle.  Two faithful BF16 implementations
# that accumulate in different orders flip a few per cent of the elements at each of the layer's
# rounding points by one bf16 ulp (fp32 sums over K ~ 2560 terms differ by ~K * 2^-24 relative,
# against the bf16 half-spacing 2^-9), so their updates differ by a fraction of an ulp; one ulp,
# 2^-8, bounds it.  FP8 uses the hidden-state bound of the FP8 path.
LAYER_TOL = {"bf16": 2.0 ** -8, "fp8": 6e-2}
KV_TOL = {"bf16": 1e-2, "fp8": 6e-2}
E2E_RATIO = 1.25                           # end to end: GPU-to-exact over oracle-storage-to-exact


def _say(msg):
    print(msg, flush=True)


# ----------------------------------------------------------------------------- fixtures
@pytest.fixture(scope="module")
def w():
    t0 = time.time()
    out = S.make_weights(SH, S.SEEDS["full_weights"], "bf16")
    _say(f"[full] weights generated in {time.time() - t0:.1f} s")
    return out


@pytest.fixture(scope="module")
def oracle_e(w):
    return OracleModel(SH, w, "bf16", "E", storage=F32, max_seq=MAX_SEQ)


@pytest.fixture(scope="module")
def oracle_sb(w):
    return OracleModel(SH, w, "bf16", "S", storage=F32, max_seq=MAX_SEQ)


@pytest.fixture(scope="module")
def gpu_bf16(w):
    ctx = gpu_context(SH, w, "bf16", max_seq=MAX_SEQ, max_prefill=MAX_PREFILL)
    yield ctx
    ctx.close()


@pytest.fixture(scope="module")
def calibration(w, gpu_bf16):
    """(oracle scales, oracle codes, GPU scales) for the seeded 16-token prompt + 16 frames."""
    calib = S.token_ids(S.SEEDS["calib_prompt"], 16, SH.text_vocab)
    s_o, _, codes_o = calibrate(SH, w, calib, 16, storage=F32)
    s_g = gpu_bf16.calibrate(calib, 16, forced_codes=codes_o)
    return s_o, codes_o, s_g


@pytest.fixture(scope="module")
def gpu_fp8(w, calibration):
    ctx = gpu_context(SH, w, "fp8", max_seq=MAX_SEQ, max_prefill=MAX_PREFILL, act_scales=calibration[2])
    yield ctx
    ctx.close()


@pytest.fixture(scope="module")
def oracle_s8(w, calibration):
    return OracleModel(SH, w, "fp8", "S", act_scales=calibration[2], storage=F32, max_seq=MAX_SEQ)


def _ctx_and_oracle(request, precision):
    if precision == "bf16":
        return request.getfixturevalue("gpu_bf16"), request.getfixturevalue("oracle_sb")
    return request.getfixturevalue("gpu_fp8"), request.getfixturevalue("oracle_s8")


# ----------------------------------------------------------------------------- re-anchored checks
def _check_layer(ctx, oracle, layer, h_in, h_out, positions, precision, what):
    """Oracle layer from the GPU's input rows and the GPU's KV before positions[0]; returns
    (update rel, K rel, V rel) and asserts the per-layer bounds."""
    p0 = int(positions[0])
    kp, vp = _kv_rows(ctx, layer, p0)
    oracle.set_kv(layer, kp, vp)
    ref = oracle.layer(layer, np.asarray(h_in, np.float64), np.asarray(positions))
    upd = rel_l2(h_out - h_in, ref - h_in)
    n = int(positions[-1]) + 1
    kg, vg = _kv_rows(ctx, layer, n)
    k_rel = rel_l2(kg[p0:n], oracle.k_cache[layer, p0:n])
    v_rel = rel_l2(vg[p0:n], oracle.v_cache[layer, p0:n])
    assert upd <= LAYER_TOL[precision], f"{what} layer {layer}: update rel {upd:.3e}"
    assert k_rel <= KV_TOL[precision] and v_rel <= KV_TOL[precision], f"{what} layer {layer}: K {k_rel:.3e} V {v_rel:.3e}"
    return upd, k_rel, v_rel


def _check_head(ctx, oracle, taps, t, state_before, what):
    """Head from the GPU's final residual; logits cosine and robust greedy ids."""
    ref = oracle.head(taps[-1])
    got = ctx.tap_logits().astype(np.float64)
    cos = cosines(got, ref).min()
    codes = ctx.tap_state()["codes"]
    n = 0
    for k in range(SH.n_codebooks):
        if t < k or state_before["eoc"] >= 0 or int(state_before["prev"][0]) == SH.eos_id:
            continue  # BOS forced, or the EOS rule decides
        mask = allowed_mask(SH, k)
        if top2_margin(ref[k], mask) > MARGIN:
            n += 1
            want = int(np.flatnonzero(mask)[np.argmax(ref[k][mask])])
            assert int(codes[k]) == want, f"{what} t={t} codebook {k}: gpu {codes[k]} oracle {want}"
    assert cos >= COS_MIN, f"{what} t={t}: logits cos {cos:.6f}"
    return cos, n


def _reanchored_frames(ctx, oracle, precision, n_frames, what):
    """Decode n_frames frames (greedy, the GPU's own codes fed back) with taps on and check
    the frame input, every rounding point of every layer and the head of each against the
    oracle (site-anchored; module docstring)."""
    flips = np.zeros(4, np.int64)
    kv_flips, worst_upd = 0, 0.0
    FLIP_LOG.clear()
    worst_cos, n_ids = 1.0, 0
    sh = SH
    for _ in range(n_frames):
        st = ctx.tap_state()
        pos, t = st["len"], st["t"]
        ctx.decode_frame()
        taps = ctx.tap_layers().astype(np.float64)
        acts = ctx.tap_acts()
        q_tap = ctx.tap_q()
        x = sum(oracle.e_aud[k, int(st["prev"][k])].astype(np.float64) for k in range(sh.n_codebooks))
        assert rel_l2(taps[0], x) <= 1e-6, f"{what} t={t}: frame input"
        for layer in range(sh.n_layers):
            f, kvf, upd = check_layer_sites(ctx, oracle, layer, taps[layer], taps[layer + 1], acts, q_tap, pos,
                                            f"{what} t={t}")
            flips += f
            kv_flips += kvf
            worst_upd = max(worst_upd, upd)
        z = bf16_values(acts[5 * sh.n_layers][:sh.hidden])
        pre_z, lg = oracle.head_anchored(taps[-1], z)
        head_flips, _ = check_site(oracle, 4 * sh.n_layers, z, pre_z, HEAD_BAND, f"{what} t={t} head")
        flips[0] += head_flips
        got = ctx.tap_logits().astype(np.float64)
        assert rel_l2(got, lg) <= 1e-5, f"{what} t={t}: logits from the GPU's own head input off by {rel_l2(got, lg):.3e}"
        cos, n = _check_head(ctx, oracle, taps, t, st, f"{what}")
        worst_cos, n_ids = min(worst_cos, cos), n_ids + n
        assert np.array_equal(taps[-1], ctx.tap_hidden().astype(np.float64))
    n_dec = n_frames * (sh.n_layers * (2 * sh.hidden + sh.q_dim + sh.ffn) + sh.hidden)
    per_site = {}
    for (_, site, n, wr, wm) in FLIP_LOG:
        k = "head" if site == 4 * sh.n_layers else site % 4
        a = per_site.setdefault(k, [0, 0.0, 0.0])
        a[0] += n
        a[1] = max(a[1], wr)
        a[2] = max(a[2], wm)
    FLIP_LOG.clear()
    _say(f"[full] {what}: flips by site kind (count, worst rel distance, worst RMS distance): {per_site}")
    _say(f"[full] {what}: {n_frames} frames x {sh.n_layers} layers site-anchored: {int(flips.sum())} rounding flips "
         f"of {n_dec} decisions at boundaries (per site {flips.tolist()}), {kv_flips} q/k/v flips, worst layer output "
         f"rel {worst_upd:.2e}; head cos >= {worst_cos:.6f}; {n_ids} robust ids equal")


@pytest.mark.parametrize("precision", ["bf16", "fp8"])
def test_full_decode_layers_reanchored(request, precision):
    ctx, oracle = _ctx_and_oracle(request, precision)
    prompt = S.token_ids(S.SEEDS["full_prompt"], 13, SH.text_vocab)
    ctx.set_option(hta.OPT_TAPS, 1)
    try:
        ctx.reset(0)
        ctx.prefill(prompt)
        _reanchored_frames(ctx, oracle, precision, 3, f"{precision} decode")
    finally:
        ctx.set_option(hta.OPT_TAPS, 0)


def _prefill_reanchored(ctx, oracle, precision, P, what):
    """Layers 0, 18 and 35 of a P-row prefill re-anchored on the oracle; returns the worst
    (update rel, K rel, V rel) and the rows leaving the last layer."""
    ids = S.token_ids(S.SEEDS[f"prefill_{P}"], P, SH.text_vocab)
    ctx.set_option(hta.OPT_TAPS, 1)
    worst = [0.0, 0.0, 0.0]
    last = None
    try:
        for layer in (0, SH.n_layers // 2, SH.n_layers - 1):
            ctx.set_option(hta.OPT_PREFILL_TAP_LAYER, layer)
            ctx.reset(0)
            ctx.prefill(ids)
            rows = ctx.tap_prefill_layer(P).astype(np.float64)
            r = _check_layer(ctx, oracle, layer, rows[0], rows[1], np.arange(P), precision, what)
            worst = [max(a, b) for a, b in zip(worst, r)]
            if layer == SH.n_layers - 1:
                assert np.array_equal(rows[1], ctx.tap_prefill_hidden(P).astype(np.float64))
                last = rows[1]
    finally:
        ctx.set_option(hta.OPT_TAPS, 0)
        ctx.set_option(hta.OPT_PREFILL_TAP_LAYER, 0)
    return worst, last


@pytest.mark.parametrize("precision", ["bf16", "fp8"])
@pytest.mark.parametrize("P", [13, 128, 512])
def test_full_prefill_layers_reanchored(request, precision, P):
    ctx, oracle = _ctx_and_oracle(request, precision)
    worst, _ = _prefill_reanchored(ctx, oracle, precision, P, f"{precision} prefill P={P}")
    _say(f"[full] {precision} prefill P={P}: layers 0/18/35 re-anchored: worst update rel {worst[0]:.3e}, "
         f"K {worst[1]:.3e}, V {worst[2]:.3e}")


@pytest.mark.parametrize("P", [13, 512])
def test_full_prefill_fp8_mfma_option_reanchored(request, P):
    """The opt-in e4m3 MFMA form of the prefill GEMMs: its sums carry fewer bits than fp32
    (tests/test_gpu_gemm.py), yet each re-anchored layer stays within the FP8 layer
    tolerance; the option is live (the last layer's rows differ from the default path's)."""
    ctx, oracle = _ctx_and_oracle(request, "fp8")
    _, base = _prefill_reanchored(ctx, oracle, "fp8", P, f"fp8 prefill P={P}")
    ctx.set_option(hta.OPT_FP8_MFMA, 1)
    try:
        worst, rows = _prefill_reanchored(ctx, oracle, "fp8", P, f"fp8 e4m3-MFMA prefill P={P}")
    finally:
        ctx.set_option(hta.OPT_FP8_MFMA, 0)
    assert not np.array_equal(rows, base)
    _say(f"[full] fp8 e4m3-MFMA prefill P={P}: layers 0/18/35 re-anchored: worst update rel {worst[0]:.3e}, "
         f"K {worst[1]:.3e}, V {worst[2]:.3e}; last layer vs default rel {rel_l2(rows, base):.3e}")


# ----------------------------------------------------------------------------- end to end
def _teacher_forced(ctx, oracles, prompt, n, driver):
    for o in oracles.values():
        o.reset(0)
        o.prefill(prompt)
    ctx.reset(0)
    ctx.prefill(prompt)
    recs = []
    for f in range(n):
        rec = {"t": f}
        for m, o in oracles.items():
            codes, _ = o.decode_frame()
            rec[m] = {"codes": codes, "hidden": o.last_hidden.copy(), "logits": o.last_logits.copy()}
        g, _ = ctx.decode_frame()
        rec["gpu"] = {"codes": g, "hidden": ctx.tap_hidden().astype(np.float64),
                      "logits": ctx.tap_logits().astype(np.float64)}
        for o in oracles.values():
            o.force_codes(rec[driver]["codes"])
        ctx.force_codes(rec[driver]["codes"])
        recs.append(rec)
    return recs


def _worst(recs, a, b):
    return (max(rel_l2(r[a]["hidden"], r[b]["hidden"]) for r in recs),
            min(cosines(r[a]["logits"], r[b]["logits"]).min() for r in recs))


def _robust_ids(recs, ref, who="gpu"):
    """Greedy decisions with oracle top-2 margin > MARGIN: (count, disagreements as (t, k, margin)),
    and sigma_delta, the RMS of (who - ref) logits over the run."""
    n, bad, deltas = 0, [], []
    for rec in recs:
        deltas.append((rec[who]["logits"] - rec[ref]["logits"]).ravel())
        for k in range(SH.n_codebooks):
            if rec["t"] < k:
                continue
            mg = top2_margin(rec[ref]["logits"][k], allowed_mask(SH, k))
            if mg > MARGIN:
                n += 1
                if int(rec[ref]["codes"][k]) != int(rec[who]["codes"][k]):
                    bad.append((rec["t"], k, round(mg, 4)))
    return n, bad, float(np.sqrt(np.mean(np.concatenate(deltas) ** 2)))


def test_full_bf16_end_to_end(gpu_bf16, oracle_e, oracle_sb):
    prompt = S.token_ids(S.SEEDS["full_prompt"], 13, SH.text_vocab)
    recs = _teacher_forced(gpu_bf16, {"E": oracle_e, "S": oracle_sb}, prompt, 6, "E")
    rel, cos = _worst(recs, "gpu", "E")
    rel_s, cos_s = _worst(recs, "S", "E")
    n, bad, sigma = _robust_ids(recs, "E")
    _, bad_s, sigma_s = _robust_ids(recs, "E", who="S")
    _say(f"[full] bf16 end to end (6 frames, vs exact): hidden rel {rel:.3e} (oracle bf16 storage {rel_s:.3e}), "
         f"logits cos {cos:.6f} (oracle {cos_s:.6f}); {n} robust ids, disagreements {bad} at sigma_delta "
         f"{sigma:.3e} (oracle bf16 storage: {bad_s} at {sigma_s:.3e})")
    assert rel <= HIDDEN_TOL["bf16"]  # the stated end-to-end bound
    assert rel <= E2E_RATIO * rel_s
    assert cos >= COS_MIN
    # Over 36 layers the logit noise of any BF16-storage run (sigma_delta ~ 1.7e-2 here) exceeds the
    # 1e-2 margin, so an id whose margin is a few sigma_delta can flip; every disagreement must lie
    # within 4 sigma_delta.  The exact 1e-2 rule is checked on the head re-anchored to the GPU's
    # own residual (test_full_decode_layers_reanchored).
    assert n >= 20
    assert all(m < 4 * sigma for (_, _, m) in bad)
    assert len(bad) <= len(bad_s) + 2


def test_full_batched_bf16_stream_against_exact(w, oracle_e, oracle_sb):
    """Batched decode at the 36-layer shape: stream 0 of a two-stream BF16 context (stream 1
    decodes another prompt alongside), teacher-forced by the exact oracle, meets the
    single-stream end-to-end gates."""
    prompt = S.token_ids(S.SEEDS["full_prompt"], 13, SH.text_vocab)
    other = S.token_ids(S.SEEDS["full_prompt"] + 1, 21, SH.text_vocab)
    oracles = {"E": oracle_e, "S": oracle_sb}
    for o in oracles.values():
        o.reset(0)
        o.prefill(prompt)
    recs = []
    with gpu_context(SH, w, "bf16", max_seq=64, max_prefill=32, n_streams=2) as ctx:
        ctx.select_stream(1)
        ctx.prefill(other)
        ctx.select_stream(0)
        ctx.prefill(prompt)
        for f in range(4):
            rec = {"t": f}
            for m, o in oracles.items():
                codes, _ = o.decode_frame()
                rec[m] = {"codes": codes, "hidden": o.last_hidden.copy(), "logits": o.last_logits.copy()}
            g, _ = ctx.decode_frame()
            rec["gpu"] = {"codes": g[0], "hidden": ctx.tap_hidden().astype(np.float64),
                          "logits": ctx.tap_logits().astype(np.float64)}
            for o in oracles.values():
                o.force_codes(rec["E"]["codes"])
            ctx.force_codes(rec["E"]["codes"])
            recs.append(rec)
    rel, cos = _worst(recs, "gpu", "E")
    rel_s, cos_s = _worst(recs, "S", "E")
    _say(f"[full] batched bf16 stream 0 of 2 (4 frames, vs exact): hidden rel {rel:.3e} (oracle bf16 storage "
         f"{rel_s:.3e}), logits cos {cos:.6f} (oracle {cos_s:.6f})")
    assert rel <= HIDDEN_TOL["bf16"]
    assert rel <= E2E_RATIO * rel_s
    assert cos >= COS_MIN


def test_full_fp8_end_to_end(gpu_fp8, oracle_e, oracle_s8):
    prompt = S.token_ids(S.SEEDS["full_prompt"], 13, SH.text_vocab)
    recs = _teacher_forced(gpu_fp8, {"E": oracle_e, "S": oracle_s8}, prompt, 4, "E")
    rel, cos = _worst(recs, "gpu", "E")
    rel_s, cos_s = _worst(recs, "S", "E")
    rel_gs, cos_gs = _worst(recs, "gpu", "S")
    _say(f"[full] fp8 end to end (4 frames, vs exact): hidden rel {rel:.3e} (oracle fp8 storage {rel_s:.3e}), "
         f"logits cos {cos:.6f} (oracle {cos_s:.6f}); gpu vs fp8 oracle: hidden rel {rel_gs:.3e}, cos {cos_gs:.6f}")
    assert rel <= E2E_RATIO * rel_s
    assert cos >= cos_s - 0.02


def test_full_calibration_matches_oracle(calibration):
    s_o, _, s_g = calibration
    r = np.abs(s_g.astype(np.float64) / s_o - 1.0)
    _say(f"[full] calibration: worst per-scale rel diff {r.max():.3e} at site {int(r.argmax())}, median {np.median(r):.3e}")
    assert s_g.shape == (4 * SH.n_layers + 1,)
    # a scale is a maximum over the site's activations, which two BF16-storage runs reproduce
    # only to the BF16 hidden-state tolerance; the typical site agrees far closer
    assert r.max() <= HIDDEN_TOL["bf16"]
    assert np.median(r) <= 5e-3


@pytest.mark.parametrize("precision", ["bf16", "fp8"])
@pytest.mark.parametrize("P", [13, 128, 512])
def test_full_prefill_end_to_end(request, precision, P):
    ctx, oracle_s = _ctx_and_oracle(request, precision)
    oracle_e = request.getfixturevalue("oracle_e")
    ids = S.token_ids(S.SEEDS[f"prefill_{P}"], P, SH.text_vocab)
    ctx.reset(0)
    ctx.prefill(ids)
    got = ctx.tap_prefill_hidden(P).astype(np.float64)
    for o in (oracle_e, oracle_s):
        o.reset(0)
        o.prefill(ids)
    rel = rel_l2(got, oracle_e.last_hidden)
    rel_s = rel_l2(oracle_s.last_hidden, oracle_e.last_hidden)
    _say(f"[full] {precision} prefill P={P} end to end (vs exact): rows rel {rel:.3e} (oracle storage {rel_s:.3e})")
    assert rel <= E2E_RATIO * rel_s


# ----------------------------------------------------------------------------- determinism
@pytest.mark.parametrize("precision", ["bf16", "fp8"])
def test_full_decode_is_deterministic(request, precision):
    """The one-launch frame fixes every reduction order, so the same state decoded twice
    gives bit-identical hidden states, logits and codes (a stale or misplaced weight
    fetch into the LDS ring shows up here first)."""
    ctx, _ = _ctx_and_oracle(request, precision)
    prompt = S.token_ids(S.SEEDS["full_prompt"], 13, SH.text_vocab)
    runs = []
    for _ in range(2):
        ctx.reset(0)
        ctx.prefill(prompt)
        codes, _ = ctx.decode_frames(4)
        runs.append((codes, ctx.tap_hidden().copy(), ctx.tap_logits().copy()))
    assert np.array_equal(runs[0][0], runs[1][0]), "codes differ between identical runs"
    assert np.array_equal(runs[0][1], runs[1][1]), "hidden state differs between identical runs"
    assert np.array_equal(runs[0][2], runs[1][2]), "logits differ between identical runs"
    _say(f"[full] {precision} decode: two identical runs bit-identical")


def test_full_fp8_sampling_head(gpu_fp8):
    """The sampling head at the 36-layer shape: every draw of 12 frames equals the sampling
    oracle's on the GPU's own logits (a neighbour within the fp32 band)."""
    prompt = S.token_ids(S.SEEDS["full_prompt"], 13, SH.text_vocab)
    try:
        gpu_fp8.reset(0)
        gpu_fp8.set_sampling(1.0, 0xFEEDFACECAFEBEEF)
        gpu_fp8.prefill(prompt)
        _, n_draws, n_band = sampled_run(gpu_fp8, SH, 12, 1.0, 0xFEEDFACECAFEBEEF)
    finally:
        gpu_fp8.set_sampling(0.0, 0)
    _say(f"[full] fp8 sampling: {n_draws} draws checked, {n_band} within the fp32 band")
    assert n_draws >= 12 * 8 - 28 - 8 and n_band <= 3


# ----------------------------------------------------------------------------- chunked prefill
# (total rows, chunks): 100 rows in one call take the LDS-tiled GEMM below 256 rows (64 x 64
# tiles in e4m3, 128 x 128 in bf16) and the chunks the 32-row and 16-row skinny shapes; 300
# rows take the 128 x 128 three-stage tiles, and its chunks every other shape.
CHUNK_CASES = [(100, (37, 5, 16, 42)), (300, (37, 100, 163))]


@pytest.mark.parametrize("precision", ["bf16", "fp8"])
@pytest.mark.parametrize("total,chunks", CHUNK_CASES, ids=["100", "300"])
def test_full_chunked_prefill_is_bit_identical(request, precision, total, chunks):
    """A prompt prefilled in chunks leaves the same KV and last rows, bit for bit, as the
    whole prompt prefilled in one call: a row's result does not depend on the GEMM kernel or
    tile shape that computes it, nor on the attention block it shares."""
    ctx, _ = _ctx_and_oracle(request, precision)
    ids = S.token_ids(S.SEEDS["prefill_512"], total, SH.text_vocab)
    layers = (0, SH.n_layers // 2, SH.n_layers - 1)
    ctx.reset(0)
    ctx.prefill(ids)
    cold_rows = ctx.tap_prefill_hidden(total).copy()
    cold_kv = [ctx.tap_kv(l, total) for l in layers]
    ctx.reset(0)
    c0 = 0
    for n in chunks:
        ctx.prefill(ids[c0:c0 + n])
        c0 += n
        assert np.array_equal(ctx.tap_prefill_hidden(n), cold_rows[c0 - n:c0]), f"rows {c0 - n}..{c0} differ"
    assert c0 == total
    for l, (kc, vc) in zip(layers, cold_kv):
        k, v = ctx.tap_kv(l, total)
        assert np.array_equal(k, kc) and np.array_equal(v, vc), f"layer {l}: KV differs"
    _say(f"[full] {precision} prefill in chunks {'/'.join(map(str, chunks))}: bit-identical to one "
         f"{total}-row prefill")


# ----------------------------------------------------------------------------- prefix reuse
@pytest.mark.parametrize("precision", ["bf16", "fp8"])
def test_full_prefix_reuse(request, precision):
    ctx, oracle = _ctx_and_oracle(request, precision)
    pre = S.token_ids(S.SEEDS["preamble"], 64, SH.text_vocab)
    sufs = [S.token_ids(S.SEEDS["suffix_base"] + i, 16, SH.text_vocab) for i in range(8)]
    cold = []
    for s in sufs:
        ctx.reset(0)
        ctx.prefill(np.concatenate([pre, s]))
        codes, _ = ctx.decode_frames(3)
        cold.append((codes, ctx.tap_hidden().copy(), ctx.tap_kv(SH.n_layers - 1, 83)))
    ctx.reset(0)
    ctx.prefill(pre)
    for i, s in enumerate(sufs):
        ctx.reset(64)
        ctx.prefill(s)
        codes, _ = ctx.decode_frames(3)
        assert np.array_equal(codes, cold[i][0]), f"suffix {i}: codes differ"
        assert np.array_equal(ctx.tap_hidden(), cold[i][1]), f"suffix {i}: hidden state differs"
        kv = ctx.tap_kv(SH.n_layers - 1, 83)
        assert np.array_equal(kv[0], cold[i][2][0]) and np.array_equal(kv[1], cold[i][2][1]), f"suffix {i}: KV"
    # the frames after a reused prefix, re-anchored layer by layer
    ctx.set_option(hta.OPT_TAPS, 1)
    try:
        ctx.reset(64)
        ctx.prefill(sufs[-1])
        _reanchored_frames(ctx, oracle, precision, 1, f"{precision} after prefix reuse")
    finally:
        ctx.set_option(hta.OPT_TAPS, 0)
    _say(f"[full] {precision} prefix reuse: 8 suffixes bit-identical to cold 80-token prefills")


# ----------------------------------------------------------------------------- FP8 decode at KV 4096
def test_full_fp8_decode_kv4096(request, gpu_fp8, oracle_s8, oracle_e):
    ids = S.token_ids(S.SEEDS["long_prompt"], MAX_SEQ - 1, SH.text_vocab)
    ctx = gpu_fp8
    ctx.reset(0)
    for c0 in range(0, len(ids), MAX_PREFILL):
        ctx.prefill(ids[c0:c0 + MAX_PREFILL])
    assert ctx.tap_state()["len"] == MAX_SEQ - 1
    ctx.set_option(hta.OPT_TAPS, 1)
    try:
        _reanchored_frames(ctx, oracle_s8, "fp8", 1, "fp8 frame at KV 4096")
    finally:
        ctx.set_option(hta.OPT_TAPS, 0)
    assert ctx.tap_state()["len"] == MAX_SEQ
    # the same frame end to end from the GPU's cache: the oracle runs all 36 layers itself, in
    # the FP8 storage-faithful mode and exactly; as for every 36-layer end-to-end comparison the
    # gate is the oracle's own FP8 run's distance to the exact model (one flipped e4m3 rounding
    # cascades through the remaining layers)
    # a second faithful FP8 oracle that differs only in accumulation precision (float64 instead
    # of float32 products): its distance from the first is the scale at which a handful of
    # rounding-boundary flips, cascading through 36 layers, moves the end result
    twin = OracleModel(SH, request.getfixturevalue("w"), "fp8", "S", act_scales=oracle_s8.scales,
                       storage=np.float64, max_seq=MAX_SEQ)
    for o in (oracle_s8, oracle_e, twin):
        o.reset(0)
        for layer in range(SH.n_layers):
            o.set_kv(layer, *_kv_rows(ctx, layer, MAX_SEQ - 1))
        o.decode_frame()
    n_s = rel_l2(twin.last_hidden, oracle_s8.last_hidden)
    del twin
    ctx.reset(MAX_SEQ - 1)
    ctx.decode_frame()
    d_s = rel_l2(ctx.tap_hidden(), oracle_s8.last_hidden)
    d_e = rel_l2(ctx.tap_hidden(), oracle_e.last_hidden)
    q_e = rel_l2(oracle_s8.last_hidden, oracle_e.last_hidden)
    cos_e = cosines(ctx.tap_logits(), oracle_e.last_logits).min()
    cos_q = cosines(oracle_s8.last_logits, oracle_e.last_logits).min()
    _say(f"[full] fp8 frame at KV 4096 end to end from the same cache: hidden rel vs fp8 oracle {d_s:.3e} (the float64 "
         f"fp8 oracle vs the float32 one {n_s:.3e}), vs exact {d_e:.3e} (fp8 oracle vs exact {q_e:.3e}); logits cos "
         f"vs exact {cos_e:.6f} (fp8 oracle {cos_q:.6f})")
    assert d_s <= max(HIDDEN_TOL["fp8"], 2.0 * n_s)
    assert d_e <= E2E_RATIO * q_e
    assert cos_e >= cos_q - 0.02
    # a full cache refuses another frame
    with pytest.raises(hta.HtaError):
        ctx.decode_frame()



# ----------------------------------------------------------------------------- whole utterances
@pytest.mark.parametrize("precision,frames", [("fp8", 1017), ("bf16", 256)])
def test_full_utterance_repeatable_and_last_frame_anchored(request, precision, frames):
    """The benchmark's utterances: a P = 13 prompt, then 1017 FP8 frames (KV 14 -> 1030) or 256
    BF16 frames (KV 14 -> 269), decoded twice from the same state in one graph-replayed run:
    the codes agree bit for bit (the persistent frame's exchange words repeat their 16-bit
    tags over a long run, and a stale word would show here).  The last frame is then decoded
    again with the taps on and checked site by site at its full KV length."""
    ctx, oracle = _ctx_and_oracle(request, precision)
    prompt = S.token_ids(S.SEEDS["full_prompt"], 13, SH.text_vocab)
    runs = []
    for _ in range(2):
        ctx.reset(0)
        ctx.prefill(prompt)
        codes, _ = ctx.decode_frames(frames)
        runs.append((codes, ctx.tap_hidden().copy()))
    assert np.array_equal(runs[0][0], runs[1][0]), f"{precision}: codes of two identical utterances differ"
    assert np.array_equal(runs[0][1], runs[1][1])
    ctx.reset(0)
    ctx.prefill(prompt)
    ctx.decode_frames(frames - 1)
    ctx.set_option(hta.OPT_TAPS, 1)
    try:
        _reanchored_frames(ctx, oracle, precision, 1, f"{precision} frame {frames} at KV {13 + frames}")
    finally:
        ctx.set_option(hta.OPT_TAPS, 0)
    st = ctx.tap_state()
    assert st["len"] == 13 + frames and st["t"] == frames
    _say(f"[full] {precision} utterance of {frames} frames: two runs bit-identical")
