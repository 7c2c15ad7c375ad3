"""Shared helpers of the GPU parity tests: build a device context from seeded
weights, run the CPU oracle and the GPU side by side under teacher forcing,
and compare with the tolerances of the decode path:

* final hidden state (residual after the last layer) relative L2 against the
  exact oracle: <= 2e-2 (BF16), <= 6e-2 (FP8);
* per-codebook logits cosine against the exact oracle >= 0.999;
* greedy ids equal to the oracle's wherever the oracle's top-2 margin over
  the allowed ids exceeds 1e-2;
* everything integer (delay bookkeeping, KV slots, states) exact.
"""
from __future__ import annotations

import numpy as np

import synthetic as S
from autoregressive_codebook_tts_amd import hta
from oracle import numerics as nx
from oracle import sampling as smp
from oracle.delay import DelayState
from oracle.model import OracleModel

HIDDEN_TOL = {"bf16": 2e-2, "fp8": 6e-2}
COS_MIN = 0.999
MARGIN = 1e-2


def gpu_context(shape, weights, precision="bf16", max_seq=256, max_prefill=128, act_scales=None, fill_byte=None,
                n_streams=1):
    ctx = hta.Hta(shape, precision, max_seq=max_seq, max_prefill=max_prefill, fill_byte=fill_byte, n_streams=n_streams)
    tensors, src = hta.weights_to_device(weights, shape.n_layers)
    ctx.load_weights(tensors, src, act_scales=act_scales)
    del tensors
    return ctx


def rel_l2(a, b) -> float:
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    return float(np.linalg.norm(a - b) / np.linalg.norm(b))


def cosines(a, b) -> np.ndarray:
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    return np.sum(a * b, axis=1) / (np.linalg.norm(a, axis=1) * np.linalg.norm(b, axis=1))


def top2_margin(logits_row, allowed) -> float:
    v = np.sort(np.asarray(logits_row, np.float64)[allowed])
    return float(v[-1] - v[-2])


def allowed_mask(shape, k) -> np.ndarray:
    m = np.zeros(shape.codebook_size, dtype=bool)
    m[: shape.bos_id] = True
    if k == 0:
        m[shape.eos_id] = True
    return m


def teacher_forced_run(shape, weights, prompt, n_frames, precision, act_scales=None, oracle_modes=("E",),
                       ctx=None, storage=np.float64, max_seq=256):
    """Free-run the oracle (mode of oracle_modes[0] drives the codes), force its codes into the
    GPU context and the other oracle modes; return per-frame records."""
    oracles = {m: OracleModel(shape, weights, precision, m, act_scales=act_scales if m == "S" else None,
                              storage=storage, max_seq=max_seq) for m in oracle_modes}
    for o in oracles.values():
        o.prefill(prompt)
    own = ctx is None
    if own:
        ctx = gpu_context(shape, weights, precision, max_seq=max_seq, max_prefill=max(len(prompt), 16),
                          act_scales=act_scales)
    ctx.prefill(prompt)
    recs = []
    driver = oracles[oracle_modes[0]]
    for f in range(n_frames):
        rec = {"t": f}
        for m, o in oracles.items():
            codes, done = o.decode_frame()
            rec[m] = {"codes": codes, "done": done, "hidden": o.last_hidden.copy(), "logits": o.last_logits.copy()}
        gcodes, gdone = ctx.decode_frame()
        rec["gpu"] = {"codes": gcodes, "done": gdone, "hidden": ctx.tap_hidden().astype(np.float64),
                      "logits": ctx.tap_logits().astype(np.float64)}
        forced = rec[oracle_modes[0]]["codes"]
        for o in oracles.values():
            o.force_codes(forced)
        ctx.force_codes(forced)
        recs.append(rec)
    if own:
        ctx.close()
    return recs, driver


def id_agreement(shape, recs, ref_mode):
    """(n_compared, mismatches) over argmax decisions whose oracle margin exceeds MARGIN."""
    n, bad = 0, []
    for rec in recs:
        t = rec["t"]
        lg = rec[ref_mode]["logits"]
        for k in range(shape.n_codebooks):
            if t < k:
                continue  # BOS forced
            ref_c = int(rec[ref_mode]["codes"][k])
            if ref_c == shape.eos_id and k > 0:
                continue  # EOS forced after EOC
            mask = allowed_mask(shape, k)
            if top2_margin(lg[k], mask) > MARGIN:
                n += 1
                if int(rec["gpu"]["codes"][k]) != ref_c:
                    bad.append((t, k, ref_c, int(rec["gpu"]["codes"][k])))
    return n, bad


def tiny_weights():
    return S.make_weights(S.TINY, S.SEEDS["tiny_weights"], "f32")


# ----------------------------------------------------------------------------- site-anchored checks
# A rounding decision may differ between the GPU (fp32 arithmetic) and the oracle (float64,
# or float32 BLAS products for the 36-layer weights) only where the value being rounded lies
# within the two sides' arithmetic difference of a rounding boundary (the midpoint of two
# neighbouring grid values).  That difference has a relative part and, where the value is a
# sum of many terms that cancel (a dot product over the hidden width, a P.V sum), an absolute
# part of the order of the accumulated terms, i.e. of the vector's RMS.  A flip is accepted
# when its distance from the boundary is within either band:
#  * norm inputs (attention input, MLP input, head input): a sum of squares over the row,
#    rsqrt, two products and (FP8) one division: relative 2^-16, absolute 2^-18 RMS;
#  * SiLU*mul output: the product of two fp32 dot products over the hidden width:
#    relative 2^-14, absolute 2^-12 RMS;
#  * attention output, computed by the oracle from the GPU's own rounded q, k and v: fp32
#    scores, softmax and P.V over the keys: relative 2^-14, absolute 2^-14 RMS.
#  * q, k and v rows: q/k-norm and RoPE (q, k) after an fp32 dot product (all three):
#    relative 2^-12, absolute 2^-12 RMS.
# The fraction of a vector's decisions that may flip is capped: 0.2 % at every GEMV input,
# 0.5 % in a q/k/v row.
SITE_BANDS = ((2.0 ** -16, 2.0 ** -18), (2.0 ** -14, 2.0 ** -14), (2.0 ** -16, 2.0 ** -18), (2.0 ** -14, 2.0 ** -12))
HEAD_BAND = (2.0 ** -16, 2.0 ** -18)
KV_BAND = (2.0 ** -12, 2.0 ** -12)
SITE_FLIP_FRAC = (2e-3, 2e-3, 2e-3, 2e-3)
KV_FLIP_FRAC = 5e-3
FLIP_LOG = []  # (what, site, flips, worst relative distance, worst distance in RMS units) of every check


def bf16_values(bits) -> np.ndarray:
    """float64 values of bf16 bit patterns (uint16)."""
    return (np.asarray(bits, np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def rounding_flips(gpu_vals, oracle_vals, x):
    """Positions where the GPU's rounded values differ from the oracle's rounding of the same
    pre-rounding values x (in the rounding's own units), and each one's distance from the
    midpoint of the two values, relative to |x| and in units of the RMS of x: a flip at a
    true boundary has distance ~0, a wrong value is at least half a grid step away."""
    g = np.asarray(gpu_vals, np.float64)
    o = np.asarray(oracle_vals, np.float64)
    x = np.asarray(x, np.float64)
    idx = np.flatnonzero(g != o)
    gap = np.abs(x[idx] - 0.5 * (g[idx] + o[idx]))
    rms = float(np.sqrt(np.mean(x * x))) or 1e-30
    return idx, gap / np.maximum(np.abs(x[idx]), 1e-30), gap / rms


def check_site(oracle, site, gpu_vals, pre, band, what, max_frac=2e-3):
    """GPU rounded GEMV input vs the oracle's rounding of its own pre-rounding values at
    `site`; returns (flips, worst relative distance).  The rounding is compared in the units
    it is taken in: bf16 values, or fp32(x) / scale for e4m3 codes.  `band` = (relative,
    absolute in RMS units): every flip must lie within one of the two."""
    ref = oracle.round_site(pre, site)
    if oracle.precision == "fp8":
        x = np.asarray(pre, np.float64).astype(np.float32) / np.float32(oracle.scales[site])
    else:
        x = np.asarray(pre, np.float64)
    idx, d_rel, d_rms = rounding_flips(gpu_vals, ref, x)
    ok = (d_rel <= band[0]) | (d_rms <= band[1])
    worst_rel = float(d_rel.max()) if idx.size else 0.0
    worst_rms = float(np.minimum(d_rms, d_rel * 1e9).max()) if idx.size else 0.0
    FLIP_LOG.append((what, site, int(idx.size), worst_rel, worst_rms))
    if not np.all(ok):
        bad = idx[~ok][:4]
        vals = [(int(i), float(x[i]), float(np.asarray(gpu_vals)[i]), float(ref[i])) for i in bad]
        raise AssertionError(f"{what} site {site}: {idx.size} flips, {int((~ok).sum())} outside the bands "
                             f"(rel {band[0]:.1e} / rms {band[1]:.1e}): (index, x, gpu, oracle) {vals}; "
                             f"worst rel {worst_rel:.2e}, worst rms {float(d_rms.max()):.2e}")
    assert idx.size <= max_frac * len(ref) + 1, f"{what} site {site}: {idx.size} flips of {len(ref)}"
    return idx.size, worst_rel


def check_kv_row(gpu_bits, pre, what):
    """The K or V row the GPU stored (bf16 bits) against the oracle's bf16 rounding of its own
    pre-rounding row `pre` for the same inputs: flips only within KV_BAND of a boundary;
    returns the flip count."""
    g = bf16_values(gpu_bits).ravel()
    x = np.asarray(pre, np.float64).ravel()
    o = nx.round_bf16(x)
    idx, d_rel, d_rms = rounding_flips(g, o, x)
    ok = (d_rel <= KV_BAND[0]) | (d_rms <= KV_BAND[1])
    assert np.all(ok), (f"{what}: {int((~ok).sum())} of {idx.size} flips outside the bands; worst rel "
                        f"{float(d_rel.max()):.2e}, worst rms {float(d_rms.max()):.2e}")
    assert idx.size <= KV_FLIP_FRAC * g.size + 1, f"{what}: {idx.size} K/V flips of {g.size}"
    return idx.size


def kv_rows(ctx, layer, n):
    """GPU K, V of positions [0, n) as oracle values [n][Hkv][hd]."""
    k, v = ctx.tap_kv(layer, max(n, 1))
    return (nx.bf16_bits_to_float(k[:, :n]).transpose(1, 0, 2), nx.bf16_bits_to_float(v[:, :n]).transpose(1, 0, 2))


def check_layer_sites(ctx, oracle, layer, h_in, h_out, acts, q_tap, pos, what):
    """Layer `layer` of the last decode frame, rounding point by rounding point: the oracle
    recomputes the layer from the GPU's input residual h_in and KV cache before `pos`, every
    GEMV fed the GPU's own rounded input (the TAP_ACT rows `acts`) and the attention fed the
    GPU's own rounded q, k and v (TAP_Q rows `q_tap` and the cache row at `pos`).  Each GEMV
    input and each q/k/v row must equal the oracle's rounding of the same values up to
    counted boundary flips, and the layer output h_out must match the oracle's output from
    those inputs to fp32 accumulation.  Returns (flips per site [4], q/k/v flips, output rel)."""
    sh = oracle.shape
    kp, vp = kv_rows(ctx, layer, pos)
    oracle.set_kv(layer, kp, vp)
    widths = (sh.hidden, sh.q_dim, sh.hidden, sh.ffn)
    phases = (5 * layer, 5 * layer + 2, 5 * layer + 3, 5 * layer + 4)
    gv = [bf16_values(acts[p][:n]) for p, n in zip(phases, widths)]
    kg, vg = ctx.tap_kv(layer, pos + 1)
    q_gpu = bf16_values(q_tap[layer])
    k_gpu, v_gpu = bf16_values(kg[:, pos]), bf16_values(vg[:, pos])
    pre, _, _, h_o, (q_pre, k_pre, v_pre) = oracle.layer_anchored(layer, h_in, gv, qkv=(q_gpu, k_gpu, v_gpu))
    s0 = 4 * layer
    flips = [check_site(oracle, s0 + i, gv[i], pre[i], SITE_BANDS[i], f"{what} layer {layer}",
                        max_frac=SITE_FLIP_FRAC[i])[0] for i in range(4)]
    qkv_flips = (check_kv_row(q_tap[layer], q_pre, f"{what} layer {layer} q") +
                 check_kv_row(kg[:, pos], k_pre, f"{what} layer {layer} k") +
                 check_kv_row(vg[:, pos], v_pre, f"{what} layer {layer} v"))
    upd = rel_l2(h_out - h_in, h_o - h_in)
    assert upd <= 1e-5, f"{what} layer {layer}: output from the GPU's own site values off by {upd:.3e}"
    return flips, qkv_flips, upd


# ----------------------------------------------------------------------------- sampling head
# The kernel's fp32 error relative to the total weight: a lane's sequential sum of at most
# 17 weights, six scan additions, the exponentials and the product u * total, each within
# 2^-24 relative.  A draw whose target lies within this of a cumulative boundary may fall
# on either side of it.
SAMPLE_BAND = 2e-6


def sample_neighbours(z, allowed, T, u):
    """Ids on both sides of the cumulative boundary nearest to u * total."""
    wts = smp.weights(z, allowed, T)
    c = np.cumsum(wts)
    target = u * c[-1]
    pos = np.nonzero(wts > 0)[0]
    j = int(np.argmin(np.abs(c[pos[:-1]] - target)))
    return {int(pos[j]), int(pos[j + 1])}


def sampled_run(ctx, SH, n, T, seed):
    """Decode n frames one at a time; check every draw against the oracle on the GPU's logits."""
    st = DelayState(SH.n_codebooks, SH.codebook_size, SH.bos_id, SH.eos_id)
    codes_all, n_band, n_draws = [], 0, 0
    for f in range(n):
        st.begin_frame()
        codes, _ = ctx.decode_frame()
        z = ctx.tap_logits().reshape(SH.n_codebooks, SH.codebook_size).astype(np.float64)
        want, margins = smp.choose_sampled(st, z, T, seed)
        for k in range(SH.n_codebooks):
            if np.isinf(margins[k]):  # forced by the delay rule (or no finite logit)
                assert codes[k] == want[k], (f, k, codes[k], want[k])
                continue
            n_draws += 1
            if margins[k] > SAMPLE_BAND:
                assert codes[k] == want[k], (f, k, int(codes[k]), int(want[k]), float(margins[k]))
            else:
                n_band += 1
                u = float(smp.uniform(seed, st.t, k))
                assert int(codes[k]) in sample_neighbours(z[k], st.allowed_mask(k), T, u), (f, k)
        st.finish(codes)
        codes_all.append(codes.copy())
    return np.array(codes_all), n_draws, n_band


