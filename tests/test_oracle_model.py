"""Pins of the oracle's model, delay bookkeeping and calibration (CPU only).

The model is checked against an independent formulation written with torch's
library routines (F.linear, F.rms_norm, complex-multiply RoPE,
scaled_dot_product_attention with GQA, F.silu), against the causal-mask
equivalence of batched prefill and step-by-step decoding, and against MHA with
repeated K/V.  The delay bookkeeping is enumerated by brute force against the
frame-view of the pattern."""
import dataclasses

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import synthetic as S
from oracle import numerics as nx
from oracle.delay import DelayState, delay_frames, find_eoc, undelay
from oracle.model import OracleModel, calibrate

TINY = S.TINY


@pytest.fixture(scope="module")
def tiny_weights():
    return S.make_weights(TINY, S.SEEDS["tiny_weights"], "f32")


# ----------------------------------------------------------------------------- independent torch formulation
SITES = 4  # per layer: attention input, attention output, MLP input, down input; then the head input


class TorchStorage:
    """Rounding at the storage points of one precision, written with torch's own casts.

    ``None``: no rounding (the exact model).  ``"bf16"``: weights, embeddings, the five
    GEMV inputs and q/k/v through ``torch.bfloat16``.  ``"fp8"``: projection and head
    weights through ``torch.float8_e4m3fn`` with per-row float32 scales amax/448, and
    the five GEMV inputs as float8_e4m3fn codes of fp32(x) / s (clamped to +-448, the
    saturating reading of FlashRT section 8), dequantised before the product; embeddings
    bf16; q/k/v bf16 in both.  ``record`` (a float64 array) receives max |x| of every
    GEMV input before rounding."""

    def __init__(self, kind=None, scales=None, record=None):
        self.kind, self.record = kind, record
        self.scales = None if scales is None else torch.from_numpy(np.asarray(scales, np.float32))

    @staticmethod
    def bf16(t):
        """float64 -> bfloat16 with one correct rounding.  torch converts float64 to bfloat16
        through float32, and that double rounding lands on a bf16 tie for about one value in
        2^16.  Rounding to odd at the float32 step (truncate, then set the last bit when
        inexact; Boldo and Melquiond, IEEE Trans. Computers 57(4), 2008) makes the second
        rounding (torch's RNE float32 -> bfloat16) the correctly rounded result."""
        f = t.to(torch.float32)
        f = torch.where(f.to(torch.float64).abs() > t.abs(), torch.nextafter(f, torch.zeros_like(f)), f)
        inexact = (f.to(torch.float64) != t).to(torch.int32)
        f = (f.view(torch.int32) | inexact).view(torch.float32)
        return f.to(torch.bfloat16).to(torch.float64)

    def embedding(self, t):
        return t if self.kind is None else self.bf16(t)

    def weight(self, t):
        if self.kind is None:
            return t
        if self.kind == "bf16":
            return self.bf16(t)
        w32 = t.to(torch.float32)
        amax = w32.abs().amax(dim=-1)
        s = torch.where(amax > 0, amax / 448.0, torch.ones_like(amax))
        codes = (w32 / s[:, None]).to(torch.float8_e4m3fn)
        return codes.to(torch.float64) * s.to(torch.float64)[:, None]

    def act(self, t, site):
        if self.record is not None:
            self.record[site] = max(self.record[site], float(t.abs().max()))
        if self.kind is None:
            return t
        if self.kind == "bf16":
            return self.bf16(t)
        s = self.scales[site]
        codes = (t.to(torch.float32) / s).clamp(-448.0, 448.0).to(torch.float8_e4m3fn)
        return codes.to(torch.float64) * s.to(torch.float64)

    def kv(self, t):
        return t if self.kind is None else self.bf16(t)


def torch_forward(shape, w, ids_frames, store=None):
    """Causal forward over an input sequence given as a list of ("text", id) / ("audio", codes[8]);
    ``store`` (a TorchStorage) rounds at the storage points.  Returns the final residual of every
    row and the head's logits of every row."""
    store = store or TorchStorage()
    d, hd, Hq, Hkv = shape.hidden, shape.head_dim, shape.n_q_heads, shape.n_kv_heads
    T = lambda a: torch.from_numpy(np.asarray(a, dtype=np.float64))
    e_text, e_aud = store.embedding(T(w["e_text"])), store.embedding(T(w["e_aud"]))
    rows = []
    for kind, val in ids_frames:
        if kind == "text":
            rows.append(e_text[val])
        else:
            rows.append(sum(e_aud[k, int(c)] for k, c in enumerate(val)))
    x = torch.stack(rows)  # [N, d]
    N = x.shape[0]
    pos = torch.arange(N, dtype=torch.float64)
    inv = shape.rope_theta ** (-torch.arange(hd // 2, dtype=torch.float64) * 2.0 / hd)
    rot = torch.polar(torch.ones(N, hd // 2, dtype=torch.float64), pos[:, None] * inv[None, :])

    def rope(t):  # t [N, H, hd]
        z = torch.complex(t[..., : hd // 2], t[..., hd // 2:]) * rot[:, None, :]
        return torch.cat([z.real, z.imag], dim=-1)

    for layer in range(shape.n_layers):
        p = f"layers.{layer}."
        G = lambda n: T(w[p + n])
        Wt = lambda n: store.weight(T(w[p + n]))
        s0 = SITES * layer
        u = store.act(F.rms_norm(x, (d,), G("g_attn"), eps=shape.rms_eps), s0)
        q = F.linear(u, Wt("wq")).view(N, Hq, hd)
        k = F.linear(u, Wt("wk")).view(N, Hkv, hd)
        v = store.kv(F.linear(u, Wt("wv")).view(N, Hkv, hd))
        q = store.kv(rope(F.rms_norm(q, (hd,), G("g_q"), eps=shape.rms_eps)))
        k = store.kv(rope(F.rms_norm(k, (hd,), G("g_k"), eps=shape.rms_eps)))
        o = F.scaled_dot_product_attention(q.transpose(0, 1)[None], k.transpose(0, 1)[None], v.transpose(0, 1)[None],
                                           is_causal=True, enable_gqa=True)[0].transpose(0, 1).reshape(N, Hq * hd)
        x = x + F.linear(store.act(o, s0 + 1), Wt("wo"))
        u2 = store.act(F.rms_norm(x, (d,), G("g_mlp"), eps=shape.rms_eps), s0 + 2)
        a = store.act(F.silu(F.linear(u2, Wt("wg"))) * F.linear(u2, Wt("wu")), s0 + 3)
        x = x + F.linear(a, Wt("wd"))
    return x.numpy(), x


def torch_head(shape, w, x_rows, store=None):
    """Logits [rows][C][V] of the fused head for final residual rows (torch tensor)."""
    store = store or TorchStorage()
    T = lambda a: torch.from_numpy(np.asarray(a, dtype=np.float64))
    z = store.act(F.rms_norm(x_rows, (shape.hidden,), T(w["g_final"]), eps=shape.rms_eps), SITES * shape.n_layers)
    return F.linear(z, store.weight(T(w["w_head"]))).view(-1, shape.n_codebooks, shape.codebook_size).numpy()


def test_oracle_matches_torch_formulation(tiny_weights):
    w = tiny_weights
    ids = S.token_ids(S.SEEDS["tiny_prompt"], 8, TINY.text_vocab)
    m = OracleModel(TINY, w, "bf16", "E", max_seq=64)
    m.prefill(ids)
    seq = [("text", int(i)) for i in ids]
    hid, logit_list, codes_list = [], [], []
    forced = S.code_frames(77, 6)
    for f in range(6):
        codes, _ = m.decode_frame()
        hid.append(m.last_hidden.copy())
        logit_list.append(m.last_logits.copy())
        seq.append(("audio", np.full(8, 1024) if f == 0 else forced[f - 1]))
        m.force_codes(forced[f])
    x_ref, xt = torch_forward(TINY, w, seq)
    lg_ref = torch_head(TINY, w, xt)
    P = len(ids)
    for f in range(6):
        assert np.allclose(hid[f], x_ref[P + f], rtol=1e-10, atol=1e-13)
        assert np.allclose(logit_list[f], lg_ref[P + f], rtol=1e-10, atol=1e-12)


@pytest.mark.parametrize("precision", ["bf16", "fp8"])
def test_mode_s_matches_torch_storage_formulation(tiny_weights, precision):
    """Mode S rounds exactly at the storage points: the same teacher-forced run through the
    torch formulation that casts with torch.bfloat16 / torch.float8_e4m3fn at the five GEMV
    inputs, q/k/v and the weights (FP8: dequantised weights and activations, where the
    oracle scales the code products) agrees to 1e-10.  A rounding moved to another point, a
    dropped rounding or an activation scale taken from the wrong site moves the result by
    far more (at least one bf16 / e4m3 rounding step of some element)."""
    w = tiny_weights
    calib_ids = S.token_ids(S.SEEDS["calib_prompt"], 16, TINY.text_vocab)
    scales = calibrate(TINY, w, calib_ids, 8)[0] if precision == "fp8" else None
    ids = S.token_ids(S.SEEDS["tiny_prompt"], 8, TINY.text_vocab)
    m = OracleModel(TINY, w, precision, "S", act_scales=scales, max_seq=64)
    m.prefill(ids)
    seq = [("text", int(i)) for i in ids]
    forced = S.code_frames(78, 6)
    hid, lgs = [], []
    for f in range(6):
        m.decode_frame()
        hid.append(m.last_hidden.copy())
        lgs.append(m.last_logits.copy())
        seq.append(("audio", np.full(8, 1024) if f == 0 else forced[f - 1]))
        m.force_codes(forced[f])
    store = TorchStorage(precision, scales)
    x_ref, xt = torch_forward(TINY, w, seq, store)
    lg_ref = torch_head(TINY, w, xt[len(ids):], store)
    P = len(ids)
    for f in range(6):
        assert np.max(np.abs(hid[f] - x_ref[P + f])) <= 1e-10 * np.max(np.abs(x_ref[P + f])), f
        assert np.max(np.abs(lgs[f] - lg_ref[f])) <= 1e-10 * np.max(np.abs(lg_ref[f])), f
    # the formulation is sharp: without the storage rounding it lands far away
    x_e, _ = torch_forward(TINY, w, seq)
    assert np.max(np.abs(x_e[P:] - x_ref[P:])) > 1e-4 * np.max(np.abs(x_ref[P:]))


def test_calibration_records_each_site_before_rounding(tiny_weights):
    """calibrate() records max |x| of every GEMV input before its bf16 rounding, over every
    prefill row and every decode frame (the head input over the frames only, as a prefill
    evaluates no head), at the site index the activation-scale table uses.  The torch
    formulation records the same maxima on the same rows independently; both agree to
    1e-12 and give bit-identical float32 scales."""
    w = tiny_weights
    calib_ids = S.token_ids(S.SEEDS["calib_prompt"], 16, TINY.text_vocab)
    n = 8
    scales, amax, codes = calibrate(TINY, w, calib_ids, n)
    seq = [("text", int(i)) for i in calib_ids]
    seq += [("audio", np.full(8, 1024) if f == 0 else codes[f - 1]) for f in range(n)]
    rec = np.zeros(SITES * TINY.n_layers + 1)
    store = TorchStorage("bf16", record=rec)
    _, xt = torch_forward(TINY, w, seq, store)
    torch_head(TINY, w, xt[len(calib_ids):], store)
    assert np.all(rec > 0)
    assert np.allclose(amax, rec, rtol=1e-12, atol=0.0), np.abs(amax / rec - 1).max()
    assert np.array_equal(scales, np.array([nx.act_scale(a) for a in rec], np.float32))
    # the sites are distinct enough that a permuted table would not pass
    assert len(np.unique(np.round(rec, 6))) == len(rec)


def test_prefill_equals_step_by_step(tiny_weights):
    ids = S.token_ids(11, 12, TINY.text_vocab)
    a = OracleModel(TINY, tiny_weights, "bf16", "E", max_seq=32)
    a.prefill(ids)
    b = OracleModel(TINY, tiny_weights, "bf16", "E", max_seq=32)
    for i in ids:
        b.prefill([i])
    assert np.allclose(a.last_hidden[-1], b.last_hidden[-1], rtol=1e-10, atol=1e-14)
    assert np.allclose(a.k_cache[:, :12], b.k_cache[:, :12], rtol=1e-10, atol=1e-14)
    assert np.allclose(a.v_cache[:, :12], b.v_cache[:, :12], rtol=1e-10, atol=1e-14)
    ca, _ = a.decode_frame()
    cb, _ = b.decode_frame()
    assert np.array_equal(ca, cb)
    assert np.allclose(a.last_logits, b.last_logits, rtol=1e-10, atol=1e-13)


def test_gqa_equals_mha_with_repeated_kv(tiny_weights):
    w = dict(tiny_weights)
    group = TINY.n_q_heads // TINY.n_kv_heads
    hd = TINY.head_dim
    mha_shape = dataclasses.replace(TINY, n_kv_heads=TINY.n_q_heads)
    for layer in range(TINY.n_layers):
        for n in ("wk", "wv"):
            key = f"layers.{layer}.{n}"
            heads = w[key].reshape(TINY.n_kv_heads, hd, -1)
            w[key] = np.repeat(heads, group, axis=0).reshape(TINY.n_q_heads * hd, -1)
    ids = S.token_ids(12, 9, TINY.text_vocab)
    a = OracleModel(TINY, tiny_weights, "bf16", "E", max_seq=32)
    b = OracleModel(mha_shape, w, "bf16", "E", max_seq=32)
    a.prefill(ids)
    b.prefill(ids)
    a.decode_frame()
    b.decode_frame()
    assert np.allclose(a.last_logits, b.last_logits, rtol=1e-11, atol=1e-13)


def test_prefix_reuse_equals_cold(tiny_weights):
    pre = S.token_ids(20, 10, TINY.text_vocab)
    suf = S.token_ids(21, 5, TINY.text_vocab)
    cold = OracleModel(TINY, tiny_weights, "bf16", "S", max_seq=64)
    cold.prefill(np.concatenate([pre, suf]))
    warm = OracleModel(TINY, tiny_weights, "bf16", "S", max_seq=64)
    warm.prefill(pre)
    warm.prefill(S.token_ids(22, 7, TINY.text_vocab))  # an earlier request
    for _ in range(3):
        warm.decode_frame()
    warm.reset(keep_len=10)
    warm.prefill(suf)
    for _ in range(4):
        ca, _ = cold.decode_frame()
        cw, _ = warm.decode_frame()
        assert np.array_equal(ca, cw)
        assert np.allclose(cold.last_logits, warm.last_logits, rtol=1e-10, atol=1e-13)


def test_mode_s_rounds_at_storage_points(tiny_weights):
    ids = S.token_ids(S.SEEDS["tiny_prompt"], 8, TINY.text_vocab)
    e = OracleModel(TINY, tiny_weights, "bf16", "E", max_seq=32)
    s = OracleModel(TINY, tiny_weights, "bf16", "S", max_seq=32)
    e.prefill(ids)
    s.prefill(ids)
    # KV is stored in bfloat16 in mode S, unrounded in mode E
    kv = s.k_cache[:, :8]
    assert np.array_equal(nx.round_bf16(kv), kv)
    assert not np.array_equal(nx.round_bf16(e.k_cache[:, :8]), e.k_cache[:, :8])
    e.decode_frame()
    s.decode_frame()
    rel = np.linalg.norm(s.last_hidden - e.last_hidden) / np.linalg.norm(e.last_hidden)
    assert 1e-5 < rel < 2e-2


def test_fp8_mode_close_to_exact(tiny_weights):
    calib_ids = S.token_ids(S.SEEDS["calib_prompt"], 16, TINY.text_vocab)
    scales, amax, _ = calibrate(TINY, tiny_weights, calib_ids, 16)
    # the calibrated maximum of each site quantises exactly to the largest code
    for site in range(len(scales)):
        assert nx.quantize_static(np.array([amax[site]]), scales[site])[0] == 448.0
    ids = S.token_ids(S.SEEDS["tiny_prompt"], 8, TINY.text_vocab)
    e = OracleModel(TINY, tiny_weights, "fp8", "E", max_seq=32)
    q = OracleModel(TINY, tiny_weights, "fp8", "S", act_scales=scales, max_seq=32)
    e.prefill(ids)
    q.prefill(ids)
    e.decode_frame()
    q.decode_frame()
    rel = np.linalg.norm(q.last_hidden - e.last_hidden) / np.linalg.norm(e.last_hidden)
    assert 1e-3 < rel < 0.15
    cos = np.sum(q.last_logits * e.last_logits, 1) / (np.linalg.norm(q.last_logits, axis=1) * np.linalg.norm(e.last_logits, axis=1))
    assert np.all(cos > 0.98)


def test_calibration_is_deterministic_and_order_free(tiny_weights):
    calib_ids = S.token_ids(S.SEEDS["calib_prompt"], 16, TINY.text_vocab)
    s1, _, c1 = calibrate(TINY, tiny_weights, calib_ids, 8)
    s2, _, c2 = calibrate(TINY, tiny_weights, calib_ids, 8)
    assert np.array_equal(s1, s2) and np.array_equal(c1, c2)
    # teacher-forced calibration with the free run's own codes reproduces the free run
    s3, _, _ = calibrate(TINY, tiny_weights, calib_ids, 8, forced_codes=c1)
    assert np.array_equal(s1, s3)


# ----------------------------------------------------------------------------- delay pattern
def _logits_for(step_choice, C=8, V=1026, rng=None):
    lg = rng.standard_normal((C, V)) * 0.1
    for k, c in enumerate(step_choice):
        lg[k, c] = 10.0
    return lg


@pytest.mark.parametrize("T", [12, 24])
def test_delay_bruteforce_every_eoc_step(T):
    """For every EOC step e, drive the state machine with logits whose argmax is a chosen
    frame code, and compare with the frame view of the pattern (frame f, codebook k at step f+k)."""
    rng = np.random.default_rng(T)
    C = 8
    for e in range(T):
        frames = rng.integers(0, 1024, size=(e, C))
        expect = delay_frames(frames)  # e + C steps through codebook 7's EOS
        st = DelayState()
        got, dones = [], []
        for t in range(min(T, e + C) if e + C <= T else T):
            want = np.array([frames[t - k, k] if 0 <= t - k < e else (1025 if k == 0 else 0) for k in range(C)])
            st.begin_frame()
            codes = st.choose(_logits_for(want, rng=rng))
            dones.append(st.finish(codes))
            got.append(codes)
        got = np.array(got)
        n = got.shape[0]
        assert np.array_equal(got, expect[:n]), e
        if e + C <= T:
            assert dones[-1] and not any(dones[:-1])
            assert find_eoc(got) == e
            assert np.array_equal(undelay(got, e), frames)


def test_delay_after_done_is_all_eos():
    st = DelayState()
    rng = np.random.default_rng(5)
    for t in range(20):
        st.begin_frame()
        want = np.full(8, 3)
        want[0] = 1025 if t == 2 else 3
        codes = st.choose(_logits_for(want, rng=rng))
        done = st.finish(codes)
        if t >= 9:
            assert done and np.all(codes == 1025)


def test_argmax_ties_and_masks():
    st = DelayState()
    st.t = 8
    lg = np.zeros((8, 1026))
    lg[:, 1024] = 5.0  # BOS never chosen by argmax
    lg[1:, 1025] = 5.0  # EOS only for codebook 0
    lg[0, 1025] = 5.0
    lg[:, 7] = 1.0
    lg[:, 3] = 1.0  # tie between 3 and 7: lowest id wins
    codes = st.choose(lg)
    assert codes[0] == 1025 and np.all(codes[1:] == 3)


def test_teacher_forcing_drives_eoc():
    st = DelayState()
    rng = np.random.default_rng(6)
    for t in range(4):
        st.begin_frame()
        st.finish(st.choose(_logits_for(np.full(8, 5), rng=rng)))
    st.prev = np.array([1025, 1, 2, 3, 4, 5, 6, 7])  # forced: codebook 0 at step 3 was EOS
    st.begin_frame()
    assert st.eoc == 3
    codes = st.choose(_logits_for(np.full(8, 5), rng=rng))
    assert codes[0] == 1025 and codes[1] == 1025 and codes[2] == 5


def test_undelay_inverts_delay():
    rng = np.random.default_rng(7)
    for n in (0, 1, 5, 40):
        frames = rng.integers(0, 1024, size=(n, 8))
        steps = delay_frames(frames)
        assert np.array_equal(undelay(steps, find_eoc(steps)), frames)
        # without EOC (a capped run), T - 7 frames come back
        assert np.array_equal(undelay(steps[: n + 7][:, :], None)[:n], frames)


def test_forced_eos_weight_set_stops_at_step_zero(tiny_weights):
    w = dict(tiny_weights)
    head = w["w_head"].copy()
    head[1025] *= 100.0  # EOS row of codebook 0
    w["w_head"] = head
    m = OracleModel(TINY, w, "bf16", "E", max_seq=64)
    m.prefill(S.token_ids(3, 4, TINY.text_vocab))
    # the EOS logit of codebook 0 must dominate for the test to mean anything
    codes, done = m.decode_frame()
    assert codes[0] == 1025 and np.all(codes[1:] == 1024) and not done
    for t in range(1, 8):
        codes, done = m.decode_frame()
        assert np.all(codes[: t + 1] == 1025) and np.all(codes[t + 1:] == 1024)
        assert done == (t == 7)


@pytest.mark.parametrize("precision", ["bf16", "fp8"])
def test_layer_anchored_equals_layer_on_own_site_values(tiny_weights, precision):
    """Fed the oracle's own rounded GEMV inputs, the site-anchored step reproduces the plain
    layer: the same pre-rounding values at the four sites, the same K/V row and the same
    output; fed values moved by one rounding step at one site, its output moves."""
    w = tiny_weights
    calib_ids = S.token_ids(S.SEEDS["calib_prompt"], 16, TINY.text_vocab)
    scales = calibrate(TINY, w, calib_ids, 4)[0] if precision == "fp8" else None
    ids = S.token_ids(S.SEEDS["tiny_prompt"], 8, TINY.text_vocab)
    a = OracleModel(TINY, w, precision, "S", act_scales=scales, max_seq=32)
    b = OracleModel(TINY, w, precision, "S", act_scales=scales, max_seq=32)
    a.prefill(ids)
    b.prefill(ids)
    h = a.frame_input()
    seen = {}
    orig = a._act

    def capture(x, site):
        seen[site] = (np.array(x, copy=True), orig(x, site))
        return seen[site][1]

    a._act = capture
    out_a = a.layer(0, h[None, :], np.array([a.length]))[0]
    vals = [seen[s][1][0] for s in range(4)]
    pre, k, v, out_b, (q_pre, k_pre, v_pre) = b.layer_anchored(0, h, vals)
    assert np.array_equal(nx.round_bf16(k_pre), k) and np.array_equal(nx.round_bf16(v_pre), v)
    # given the oracle's own rounded q, k, v explicitly, the step is the same
    b2 = OracleModel(TINY, w, precision, "S", act_scales=scales, max_seq=32)
    b2.prefill(ids)
    out_b2 = b2.layer_anchored(0, h, vals, qkv=(nx.round_bf16(q_pre), k, v))[3]
    assert np.array_equal(out_b2, out_b)
    for s in range(4):
        assert np.allclose(pre[s], seen[s][0][0], rtol=1e-12, atol=1e-14), s
        assert np.array_equal(b.round_site(pre[s], s), vals[s]), s
    assert np.array_equal(k, a.k_cache[0, 8]) and np.array_equal(v, a.v_cache[0, 8])
    assert np.allclose(out_b, out_a, rtol=1e-12, atol=1e-14)
    # one site value moved to its neighbour on the grid changes the output
    moved = [x.copy() for x in vals]
    moved[3][0] = vals[3][0] * (1 + 2.0 ** -6) if vals[3][0] != 0 else 2.0 ** -9
    c = OracleModel(TINY, w, precision, "S", act_scales=scales, max_seq=32)
    c.prefill(ids)
    out_c = c.layer_anchored(0, h, moved)[3]
    assert not np.allclose(out_c, out_a, rtol=1e-9, atol=0)
