"""Plain CPU forward pass of the codebook-TTS backbone: prefill, decode frame,
FP8 calibration.  Slow on purpose; every step is written out as the pages
describe it.

TEST INFRASTRUCTURE ONLY: nothing in the product path may import this package.

Sources (reference pages):
* FlashRT "Higgs Audio v3 TTS-4B" page, summary paragraph: dense Qwen3-4B
  backbone (36 layers, hidden 2560, GQA 32q/8kv, head_dim 128, SwiGLU, RoPE
  theta 1e6) plus a fused head of 8 codebooks x 1026.
* same page, section 5: the decode chain RMSNorm -> qkv -> q/k-norm + RoPE ->
  attention -> o_proj with residual -> RMSNorm -> gate/up -> SiLU*mul ->
  down with residual -> final RMSNorm -> fused 8-codebook head -> argmax with
  the delay mask -> embedding of the chosen codes as the next input.
* SGLang-Omni Higgs Audio v3 page, architecture paragraph: the next input is
  the sum of the embeddings of the 8 codes of the previous frame.
* FlashRT page, section 7: the prompt is prefilled in one batched pass that
  writes the KV cache; a shared preamble's KV can be kept and only a suffix
  prefilled.
* FlashRT page, section 8: FP8 W8A8 with per-tensor static activation scales
  amax/448 calibrated once from a short BF16 free run of a fixed prompt.

Two modes:
* ``mode="E"``: the exact model on the weights as stored; no activation rounding.
* ``mode="S"``: the same arithmetic, rounded only at the storage points of the
  given precision -- BF16: weights and embeddings in bfloat16, the five GEMV
  inputs (attention input, attention output, MLP input, SiLU*mul output, head
  input) rounded to bfloat16; FP8: projection and head weights as e4m3 codes
  with per-row scales, the five GEMV inputs quantised to e4m3 with the static
  scales; both: q, k, v (after q/k-norm and RoPE) rounded to bfloat16, which is
  also the KV-cache format.
Everything else is float64 (float32 storage for the 36-layer weights, whose
matrix products then run in float32 BLAS; see the design notes).
"""
from __future__ import annotations

import numpy as np

from . import numerics as nx
from .delay import DelayState

SITES_PER_LAYER = 4  # attention input, attention output, MLP input, down input


class OracleModel:
    def __init__(self, shape, weights: dict, precision: str = "bf16", mode: str = "E",
                 act_scales=None, storage=np.float64, max_seq: int = 4096, layers_only: bool = False):
        if precision not in ("bf16", "fp8"):
            raise ValueError(precision)
        if mode not in ("E", "S"):
            raise ValueError(mode)
        if mode == "S" and precision == "fp8" and act_scales is None:
            raise ValueError("FP8 storage-faithful mode needs activation scales")
        self.shape, self.precision, self.mode, self.storage = shape, precision, mode, storage
        self.scales = None if act_scales is None else np.asarray(act_scales, dtype=np.float32)
        self.max_seq = max_seq
        self.record = None
        sh = shape
        self.layers = []

        def build(layer):
            p = f"layers.{layer}."
            L = {"g_attn": self._plain(weights[p + "g_attn"]), "g_q": self._plain(weights[p + "g_q"]),
                 "g_k": self._plain(weights[p + "g_k"]), "g_mlp": self._plain(weights[p + "g_mlp"])}
            for name in ("wq", "wk", "wv", "wo", "wg", "wu", "wd"):
                L[name] = self._matrix(weights[p + name])
            return L

        # layers are independent: build them on a few threads (numpy releases the GIL)
        from concurrent.futures import ThreadPoolExecutor
        with ThreadPoolExecutor(max(1, min(8, sh.n_layers))) as ex:
            self.layers = list(ex.map(build, range(sh.n_layers)))
        if not layers_only:
            self.e_text = self._embedding(weights["e_text"])
            self.e_aud = self._embedding(weights["e_aud"])
            self.g_final = self._plain(weights["g_final"])
            self.w_head = self._matrix(weights["w_head"])
        self.k_cache = np.zeros((sh.n_layers, max_seq, sh.n_kv_heads, sh.head_dim), dtype=np.float64)
        self.v_cache = np.zeros_like(self.k_cache)
        self.length = 0
        self.state = DelayState(sh.n_codebooks, sh.codebook_size, sh.bos_id, sh.eos_id)
        self.last_hidden = None
        self.last_logits = None
        self.layer_out = []

    # ------------------------------------------------------------------ weights
    @staticmethod
    def _values(w) -> np.ndarray:
        w = np.asarray(w)
        if w.dtype == np.uint16:  # bfloat16 bit patterns
            return nx.bf16_bits_to_float(w)
        return w.astype(np.float64)

    def _plain(self, w) -> np.ndarray:
        return self._values(w)

    def _embedding(self, w) -> np.ndarray:
        v = self._values(w)
        if self.mode == "S":
            v = nx.round_bf16(v)
        return v.astype(self.storage)

    def _matrix(self, w):
        v = self._values(w)
        if self.mode == "E":
            return v.astype(self.storage)
        if self.precision == "bf16":
            return nx.round_bf16(v).astype(self.storage)
        q, s = nx.quantize_weight_rows(v)
        return (q.astype(self.storage), s)

    # ------------------------------------------------------------------ activation sites
    def _act(self, x, site: int):
        """Round a GEMV input at activation site ``site`` (index into the scale table)."""
        if self.record is not None:
            self.record[site] = max(self.record[site], float(np.max(np.abs(x))))
        if self.mode == "E":
            return x
        if self.precision == "bf16":
            return nx.round_bf16(x)
        return nx.quantize_static(x, self.scales[site])

    def _linear(self, xa, W, site: int) -> np.ndarray:
        """y = xa . W^T for rows of xa (the already-rounded GEMV input)."""
        if isinstance(W, tuple):
            q, s_w = W
            acc = (xa.astype(self.storage) @ q.T).astype(np.float64)
            return acc * (np.float64(self.scales[site]) * s_w.astype(np.float64))[None, :]
        return (xa.astype(W.dtype) @ W.T).astype(np.float64)

    def _kv_round(self, x):
        return nx.round_bf16(x) if self.mode == "S" else x

    # ------------------------------------------------------------------ layer
    def layer(self, layer: int, H: np.ndarray, positions: np.ndarray) -> np.ndarray:
        """One decoder layer over rows H [T, d] at absolute ``positions`` [T]; writes the KV cache."""
        sh, Lw = self.shape, self.layers[layer]
        T = H.shape[0]
        hd, Hq, Hkv = sh.head_dim, sh.n_q_heads, sh.n_kv_heads
        s0 = SITES_PER_LAYER * layer
        u = self._act(nx.rmsnorm(H, Lw["g_attn"], sh.rms_eps), s0)
        q = self._linear(u, Lw["wq"], s0).reshape(T, Hq, hd)
        k = self._linear(u, Lw["wk"], s0).reshape(T, Hkv, hd)
        v = self._linear(u, Lw["wv"], s0).reshape(T, Hkv, hd)
        q = nx.rope(nx.rmsnorm(q, Lw["g_q"], sh.rms_eps), positions, sh.rope_theta)
        k = nx.rope(nx.rmsnorm(k, Lw["g_k"], sh.rms_eps), positions, sh.rope_theta)
        q, k, v = self._kv_round(q), self._kv_round(k), self._kv_round(v)
        self.k_cache[layer, positions] = k
        self.v_cache[layer, positions] = v
        o = np.empty((T, Hq, hd), dtype=np.float64)
        group = Hq // Hkv
        n_keys = int(positions.max()) + 1
        # causal mask: query i sees the keys at positions 0..p_i
        visible = np.arange(n_keys)[None, :] <= np.asarray(positions)[:, None]
        for h in range(Hq):
            j = h // group
            K = self.k_cache[layer, :n_keys, j]
            V = self.v_cache[layer, :n_keys, j]
            scores = (q[:, h] @ K.T) / np.sqrt(hd)
            scores = np.where(visible, scores, -np.inf)
            o[:, h] = nx.softmax(scores, axis=-1) @ V
        oa = self._act(o.reshape(T, Hq * hd), s0 + 1)
        H = H + self._linear(oa, Lw["wo"], s0 + 1)
        u2 = self._act(nx.rmsnorm(H, Lw["g_mlp"], sh.rms_eps), s0 + 2)
        g = self._linear(u2, Lw["wg"], s0 + 2)
        up = self._linear(u2, Lw["wu"], s0 + 2)
        a = self._act(nx.silu(g) * up, s0 + 3)
        return H + self._linear(a, Lw["wd"], s0 + 3)

    def run_layers(self, H: np.ndarray, positions: np.ndarray) -> np.ndarray:
        self.layer_out = []
        for layer in range(self.shape.n_layers):
            H = self.layer(layer, H, positions)
            self.layer_out.append(H.copy())
        return H

    # ------------------------------------------------------------------ API
    def reset(self, keep_len: int = 0) -> None:
        """Start a new utterance, keeping the KV of positions [0, keep_len) (prefix reuse)."""
        if keep_len < 0 or keep_len > self.length:
            raise ValueError("keep_len out of range")
        self.length = keep_len
        sh = self.shape
        self.state = DelayState(sh.n_codebooks, sh.codebook_size, sh.bos_id, sh.eos_id)

    def prefill(self, ids) -> None:
        """Append the prompt ``ids`` at positions length .. length+P-1 in one batched pass (no head)."""
        ids = np.asarray(ids, dtype=np.int64)
        P = ids.shape[0]
        if self.length + P > self.max_seq:
            raise ValueError("capacity")
        H = self.e_text[ids].astype(np.float64)
        positions = np.arange(self.length, self.length + P)
        self.last_hidden = self.run_layers(H, positions)
        self.length += P

    def frame_input(self) -> np.ndarray:
        """x = sum over codebooks k of E_aud[k][prev_k]."""
        prev = self.state.prev
        return sum(self.e_aud[k, int(prev[k])].astype(np.float64) for k in range(self.shape.n_codebooks))

    def decode_frame(self):
        """One decode step; returns (codes [C], done)."""
        sh = self.shape
        if self.length + 1 > self.max_seq:
            raise ValueError("capacity")
        self.state.begin_frame()
        x = self.frame_input()
        H = self.run_layers(x[None, :], np.array([self.length]))
        self.length += 1
        h = H[0]
        self.last_hidden = h
        self.last_logits = self.head(h)
        codes = self.state.choose(self.last_logits)
        done = self.state.finish(codes)
        return codes, done

    def head(self, h) -> np.ndarray:
        """Logits [C][V] of the fused codebook head for a final residual h [d]:
        final RMSNorm, the head-input rounding of the mode, the head GEMV."""
        sh = self.shape
        z = self._act(nx.rmsnorm(np.asarray(h, np.float64)[None, :], self.g_final, sh.rms_eps),
                      SITES_PER_LAYER * sh.n_layers)
        return self._linear(z, self.w_head, SITES_PER_LAYER * sh.n_layers)[0].reshape(sh.n_codebooks, sh.codebook_size)

    def force_codes(self, codes) -> None:
        """Teacher forcing: the next frame embeds ``codes`` instead of the last choice."""
        self.state.prev = np.asarray(codes, dtype=np.int64).copy()

    # ------------------------------------------------------------------ site-anchored checks
    def layer_anchored(self, layer: int, h, site_vals, qkv=None):
        """One decode step of ``layer`` for a single row ``h`` at position ``length`` in which
        each GEMV multiplies with the given rounded input instead of the oracle's own:
        ``site_vals`` holds the four GEMV inputs (attention input, attention output, MLP
        input, down input) in GEMV units -- bfloat16 values (BF16) or e4m3 code values
        (FP8).  This is how an implementation is checked rounding decision by rounding
        decision: every rounding point then starts from the same values on both sides.

        ``qkv`` (optional): the rounded rotated queries [Hq][hd], key and value [Hkv][hd]
        to attend with and append to the cache in place of the oracle's own (the
        implementation's, so that its attention output is checked on its own inputs).

        Returns (pre, k, v, h_out, qkv_pre): the four sites' values before rounding
        (float64), the key and value row appended to the cache (rounded as stored), the
        layer output computed from the given site values, and the oracle's own q, k and v
        rows before their rounding."""
        sh, Lw = self.shape, self.layers[layer]
        hd, Hq, Hkv = sh.head_dim, sh.n_q_heads, sh.n_kv_heads
        s0 = SITES_PER_LAYER * layer
        pos = self.length
        h = np.asarray(h, np.float64)[None, :]
        x = [np.asarray(v, np.float64)[None, :] for v in site_vals]
        pre = [nx.rmsnorm(h, Lw["g_attn"], sh.rms_eps)]
        q = self._linear(x[0], Lw["wq"], s0).reshape(1, Hq, hd)
        k = self._linear(x[0], Lw["wk"], s0).reshape(1, Hkv, hd)
        v = self._linear(x[0], Lw["wv"], s0).reshape(1, Hkv, hd)
        p = np.array([pos])
        q_pre = nx.rope(nx.rmsnorm(q, Lw["g_q"], sh.rms_eps), p, sh.rope_theta)
        k_pre = nx.rope(nx.rmsnorm(k, Lw["g_k"], sh.rms_eps), p, sh.rope_theta)
        v_pre = v
        if qkv is None:
            q, k, v = self._kv_round(q_pre), self._kv_round(k_pre), self._kv_round(v_pre)
        else:
            q, k, v = (np.asarray(a, np.float64)[None] for a in qkv)
        self.k_cache[layer, pos] = k[0]
        self.v_cache[layer, pos] = v[0]
        group = Hq // Hkv
        o = np.empty((Hq, hd))
        for hh in range(Hq):
            j = hh // group
            o[hh] = nx.attention_one(q[0, hh], self.k_cache[layer, :pos + 1, j], self.v_cache[layer, :pos + 1, j])
        pre.append(o.reshape(1, Hq * hd))
        h_mid = h + self._linear(x[1], Lw["wo"], s0 + 1)
        pre.append(nx.rmsnorm(h_mid, Lw["g_mlp"], sh.rms_eps))
        g = self._linear(x[2], Lw["wg"], s0 + 2)
        up = self._linear(x[2], Lw["wu"], s0 + 2)
        pre.append(nx.silu(g) * up)
        h_out = h_mid + self._linear(x[3], Lw["wd"], s0 + 3)
        self.length += 1
        return [a[0] for a in pre], k[0], v[0], h_out[0], (q_pre[0], k_pre[0], v_pre[0])

    def head_anchored(self, h, z_val):
        """The head for final residual ``h`` with the given rounded head input ``z_val`` (GEMV
        units): (the head input before rounding, logits [C][V])."""
        sh = self.shape
        site = SITES_PER_LAYER * sh.n_layers
        pre = nx.rmsnorm(np.asarray(h, np.float64)[None, :], self.g_final, sh.rms_eps)[0]
        lg = self._linear(np.asarray(z_val, np.float64)[None, :], self.w_head, site)[0]
        return pre, lg.reshape(sh.n_codebooks, sh.codebook_size)

    def round_site(self, x, site: int):
        """The oracle's rounding of GEMV input values ``x`` at activation site ``site``, in GEMV
        units (bfloat16 value, or e4m3 code value of fp32(x) / scale)."""
        if self.precision == "bf16":
            return nx.round_bf16(x)
        return nx.quantize_static(x, self.scales[site])

    # ------------------------------------------------------------------ one layer at a preset KV
    def set_kv(self, layer: int, k, v) -> None:
        """Fill positions [0, n) of ``layer`` with given K/V rows [n][Hkv][hd] (as stored) and set length n."""
        n = k.shape[0]
        self.k_cache[layer, :n] = self._kv_round(np.asarray(k, np.float64))
        self.v_cache[layer, :n] = self._kv_round(np.asarray(v, np.float64))
        self.length = n

    def layer_step(self, layer: int, h) -> np.ndarray:
        """One decoder layer for a single input row ``h`` at position ``length``."""
        out = self.layer(layer, np.asarray(h, np.float64)[None, :], np.array([self.length]))
        self.length += 1
        return out[0]


def calibrate(shape, weights, prompt, n_frames: int, forced_codes=None, storage=np.float64):
    """FP8 activation scales from a BF16 storage-faithful run: prefill ``prompt``,
    then ``n_frames`` greedy frames (or frames fed with ``forced_codes``),
    recording max |x| at every activation site; scale = amax / 448.

    Returns (scales [4 * n_layers + 1] float32, amax float64, codes [n_frames][C])."""
    n_sites = SITES_PER_LAYER * shape.n_layers + 1
    m = OracleModel(shape, weights, precision="bf16", mode="S", storage=storage,
                    max_seq=len(prompt) + n_frames + 1)
    m.record = np.zeros(n_sites, dtype=np.float64)
    m.prefill(prompt)
    codes = []
    for f in range(n_frames):
        c, _ = m.decode_frame()
        codes.append(c)
        if forced_codes is not None:
            m.force_codes(forced_codes[f])
    amax = m.record.copy()
    scales = np.array([nx.act_scale(a) for a in amax], dtype=np.float32)
    return scales, amax, np.array(codes)
