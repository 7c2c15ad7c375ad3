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
from oracle.model import OracleModel

HIDDEN_TOL = {"bf16": 2e-2, "fp8": 6e-2}
COS_MIN = 0.999
MARGIN = 1e-2


def gpu_context(shape, weights, precision="bf16", max_seq=256, max_prefill=128, act_scales=None, fill_byte=None):
    ctx = hta.Hta(shape, precision, max_seq=max_seq, max_prefill=max_prefill, fill_byte=fill_byte)
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
