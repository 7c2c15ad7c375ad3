"""Delay pattern of the 8-codebook head: per-step code choice and un-delay.

TEST INFRASTRUCTURE ONLY: nothing in the product path may import this package.

Sources: FlashRT "Higgs Audio v3 TTS-4B" page, section 5 (greedy generation
applies the delay pattern, BOC/EOC, and un-delays the codes before the codec)
and the Performance section (an utterance ends at EOC, with a 40.68 s cap);
SGLang-Omni Higgs Audio v3 page, architecture paragraph (8 codebooks, delay
pattern).  The pages give no finer rule, so this module fixes the plainest
reading:

* at step t, codebook k lags k steps: while t < k it emits BOS (1024);
* codebook 0 ends the utterance: the first step e at which it picks EOS
  (1025) is the EOC step, and from step e + k on codebook k emits EOS;
* otherwise the code is the argmax over the allowed ids: codebook 0 may pick
  a code 0..1023 or EOS; codebooks 1..7 may pick only codes 0..1023 (BOS is
  never chosen by argmax); ties go to the lowest id;
* the utterance is done once codebook 7 has emitted EOS, i.e. after step e + 7;
* e is taken from the code of codebook 0 that is fed back into the next
  frame, so forcing codes (teacher forcing) drives the same bookkeeping.

The same page's Performance section mentions a deterministic repeated-code stop guard that
ends pathological runs without EOC before the generation cap, and section 4 a streaming
generator whose output equals the one-shot output; neither gives a rule.  The reading
taken here (``repeat_guard``): the guard watches the complete (un-delayed) frames and fires
at the first frame f that ends a window of ``window`` frames repeating with some period
p <= ``max_period`` (frame g equals frame g - p for every g of the window after its first
p); the frames up to and including f are the output.  Streaming emits the un-delayed frames
in chunks as they complete; the chunks concatenated equal ``undelay`` of all the steps.
"""
from __future__ import annotations

import numpy as np


class DelayState:
    """Bookkeeping of one utterance: step t, EOC step, previous (fed-back) codes."""

    def __init__(self, n_codebooks: int = 8, codebook_size: int = 1026, bos: int = 1024, eos: int = 1025):
        self.C, self.V, self.bos, self.eos = n_codebooks, codebook_size, bos, eos
        self.t = 0
        self.eoc = None
        self.prev = np.full(n_codebooks, bos, dtype=np.int64)

    def begin_frame(self) -> None:
        """Derive the EOC step from the fed-back code of codebook 0."""
        if self.eoc is None and self.t > 0 and int(self.prev[0]) == self.eos:
            self.eoc = self.t - 1

    def allowed_mask(self, k: int) -> np.ndarray:
        m = np.zeros(self.V, dtype=bool)
        m[: self.bos] = True
        if k == 0:
            m[self.eos] = True
        return m

    def choose(self, logits) -> np.ndarray:
        """Codes for the current step t from logits [C][V]; does not advance the state."""
        logits = np.asarray(logits)
        codes = np.empty(self.C, dtype=np.int64)
        for k in range(self.C):
            if self.t < k:
                codes[k] = self.bos
            elif self.eoc is not None and self.t >= self.eoc + k:
                codes[k] = self.eos
            else:
                masked = np.where(self.allowed_mask(k), logits[k], -np.inf)
                codes[k] = int(np.argmax(masked))  # first maximum = lowest id
        return codes

    def finish(self, codes) -> bool:
        """Feed ``codes`` back, advance t; True when the utterance is done after this step."""
        step = self.t
        eoc = self.eoc
        if eoc is None and int(codes[0]) == self.eos:
            eoc = step
        self.prev = np.asarray(codes, dtype=np.int64).copy()
        self.t += 1
        return eoc is not None and step >= eoc + self.C - 1


def delay_frames(frames, n_codebooks: int = 8, bos: int = 1024, eos: int = 1025) -> np.ndarray:
    """Apply the delay pattern to n un-delayed frames [n][C], giving the n + C steps a
    greedy run emits up to and including the step at which codebook C-1 emits EOS:
    step s, codebook k holds frame s - k, BOS before the first frame and EOS after the last."""
    frames = np.asarray(frames, dtype=np.int64)
    n, C = frames.shape
    T = n + C
    steps = np.empty((T, C), dtype=np.int64)
    for s in range(T):
        for k in range(C):
            f = s - k
            steps[s, k] = bos if f < 0 else (eos if f >= n else frames[f, k])
    return steps


def undelay(step_codes, eoc=None, n_codebooks: int = 8) -> np.ndarray:
    """frames[f][k] = step_codes[f + k][k] for f < n; n = eoc if EOC occurred, else T - (C - 1)."""
    step_codes = np.asarray(step_codes, dtype=np.int64)
    T = step_codes.shape[0]
    C = n_codebooks
    n = eoc if eoc is not None else max(0, T - (C - 1))
    out = np.empty((n, C), dtype=np.int64)
    for f in range(n):
        for k in range(C):
            out[f, k] = step_codes[f + k, k]
    return out


def find_eoc(step_codes, eos: int = 1025):
    """First step at which codebook 0 holds EOS, or None."""
    col = np.asarray(step_codes)[:, 0]
    hits = np.nonzero(col == eos)[0]
    return int(hits[0]) if hits.size else None


def repeat_guard(frames, window: int, max_period: int):
    """First frame index f at which the last ``window`` complete frames repeat with some
    period p in 1..max_period, or None."""
    frames = np.asarray(frames, dtype=np.int64)
    for f in range(window - 1, frames.shape[0]):
        w = frames[f - window + 1: f + 1]
        for p in range(1, max_period + 1):
            if p < window and all(np.array_equal(w[g], w[g - p]) for g in range(p, window)):
                return f
    return None
