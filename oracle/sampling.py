"""Temperature sampling of the codebook head: a counter-based generator and the categorical
draw over each codebook's allowed ids.

TEST INFRASTRUCTURE ONLY: nothing in the product path may import this package.

Sources: FlashRT "Higgs Audio v3 TTS-4B" page, section 4 (the sampling policy: greedy is
the default; an explicit positive temperature runs a native stable softmax, a stateless
categorical draw, the delay masking and the codebook embedding; an optional uint64 seed
repeats the same draws), section 5 (the draw and the embedding are a separate helper at
the end of the frame; the backbone is unchanged) and section 8 (decode policy: no top-p or
top-k).  The pages name neither the generator nor the way the draw is made.  The readings
taken here:

* generator: Philox4x32-10 (J. Salmon, M. Moraes, R. Dror, D. Shaw, "Parallel random
  numbers: as easy as 1, 2, 3", SC'11), keyed by the 64-bit seed (low word first) with the
  counter (step t, codebook k, 0, 0), so every draw depends only on (seed, t, k);
* uniform: the top 24 bits of the first output word, u = (x0 >> 8) / 2^24, in [0, 1);
* distribution: weight exp((z_i - m) / T) for every allowed id i of the codebook (the
  greedy path's allowed set), m the largest allowed logit; a NaN logit weighs nothing;
  with no allowed finite logit the lowest allowed id is taken, as in the greedy path;
* draw: inversion in id order: the id i whose cumulative interval [W_{i-1}, W_i) holds
  u * W_total;
* the delay rule forces BOS and EOS exactly as in the greedy path.
"""
from __future__ import annotations

import numpy as np

# Philox4x32 round multipliers and key increments (the "Weyl" constants), from the paper.
PHILOX_M0, PHILOX_M1 = 0xD2511F53, 0xCD9E8D57
PHILOX_W0, PHILOX_W1 = 0x9E3779B9, 0xBB67AE85
MASK32 = 0xFFFFFFFF


def philox4x32_10(counter, key):
    """Philox4x32 with 10 rounds.  counter: four uint32 (scalars or equal-shape arrays),
    key: two uint32.  Each round multiplies words 0 and 2 by the two constants into
    64-bit products; the new words are (hi(M1*x2) ^ x1 ^ k0, lo(M1*x2), hi(M0*x0) ^ x3 ^ k1,
    lo(M0*x0)); the key is advanced by the two Weyl constants between rounds."""
    x0, x1, x2, x3 = (np.asarray(c, dtype=np.uint64) & MASK32 for c in counter)
    k0 = np.uint64(int(key[0]) & MASK32)
    k1 = np.uint64(int(key[1]) & MASK32)
    m0, m1 = np.uint64(PHILOX_M0), np.uint64(PHILOX_M1)
    mask = np.uint64(MASK32)
    sh = np.uint64(32)
    for r in range(10):
        if r:
            k0 = (k0 + np.uint64(PHILOX_W0)) & mask
            k1 = (k1 + np.uint64(PHILOX_W1)) & mask
        p0 = x0 * m0  # < 2^64: exact in uint64
        p1 = x2 * m1
        x0, x1, x2, x3 = ((p1 >> sh) ^ x1 ^ k0, p1 & mask, (p0 >> sh) ^ x3 ^ k1, p0 & mask)
    return tuple(np.asarray(v, dtype=np.uint64).astype(np.uint32) for v in (x0, x1, x2, x3))


def seed_key(seed: int):
    seed = int(seed) & 0xFFFFFFFFFFFFFFFF
    return seed & MASK32, seed >> 32


def uniform(seed: int, step, codebook):
    """The draw's uniform for (seed, step t, codebook k): top 24 bits of Philox word 0."""
    x0, _, _, _ = philox4x32_10((step, codebook, 0, 0), seed_key(seed))
    return (np.asarray(x0, dtype=np.uint64) >> np.uint64(8)).astype(np.float64) / float(1 << 24)


def weights(logits_row, allowed, temperature: float):
    """Unnormalised weights exp((z - m) / T) over the allowed finite logits (float64);
    None when no allowed logit is finite."""
    z = np.asarray(logits_row, dtype=np.float64)
    ok = np.asarray(allowed, dtype=bool) & ~np.isnan(z)
    if not ok.any():
        return None
    m = z[ok].max()
    if not np.isfinite(m):
        return None
    w = np.zeros_like(z)
    w[ok] = np.exp((z[ok] - m) / float(temperature))
    return w


def draw(logits_row, allowed, temperature: float, u: float):
    """Inversion draw: returns (id, margin), margin = distance of u * W_total from the
    nearest cumulative boundary W_j (j < last) over W_total.  Where no allowed logit is
    finite, the lowest allowed id with margin inf."""
    allowed = np.asarray(allowed, dtype=bool)
    w = weights(logits_row, allowed, temperature)
    if w is None:
        return int(np.nonzero(allowed)[0][0]), np.inf
    c = np.cumsum(w)
    total = c[-1]
    target = u * total
    i = int(np.searchsorted(c, target, side="right"))  # first id with W_i > target
    i = min(i, len(c) - 1)
    bounds = c[w > 0][:-1]  # interior boundaries between ids of positive weight
    margin = float(np.min(np.abs(bounds - target)) / total) if bounds.size else np.inf
    return i, margin


def choose_sampled(state, logits, temperature: float, seed: int):
    """Codes of one step under sampling, with the delay rule of ``state`` (an
    oracle.delay.DelayState at the step's t): (codes [C], margins [C]); forced codes have
    margin inf.  Does not advance the state."""
    logits = np.asarray(logits)
    codes = np.empty(state.C, dtype=np.int64)
    margins = np.full(state.C, np.inf)
    for k in range(state.C):
        if state.t < k:
            codes[k] = state.bos
        elif state.eoc is not None and state.t >= state.eoc + k:
            codes[k] = state.eos
        else:
            u = float(uniform(seed, state.t, k))
            codes[k], margins[k] = draw(logits[k], state.allowed_mask(k), temperature, u)
    return codes, margins
