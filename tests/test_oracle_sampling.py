"""Pins of the sampling oracle (oracle/sampling.py) against what fixes it from outside:
the generator's published known-answer vectors, the softmax distribution as torch computes
it (chi-square over many counters), a hand-worked inversion, and the limit cases."""
import math

import numpy as np
import pytest
import scipy.stats
import torch

from oracle import sampling as smp
from oracle.delay import DelayState

# Known-answer vectors of Philox4x32-10 published with the generator (Salmon et al., SC'11,
# Random123 distribution): (counter, key) -> output.
PHILOX_KAT = [
    ((0x00000000, 0x00000000, 0x00000000, 0x00000000), (0x00000000, 0x00000000),
     (0x6627E8D5, 0xE169C58D, 0xBC57AC4C, 0x9B00DBD8)),
    ((0xFFFFFFFF, 0xFFFFFFFF, 0xFFFFFFFF, 0xFFFFFFFF), (0xFFFFFFFF, 0xFFFFFFFF),
     (0x408F276D, 0x41C83B0E, 0xA20BC7C6, 0x6D5451FD)),
    ((0x243F6A88, 0x85A308D3, 0x13198A2E, 0x03707344), (0xA4093822, 0x299F31D0),
     (0xD16CFE09, 0x94FDCCEB, 0x5001E420, 0x24126EA1)),
]


@pytest.mark.parametrize("counter,key,expect", PHILOX_KAT)
def test_philox_known_answers(counter, key, expect):
    assert tuple(int(v) for v in smp.philox4x32_10(counter, key)) == expect


def test_philox_vectorised_equals_scalar():
    rng = np.random.default_rng(7)
    c = rng.integers(0, 2 ** 32, size=(4, 64), dtype=np.uint64)
    key = (0x1234ABCD, 0x0BADF00D)
    vec = smp.philox4x32_10(tuple(c), key)
    for j in range(64):
        one = smp.philox4x32_10(tuple(int(c[i, j]) for i in range(4)), key)
        assert all(int(vec[i][j]) == int(one[i]) for i in range(4))


def test_uniform_is_24_bit_in_unit_interval():
    u = smp.uniform(0xDEADBEEFCAFEF00D, np.arange(100000, dtype=np.uint64), 3)
    assert u.min() >= 0.0 and u.max() < 1.0
    assert np.all(u * (1 << 24) == np.floor(u * (1 << 24)))
    # the uniform is the top 24 bits of word 0 of Philox(counter (t, k, 0, 0), key (lo, hi))
    x0 = smp.philox4x32_10((5, 3, 0, 0), (0xCAFEF00D, 0xDEADBEEF))[0]
    assert smp.uniform(0xDEADBEEFCAFEF00D, 5, 3) == (int(x0) >> 8) / 2.0 ** 24
    # mean and variance of a uniform on [0, 1)
    assert abs(u.mean() - 0.5) < 4 * math.sqrt(1 / 12 / u.size)
    assert abs(u.var() - 1 / 12) < 0.002


def test_hand_worked_inversion():
    # weights 1, 2, (masked), 5 at T = 1: cumulative 1, 3, 3, 8
    z = np.array([0.0, math.log(2.0), math.log(3.0), math.log(5.0)])
    allowed = np.array([True, True, False, True])
    for u, want in ((0.1, 0), (0.124, 0), (0.125, 1), (0.126, 1), (0.374, 1), (0.376, 3), (0.99, 3), (0.0, 0)):
        assert smp.draw(z, allowed, 1.0, u)[0] == want
    # T = 2: weights 1, sqrt 2, sqrt 5
    w = np.array([1.0, math.sqrt(2.0), math.sqrt(5.0)])
    c = np.cumsum(w) / w.sum()
    assert smp.draw(z, allowed, 2.0, c[0] - 1e-9)[0] == 0
    assert smp.draw(z, allowed, 2.0, c[0] + 1e-9)[0] == 1
    assert smp.draw(z, allowed, 2.0, c[1] + 1e-9)[0] == 3
    # margin: distance to the nearest interior boundary over the total
    _, margin = smp.draw(z, allowed, 1.0, 0.2)
    assert abs(margin - abs(0.2 * 8 - 1.0) / 8) < 1e-15


def _torch_probs(z, allowed, T):
    zt = torch.tensor(z, dtype=torch.float64) / T
    zt[~torch.tensor(allowed)] = -math.inf
    return torch.softmax(zt, dim=0).numpy()


@pytest.mark.parametrize("T,k", [(1.0, 0), (0.7, 3), (1.6, 0)])
def test_draws_follow_torch_softmax(T, k):
    """Chi-square of 60000 draws (counters t = 0..59999) against torch.softmax."""
    rng = np.random.default_rng(11 + k)
    V = 1026
    z = rng.normal(0.0, 1.5, V)
    z[1025] = 2.0  # EOS reachable for codebook 0
    allowed = DelayState().allowed_mask(k)
    p = _torch_probs(z, allowed, T)
    n = 60000
    u = smp.uniform(987654321, np.arange(n, dtype=np.uint64), k)
    ids = np.array([smp.draw(z, allowed, T, float(x))[0] for x in u])
    assert allowed[ids].all()
    counts = np.bincount(ids, minlength=V).astype(np.float64)
    exp = p * n
    # merge the categories expected below 5 into one bin
    big = exp >= 5
    obs_b = np.append(counts[big], counts[~big].sum())
    exp_b = np.append(exp[big], exp[~big].sum())
    if exp_b[-1] < 5:
        obs_b[-2] += obs_b[-1]
        exp_b[-2] += exp_b[-1]
        obs_b, exp_b = obs_b[:-1], exp_b[:-1]
    stat = float(((obs_b - exp_b) ** 2 / exp_b).sum())
    pval = scipy.stats.chi2.sf(stat, df=obs_b.size - 1)
    assert pval > 1e-4, (stat, obs_b.size, pval)


def test_limits():
    rng = np.random.default_rng(3)
    z = rng.normal(0.0, 1.0, 1026)
    allowed = DelayState().allowed_mask(1)
    best = int(np.argmax(np.where(allowed, z, -np.inf)))
    # a tiny temperature gives the argmax for every uniform
    assert all(smp.draw(z, allowed, 1e-4, u)[0] == best for u in (0.0, 0.3, 0.999999))
    # NaN logits weigh nothing; with none finite the lowest allowed id is taken
    zn = z.copy()
    zn[best] = np.nan
    assert smp.draw(zn, allowed, 1e-4, 0.5)[0] != best
    assert smp.draw(np.full(1026, np.nan), allowed, 1.0, 0.5)[0] == 0
    assert smp.draw(np.full(1026, -np.inf), allowed, 1.0, 0.5)[0] == 0
    # a single allowed id is always drawn
    one = np.zeros(1026, dtype=bool)
    one[17] = True
    assert smp.draw(z, one, 1.0, 0.9)[0] == 17


def test_delay_rule_forces_codes_under_sampling():
    st = DelayState()
    z = np.random.default_rng(5).normal(0.0, 1.0, (8, 1026))
    st.t = 2
    codes, margins = smp.choose_sampled(st, z, 1.0, 42)
    assert list(codes[3:]) == [1024] * 5 and np.isinf(margins[3:]).all()
    assert np.all(codes[:3] < 1024) or codes[0] == 1025
    st.t, st.eoc = 10, 7
    codes, _ = smp.choose_sampled(st, z, 1.0, 42)
    assert list(codes[:4]) == [1025] * 4 and np.all(codes[4:] < 1024)
    # fixed (seed, t, k): the same draws; another seed: other draws
    st = DelayState()
    st.t = 20
    a = smp.choose_sampled(st, z, 1.0, 42)[0]
    assert np.array_equal(a, smp.choose_sampled(st, z, 1.0, 42)[0])
    assert not np.array_equal(a, smp.choose_sampled(st, z, 1.0, 43)[0])
