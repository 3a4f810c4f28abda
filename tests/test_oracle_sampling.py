"""Pins of the oracle's seeded Gumbel-max sampling (hidekazu-konishi.com,
section 9.3 "Non-Greedy Sampling Can Be Deterministic Too") against things
other than itself: the generator's published known-answer vectors, the Gumbel
distribution's closed-form moments and range, the Gumbel-max identity (the
sample frequencies follow softmax(logits / T)), and greedy argmax at T <= 0.
"""
import math

import numpy as np
import pytest

import oracle
from tests.conftest import golden_lines


def test_philox_known_answers():
    for line in golden_lines("philox4x32_10_kat.txt"):
        w = [int(x, 16) for x in line.split()]
        assert oracle.philox4x32_10(w[0:4], w[4:6]) == tuple(w[6:10]), line


def test_gumbel_moments_and_range():
    # standard Gumbel: mean = Euler-Mascheroni constant, variance = pi^2 / 6; the
    # 23-bit uniforms bound the noise to [-ln(-ln 2^-24), -ln(-ln(1 - 2^-24))]
    n = 1_000_000
    g = np.concatenate([oracle.gumbel_noise(seed, 3, n // 4) for seed in (1, 2, 3, 4)])
    gamma = 0.5772156649015329
    se = math.sqrt(math.pi ** 2 / 6 / n)
    assert abs(g.mean() - gamma) < 5 * se
    assert abs(g.var() - math.pi ** 2 / 6) < 0.02
    lo = -math.log(-math.log(2.0 ** -24))
    hi = -math.log(-math.log1p(-2.0 ** -24))
    assert g.min() >= lo - 1e-12 and g.max() <= hi + 1e-9
    # exceedance of a quantile: P(g > x) = 1 - exp(-exp(-x))
    for x in (-1.0, 0.0, 2.0):
        p = 1 - math.exp(-math.exp(-x))
        assert abs((g > x).mean() - p) < 5 * math.sqrt(p * (1 - p) / n)


def test_noise_is_a_function_of_seed_position_and_id():
    a = oracle.gumbel_noise(7, 100, 1000)
    assert np.array_equal(a[:333], oracle.gumbel_noise(7, 100, 333))   # prefix-stable
    assert not np.array_equal(a, oracle.gumbel_noise(8, 100, 1000))   # seed matters
    assert not np.array_equal(a, oracle.gumbel_noise(7, 101, 1000))   # position matters
    big = oracle.gumbel_noise(2**64 - 1, 2**40 + 5, 8)                 # 64-bit seed / position
    assert np.isfinite(big).all()
    assert not np.array_equal(big, oracle.gumbel_noise(2**32 - 1, 5, 8))


def test_gumbel_max_follows_softmax():
    # P(argmax(l / T + g) = i) = softmax(l / T)_i; 40000 seeds, chi-square
    logits = np.array([0.3, -1.0, 1.2, 0.0, 0.9, -0.4], dtype=np.float32)
    for T in (0.7, 1.0, 2.5):
        n = 40000
        rows = np.repeat(logits[None], n, 0)
        tok, _, _ = oracle.sample_gumbel(rows, np.arange(n, dtype=np.uint64) * 7919 + 11,
                                         np.full(n, 42), np.full(n, T, dtype=np.float32))
        p = np.exp(logits.astype(np.float64) / T)
        p /= p.sum()
        counts = np.bincount(tok, minlength=len(logits))
        chi2 = float(((counts - n * p) ** 2 / (n * p)).sum())
        assert chi2 < 25.0, (T, chi2, counts, n * p)   # 5 dof: P(chi2 > 25) < 2e-4


def test_greedy_and_special_values():
    rng = np.random.default_rng(5)
    x = rng.standard_normal((6, 50)).astype(np.float32)
    x[1, 7] = x[1, 30] = 9.0                      # tie: the lower index wins
    x[2, :] = np.nan
    x[3, 4] = np.nan                              # NaN never chosen
    x[3, 5] = 50.0
    tok, best, gap = oracle.sample_gumbel(x, np.arange(6), np.zeros(6), np.array(
        [0, 0, 0, 0, -1, 0], dtype=np.float32))
    clean = np.where(np.isnan(x), -np.inf, x)
    assert tok[0] == np.argmax(clean[0]) and tok[1] == 7 and tok[2] == 0 and tok[3] == 5
    assert tok[4] == np.argmax(clean[4]) and tok[5] == np.argmax(clean[5])
    assert gap[1] == 0.0 and best[3] == 50.0
    # a tiny temperature scales the logits past any noise: greedy again
    tok_t, _, _ = oracle.sample_gumbel(x[[0, 4, 5]], [1, 2, 3], [0, 0, 0], [1e-6] * 3)
    assert list(tok_t) == [tok[0], tok[4], tok[5]]


def test_scores_are_logit_over_t_plus_noise():
    rng = np.random.default_rng(9)
    x = rng.standard_normal((3, 257)).astype(np.float32)
    seeds, pos, T = [5, 6, 7], [0, 9, 2**33], [0.5, 1.0, 3.0]
    tok, best, gap = oracle.sample_gumbel(x, seeds, pos, np.array(T, dtype=np.float32))
    for r in range(3):
        s = x[r].astype(np.float64) / np.float64(np.float32(T[r])) + oracle.gumbel_noise(
            seeds[r], pos[r], 257)
        assert tok[r] == int(np.argmax(s)) and best[r] == s.max()
        assert gap[r] == s.max() - np.sort(s)[-2]
