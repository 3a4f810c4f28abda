"""CPU checks of the attention parity criterion (tests/conftest.attn_tol): a one-step
bf16 rounding flip is excused only where the reference lies at a rounding midpoint
(within FLIP_TAU relative), and any other deviation counts in full."""
import numpy as np
import torch

import oracle
from tests.conftest import FLIP_TAU, attn_tol


def _row(values):
    return np.asarray(values, dtype=np.float64)[None, :]


def _bf16(x):
    return torch.from_numpy(oracle.bf16_to_f64(oracle.round_bf16(np.asarray(x))))


def test_exact_rounding_passes():
    ref = _row(np.linspace(-3, 3, 64) + 1e-3)
    ok, ratio, _ = attn_tol(_bf16(ref), ref)
    assert ok and ratio == 0


def test_flip_at_a_midpoint_is_excused():
    # 3.0078125 is the midpoint of the bf16 neighbours 3.0 and 3.015625; a reference a
    # hair above it rounds up, and an fp32 result a hair below it rounds down to 3.0
    ref = _row([3.0078125 * (1 + 1e-6)] + [0.5] * 63)
    out = _bf16(ref).clone()
    out[0, 0] = 3.0
    ok, ratio, _ = attn_tol(out, ref)
    assert ok and ratio == 0
    # without the exception the one step (0.015625) is ~0.037 of this row's RMS
    assert 0.015625 / np.sqrt(np.mean(ref ** 2)) > 0.02


def test_flip_away_from_a_midpoint_counts():
    ref = _row([3.0078125 * (1 + 30 * FLIP_TAU)] + [0.5] * 63)
    out = _bf16(ref).clone()
    out[0, 0] = 3.0
    ok, ratio, _ = attn_tol(out, ref)
    assert not ok and ratio > 0.02


def test_a_real_error_counts():
    ref = _row(np.full(64, 1.0))
    out = _bf16(ref).clone()
    out[0, 7] = 1.03125   # four steps off
    ok, ratio, _ = attn_tol(out, ref)
    assert not ok and ratio > 0.02
