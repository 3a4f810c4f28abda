"""Shared pytest set-up.

Markers:
  gpu -- needs an MI355X (gfx950) and the built HIP library; parity and
         invariance tests proper.  Everything else runs on the CPU.
"""
import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X GPU and the built HIP library")


def read_golden(name: str) -> dict:
    """key = value lines of a golden fixture (comments start with '#')."""
    out = {}
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if "=" in line:
                k, v = (s.strip() for s in line.split("=", 1))
                out[k] = float(v)
    return out


def golden_lines(name: str) -> list:
    with open(os.path.join(GOLDEN, name)) as f:
        return [l.strip() for l in f if l.strip() and not l.lstrip().startswith("#")]


def attn_tol(out, ref, bar: float = 2e-2):
    """Attention parity, per row (each row is its own attention problem):
        max_i max(0, |out_i - ref_i| - u_i) <= bar * RMS(ref row),
    where u_i is half a bf16 step at ref_i -- the rounding of the exact result to
    the bf16 output, which no bf16-output kernel avoids.  (A head that attends to
    few tokens has outputs near |v| ~ 1 while the row's RMS can be ~0.07; its
    output rounding alone is then ~2.7 % of the RMS.)
    out: torch tensor [rows, ...]; ref: float64 array of the same shape.
    Returns (ok, worst ratio, its row)."""
    import numpy as np
    r = np.asarray(ref, dtype=np.float64).reshape(ref.shape[0], -1)
    o = out.double().cpu().numpy().reshape(r.shape)
    mag = np.abs(r)
    e = np.floor(np.log2(np.where(mag > 0, mag, 1.0)))
    half = np.where(mag > 0, np.exp2(np.maximum(e, -126) - 8), 0.0)
    err = np.maximum(np.abs(o - r) - half, 0.0).max(1)
    ratio = err / np.sqrt(np.mean(r ** 2, 1))
    worst = int(np.argmax(ratio))
    return bool((ratio <= bar).all()), float(ratio[worst]), worst
