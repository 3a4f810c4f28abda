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


def attn_tol(out, ref, bar: float = 2e-2, name: str = ""):
    """Attention parity, per row (each row is its own attention problem, so a
    batch-wide RMS would let short rows hide behind long ones):
        max_i |out_i - RNE_bf16(ref_i)| <= bar * RMS(ref row),
    ref in fp64 from the oracle, RNE_bf16 its one rounding to the output type.
    Prints the worst ratio (and the same ratio against the RMS of the whole call,
    the form the bar is stated in) so the margin stays visible.
    out: torch tensor [rows, ...]; ref: float64 array of the same shape.
    Returns (ok, worst per-row ratio, its row)."""
    import numpy as np

    import oracle
    r = np.asarray(ref, dtype=np.float64).reshape(ref.shape[0], -1)
    o = out.double().cpu().numpy().reshape(r.shape)
    rr = oracle.bf16_to_f64(oracle.round_bf16(r))
    err = np.abs(o - rr).max(1)
    ratio = err / np.sqrt(np.mean(r ** 2, 1))
    worst = int(np.argmax(ratio))
    call = float(err.max() / np.sqrt(np.mean(r ** 2)))
    print(f"parity {name or 'attention'}: worst max|out - RNE(ref)| / RMS(row) = "
          f"{ratio[worst]:.4g} (row {worst}), / RMS(call) = {call:.4g}; bar {bar}", flush=True)
    return bool((ratio <= bar).all()), float(ratio[worst]), worst
