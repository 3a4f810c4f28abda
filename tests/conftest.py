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


def _bf16_neighbour(bits, up):
    """The bf16 value next to each bf16 bit pattern, toward +inf (up) or -inf."""
    import numpy as np
    bits = np.asarray(bits, dtype=np.uint16)
    neg = (bits >> 15).astype(bool)
    mag = (bits & 0x7fff).astype(np.int32)
    grow = neg != up                      # the magnitude grows going outward
    mag2 = np.where(grow, mag + 1, mag - 1)
    cross = mag2 < 0                      # past zero: the smallest value of the other sign
    out = np.where(cross, 1, mag2) | np.where(cross, np.where(neg, 0, 0x8000),
                                              np.where(neg, 0x8000, 0))
    return out.astype(np.uint16)


# A bf16 output is the exactly rounded value unless the fp32 result it was rounded
# from fell on the other side of a rounding midpoint.  The kernels' fp32 results are
# within ~1e-5 of the exact value relative to it (the softmax weights carry 16
# significant bits), so a reference value within FLIP_TAU of a midpoint, relative to
# itself, may come out as either neighbour: that one-step flip is excused; any other
# deviation counts in full.
FLIP_TAU = 1e-4


def attn_tol(out, ref, bar: float = 2e-2, name: str = ""):
    """Attention parity, per row (each row is its own attention problem, so a
    batch-wide RMS would let short rows hide behind long ones):
        max_i |out_i - RNE_bf16(ref_i)| <= bar * RMS(ref row),
    ref in fp64 from the oracle, RNE_bf16 its one rounding to the output type, except
    that out_i may be the other bf16 neighbour of ref_i when ref_i lies within
    FLIP_TAU (relative) of the midpoint between the two (a rounding flip of an fp32
    result that is itself within tolerance by orders of magnitude).
    Prints the worst ratio without the exception, the worst with it, and how many
    elements the exception covered, together with the ratio against the RMS of the
    whole call (the form the bar is stated in), so the margin stays visible.
    out: torch tensor [rows, ...]; ref: float64 array of the same shape.
    Returns (ok, worst per-row ratio with the exception, its row)."""
    import numpy as np

    import oracle
    r = np.asarray(ref, dtype=np.float64).reshape(ref.shape[0], -1)
    o = out.double().cpu().numpy().reshape(r.shape)
    rb = oracle.round_bf16(r)
    rr = oracle.bf16_to_f64(rb)
    other = oracle.bf16_to_f64(np.where(r > rr, _bf16_neighbour(rb, True),
                                        _bf16_neighbour(rb, False)))
    mid = 0.5 * (rr + other)
    flip = (r != rr) & (o == other) & (np.abs(r - mid) <= FLIP_TAU * np.abs(r))
    err_strict = np.abs(o - rr)
    err = np.where(flip, 0.0, err_strict)
    rms = np.sqrt(np.mean(r ** 2, 1))
    ratio = err.max(1) / rms
    strict = err_strict.max(1) / rms
    worst = int(np.argmax(ratio))
    call = float(err.max() / np.sqrt(np.mean(r ** 2)))
    print(f"parity {name or 'attention'}: worst max|out - RNE(ref)| / RMS(row) = "
          f"{ratio[worst]:.4g} (row {worst}); without the midpoint-flip exception "
          f"{strict.max():.4g} (row {int(np.argmax(strict))}), {int(flip.sum())} flips of "
          f"{flip.size}; / RMS(call) = {call:.4g}; bar {bar}", flush=True)
    return bool((ratio <= bar).all()), float(ratio[worst]), worst
