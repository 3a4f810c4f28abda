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
