"""CPU oracle for batch-invariant RMSNorm, matmul and paged decode attention.

TEST INFRASTRUCTURE ONLY.  Only the test suite, ``__graft_entry__.smoke()`` and
the bench's ``cpu_baseline`` leg may import this package.  The product path (the
HIP library and its binding) never calls it and shares no code with it.

The arithmetic lives in ``oracle.c`` (plain fp64 loops, OpenMP over independent
rows); this module loads it with ctypes, marshals numpy arrays, and composes the
dense decode layer of the config-5 workload from those definitions
(``layer.py``).  Every function returns float64 results computed from the exact
input values; bf16 inputs are passed as their raw uint16 bits.

Pinning (see ``tests/test_oracle_pins.py``): every function here is checked
against values the pages print, closed forms, invariants and independent library
routines (numpy, torch CPU fp64).  No function is "parity unpinned".
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

F32, BF16, F64 = 0, 1, 2


def build(force: bool = True) -> str:
    """Compile oracle.c with gcc (-O2, OpenMP, strict IEEE: no fast-math, no FMA
    contraction) into liboracle.so next to the source."""
    if not force and os.path.exists(_LIB) and os.path.getmtime(_LIB) >= os.path.getmtime(_SRC):
        return _LIB
    tmp = _LIB + ".tmp%d" % os.getpid()
    cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp", "-ffp-contract=off",
           "-fno-fast-math", "-o", tmp, _SRC, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, _LIB)
    return _LIB


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
            build()
        L = ctypes.CDLL(_LIB)
        p, i64, i32, d = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_double
        L.orc_num_threads.restype = i32
        L.orc_round_bf16.argtypes = [p, p, i64]
        L.orc_rmsnorm.argtypes = [p, i32, i64, p, i32, p, i64, i64, d]
        L.orc_matmul.argtypes = [p, i32, i64, p, i32, i64, p, i64, i64, i64, i64]
        L.orc_decode_attn.argtypes = [p, i64, p, p, p, i64, p, p, i64, i32, i32, i32, i32, d]
        L.orc_decode_attn_split.argtypes = [p, i64, p, p, p, i64, p, p, i64, i32, i32, i32, i32,
                                             d, i64]
        L.orc_decode_attn_split_groups.argtypes = [p, i64, p, p, p, i64, p, p, i64, i32, i32,
                                                    i32, i32, d, i64, i64]
        L.orc_split_plan.argtypes = [i64, i64, p, i64]
        L.orc_philox4x32_10.argtypes = [p, p, p]
        L.orc_gumbel_noise.argtypes = [ctypes.c_uint64, i64, i64, p]
        L.orc_sample_gumbel.argtypes = [p, i64, i64, i64, p, p, p, p, p, p]
        L.orc_split_plan.restype = i64
        _lib = L
    return _lib


def num_threads() -> int:
    return int(lib().orc_num_threads())


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


def _as(a, dtype_code):
    """Contiguous numpy view with the dtype the C code expects for ``dtype_code``."""
    want = {F32: np.float32, BF16: np.uint16, F64: np.float64}[dtype_code]
    a = np.ascontiguousarray(a)
    if a.dtype != want:
        if dtype_code == BF16 and a.dtype == np.int16:
            a = a.view(np.uint16)
        else:
            raise TypeError(f"expected {want}, got {a.dtype}")
    return a


def _code(a: np.ndarray) -> int:
    if a.dtype == np.float32:
        return F32
    if a.dtype in (np.uint16, np.int16):
        return BF16
    if a.dtype == np.float64:
        return F64
    raise TypeError(a.dtype)


# ---------------------------------------------------------------------------------------
# element conversions
# ---------------------------------------------------------------------------------------

def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bits to float64."""
    b = np.ascontiguousarray(bits).view(np.uint16).astype(np.uint32) << 16
    return b.view(np.float32).astype(np.float64)


def round_bf16(x: np.ndarray) -> np.ndarray:
    """float64 -> nearest bf16 (ties to even) in a single rounding; uint16 bits."""
    x = np.ascontiguousarray(x, dtype=np.float64)
    out = np.empty(x.shape, dtype=np.uint16)
    lib().orc_round_bf16(_ptr(x), _ptr(out), x.size)
    return out


# ---------------------------------------------------------------------------------------
# the three reductions
# ---------------------------------------------------------------------------------------

def rmsnorm(x: np.ndarray, w: np.ndarray, eps: float) -> np.ndarray:
    """y = x * w / sqrt(mean(x^2) + eps) per row, fp64.  x: [rows, H] (fp32 array,
    bf16 uint16 bits, or fp64), w: [H]."""
    x = np.ascontiguousarray(x)
    w = np.ascontiguousarray(w)
    rows, H = x.shape
    assert w.shape == (H,)
    y = np.empty((rows, H), dtype=np.float64)
    lib().orc_rmsnorm(_ptr(x), _code(x), H, _ptr(w), _code(w), _ptr(y), rows, H, float(eps))
    return y


def matmul(A: np.ndarray, W: np.ndarray) -> np.ndarray:
    """C = A @ W.T in fp64, W stored [N, K].  A: [M, K]."""
    A = np.ascontiguousarray(A)
    W = np.ascontiguousarray(W)
    M, K = A.shape
    N, K2 = W.shape
    assert K == K2
    C = np.empty((M, N), dtype=np.float64)
    lib().orc_matmul(_ptr(A), _code(A), K, _ptr(W), _code(W), K, _ptr(C), N, M, N, K)
    return C


def decode_attn(q: np.ndarray, k_cache: np.ndarray, v_cache: np.ndarray,
                block_table: np.ndarray, kv_lens: np.ndarray, scale: float,
                split: int | None = None, group: int = 1) -> np.ndarray:
    """Unsplit decode attention (``split=None``) or the fixed-split-size
    evaluation with log-sum-exp combine (``split=S``), fp64; with ``group=G`` the
    splits are first combined within each group of G consecutive splits and the
    group partials then combined.

    q: [rows, Hq, D] bf16 bits; k_cache: [pages, Hkv, page, D] bf16 bits (token-major
    pages); v_cache: [pages, Hkv, D, page] bf16 bits (head-dim-major pages);
    block_table: [rows, max_pages] int32; kv_lens: [rows] int32 (each >= 1).
    Returns [rows, Hq, D] float64.
    """
    q = _as(q, BF16)
    kc = _as(k_cache, BF16)
    vc = _as(v_cache, BF16)
    bt = np.ascontiguousarray(block_table, dtype=np.int32)
    lens = np.ascontiguousarray(kv_lens, dtype=np.int32)
    rows, hq, d = q.shape
    _, hkv, page, d2 = kc.shape
    assert d == d2 and hq % hkv == 0 and lens.shape == (rows,)
    assert vc.shape == (kc.shape[0], hkv, d, page)
    assert (lens >= 1).all()
    out = np.empty((rows, hq, d), dtype=np.float64)
    args = (_ptr(q), hq * d, _ptr(kc), _ptr(vc), _ptr(bt), bt.shape[1], _ptr(lens), _ptr(out),
            rows, hq, hkv, d, page, float(scale))
    if split is None:
        lib().orc_decode_attn(*args)
    elif group == 1:
        lib().orc_decode_attn_split(*args, int(split))
    else:
        lib().orc_decode_attn_split_groups(*args, int(split), int(group))
    return out


def split_plan(L: int, S: int) -> list[tuple[int, int]]:
    """[(start, end)] of the fixed-size splits of a length-L sequence."""
    cap = max(1, -(-L // S))
    starts = np.zeros(cap, dtype=np.int64)
    n = lib().orc_split_plan(L, S, _ptr(starts), cap)
    return [(int(starts[s]), int(min(starts[s] + S, L))) for s in range(n)]


def silu_mul(g: np.ndarray, u: np.ndarray) -> np.ndarray:
    """SwiGLU gate: silu(g) * u = g / (1 + e^-g) * u, fp64 (element-wise, no
    reduction: batch-invariant by construction, hidekazu-konishi.com section 5.4)."""
    g = np.asarray(g, dtype=np.float64)
    return g / (1.0 + np.exp(-g)) * np.asarray(u, dtype=np.float64)


def argmax_lowest(x: np.ndarray) -> np.ndarray:
    """Row-wise argmax; the lowest index wins a tie."""
    x = np.asarray(x)
    assert not np.isnan(x).any()
    return np.argmax(x, axis=-1)  # numpy returns the first occurrence of the maximum


def philox4x32_10(ctr, key) -> tuple:
    """Philox4x32-10 (Salmon et al., SC 2011) of a 4-word counter and a 2-word key."""
    c = np.ascontiguousarray(np.asarray(ctr, dtype=np.uint32))
    k = np.ascontiguousarray(np.asarray(key, dtype=np.uint32))
    out = np.zeros(4, dtype=np.uint32)
    lib().orc_philox4x32_10(_ptr(c), _ptr(k), _ptr(out))
    return tuple(int(x) for x in out)


def gumbel_noise(seed: int, position: int, n: int) -> np.ndarray:
    """Gumbel noise g_0 .. g_{n-1} of one (seed, position): -ln(-ln u) with u from
    Philox4x32-10 (see orc_gumbel_noise), float64."""
    g = np.zeros(n, dtype=np.float64)
    lib().orc_gumbel_noise(int(seed) & (2**64 - 1), int(position), int(n), _ptr(g))
    return g


def sample_gumbel(logits: np.ndarray, seeds, positions, temperatures):
    """Seeded Gumbel-max sampling per row (hidekazu-konishi.com, section 9.3):
    token = argmax(logit / T + g), greedy when T <= 0.  logits: fp32 [rows, vocab].
    Returns (tokens int32 [rows], best score float64 [rows], gap to the runner-up
    float64 [rows])."""
    x = np.ascontiguousarray(logits, dtype=np.float32)
    rows, vocab = x.shape
    sd = np.ascontiguousarray(np.asarray(seeds, dtype=np.uint64).reshape(rows))
    ps = np.ascontiguousarray(np.asarray(positions, dtype=np.int64).reshape(rows))
    tp = np.ascontiguousarray(np.asarray(temperatures, dtype=np.float32).reshape(rows))
    tok = np.zeros(rows, dtype=np.int32)
    best = np.zeros(rows, dtype=np.float64)
    gap = np.zeros(rows, dtype=np.float64)
    lib().orc_sample_gumbel(_ptr(x), vocab, rows, vocab, _ptr(sd), _ptr(ps), _ptr(tp), _ptr(tok),
                            _ptr(best), _ptr(gap))
    return tok, best, gap
