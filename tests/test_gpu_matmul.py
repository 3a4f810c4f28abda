"""GPU tests of matmul_bi / matmul_tuned: parity with the CPU oracle (exact on
integer inputs, max|C - ref| <= 2e-2 * RMS(ref) on normal inputs) and bitwise
batch invariance over M, position and neighbours.
"""
import numpy as np
import pytest
import torch

import invariant_rmsnorm_bi_amd as rbi
import oracle
import synth

pytestmark = pytest.mark.gpu
DEV = "cuda"
QKV = (9216, 4096)     # [N, K] of the attention QKV projection
OPROJ = (4096, 8192)   # [N, K] of o_proj


def _tol_ok(c: torch.Tensor, ref: np.ndarray) -> tuple:
    """max|C - ref| <= 2e-2 * RMS(ref) over the call; also prints the distance from the
    reference rounded once to C's type (for bf16 output that rounding alone is up to
    half a bf16 step of the largest |C|, most of the measured ratio)."""
    cc = c.double().cpu().numpy()
    err = np.abs(cc - ref).max()
    rms = np.sqrt(np.mean(ref ** 2))
    rr = oracle.bf16_to_f64(oracle.round_bf16(ref)) if c.dtype == torch.bfloat16 else ref
    print(f"parity matmul {tuple(c.shape)}: max|C - ref| / RMS = {err / rms:.4g}, "
          f"max|C - RNE(ref)| / RMS = {np.abs(cc - rr).max() / rms:.4g}; bar 0.02", flush=True)
    return err <= 2e-2 * rms, err, rms


def test_c1_parity_and_rows_bitwise_across_batch():
    A = synth.normal((8, 256), seed=synth.SEED_DATA)
    W = synth.normal((512, 256), std=0.02, seed=synth.SEED_WEIGHTS)
    ref = oracle.matmul(synth.bf16_bits(A), synth.bf16_bits(W))
    Ag, Wg = A.to(DEV), W.to(DEV)
    outs = {}
    for B in (1, 3, 8):
        c = rbi.matmul_bi(Ag[:B].contiguous(), Wg)
        ok, err, rms = _tol_ok(c, ref[:B])
        assert ok, (B, err, rms)
        outs[B] = c
    assert torch.equal(outs[3][:1], outs[1]) and torch.equal(outs[8][:3], outs[3])
    for r in range(8):
        assert torch.equal(rbi.matmul_bi(Ag[r:r + 1].contiguous(), Wg)[0], outs[8][r])


SMALL_EXACT_CASES = [(1, 512, 256), (17, 4096, 4096), (130, 260, 1032),
                     (257, 9216, 512), (64, 128, 8), (300, 260, 576),
                     (600, 1004, 128),
                     # the register-streaming tile (M <= 16, <= 256 tiles of 16
                     # columns): ragged N, a single k step, a step count that
                     # is not a multiple of its ring, M at its limit
                     (5, 20, 32), (3, 36, 4000), (16, 4096, 352),
                     # the two-wave 32 x 32 tile (33 <= M <= 64, N <= 4096):
                     # ragged M and N
                     (40, 100, 320), (64, 4096, 1024),
                     # the 32 x 16 LDS tile (9 <= M <= 32, more than 1024 16 x 16 tiles)
                     (24, 24576, 256)]


@pytest.mark.parametrize("M,N,K", SMALL_EXACT_CASES)
@pytest.mark.parametrize("out_dtype", [torch.bfloat16, torch.float32])
def test_integer_inputs_exact(M, N, K, out_dtype):
    # integers in [-4, 4]: every partial sum is an integer below 2^24, so fp32 is exact
    # in any order and the result must equal the oracle's rounded value bit for bit
    A = synth.integer_valued((M, K), seed=M + K)
    W = synth.integer_valued((N, K), seed=N + 1)
    ref = oracle.matmul(synth.bf16_bits(A), synth.bf16_bits(W))
    c = rbi.matmul_bi(A.to(DEV), W.to(DEV), out_dtype=out_dtype).cpu()
    if out_dtype == torch.float32:
        assert np.array_equal(c.double().numpy(), ref)
    else:
        assert np.array_equal(synth.bf16_bits(c), oracle.round_bf16(ref))
    ct = rbi.matmul_tuned(A.to(DEV), W.to(DEV), out_dtype=out_dtype).cpu()
    assert torch.equal(ct, c)


# Full-size integer cases through the multi-wave tiles the large-M plans launch: each
# (M, N, K) with the launches matmul_bi makes for it (matmul_bi_plan).  Together with
# the cases of test_integer_inputs_exact they reach every tile shape of the plan table
# (checked on the CPU by tests/test_capi_host.py).
BIG_EXACT_CASES = [
    ((4096, 9216, 4096), ((256, 256, 0), 8192, (128, 128, 0))),   # QKV: column split
    ((2048, 9216, 4096), ((256, 256, 0), 8192, (128, 64, 0))),    # other right-hand tile
    ((4096, 4096, 8192), ((256, 256, 0), 4096, None)),            # o_proj: one launch
    ((768, 9216, 4096), ((256, 128, 0), 9216, None)),
    ((1024, 4096, 8192), ((128, 128, 0), 4096, None)),
    ((1536, 4096, 8192), ((256, 128, 0), 4096, None)),
    ((509, 4096, 8192), ((128, 64, 0), 4096, None)),
    # K = 32 mod 64: every LDS tile shape in its 32-k-stage kernel (the shapes above
    # run the 64-k-stage kernel)
    ((4096, 4096, 4128), ((256, 256, 0), 4096, None)),
    ((1536, 4096, 4128), ((256, 128, 0), 4096, None)),
    ((600, 4096, 4128), ((128, 128, 0), 4096, None)),
    ((300, 4096, 4128), ((128, 64, 0), 4096, None)),
    ((130, 4096, 4128), ((64, 64, 0), 4096, None)),
    ((65, 4096, 4128), ((64, 32, 0), 4096, None)),
    ((33, 4096, 4128), ((32, 32, 0), 4096, None)),
    ((17, 9216, 4128), ((32, 16, 0), 9216, None)),
    ((17, 4096, 4128), ((16, 16, 0), 4096, None)),
]


@pytest.mark.parametrize("mnk,plan", BIG_EXACT_CASES, ids=lambda v: str(v))
def test_integer_exact_big_tiles(mnk, plan):
    # integers in [-4, 4]: |partial sums| <= 16 K <= 2^17, exact in fp32 in any order,
    # so sampled rows must equal the oracle bit for bit; rows on both sides of tile
    # boundaries, every column (both sides of the column split included)
    M, N, K = mnk
    got = rbi.matmul_bi_plan(M, N, K)
    assert (got["first"], got["n1"], got["second"]) == plan
    A = synth.integer_valued((M, K), seed=7 * M + K)
    W = synth.integer_valued((N, K), seed=N + 3)
    Ag, Wg = A.to(DEV), W.to(DEV)
    c32 = rbi.matmul_bi(Ag, Wg, out_dtype=torch.float32)
    c16 = rbi.matmul_bi(Ag, Wg)
    rng = np.random.default_rng(M + N)
    rows = sorted({0, 1, 15, 16, 63, 64, 127, 128, 255, 256, M // 2, M - 2, M - 1} |
                  set(rng.integers(0, M, 3).tolist()))
    rows = [r for r in rows if r < M]
    ref = oracle.matmul(synth.bf16_bits(A[rows]), synth.bf16_bits(W))
    assert np.array_equal(c32[rows].double().cpu().numpy(), ref)
    assert np.array_equal(synth.bf16_bits(c16[rows]), oracle.round_bf16(ref))


# the twin's split-K schedules (one per row of its table, plus a K = 32 mod 64 split
# that runs its ranges in 32-k stages): (M, N, K) and the expected number of K ranges
TWIN_EXACT_CASES = [((16, 4096, 8192), 2), ((32, 4096, 8192), 2), ((64, 4096, 8192), 4),
                    ((127, 4096, 8192), 4), ((200, 4096, 8192), 2), ((509, 4096, 14336), 4),
                    ((768, 4096, 14336), 4), ((160, 9216, 4096), 2), ((32, 24576, 4096), 2),
                    ((64, 4096, 8224), 4)]


@pytest.mark.parametrize("mnk,splits", TWIN_EXACT_CASES, ids=lambda v: str(v))
def test_integer_exact_twin_splits(mnk, splits):
    # integers in [-4, 4]: each K range's partial sums and their fp32 sum are exact,
    # so the split-K twin must equal the oracle bit for bit on sampled rows (tile
    # boundaries included), like matmul_bi
    M, N, K = mnk
    assert rbi.matmul_tuned_workspace_size(M, N, K) == splits * M * N * 4
    A = synth.integer_valued((M, K), seed=5 * M + K)
    W = synth.integer_valued((N, K), seed=N + 7)
    Ag, Wg = A.to(DEV), W.to(DEV)
    c32 = rbi.matmul_tuned(Ag, Wg, out_dtype=torch.float32)
    c16 = rbi.matmul_tuned(Ag, Wg)
    rows = sorted({0, 1, 15, 16, 63, 64, 127, 128, M // 2, M - 2, M - 1})
    rows = [r for r in rows if r < M]
    ref = oracle.matmul(synth.bf16_bits(A[rows]), synth.bf16_bits(W))
    assert np.array_equal(c32[rows].double().cpu().numpy(), ref)
    assert np.array_equal(synth.bf16_bits(c16[rows]), oracle.round_bf16(ref))


@pytest.mark.parametrize("shape", [QKV, OPROJ])
@pytest.mark.parametrize("M", [1, 7, 64, 127, 256])
def test_c3_parity_normal_inputs(shape, M):
    N, K = shape
    A = synth.normal((M, K), seed=1000 + M)   # not a weight seed: keeps A and W independent
    W = synth.normal((N, K), std=0.02, seed=synth.SEED_WEIGHTS)
    ref = oracle.matmul(synth.bf16_bits(A), synth.bf16_bits(W))
    Ag, Wg = A.to(DEV), W.to(DEV)
    for fn in (rbi.matmul_bi, rbi.matmul_tuned):
        ok, err, rms = _tol_ok(fn(Ag, Wg), ref)
        assert ok, (fn.__name__, err, rms)


@pytest.mark.parametrize("shape", [QKV, OPROJ])
def test_c3_sampled_rows_at_m4096(shape):
    N, K = shape
    M = 4096
    A = synth.normal((M, K), seed=11)
    W = synth.normal((N, K), std=0.02, seed=synth.SEED_WEIGHTS)
    c = rbi.matmul_bi(A.to(DEV), W.to(DEV))
    rows = [0, 1, 127, 128, 2047, 4095]
    ref = oracle.matmul(synth.bf16_bits(A[rows]), synth.bf16_bits(W))
    ok, err, rms = _tol_ok(c[rows], ref)
    assert ok, (err, rms)


@pytest.mark.parametrize("shape", [QKV, OPROJ])
def test_every_position_same_bits(shape):
    # one row repeated M = 4096 times: every tile, wave and MFMA slot must produce the
    # bits the row gets alone
    N, K = shape
    p = synth.normal((1, K), seed=21).to(DEV)
    W = synth.normal((N, K), std=0.02, seed=synth.SEED_WEIGHTS).to(DEV)
    alone = rbi.matmul_bi(p, W)
    full = rbi.matmul_bi(p.repeat(4096, 1), W)
    assert torch.equal(full, alone.expand_as(full))


@pytest.mark.parametrize("shape", [QKV, OPROJ])
def test_rows_bitwise_over_m_sweep(shape):
    # M = 1..4096 (every value: odd, prime and tile-straddling M included); probe rows
    # at the first, last and a seeded random position among N(0,1) neighbours
    N, K = shape
    pool = synth.normal((4096, K), seed=31).to(DEV)
    W = synth.normal((N, K), std=0.02, seed=synth.SEED_WEIGHTS).to(DEV)
    probe = synth.normal((1, K), seed=32).to(DEV)
    alone = rbi.matmul_bi(probe, W)[0]
    out = torch.empty((4096, N), dtype=torch.bfloat16, device=DEV)
    rng = np.random.default_rng(synth.SEED_BATCH)
    bad = torch.zeros((), dtype=torch.int64, device=DEV)
    for M in range(1, 4097):
        pos = int(rng.integers(0, M)) if M % 3 else (M - 1 if M % 2 else 0)
        keep = pool[pos].clone()
        pool[pos] = probe[0]
        rbi.matmul_bi(pool[:M], W, out=out[:M])
        bad += (out[pos] != alone).sum()
        pool[pos] = keep
    assert int(bad) == 0


def test_p1_batch_slice_example():
    # hidekazu-konishi.com section 3.3: row 0 of a[:1] @ b versus row 0 of a @ b with
    # linspace matrices (here bf16 inputs, fp32 output, b stored as W = b^T [N, K]).
    # The invariant kernel must give exactly 0 difference.
    B, D = 2048, 4096
    a = synth.linspace_matrix(B, D, dtype=torch.bfloat16).to(DEV)
    W = synth.linspace_matrix(D, D, dtype=torch.bfloat16).T.contiguous().to(DEV)
    one = rbi.matmul_bi(a[:1], W, out_dtype=torch.float32)
    full = rbi.matmul_bi(a, W, out_dtype=torch.float32)[:1]
    assert float((one - full).abs().max()) == 0.0
    # the split-K twin is free to change with the batch.  At this N = 4096, K = 4096 it
    # runs matmul_bi's plan at both sizes, so the twin is shown on a linspace W four
    # times as wide, where it splits K in two at M <= 16 and not at M = 2048.
    W2 = synth.linspace_matrix(D, 4 * D, dtype=torch.bfloat16).T.contiguous().to(DEV)
    assert rbi.matmul_tuned_differs(1, 4 * D, D) and not rbi.matmul_tuned_differs(B, 4 * D, D)
    t_one = rbi.matmul_tuned(a[:1], W2, out_dtype=torch.float32)
    t_full = rbi.matmul_tuned(a, W2, out_dtype=torch.float32)[:1]
    assert float((t_one - t_full).abs().max()) > 0.0, "inputs lack the power to show a change"


@pytest.mark.parametrize("shape,m_small", [(OPROJ, 64), (QKV, 160)])
def test_tuned_twin_sensitivity_normal_inputs(shape, m_small):
    # the twin splits K at these M (o_proj: four ranges, QKV: two) and not at M = 4096,
    # so a row's bits move with the batch; matmul_bi's do not
    N, K = shape
    assert rbi.matmul_tuned_differs(m_small, N, K) and not rbi.matmul_tuned_differs(4096, N, K)
    pool = synth.normal((4096, K), seed=41).to(DEV)
    W = synth.normal((N, K), std=0.02, seed=synth.SEED_WEIGHTS).to(DEV)
    small = rbi.matmul_tuned(pool[:m_small], W, out_dtype=torch.float32)[:1]
    big = rbi.matmul_tuned(pool, W, out_dtype=torch.float32)[:1]
    assert not torch.equal(small, big)
    assert torch.equal(rbi.matmul_bi(pool[:m_small], W, out_dtype=torch.float32)[:1],
                       rbi.matmul_bi(pool, W, out_dtype=torch.float32)[:1])


def test_run_to_run_1000():
    # hidekazu-konishi.com section 4.2: the same bf16 2048x2048 product 1000 times
    A = synth.normal((2048, 2048), seed=51).to(DEV)
    W = synth.normal((2048, 2048), seed=52).to(DEV)
    ref = rbi.matmul_bi(A, W)
    out = torch.empty_like(ref)
    diff = torch.zeros((), dtype=torch.int64, device=DEV)
    for _ in range(1000):
        rbi.matmul_bi(A, W, out=out)
        diff += (out != ref).sum()
    assert int(diff) == 0


def test_strided_views():
    # A and C as column slices of wider buffers (row strides > K, > N)
    A = synth.normal((40, 512), seed=61).to(DEV)
    W = synth.normal((96, 256), std=0.02, seed=62).to(DEV)
    out = torch.zeros((40, 200), dtype=torch.float32, device=DEV)
    c = rbi.matmul_bi(A[:, 128:384], W, out_dtype=torch.float32, out=out[:, 100:196])
    ref = oracle.matmul(synth.bf16_bits(A[:, 128:384].contiguous()), synth.bf16_bits(W))
    ok, err, rms = _tol_ok(c, ref)
    assert ok
    assert float(out[:, :100].abs().max()) == 0 and float(out[:, 196:].abs().max()) == 0
