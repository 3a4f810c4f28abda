"""Pins for the CPU oracle: each check ties an oracle function to something other
than itself -- numbers the pages print, closed forms, invariants, exact rational
brute force, or an independent library routine (numpy / torch CPU fp64) -- so
that a dropped term, a wrong sign or index, or a transposed operand fails here.

Pages: [P1] "Reproducible LLM Inference - Batch Invariance, the Cost of
Determinism, ..." (hidekazu-konishi.com); [P3] "Your Answer Depends on Who Else
Is in the Batch" (praveentn.live).
"""
import math
import struct
from fractions import Fraction

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle
import synth
from tests.conftest import golden_lines, read_golden


def f64(bits):
    return oracle.bf16_to_f64(bits)


# -------------------------------------------------------------------------------------
# bf16 conversion
# -------------------------------------------------------------------------------------

def test_round_bf16_matches_torch_on_fp32_values():
    # library routine: torch's fp32 -> bf16 conversion is round-to-nearest-even;
    # on values that are exactly fp32 there is no double-rounding question.
    g = torch.Generator().manual_seed(11)
    x = torch.randn(200000, generator=g, dtype=torch.float32) * torch.exp(
        torch.randn(200000, generator=g) * 20)
    ref = x.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = oracle.round_bf16(x.double().numpy())
    assert np.array_equal(got, ref)


@pytest.mark.parametrize("x,bits", [
    (1.0, 0x3F80),
    (1.0 + 2.0 ** -8, 0x3F80),                  # exact midpoint -> even (down)
    (1.0 + 3 * 2.0 ** -8, 0x3F82),              # exact midpoint -> even (up)
    (1.0 + 2.0 ** -8 + 2.0 ** -40, 0x3F81),     # just above midpoint: a pass through
                                                # fp32 would land on the midpoint and
                                                # round to even (0x3F80): double rounding
    (-(1.0 + 2.0 ** -8 + 2.0 ** -40), 0xBF81),
    (2.0 ** -133, 0x0001),                      # smallest subnormal
    (2.0 ** -134, 0x0000),                      # half of it: tie -> even (zero)
    (3 * 2.0 ** -135, 0x0001),                  # 0.75 step -> 1
    (3.3895313892515355e38, 0x7F7F),            # largest finite
    (3.3961775292304957e38, 0x7F80),            # at the midpoint above it -> inf
    (float("inf"), 0x7F80),
    (-0.0, 0x8000),
])
def test_round_bf16_closed_forms(x, bits):
    assert int(oracle.round_bf16(np.array([x]))[0]) == bits


def test_round_bf16_nan():
    b = int(oracle.round_bf16(np.array([float("nan")]))[0])
    assert (b & 0x7F80) == 0x7F80 and (b & 0x007F) != 0


# -------------------------------------------------------------------------------------
# RMSNorm
# -------------------------------------------------------------------------------------

def test_rmsnorm_p3_worked_example_exact_sum():
    # [P3] "A Concrete Example" step 1: x_1^2 = 1, 4095 squares of 3e-8, exact total
    # 1.00012285.  With w = 1 and eps = 0 the first output is 1 / sqrt(total / H).
    gd = read_golden("p3_rmsnorm_example.txt")
    H = int(gd["hidden"])
    x = np.full(H, math.sqrt(gd["small_sq"]), dtype=np.float64)
    x[0] = 1.0
    y = oracle.rmsnorm(x[None, :], np.ones(H), 0.0)[0]
    expect = 1.0 / math.sqrt(gd["exact_sum"] / H)
    assert abs(y[0] - expect) / expect < 1e-12
    # the page's sequential-fp32 sum (1.0) would move the scale by ~6e-5 relative
    seq_scale = 1.0 / math.sqrt(gd["sequential_fp32"] / H)
    assert abs(seq_scale - expect) / expect == pytest.approx(gd["scale_rel_diff"], rel=0.05)


def test_p3_rmsnorm_example_fp32_models():
    # The page's step-2 and step-3 numbers reproduce with an fp32 model of the two
    # reduction layouts; this fixes what the kernel must avoid (a single sequential
    # accumulator) and what a tree achieves.
    gd = read_golden("p3_rmsnorm_example.txt")
    H = int(gd["hidden"])
    sq = np.full(H, np.float32(gd["small_sq"]), dtype=np.float32)
    sq[0] = np.float32(1.0)
    acc = np.float32(0.0)
    for v in sq:
        acc = np.float32(acc + v)
    assert acc == np.float32(gd["sequential_fp32"])

    def tree(v):
        v = list(v)
        while len(v) > 1:
            v = [np.float32(v[i] + v[i + 1]) for i in range(0, len(v), 2)]
        return v[0]

    nb, bl = int(gd["blocks"]), int(gd["block_len"])
    # block 0: the shuffle tree pairs the small values first, the large one last
    b0 = np.float32(tree(sq[1:bl].tolist() + [np.float32(0.0)]) + sq[0])
    assert abs(float(b0) - gd["block0"]) < 1e-7
    others = [tree(sq[i * bl:(i + 1) * bl]) for i in range(1, nb)]
    assert abs(float(others[0]) - gd["small_block"]) < 1e-8
    total = tree([b0] + others)
    assert abs(float(total) - gd["tree_fp32"]) < 1.5e-7


def test_p3_absorption_fp32_model():
    gd = read_golden("p3_absorption.txt")
    n = int(gd["n_small"])
    small = np.float32(gd["small"])
    acc = np.float32(1.0)
    for _ in range(n):
        acc = np.float32(acc + small)
    assert acc == np.float32(gd["sequential"])
    s = np.float32(0.0)
    for _ in range(n):
        s = np.float32(s + small)
    split = np.float32(s + np.float32(1.0))
    assert abs(float(split) - gd["split"]) < 1e-7
    ulps = (float(split) - 1.0) / 2.0 ** -23
    assert abs(ulps - gd["ulp_difference_approx"]) <= 1
    assert float(small) < gd["half_ulp_threshold"]


def test_rmsnorm_vs_torch_library():
    g = torch.Generator().manual_seed(3)
    x = torch.randn(37, 300, generator=g, dtype=torch.float64) * 3
    w = torch.randn(300, generator=g, dtype=torch.float64)
    ref = F.rms_norm(x, (300,), w, eps=1e-6).numpy()
    got = oracle.rmsnorm(x.numpy(), w.numpy(), 1e-6)
    assert np.abs(got - ref).max() <= 1e-13 * np.abs(ref).max()


@pytest.mark.parametrize("H", [1, 5, 256, 4096])
@pytest.mark.parametrize("a", [1e-4, 0.5, 3.0])
def test_rmsnorm_constant_row_closed_form(H, a):
    # constant row a, w = 1: mean of squares is a^2, so y = a / sqrt(a^2 + eps)
    eps = 1e-6
    y = oracle.rmsnorm(np.full((1, H), a), np.ones(H), eps)
    assert np.allclose(y, a / math.sqrt(a * a + eps), rtol=1e-14, atol=0)


def test_rmsnorm_exact_rational_bruteforce():
    # tiny rows of bf16 values: the sum of squares as an exact fraction, the root
    # and quotient in 60-digit decimal arithmetic
    from decimal import Decimal, getcontext
    getcontext().prec = 60
    x = synth.normal((4, 13), seed=21)
    w = synth.normal((13,), seed=22, std=0.1, mean=1.0)
    xb, wb = synth.bf16_bits(x), synth.bf16_bits(w)
    eps = Fraction(1, 10 ** 6)
    got = oracle.rmsnorm(xb, wb, 1e-6)
    xs, ws = f64(xb), f64(wb)
    for r in range(4):
        ss = sum(Fraction(float(v)) ** 2 for v in xs[r])
        ms = ss / 13 + Fraction(1e-6)  # eps as the double the oracle receives
        den = Decimal(ms.numerator) / Decimal(ms.denominator)
        den = den.sqrt()
        for i in range(13):
            ref = Decimal(float(xs[r, i])) * Decimal(float(ws[i])) / den
            assert abs(Decimal(got[r, i]) - ref) <= abs(ref) * Decimal(1e-15) + Decimal(1e-300)
    assert eps  # (eps written as a fraction for the reader)


def test_rmsnorm_scale_invariance_and_row_independence():
    x = np.random.default_rng(4).standard_normal((6, 64))
    w = np.random.default_rng(5).standard_normal(64)
    y = oracle.rmsnorm(x, w, 0.0)
    y2 = oracle.rmsnorm(x * 7.5, w, 0.0)
    assert np.allclose(y, y2, rtol=1e-13)
    # each row is a function of that row only
    y3 = oracle.rmsnorm(x[[3]], w, 0.0)
    assert np.array_equal(y3[0], y[3])


def test_rmsnorm_f32_and_bf16_inputs():
    x = synth.normal((3, 40), seed=9, dtype=torch.float32)
    w = synth.normal((40,), seed=10, dtype=torch.float32)
    a = oracle.rmsnorm(x.numpy(), w.numpy(), 1e-6)
    b = oracle.rmsnorm(x.double().numpy(), w.double().numpy(), 1e-6)
    assert np.array_equal(a, b)
    xb = x.to(torch.bfloat16)
    c = oracle.rmsnorm(synth.bf16_bits(xb), w.numpy(), 1e-6)
    d = oracle.rmsnorm(xb.double().numpy(), w.double().numpy(), 1e-6)
    assert np.array_equal(c, d)


# -------------------------------------------------------------------------------------
# Matmul
# -------------------------------------------------------------------------------------

@pytest.mark.parametrize("M,N,K", [(1, 7, 5), (9, 3, 33), (17, 40, 64)])
def test_matmul_vs_numpy_library(M, N, K):
    A = synth.normal((M, K), seed=M, dtype=torch.bfloat16)
    W = synth.normal((N, K), seed=N + 100, dtype=torch.bfloat16)
    got = oracle.matmul(synth.bf16_bits(A), synth.bf16_bits(W))
    ref = A.double().numpy() @ W.double().numpy().T       # W is [N, K]: C = A W^T
    assert got.shape == (M, N)
    assert np.abs(got - ref).max() <= 1e-13 * max(1.0, np.abs(ref).max())


def test_matmul_integer_exact():
    A = synth.integer_valued((11, 48), seed=1)
    W = synth.integer_valued((13, 48), seed=2)
    got = oracle.matmul(synth.bf16_bits(A), synth.bf16_bits(W))
    ref = (A.to(torch.int64) @ W.to(torch.int64).T).numpy()
    assert np.array_equal(got, ref.astype(np.float64))


def test_matmul_fraction_bruteforce():
    A = synth.normal((3, 16), seed=31)
    W = synth.normal((4, 16), seed=32)
    a, w = f64(synth.bf16_bits(A)), f64(synth.bf16_bits(W))
    got = oracle.matmul(synth.bf16_bits(A), synth.bf16_bits(W))
    for m in range(3):
        for n in range(4):
            ex = sum(Fraction(float(a[m, k])) * Fraction(float(w[n, k])) for k in range(16))
            assert abs(Fraction(got[m, n]) - ex) <= abs(ex) * Fraction(1, 10 ** 14) + Fraction(1, 10 ** 300)


def test_matmul_transposed_operand_is_caught():
    # a non-square W makes the [N, K] layout observable: swapping the role of the
    # operands cannot produce a result of the right shape and values
    A = np.arange(6, dtype=np.float64).reshape(2, 3)
    W = np.array([[1.0, 0.0, 0.0], [0.0, 0.0, 1.0], [1.0, 1.0, 1.0], [0.0, 2.0, 0.0]])
    C = oracle.matmul(A, W)
    assert np.array_equal(C, np.array([[0.0, 2.0, 3.0, 2.0], [3.0, 5.0, 12.0, 8.0]]))


# -------------------------------------------------------------------------------------
# Decode attention
# -------------------------------------------------------------------------------------

def _kv(lens, hkv=2, d=16, page=4, seed=0):
    return synth.paged_kv(lens, hkv, d, page, seed=seed)


def _attn(q, kv, scale, split=None, group=1):
    return oracle.decode_attn(synth.bf16_bits(q), synth.bf16_bits(kv.k_cache),
                              synth.bf16_bits(kv.v_cache), kv.block_table.numpy(),
                              kv.kv_lens.numpy(), scale, split=split, group=group)


def _gather(kv, r):
    """Logical [L, Hkv, D] K and V of request r, gathered page by page (test helper)."""
    L = int(kv.kv_lens[r])
    pg = kv.page_size
    ks, vs = [], []
    for j in range(L):
        p = int(kv.block_table[r, j // pg])
        ks.append(kv.k_cache[p, :, j % pg, :])
        vs.append(kv.v_cache[p, :, :, j % pg])
    return torch.stack(ks).double(), torch.stack(vs).double()


def test_decode_attn_vs_torch_sdpa_library():
    lens = [1, 4, 5, 17, 33]
    hq, hkv, d = 6, 2, 16
    kv = _kv(lens, hkv=hkv, d=d)
    q = synth.normal((len(lens), hq, d), seed=7)
    scale = 1.0 / math.sqrt(d)
    got = _attn(q, kv, scale)
    for r in range(len(lens)):
        K, V = _gather(kv, r)                           # [L, Hkv, D]
        Kh = K.permute(1, 0, 2).repeat_interleave(hq // hkv, 0)   # [Hq, L, D]
        Vh = V.permute(1, 0, 2).repeat_interleave(hq // hkv, 0)
        ref = F.scaled_dot_product_attention(q[r].double()[:, None, :], Kh, Vh, scale=scale)
        assert np.abs(got[r] - ref[:, 0, :].numpy()).max() < 1e-13


def test_decode_attn_single_token_is_v0():
    kv = _kv([1, 1], hkv=2, d=8)
    q = synth.normal((2, 4, 8), seed=3)
    got = _attn(q, kv, 0.3)
    for r in range(2):
        _, V = _gather(kv, r)
        for h in range(4):
            assert np.array_equal(got[r, h], V[0, h // 2].numpy())


def test_decode_attn_equal_keys_give_mean_and_weights_sum_to_one():
    kv = _kv([9, 30], hkv=1, d=8)
    kv.k_cache[:] = 0.5                       # every key identical -> uniform softmax
    q = synth.normal((2, 3, 8), seed=4)
    got = _attn(q, kv, 0.25)
    for r in range(2):
        _, V = _gather(kv, r)
        mean = V[:, 0].mean(0).numpy()
        assert np.allclose(got[r], mean[None, :], rtol=0, atol=1e-14)
    # V == 1 everywhere: the output is the sum of the weights
    kv2 = _kv([7, 40], hkv=1, d=8, seed=5)
    kv2.v_cache[:] = 1.0
    out = _attn(synth.normal((2, 2, 8), seed=6), kv2, 0.7)
    assert np.abs(out - 1.0).max() <= 1e-12


def test_decode_attn_two_token_closed_form():
    # two keys whose scores differ by delta: weight of token 1 is sigmoid(delta)
    kv = _kv([2], hkv=1, d=4, page=4)
    p = int(kv.block_table[0, 0])
    kv.k_cache[p, 0, 0] = torch.tensor([1.0, 0, 0, 0])
    kv.k_cache[p, 0, 1] = torch.tensor([0, 1.0, 0, 0])
    kv.v_cache[p, 0, :, 0] = torch.tensor([1.0, 0, 0, 0])
    kv.v_cache[p, 0, :, 1] = torch.tensor([0, 1.0, 0, 0])
    q = torch.tensor([[[2.0, -1.0, 0, 0]]]).to(torch.bfloat16)
    scale = 0.5
    got = _attn(q, kv, scale)[0, 0]
    delta = scale * (2.0 - (-1.0))           # s0 - s1
    w0 = 1.0 / (1.0 + math.exp(-delta))
    assert abs(got[0] - w0) < 1e-15 and abs(got[1] - (1 - w0)) < 1e-15
    assert got[2] == 0 and got[3] == 0


def test_decode_attn_gqa_head_mapping():
    # V constant per kv head g (value g + 1): query head h must read kv head
    # h // (Hq / Hkv), contiguous groups
    hq, hkv = 8, 4
    kv = _kv([13, 21], hkv=hkv, d=8)
    for g in range(hkv):
        kv.v_cache[:, g] = float(g + 1)
    got = _attn(synth.normal((2, hq, 8), seed=8), kv, 0.4)
    for h in range(hq):
        assert np.allclose(got[:, h], float(h // (hq // hkv) + 1), rtol=0, atol=1e-14)


def test_decode_attn_block_table_indexing():
    # equal keys, V[j] = j in dim 0: the output is the mean of 0..L-1 = (L-1)/2 only
    # if every logical token is fetched through the right page and slot
    lens = [1, 6, 23, 64]
    kv = _kv(lens, hkv=1, d=4, page=4)
    kv.k_cache[:] = 1.0
    pg = kv.page_size
    for r, L in enumerate(lens):
        for j in range(L):
            kv.v_cache[int(kv.block_table[r, j // pg]), 0, 0, j % pg] = float(j)
    got = _attn(synth.normal((len(lens), 1, 4), seed=2), kv, 1.0)
    for r, L in enumerate(lens):
        assert abs(got[r, 0, 0] - (L - 1) / 2.0) < 1e-12


def test_decode_attn_page_permutation_is_exactly_neutral():
    lens = [5, 17, 63]
    a = _kv(lens, hkv=1, d=16, page=4, seed=0)
    b = synth.paged_kv(lens, 1, 16, 4, seed=0, page_seed=99)
    # same logical content under a different physical placement
    for r, L in enumerate(lens):
        for j in range(-(-L // 4)):
            b.k_cache[int(b.block_table[r, j])] = a.k_cache[int(a.block_table[r, j])]
            b.v_cache[int(b.block_table[r, j])] = a.v_cache[int(a.block_table[r, j])]
    q = synth.normal((3, 4, 16), seed=1)
    assert np.array_equal(_attn(q, a, 0.25), _attn(q, b, 0.25))


@pytest.mark.parametrize("S", [1, 7, 16, 256, 10 ** 6])
def test_split_merge_equals_unsplit(S):
    lens = [1, 16, 17, 300, 1000]
    kv = _kv(lens, hkv=2, d=16, page=16)
    q = synth.normal((len(lens), 4, 16), seed=12)
    full = _attn(q, kv, 0.25)
    split = _attn(q, kv, 0.25, split=S)
    assert np.abs(split - full).max() <= 1e-12 * np.abs(full).max()


@pytest.mark.parametrize("S,G", [(16, 2), (16, 4), (64, 4), (256, 4), (7, 3), (16, 64)])
def test_grouped_split_merge_equals_unsplit(S, G):
    # the two-level combine the GPU kernels use (splits folded within fixed groups of
    # G consecutive splits, then the groups) reaches the unsplit softmax as well;
    # lengths end on, before and after group boundaries
    lens = [1, 16, 17, 63, 64, 65, 300, 1000]
    kv = _kv(lens, hkv=2, d=16, page=16)
    q = synth.normal((len(lens), 4, 16), seed=13)
    full = _attn(q, kv, 0.25)
    grouped = _attn(q, kv, 0.25, split=S, group=G)
    assert np.abs(grouped - full).max() <= 1e-12 * np.abs(full).max()
    # the grouping only reassociates the combine: it matches the one-level split
    # combine to the same bound
    ref_split = _attn(q, kv, 0.25, split=S)
    assert np.abs(grouped - ref_split).max() <= 1e-12 * np.abs(full).max()


def test_decode_attn_ignores_stale_slots():
    # NaN in every slot past the length and in the poison page: never read
    kv = _kv([3, 10], hkv=1, d=8, page=4)
    out = _attn(synth.normal((2, 2, 8), seed=1), kv, 0.5)
    assert np.isfinite(out).all()


# -------------------------------------------------------------------------------------
# Split plan and prefill blocking
# -------------------------------------------------------------------------------------

def test_split_plan_golden():
    for line in golden_lines("split_plan.txt"):
        parts = line.split()
        if parts[0] == "count4":
            L = int(parts[1])
            lens = [int(x) for x in parts[3:]]
            # the contrast case: a fixed count of four splits the same L differently
            assert [len(c) for c in np.array_split(np.arange(L), 4)] == lens
            continue
        if parts[0] == "key":
            key, start = int(parts[1]), int(parts[3])
            for L in range(key + 1, 2049):
                plan = oracle.split_plan(L, 256)
                assert [s for s, e in plan if s <= key < e] == [start]
            continue
        L, S = int(parts[0]), int(parts[1])
        lens = [int(x) for x in parts[3:]]
        assert [e - s for s, e in oracle.split_plan(L, S)] == lens


def test_split_plan_boundaries_depend_only_on_length():
    for L in range(1, 3000, 7):
        plan = oracle.split_plan(L, 256)
        assert plan[0][0] == 0 and plan[-1][1] == L
        assert all(s % 256 == 0 for s, _ in plan)
        assert all(e - s == 256 for s, e in plan[:-1])
        # growing L never moves a completed boundary
        plan2 = oracle.split_plan(L + 300, 256)
        assert plan2[: len(plan) - 1] == plan[:-1]


def test_prefill_blocking_golden():
    gd = read_golden("prefill_blocks.txt")
    blk, cached, new = int(gd["block"]), int(gd["cached"]), int(gd["new"])
    separate = len(oracle.split_plan(cached, blk)) + len(oracle.split_plan(new, blk))
    whole = len(oracle.split_plan(cached + new, blk))
    assert separate == gd["separate_blocks"] and whole == gd["whole_blocks"]


# -------------------------------------------------------------------------------------
# element-wise pieces of the decode layer
# -------------------------------------------------------------------------------------

def test_silu_mul_vs_torch():
    g = torch.randn(1000, dtype=torch.float64) * 4
    u = torch.randn(1000, dtype=torch.float64)
    ref = (F.silu(g) * u).numpy()
    assert np.allclose(oracle.silu_mul(g.numpy(), u.numpy()), ref, rtol=1e-14, atol=1e-300)


def test_argmax_lowest_index_on_ties():
    x = np.array([[1.0, 3.0, 3.0, 2.0], [5.0, 5.0, 5.0, 5.0], [-1.0, -2.0, -1.0, -3.0]],
                 dtype=np.float32)
    assert list(oracle.argmax_lowest(x)) == [1, 0, 0]
