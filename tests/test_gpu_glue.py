"""GPU tests of the decode layer's glue kernels against the CPU oracle's plain
definitions: embedding gather (bit-exact), residual add and SwiGLU (the exact
result rounded to bf16, within one bf16 step where the kernel's fp32
intermediate rounds first), and the greedy row argmax (exact: the maximum, the
lowest index holding it, NaN never chosen), on the vectorised and the scalar
paths, with ragged lengths.
"""
import numpy as np
import pytest
import torch

import invariant_rmsnorm_bi_amd as rbi
import oracle
import synth

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _bits(t):
    return synth.bf16_bits(t.cpu())


def _within_one_step(got_bits, ref_bits):
    """bf16 bit patterns equal, or adjacent (one step apart, same sign)."""
    g = got_bits.astype(np.int32)
    r = ref_bits.astype(np.int32)
    same_sign = (g >> 15) == (r >> 15)
    return bool(((g == r) | (same_sign & (np.abs(g - r) == 1))).all()), float((g == r).mean())


def test_embed_is_an_exact_gather():
    table = synth.normal((1000, 4096), seed=90).to(DEV)
    ids = torch.tensor([0, 999, 17, 17, -1, 1000, 512], dtype=torch.int32, device=DEV)
    out = rbi.embed(table, ids)
    t = table.cpu()
    for i, v in enumerate(ids.cpu().tolist()):
        ref = t[v] if 0 <= v < 1000 else torch.zeros(4096, dtype=torch.bfloat16)
        assert torch.equal(out[i].cpu(), ref), i


def test_residual_add_is_the_rounded_sum():
    a = synth.normal((37, 4096), seed=91).to(DEV)
    b = synth.normal((37, 4096), std=0.1, seed=92).to(DEV)
    out = rbi.residual_add(a, b)
    ref = oracle.round_bf16(oracle.bf16_to_f64(_bits(a)) + oracle.bf16_to_f64(_bits(b)))
    ok, exact = _within_one_step(_bits(out), ref)
    assert ok and exact > 0.9999, exact
    # an odd element count runs the scalar tail
    a2, b2 = a.reshape(-1)[:1001].contiguous(), b.reshape(-1)[:1001].contiguous()
    out2 = rbi.residual_add(a2, b2)
    assert torch.equal(out2, out.reshape(-1)[:1001])


def test_swiglu_is_the_rounded_product():
    gu = synth.normal((9, 2 * 12288), seed=93).to(DEV)
    out = rbi.swiglu(gu)
    g = oracle.bf16_to_f64(_bits(gu[:, :12288]))
    u = oracle.bf16_to_f64(_bits(gu[:, 12288:]))
    ref = oracle.round_bf16(oracle.silu_mul(g, u))
    ok, exact = _within_one_step(_bits(out), ref)
    assert ok and exact > 0.99, exact


@pytest.mark.parametrize("n,stride", [(151936, 151936), (151933, 151936), (4099, 4101), (7, 8)])
def test_argmax_rows_exact(n, stride):
    # vectorised path (16-byte aligned rows, stride a multiple of 4) and scalar path
    rng = np.random.default_rng(n)
    rows = 9
    x = np.full((rows, stride), np.nan, dtype=np.float32)
    x[:, :n] = rng.standard_normal((rows, n)).astype(np.float32)
    x[1, [2, n - 1]] = 50.0                 # tie: the lower index wins
    x[2, :n] = np.nan                       # all NaN: 0
    x[3, :n] = -np.inf                      # all -inf: the first entry
    x[4, n - 1] = 1e30                      # maximum in the last entry (the tail)
    x[5, 0] = np.nan
    x[5, 1] = 1e30                          # NaN next to the maximum
    xt = torch.from_numpy(x).to(DEV)[:, :n]
    got = rbi.argmax_rows(xt).cpu().numpy()
    clean = np.where(np.isnan(x[:, :n]), -np.inf, x[:, :n])
    ref = oracle.argmax_lowest(clean)
    ref[2] = 0
    assert list(got) == list(ref)
