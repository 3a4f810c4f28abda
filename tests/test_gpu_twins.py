"""Run-to-run determinism of the shape-tuned twins (hidekazu-konishi.com sections
4.2 and 6.3: the same call 1000 times gives the same bits), each at a shape where
its schedule differs from the batch-invariant kernel's: the workgroup-per-row
RMSNorm tree, split-K matmul with its ordered second pass, and 512-token attention
splits.  The twins are deterministic; only their batch invariance is given up.
"""
import pytest
import torch

import invariant_rmsnorm_bi_amd as rbi
import synth

pytestmark = pytest.mark.gpu
DEV = "cuda"
REPS = 1000


def _repeat(fn, out):
    ref = fn().clone()
    diff = torch.zeros((), dtype=torch.int64, device=DEV)
    for _ in range(REPS):
        diff += (fn() != ref).sum()
    assert int(diff) == 0
    return ref


def test_rmsnorm_tuned_run_to_run():
    x = synth.rmsnorm_rows(512, 4096, seed=81, device=DEV)
    w = synth.normal((4096,), std=0.1, mean=1.0, seed=82, device=DEV)
    y = torch.empty_like(x)
    _repeat(lambda: rbi.rmsnorm_tuned(x, w, 1e-6, out=y), y)


def test_matmul_tuned_run_to_run_split_k():
    M, N, K = 127, 4096, 8192     # four K ranges
    assert rbi.matmul_tuned_differs(M, N, K)
    A = synth.normal((M, K), seed=83, device=DEV)
    W = synth.normal((N, K), std=0.02, seed=84, device=DEV)
    C = torch.empty((M, N), dtype=torch.bfloat16, device=DEV)
    ws = torch.empty(rbi.matmul_tuned_workspace_size(M, N, K), dtype=torch.uint8, device=DEV)
    _repeat(lambda: rbi.matmul_tuned(A, W, out=C, workspace=ws), C)


def test_decode_attn_tuned_run_to_run_long_splits():
    lens = [20000]
    assert rbi.decode_attn_tuned_split_size(1, 4, 32768, lens) == 512
    kv = synth.paged_kv(lens, 4, 128, 16, max_pages=2048, device=DEV)
    q = synth.normal((1, 64, 128), seed=85, device=DEV)
    out = torch.empty_like(q)
    ws = torch.empty(rbi.decode_attn_workspace_size(1, 64, 128, 32768, 512), dtype=torch.uint8,
                     device=DEV)
    _repeat(lambda: rbi.decode_attn_tuned(q, kv.k_cache, kv.v_cache, kv.block_table, kv.kv_lens,
                                          32768, kv_lens_host=lens, out=out, workspace=ws), out)
