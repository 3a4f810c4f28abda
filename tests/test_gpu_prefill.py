"""GPU tests of prefill_attn_bi: every prompt token's output is bit-identical to
the decode_attn_bi row with the same query, cache and length (so neither the
chunking of a prompt nor a cached prefix can move its bits), within tolerance of
the CPU oracle, and the same from run to run.  Both schedules are covered: the
fused one (enough token blocks to fill the GPU, no workspace) and the split one
(short chunks after a long prefix, partials staged in a workspace).
"""
import math

import numpy as np
import pytest
import torch

import invariant_rmsnorm_bi_amd as rbi
import oracle
import synth
from tests.conftest import attn_tol

pytestmark = pytest.mark.gpu
DEV = "cuda"


class Prompt:
    """One request's prompt of `total` tokens: seeded K/V/q, pages placed by a seeded
    permutation, caches NaN-filled where nothing was written."""

    def __init__(self, total, hkv, hq, d, seed):
        self.total, self.hkv, self.hq, self.d = total, hkv, hq, d
        npages = -(-total // 16)
        self.cache_pages = npages + 8
        self.pages = synth.page_ids(self.cache_pages, seed=seed)[:npages].to(torch.int32).to(DEV)
        self.k = synth.normal((total, hkv, d), seed=seed + 1).to(DEV)
        self.v = synth.normal((total, hkv, d), seed=seed + 2).to(DEV)
        self.q = synth.normal((total, hq, d), seed=seed + 3).to(DEV)
        pos = torch.arange(total, device=DEV)
        self.slots = (self.pages[pos // 16].long() * 16 + pos % 16).to(torch.int32)
        self.kc = torch.full((self.cache_pages, hkv, 16, d), float("nan"), dtype=torch.bfloat16,
                             device=DEV)
        self.vc = torch.full((self.cache_pages, hkv, d, 16), float("nan"), dtype=torch.bfloat16,
                             device=DEV)

    def append(self, a, b):
        rbi.kv_append(self.k[a:b], self.v[a:b], self.slots[a:b].contiguous(), self.kc, self.vc)

    def prefill(self, a, b, split):
        return rbi.prefill_attn_bi(self.q[a:b].contiguous(), self.kc, self.vc, self.pages, a,
                                   split, scale=1 / math.sqrt(self.d))

    def decode_rows(self, a, b, split):
        n = b - a
        bt = self.pages[None].repeat(n, 1).contiguous()
        lens = torch.arange(a + 1, b + 1, dtype=torch.int32, device=DEV)
        return rbi.decode_attn_bi(self.q[a:b].contiguous(), self.kc, self.vc, bt, lens, b, split,
                                  scale=1 / math.sqrt(self.d))

    def oracle_rows(self, rows):
        rows = np.asarray(rows)
        bt = np.repeat(self.pages.cpu().numpy()[None], len(rows), 0)
        return oracle.decode_attn(synth.bf16_bits(self.q.cpu()[rows]),
                                  synth.bf16_bits(self.kc.cpu()), synth.bf16_bits(self.vc.cpu()),
                                  bt, (rows + 1).astype(np.int32), 1 / math.sqrt(self.d))


CASES = [
    # d, hq, hkv, split, start, tokens      schedule (8-token blocks, one token per wave)
    (128, 64, 4, 256, 0, 700),            # fused, every length 1..700, ragged last block
    (128, 64, 4, 256, 1000, 40),          # split: a short chunk after a long prefix
    (64, 8, 1, 16, 0, 100),               # split, one-page splits, group of 8
    (128, 16, 2, 64, 37, 333),            # split, ragged start and count
    (64, 32, 4, 128, 5, 2049),            # fused, head_dim 64, one-token last block
    (128, 4, 4, 256, 0, 1),               # one token, group of one
    (128, 64, 8, 256, 3000, 513),         # fused, group of 8, long prefix
    (128, 64, 4, 32, 250, 2100),          # fused, many splits per token
    (64, 32, 4, 256, 0, 1100),            # fused, head_dim 64 with whole 256-token splits
    (128, 12, 3, 256, 17, 700),           # fused, 3 kv heads (not dividing 8), group of 4
]


@pytest.mark.parametrize("d,hq,hkv,split,start,tokens", CASES)
def test_prefill_equals_decode_rows(d, hq, hkv, split, start, tokens):
    print(f"prefill case d={d} hq={hq} hkv={hkv} split={split} start={start} tokens={tokens}",
          flush=True)
    p = Prompt(start + tokens, hkv, hq, d, seed=31)
    p.append(0, start + tokens)
    out = p.prefill(start, start + tokens, split)
    ref_rows = p.decode_rows(start, start + tokens, split)
    torch.cuda.synchronize()
    assert not torch.isnan(out.float()).any()
    diff = (out != ref_rows).reshape(tokens, -1).any(1).nonzero().flatten().tolist()
    assert not diff, f"tokens differing from their decode rows: {diff[:10]}"
    # the oracle on sampled tokens (first, last, split edges, seeded others)
    rng = np.random.default_rng(tokens)
    pick = {0, tokens - 1} | set(rng.integers(0, tokens, size=6).tolist())
    pick |= {t for t in range(tokens) if (start + t + 1) % split in (0, 1)}
    rows = sorted(pick)[:24]
    ok, ratio, worst = attn_tol(out[rows], p.oracle_rows([start + t for t in rows]),
                                name=f"prefill start={start} tokens={tokens}")
    assert ok, (ratio, rows[worst])


def test_prefill_bench_size_parity():
    # the bench's prefill launch: one 4096-token prompt from position 0, 64 query / 4 kv
    # heads of 128, split 256 (fused schedule, 2048 workgroups); every token bitwise
    # equal to its decode row, the oracle on sampled tokens (split edges included)
    T, HKV, HQ, D, S = 4096, 4, 64, 128, 256
    print("prefill bench size", flush=True)
    p = Prompt(T, HKV, HQ, D, seed=33)
    p.append(0, T)
    out = p.prefill(0, T, S)
    ref_rows = p.decode_rows(0, T, S)
    torch.cuda.synchronize()
    assert not torch.isnan(out.float()).any()
    diff = (out != ref_rows).reshape(T, -1).any(1).nonzero().flatten().tolist()
    assert not diff, f"tokens differing from their decode rows: {diff[:10]}"
    rows = [0, 1, 254, 255, 256, 1023, 1024, 2047, 2600, 4094, 4095]
    ok, ratio, worst = attn_tol(out[rows], p.oracle_rows(rows), name="prefill 4096 tokens")
    assert ok, (ratio, rows[worst])


def test_prefill_schedules_as_documented():
    # the fused schedule (no workspace) once token blocks fill the GPU
    assert rbi.prefill_attn_workspace_size(700, 64, 4, 128, 0, 256) == 0
    assert rbi.prefill_attn_workspace_size(40, 64, 4, 128, 1000, 256) > 0


def test_chunked_prefill_is_bitwise_unchunked():
    # one 1500-token prompt: a single call (fused) versus seeded random chunks (fused
    # and split schedules), each chunk appended just before it attends, so cache
    # slots past the chunk still hold NaN while it runs
    T, HKV, HQ, D, S = 1500, 4, 64, 128, 256
    full_p = Prompt(T, HKV, HQ, D, seed=41)
    full_p.append(0, T)
    full = full_p.prefill(0, T, S)
    chunk_p = Prompt(T, HKV, HQ, D, seed=41)
    rng = np.random.default_rng(42)
    cuts = sorted(set(rng.integers(1, T, size=7).tolist()) | {1, 1100})
    bounds = [0] + cuts + [T]
    chunked = torch.empty_like(full)
    for a, b in zip(bounds[:-1], bounds[1:]):
        chunk_p.append(a, b)
        chunked[a:b] = chunk_p.prefill(a, b, S)
    torch.cuda.synchronize()
    assert torch.equal(full, chunked), bounds
    assert not torch.isnan(full.float()).any()


def test_prefill_run_to_run_1000():
    # hidekazu-konishi.com sections 4.2 and 6.3: 1000 calls, every bit equal; a chunk
    # on each schedule (fused: 800 tokens; split: 40 tokens after a 900-token prefix)
    p = Prompt(940, 4, 64, 128, seed=51)
    p.append(0, 940)
    for a, b in ((100, 900), (900, 940)):
        first = p.prefill(a, b, 256)
        out = torch.empty_like(first)
        ws = torch.empty(max(16, rbi.prefill_attn_workspace_size(b - a, 64, 4, 128, a, 256)),
                         dtype=torch.uint8, device=DEV)
        q = p.q[a:b].contiguous()
        diff = torch.zeros((), dtype=torch.int64, device=DEV)
        for _ in range(1000):
            rbi.prefill_attn_bi(q, p.kc, p.vc, p.pages, a, 256, scale=1 / math.sqrt(128),
                                out=out, workspace=ws)
            diff += (out != first).sum()
        assert int(diff) == 0, (a, b)
