"""Seeded synthetic inputs shared by the oracle side and the HIP side.

This module only *draws* inputs: it holds none of the arithmetic of RMSNorm,
matmul or attention. Both the CPU oracle (through tests and the bench's
cpu_baseline leg) and the HIP kernels consume the very same bits produced here.

Every generator is driven by an explicit ``torch.Generator`` seed so that a
case is named by (generator, seed, shape).  bf16 tensors are produced by
drawing fp32 values and rounding them to bf16 with torch's round-to-nearest-even
conversion; the resulting bits are what both sides see.

Seeds used across the suite (recorded in every bench record):
  data 0, weights 1, batch composition 2, page permutation 3.

Distributions follow the workloads of the batch-invariance pages (Qwen3-235B-A22B
shaped tensors): activations N(0,1), linear weights N(0,0.02), RMSNorm weight
N(1,0.1), K/V N(0,1); a seeded 1% of RMSNorm rows scaled by 100.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np
import torch

SEED_DATA = 0
SEED_WEIGHTS = 1
SEED_BATCH = 2
SEED_PAGES = 3


def gen(seed: int, device: str | torch.device = "cpu") -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    return g


def normal(shape, std: float = 1.0, mean: float = 0.0, *, seed: int,
           dtype=torch.bfloat16, device="cpu") -> torch.Tensor:
    """N(mean, std) drawn in fp32, then stored in ``dtype`` (RNE for bf16)."""
    g = gen(seed, device)
    t = torch.randn(tuple(shape), generator=g, dtype=torch.float32, device=device)
    if std != 1.0:
        t.mul_(std)
    if mean != 0.0:
        t.add_(mean)
    return t.to(dtype)


def rmsnorm_rows(rows: int, hidden: int, *, seed: int = SEED_DATA, dtype=torch.bfloat16,
                 outlier_frac: float = 0.01, outlier_scale: float = 100.0,
                 device="cpu") -> torch.Tensor:
    """x ~ N(0,1) with a seeded subset of rows scaled by ``outlier_scale``.

    The scaling happens in fp32 before the single rounding to ``dtype``.
    """
    g = gen(seed, device)
    t = torch.randn((rows, hidden), generator=g, dtype=torch.float32, device=device)
    n_out = int(round(outlier_frac * rows))
    if n_out > 0:
        gi = gen(seed + 7919, "cpu")
        idx = torch.randperm(rows, generator=gi)[:n_out].to(device)
        t[idx] *= outlier_scale
    return t.to(dtype)


def absorption_row(hidden: int = 4096, small_sq: float = 3e-8, dtype=torch.float32) -> torch.Tensor:
    """The row of the RMSNorm worked example on the praveentn.live page
    ("A Concrete Example"): x_1 = 1 and every other coordinate sqrt(small_sq),
    so that the squares are 1 and small_sq.  Stored in ``dtype``."""
    r = torch.full((hidden,), math.sqrt(small_sq), dtype=torch.float64)
    r[0] = 1.0
    return r.to(dtype)


def integer_valued(shape, lo: int = -4, hi: int = 4, *, seed: int, dtype=torch.bfloat16,
                   device="cpu") -> torch.Tensor:
    """Uniform integers in [lo, hi], exactly representable in bf16."""
    g = gen(seed, device)
    t = torch.randint(lo, hi + 1, tuple(shape), generator=g, device=device, dtype=torch.int32)
    return t.to(dtype)


def linspace_matrix(rows: int, cols: int, lo: float = -1000.0, hi: float = 1000.0,
                    dtype=torch.float32) -> torch.Tensor:
    """The linspace-filled matrices of the batch-1-vs-batch-2048 example on the
    hidekazu-konishi.com page (section 3.3)."""
    return torch.linspace(lo, hi, rows * cols, dtype=torch.float32).reshape(rows, cols).to(dtype)


# --------------------------------------------------------------------------------------
# Paged KV cache workloads
# --------------------------------------------------------------------------------------

@dataclass
class PagedKV:
    """A paged KV cache plus per-request block tables.

    k_cache: [num_pages, Hkv, page_size, D] bf16 (token-major pages)
    v_cache: [num_pages, Hkv, D, page_size] bf16 (head-dim-major pages)
    block_table:      [num_reqs, max_pages] int32, physical page ids (seeded permutation)
    kv_lens:          [num_reqs] int32, every entry >= 1
    """
    k_cache: torch.Tensor
    v_cache: torch.Tensor
    block_table: torch.Tensor
    kv_lens: torch.Tensor
    page_size: int
    num_kv_heads: int
    head_dim: int
    extra: dict = field(default_factory=dict)

    @property
    def num_reqs(self) -> int:
        return int(self.kv_lens.shape[0])


def page_ids(num_pages: int, *, seed: int = SEED_PAGES) -> torch.Tensor:
    """A seeded random permutation of physical page ids."""
    return torch.randperm(num_pages, generator=gen(seed, "cpu")).to(torch.int32)


def paged_kv(kv_lens, num_kv_heads: int, head_dim: int, page_size: int, *,
             seed: int = SEED_DATA, page_seed: int = SEED_PAGES, spare_pages: int = 0,
             device="cpu", max_pages: int | None = None,
             stale_fill: float | None = float("nan")) -> PagedKV:
    """Allocate a paged cache holding one request per entry of ``kv_lens``.

    Pages are assigned from a seeded permutation of physical ids, so logically
    adjacent pages are scattered.  K and V are N(0,1) bf16.  One extra *poison*
    page, filled with ``stale_fill`` (NaN by default), is allocated; every block
    table entry past a request's last page points at it, and the slots past a
    request's length in its last page hold the same value.  A kernel that reads
    past a request's length therefore produces NaN instead of touching memory
    outside the cache.  ``extra["poison_page"]`` is its physical id.
    """
    lens = [int(x) for x in kv_lens]
    assert all(l >= 1 for l in lens)
    need = [-(-l // page_size) for l in lens]
    mp = max_pages if max_pages is not None else max(need)
    assert mp >= max(need)
    total = sum(need) + spare_pages + 1
    perm = page_ids(total, seed=page_seed)
    poison = int(perm[-1])
    bt = torch.full((len(lens), mp), poison, dtype=torch.int32)
    pos = 0
    for r, n in enumerate(need):
        bt[r, :n] = perm[pos:pos + n]
        pos += n
    k = normal((total, num_kv_heads, page_size, head_dim), seed=seed, device=device)
    v = normal((total, num_kv_heads, head_dim, page_size), seed=seed + 1, device=device)
    if stale_fill is not None:
        k[poison] = stale_fill
        v[poison] = stale_fill
        for r, l in enumerate(lens):
            last = int(bt[r, need[r] - 1])
            off = l - (need[r] - 1) * page_size
            if off < page_size:
                k[last, :, off:, :] = stale_fill
                v[last, :, :, off:] = stale_fill
    return PagedKV(k_cache=k, v_cache=v, block_table=bt.to(device),
                   kv_lens=torch.tensor(lens, dtype=torch.int32, device=device),
                   page_size=page_size, num_kv_heads=num_kv_heads, head_dim=head_dim,
                   extra={"poison_page": poison})


def uniform_lengths(n: int, lo: int, hi: int, *, seed: int = SEED_BATCH) -> list[int]:
    g = gen(seed, "cpu")
    return [int(x) for x in torch.randint(lo, hi + 1, (n,), generator=g)]


def batch_members(pool: int, batch: int, *, seed: int) -> list[int]:
    """A seeded random subset of ``batch`` request ids out of ``pool``, in random order."""
    g = gen(seed, "cpu")
    return [int(x) for x in torch.randperm(pool, generator=g)[:batch]]


# --------------------------------------------------------------------------------------
# bit helpers (no arithmetic: views only)
# --------------------------------------------------------------------------------------

def bf16_bits(t: torch.Tensor) -> np.ndarray:
    """The raw uint16 bits of a bf16 tensor, as a numpy array (host copy)."""
    assert t.dtype == torch.bfloat16
    return t.detach().contiguous().cpu().view(torch.int16).numpy().view(np.uint16)


def from_bf16_bits(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16)


# --------------------------------------------------------------------------------------
# dense decode layer weights (the end-to-end workload)
# --------------------------------------------------------------------------------------

def dense_layer_weights(hidden: int, num_q_heads: int, num_kv_heads: int, head_dim: int,
                        intermediate: int, vocab: int, *, seed: int = SEED_WEIGHTS,
                        device="cpu") -> dict:
    """bf16 weights of one dense pre-norm layer plus embedding and lm_head.

    Linear weights are stored [out_features, in_features] and drawn N(0, 0.02);
    RMSNorm weights N(1, 0.1); the embedding table N(0, 1) so that activations
    enter the layer at the scale of the RMSNorm and matmul workloads.
    """
    qkv_out = (num_q_heads + 2 * num_kv_heads) * head_dim
    return {
        "embed": normal((vocab, hidden), seed=seed * 100 + 1, device=device),
        "ln1": normal((hidden,), std=0.1, mean=1.0, seed=seed * 100 + 2, device=device),
        "wqkv": normal((qkv_out, hidden), std=0.02, seed=seed * 100 + 3, device=device),
        "wo": normal((hidden, num_q_heads * head_dim), std=0.02, seed=seed * 100 + 4, device=device),
        "ln2": normal((hidden,), std=0.1, mean=1.0, seed=seed * 100 + 5, device=device),
        "wgu": normal((2 * intermediate, hidden), std=0.02, seed=seed * 100 + 6, device=device),
        "wd": normal((hidden, intermediate), std=0.02, seed=seed * 100 + 7, device=device),
        "lm_head": normal((vocab, hidden), std=0.02, seed=seed * 100 + 8, device=device),
    }
