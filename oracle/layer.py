"""Oracle for one decode step of a dense pre-norm transformer layer feeding an
lm_head and greedy argmax -- the end-to-end workload used to show that a probe
request's tokens and logits do not depend on its batch neighbours.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

The chain, for each row (one request's current token at position p):
    x   = E[token]
    a   = rmsnorm(x; w_ln1)                       -> bf16
    qkv = a . Wqkv^T                              -> bf16, split q | k | v
    cache[p] <- (k, v)   (appended *before* attention, so cached and fresh
                          tokens reduce as one sequence: hidekazu-konishi.com
                          section 5.5)
    o   = attn(q, cache[0..p])                    -> bf16
    h   = x + (o . Wo^T -> bf16)                  -> bf16
    a2  = rmsnorm(h; w_ln2)                       -> bf16
    gu  = a2 . Wgu^T -> bf16;  s = silu(g) * u    -> bf16
    o2  = h + (s . Wd^T -> bf16)                  -> bf16
    logits = o2 . Wlm^T                           -> fp32
    token  = argmax(logits), lowest index on ties
Every intermediate is computed in fp64 from the exact stored values and rounded
once to the storage type the layer keeps it in (bf16 activations, fp32 logits).
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np

from . import (BF16, argmax_lowest, bf16_to_f64, decode_attn, matmul, rmsnorm, round_bf16,
               silu_mul)


@dataclass
class LayerDims:
    hidden: int
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    intermediate: int
    vocab: int
    eps: float = 1e-6
    page_size: int = 16

    @property
    def qkv_out(self) -> int:
        return (self.num_q_heads + 2 * self.num_kv_heads) * self.head_dim


def _f32_round(x: np.ndarray) -> np.ndarray:
    return np.asarray(x, dtype=np.float64).astype(np.float32)


class DenseLayerOracle:
    """Holds bf16 weights (uint16 bits) and its own paged KV cache."""

    def __init__(self, dims: LayerDims, weights: dict, num_pages: int):
        self.d = dims
        self.w = {k: np.ascontiguousarray(v).view(np.uint16) for k, v in weights.items()}
        self.k_cache = np.zeros((num_pages, dims.num_kv_heads, dims.page_size, dims.head_dim),
                                dtype=np.uint16)
        self.v_cache = np.zeros((num_pages, dims.num_kv_heads, dims.head_dim, dims.page_size),
                                dtype=np.uint16)

    def step(self, tokens, block_tables: np.ndarray, positions,
             logit_rows=None) -> tuple[np.ndarray, np.ndarray]:
        """One decode step for rows (token, block table row, position).  Returns
        (fp32 logits, argmax tokens) for the rows listed in ``logit_rows`` (all rows
        by default); the other rows still update the cache."""
        d = self.d
        tokens = np.asarray(tokens, dtype=np.int64)
        positions = np.asarray(positions, dtype=np.int64)
        bt = np.ascontiguousarray(block_tables, dtype=np.int32)
        B = tokens.shape[0]
        x = self.w["embed"][tokens]                                       # bf16 bits [B, H]
        a = round_bf16(rmsnorm(x, self.w["ln1"], d.eps))
        qkv = round_bf16(matmul(a, self.w["wqkv"]))                       # [B, qkv_out]
        hq, hkv, hd = d.num_q_heads, d.num_kv_heads, d.head_dim
        q = qkv[:, : hq * hd].reshape(B, hq, hd)
        k = qkv[:, hq * hd: (hq + hkv) * hd].reshape(B, hkv, hd)
        v = qkv[:, (hq + hkv) * hd:].reshape(B, hkv, hd)
        for b in range(B):
            p = int(positions[b])
            page = int(bt[b, p // d.page_size])
            self.k_cache[page, :, p % d.page_size, :] = k[b]
            self.v_cache[page, :, :, p % d.page_size] = v[b]
        lens = (positions + 1).astype(np.int32)
        o = decode_attn(np.ascontiguousarray(q), self.k_cache, self.v_cache, bt, lens,
                        1.0 / np.sqrt(hd))
        o = round_bf16(o.reshape(B, hq * hd))
        y = round_bf16(matmul(o, self.w["wo"]))
        h = round_bf16(bf16_to_f64(x) + bf16_to_f64(y))
        a2 = round_bf16(rmsnorm(h, self.w["ln2"], d.eps))
        gu = round_bf16(matmul(a2, self.w["wgu"]))
        g, u = bf16_to_f64(gu[:, : d.intermediate]), bf16_to_f64(gu[:, d.intermediate:])
        s = round_bf16(silu_mul(g, u))
        dn = round_bf16(matmul(s, self.w["wd"]))
        o2 = round_bf16(bf16_to_f64(h) + bf16_to_f64(dn))
        if logit_rows is not None:
            o2 = o2[list(logit_rows)]
        logits = _f32_round(matmul(o2, self.w["lm_head"]))
        return logits, argmax_lowest(logits)


__all__ = ["LayerDims", "DenseLayerOracle", "BF16"]
