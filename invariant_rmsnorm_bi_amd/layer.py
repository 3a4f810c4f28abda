"""One decode step of a dense pre-norm transformer layer feeding an lm_head and
greedy argmax, every stage a librbi kernel:

    x   = embed(token)
    a   = rmsnorm(x)                  qkv = a . Wqkv^T  -> q | k | v
    kv_append(k, v)                   (before attention: hidekazu-konishi.com, section 5.5)
    o   = decode_attn(q, cache)       h   = x + o . Wo^T
    a2  = rmsnorm(h)                  s   = swiglu(a2 . Wgu^T)
    o2  = h + s . Wd^T                logits = o2 . Wlm^T (fp32)   token = argmax

Rows are (request, position) pairs, so the same call serves decode (one row per
request) and prefill chunks (several consecutive positions of one request).
With ``tuned=False`` every reduction is batch-invariant, so a request's tokens
and logit bits do not depend on which other requests share its step, nor on how
its prompt was chunked.  ``tuned=True`` swaps in the shape-tuned twins, used to
price determinism end to end.

The host side here is scheduling bookkeeping only (which page slot each new
token goes to); all arithmetic runs in the HIP kernels.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np
import torch

from . import (argmax_rows, decode_attn_bi, decode_attn_tuned, embed, kv_append, matmul_bi,
               matmul_tuned, residual_add, rmsnorm_bi, rmsnorm_tuned, swiglu)


@dataclass
class LayerConfig:
    hidden: int = 4096
    num_q_heads: int = 64
    num_kv_heads: int = 4
    head_dim: int = 128
    intermediate: int = 12288
    vocab: int = 151936
    eps: float = 1e-6
    page_size: int = 16
    split_size: int = 256
    max_kv_len: int = 32768

    @property
    def q_width(self) -> int:
        return self.num_q_heads * self.head_dim

    @property
    def kv_width(self) -> int:
        return self.num_kv_heads * self.head_dim


class DecodeLayer:
    def __init__(self, cfg: LayerConfig, weights: dict, num_pages: int, device="cuda",
                 tuned: bool = False):
        self.cfg = cfg
        self.w = weights
        self.tuned = tuned
        self.device = device
        self.k_cache = torch.zeros((num_pages, cfg.num_kv_heads, cfg.page_size, cfg.head_dim),
                                   dtype=torch.bfloat16, device=device)
        self.v_cache = torch.zeros((num_pages, cfg.num_kv_heads, cfg.head_dim, cfg.page_size),
                                   dtype=torch.bfloat16, device=device)

    def _mm(self, a, w, out_dtype=torch.bfloat16):
        return (matmul_tuned if self.tuned else matmul_bi)(a, w, out_dtype=out_dtype)

    def _norm(self, x, w):
        return (rmsnorm_tuned if self.tuned else rmsnorm_bi)(x, w, self.cfg.eps)

    def step(self, tokens, block_table: np.ndarray, positions) -> tuple[torch.Tensor, torch.Tensor]:
        """Run rows (tokens[i] at positions[i] of the request whose block table is
        block_table[i]).  Returns (fp32 logits [B, vocab], argmax tokens [B] int32)."""
        c = self.cfg
        dev = self.device
        positions = np.asarray(positions, dtype=np.int64)
        bt = np.ascontiguousarray(block_table, dtype=np.int32)
        B = positions.shape[0]
        slots = bt[np.arange(B), positions // c.page_size].astype(np.int64) * c.page_size \
            + positions % c.page_size
        lens_h = (positions + 1).astype(np.int32)
        tok = torch.as_tensor(np.asarray(tokens, dtype=np.int32)).to(dev, non_blocking=False)
        bt_d = torch.from_numpy(bt).to(dev)
        slots_d = torch.from_numpy(slots.astype(np.int32)).to(dev)
        lens_d = torch.from_numpy(lens_h).to(dev)

        x = embed(self.w["embed"], tok)
        a = self._norm(x, self.w["ln1"])
        qkv = self._mm(a, self.w["wqkv"])
        q = qkv[:, : c.q_width].view(B, c.num_q_heads, c.head_dim)
        k = qkv[:, c.q_width: c.q_width + c.kv_width]
        v = qkv[:, c.q_width + c.kv_width:]
        kv_append(k, v, slots_d, self.k_cache, self.v_cache)
        if self.tuned:
            o = decode_attn_tuned(q, self.k_cache, self.v_cache, bt_d, lens_d, c.max_kv_len,
                                  kv_lens_host=lens_h)
        else:
            o = decode_attn_bi(q, self.k_cache, self.v_cache, bt_d, lens_d, c.max_kv_len,
                               c.split_size)
        y = self._mm(o.view(B, c.q_width), self.w["wo"])
        h = residual_add(x, y)
        a2 = self._norm(h, self.w["ln2"])
        gu = self._mm(a2, self.w["wgu"])
        s = swiglu(gu)
        dn = self._mm(s, self.w["wd"])
        o2 = residual_add(h, dn)
        logits = self._mm(o2, self.w["lm_head"], out_dtype=torch.float32)
        return logits, argmax_rows(logits)
