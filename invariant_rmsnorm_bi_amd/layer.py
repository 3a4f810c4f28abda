"""One decode step of a dense pre-norm transformer layer feeding an lm_head and
greedy argmax, every stage a librbi kernel:

    x   = embed(token)
    a   = rmsnorm(x)                  qkv = a . Wqkv^T  -> q | k | v
    kv_append(k, v)                   (before attention: hidekazu-konishi.com, section 5.5)
    o   = decode_attn(q, cache)       h   = x + o . Wo^T
    a2  = rmsnorm(h)                  s   = swiglu(a2 . Wgu^T)
    o2  = h + s . Wd^T                logits = o2 . Wlm^T (fp32)   token = argmax
                                      (exact: sample_gumbel at temperature 0)

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

from . import (decode_attn_bi, decode_attn_tuned, embed, kv_append, matmul_bi, matmul_tuned,
               prefill_attn_bi, residual_add, rmsnorm_bi, rmsnorm_tuned, sample_gumbel, swiglu)


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


class _Upload:
    """A step's int32 inputs (token ids, block tables, cache slots, lengths) packed
    into one pinned host buffer and moved by one asynchronous copy on the current
    stream, instead of one synchronous copy from pageable memory per input.  Each
    input starts on a 256-byte boundary.  The host buffer is rewritten only once the
    previous copy out of it has finished; the device buffer is reused in stream
    order, after the kernels of the previous step."""

    ALIGN = 64  # int32 elements

    def __init__(self, device):
        self.device = device
        self.host = None
        self.dev = None
        self.copied = None

    def put(self, arrays):
        arrays = [np.ascontiguousarray(a, dtype=np.int32) for a in arrays]
        offs, n = [], 0
        for a in arrays:
            offs.append(n)
            n += -(-a.size // self.ALIGN) * self.ALIGN
        if self.host is None or self.host.numel() < n:
            self.host = torch.empty(n, dtype=torch.int32, pin_memory=True)
            self.dev = torch.empty(n, dtype=torch.int32, device=self.device)
            self.copied = None
        if self.copied is not None:
            self.copied.synchronize()
        h = self.host.numpy()
        for a, o in zip(arrays, offs):
            h[o: o + a.size] = a.reshape(-1)
        self.dev[:n].copy_(self.host[:n], non_blocking=True)
        self.copied = torch.cuda.Event()
        self.copied.record()
        return [self.dev[o: o + a.size].view(a.shape) for a, o in zip(arrays, offs)]


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
        self._upload = _Upload(device)
        self._zeros = {}  # batch size -> (int64 zeros, fp32 zeros) for greedy selection

    def _mm(self, a, w, out_dtype=torch.bfloat16):
        return (matmul_tuned if self.tuned else matmul_bi)(a, w, out_dtype=out_dtype)

    def _norm(self, x, w):
        return (rmsnorm_tuned if self.tuned else rmsnorm_bi)(x, w, self.cfg.eps)

    def schedule(self, block_table: np.ndarray, positions):
        """Host bookkeeping of a step: the cache slot each row's new token goes to
        and each row's KV length (position + 1)."""
        c = self.cfg
        positions = np.asarray(positions, dtype=np.int64)
        bt = np.ascontiguousarray(block_table, dtype=np.int32)
        B = positions.shape[0]
        slots = bt[np.arange(B), positions // c.page_size].astype(np.int64) * c.page_size \
            + positions % c.page_size
        return bt, slots.astype(np.int32), (positions + 1).astype(np.int32)

    @staticmethod
    def segments(bt: np.ndarray, positions) -> list:
        """Split a step's rows into runs for attention: a run of at least two rows
        that are consecutive positions of one request (one block-table row) is a
        prompt chunk, attended by the prefill kernel; the other rows are decode
        rows.  Returns [(first_row, end_row, chunk_start_position or -1)], in row
        order; the prefill kernel gives each token its decode row's bits, so the
        split changes speed only."""
        positions = np.asarray(positions, dtype=np.int64)
        B = positions.shape[0]
        segs = []
        i = 0
        while i < B:
            j = i + 1
            while j < B and positions[j] == positions[j - 1] + 1 and np.array_equal(bt[j], bt[i]):
                j += 1
            if j - i >= 2:
                segs.append((i, j, int(positions[i])))
            elif segs and segs[-1][2] < 0:
                segs[-1] = (segs[-1][0], j, -1)
            else:
                segs.append((i, j, -1))
            i = j
        return segs

    def step(self, tokens, block_table: np.ndarray, positions) -> tuple[torch.Tensor, torch.Tensor]:
        """Run rows (tokens[i] at positions[i] of the request whose block table is
        block_table[i]).  Returns (fp32 logits [B, vocab], argmax tokens [B] int32)."""
        bt, slots, lens_h = self.schedule(block_table, positions)
        tok, bt_d, slots_d, lens_d = self._upload.put([np.asarray(tokens), bt, slots, lens_h])
        return self.forward(tok, bt_d, slots_d, lens_d, lens_h,
                            segments=self.segments(bt, positions))

    def forward(self, tok, bt_d, slots_d, lens_d, lens_h, segments=None):
        """The device part of a step on device inputs (token ids, block tables, cache
        slots, KV lengths); lens_h, the lengths on the host, only steers the twin's
        split size.  segments (from segments()) routes prompt chunks to the prefill
        kernel; without it every row is a decode row.  The twin always runs every
        row through its decode kernel."""
        c = self.cfg
        B = tok.shape[0]
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
        elif segments is None or all(p < 0 for _, _, p in segments):
            o = decode_attn_bi(q, self.k_cache, self.v_cache, bt_d, lens_d, c.max_kv_len,
                               c.split_size)
        else:
            o = torch.empty((B, c.num_q_heads, c.head_dim), dtype=torch.bfloat16, device=tok.device)
            for a, b, p0 in segments:
                if p0 < 0:
                    decode_attn_bi(q[a:b], self.k_cache, self.v_cache, bt_d[a:b], lens_d[a:b],
                                   c.max_kv_len, c.split_size, out=o[a:b])
                else:
                    prefill_attn_bi(q[a:b], self.k_cache, self.v_cache, bt_d[a], p0,
                                    c.split_size, out=o[a:b])
        y = self._mm(o.view(B, c.q_width), self.w["wo"])
        h = residual_add(x, y)
        a2 = self._norm(h, self.w["ln2"])
        gu = self._mm(a2, self.w["wgu"])
        s = swiglu(gu)
        dn = self._mm(s, self.w["wd"])
        o2 = residual_add(h, dn)
        logits = self._mm(o2, self.w["lm_head"], out_dtype=torch.float32)
        return logits, self._greedy(logits)

    def _greedy(self, logits):
        """The exact row argmax (lowest index on ties, NaN never chosen), through
        sample_gumbel at temperature 0: its two passes spread a 151936-wide row over
        38 workgroups, where a one-workgroup-per-row argmax is bound by one compute
        unit's latency (device time at 1 / 16 / 128 rows: 5.8 / 6.5 / 17.9 us
        against 16.5 / 16.8 / 19.5 us, same tokens)."""
        B = logits.shape[0]
        if B not in self._zeros:
            self._zeros[B] = (torch.zeros(B, dtype=torch.int64, device=logits.device),
                              torch.zeros(B, dtype=torch.float32, device=logits.device))
        zi, zf = self._zeros[B]
        return sample_gumbel(logits, zi, zi, zf)


class GraphedStep:
    """A decode step of one batch shape captured once as a HIP graph (through
    torch's graph capture of the library's stream launches) and replayed with new
    tokens and positions.  The block tables are fixed at capture; tokens, cache
    slots and KV lengths are copied into the captured input buffers before each
    replay.  Every kernel is the same one the eager step launches, so a replay
    gives the eager step's bits; the graph only removes per-launch host overhead.
    For the twins the split size is fixed by the batch size at capture."""

    def __init__(self, layer: DecodeLayer, block_table: np.ndarray, positions, tokens):
        dev = layer.device
        self.layer = layer
        bt, slots, lens_h = layer.schedule(block_table, positions)
        self.bt_h = bt
        self.bt = torch.from_numpy(bt).to(dev)
        # per-replay inputs: one fixed device buffer, refilled by one copy per step
        self._upload = _Upload(dev)
        self.tok, self.slots, self.lens = self._upload.put([np.asarray(tokens), slots, lens_h])
        self.lens_h = lens_h
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):  # warm up outside the capture
            layer.forward(self.tok, self.bt, self.slots, self.lens, lens_h)
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        self.graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(self.graph):
            self.logits, self.tokens = layer.forward(self.tok, self.bt, self.slots, self.lens,
                                                     lens_h)
        torch.cuda.synchronize()

    def step(self, tokens, positions) -> tuple[torch.Tensor, torch.Tensor]:
        """Replay with new tokens and positions (same rows, same block tables).
        Returns the captured output buffers (overwritten by the next replay)."""
        _, slots, lens_h = self.layer.schedule(self.bt_h, positions)
        self._upload.put([np.asarray(tokens), slots, lens_h])  # same sizes: same buffers
        self.graph.replay()
        return self.logits, self.tokens

