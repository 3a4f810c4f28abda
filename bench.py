"""Benchmark of the batch-invariant forward reductions on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu] [--no-twins]
                    [--no-layer] [--no-prefill] [--copy-probe]

A *step* is one pass of the whole hot path over one batch of synthetic
Qwen3-235B-A22B-shaped input, every kernel batch-invariant:
    rmsnorm_bi   x [8192, 4096] bf16 (1% of rows x100), eps 1e-6
    matmul_bi    QKV   [4096, 4096] . [9216, 4096]^T  (bf16 in, fp32 acc, bf16 out)
    matmul_bi    o_proj[4096, 8192] . [4096, 8192]^T
    kv_append    one new token per request (256 x 4 kv heads x 128)
    decode_attn_bi  batch 256, 64 query / 4 kv heads, head_dim 128, page 16,
                 split 256, KV lengths ~ U{1..32768}
Inputs are resident in HBM before the timed region; RMSNorm and matmul operands
rotate over 4 buffer sets (> 512 MB) so the 256 MB last-level cache does not
serve them warm.  ``value`` = algorithmic HBM bytes of the step / step time.

Printed: ONE JSON line with the metric, a per-kernel breakdown (HBM GB/s or MFMA
TFLOP/s against the chip's peak, from hipEvents around each call of the timed
steps, and again from graph-replayed calls over the same rotating buffer sets,
which leaves out the events' own cost; for the two projections also the vendor GEMM,
hipBLASLt through torch.matmul, timed interleaved on the same operands as
context), the ``roofline`` object of the dominant kernel
(decode attention), the shape-tuned twins' times and the determinism slowdown
(t_bi / t_tuned - 1), prefill attention against the same tokens as decode rows,
and the CPU oracle timed on a bounded sample of the same
workload (``cpu_baseline``).
"""
from __future__ import annotations

import argparse
import json
import math
import os
import platform
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import invariant_rmsnorm_bi_amd as rbi  # noqa: E402
import synth  # noqa: E402

METRIC = "HBM GB/s & MFMA TFLOP/s of batch-invariant kernels; % slowdown vs tuned twins"
HBM_PEAK_GBS = 8000.0        # MI355X HBM3E
MFMA_BF16_PEAK_TFS = 2500.0  # MI355X dense bf16 MFMA
DEV = "cuda"

H = 4096
RMS_ROWS = 8192
MM_M = 4096
QKV = (9216, 4096)
OPROJ = (4096, 8192)
ATT_B, HQ, HKV, D, PAGE, SPLIT, LMAX = 256, 64, 4, 128, 16, 256, 32768
SETS = 4

# The cost of determinism as the pages report it ("Reproducible LLM Inference ...",
# hidekazu-konishi.com, sections 8.2 and 8.3): end-to-end serving time on NVIDIA
# hardware, other models and workloads.  Context only, never a target; the unit is
# the increase in time, as above.
PAGES_COST_CONTEXT = {
    "thinking_machines_seconds": {
        "workload": "Qwen-3-8B API server, 1000 sequences of 90-110 output tokens, one GPU "
                    "(model not stated)",
        "default": 26, "deterministic_unoptimised": 55, "deterministic_better_attention": 42},
    "sglang_slowdown_pct": {
        "workload": "Qwen3-8B, TP1, H200 (140 GB), three rollout workloads of 256 requests, "
                    "radix cache off",
        "mean_flashinfer_fa3": 34.35, "range": [24.4, 55.1]},
    "source": "hidekazu-konishi.com, Reproducible LLM Inference, sections 8.2-8.3",
}


def log(msg: str) -> None:
    print(msg, file=sys.stderr, flush=True)


# --------------------------------------------------------------------------------------
# algorithmic work per call (the method's own bytes / flops, no implementation overhead)
# --------------------------------------------------------------------------------------

def rms_bytes(rows, hidden=H):
    return rows * hidden * 2 * 2 + hidden * 2


def mm_bytes(M, N, K):
    return 2 * (M * K + N * K + M * N)


def mm_flops(M, N, K):
    return 2 * M * N * K


def attn_bytes(lens):
    # K and V of every cached token and kv head, q in, out
    return int(sum(lens)) * HKV * D * 2 * 2 + len(lens) * HQ * D * 2 * 2


def append_bytes(tokens):
    return tokens * HKV * D * 2 * 2 * 2


# --------------------------------------------------------------------------------------
# workload
# --------------------------------------------------------------------------------------

class Workload:
    def __init__(self):
        t0 = time.time()
        self.x = [synth.rmsnorm_rows(RMS_ROWS, H, seed=synth.SEED_DATA + i, device=DEV)
                  for i in range(SETS)]
        self.y = [torch.empty_like(self.x[0]) for _ in range(SETS)]
        self.w_ln = synth.normal((H,), std=0.1, mean=1.0, seed=synth.SEED_WEIGHTS, device=DEV)
        self.a_qkv = [synth.normal((MM_M, QKV[1]), seed=10 + i, device=DEV) for i in range(SETS)]
        self.w_qkv = [synth.normal(QKV, std=0.02, seed=20 + i, device=DEV) for i in range(SETS)]
        self.a_o = [synth.normal((MM_M, OPROJ[1]), seed=30 + i, device=DEV) for i in range(SETS)]
        self.w_o = [synth.normal(OPROJ, std=0.02, seed=40 + i, device=DEV) for i in range(SETS)]
        self.c_qkv = torch.empty((MM_M, QKV[0]), dtype=torch.bfloat16, device=DEV)
        self.c_o = torch.empty((MM_M, OPROJ[0]), dtype=torch.bfloat16, device=DEV)
        # paged decode attention: lengths include this step's new token
        self.lens = synth.uniform_lengths(ATT_B, 1, LMAX, seed=synth.SEED_BATCH)
        self.kv = synth.paged_kv(self.lens, HKV, D, PAGE, max_pages=LMAX // PAGE, device=DEV)
        self.q = synth.normal((ATT_B, HQ, D), seed=50, device=DEV)
        self.k_new = synth.normal((ATT_B, HKV, D), seed=51, device=DEV)
        self.v_new = synth.normal((ATT_B, HKV, D), seed=52, device=DEV)
        bt = self.kv.block_table.cpu()
        slots = [int(bt[r, (L - 1) // PAGE]) * PAGE + (L - 1) % PAGE
                 for r, L in enumerate(self.lens)]
        self.slots = torch.tensor(slots, dtype=torch.int32, device=DEV)
        self.att_out = torch.empty((ATT_B, HQ, D), dtype=torch.bfloat16, device=DEV)
        self.ws = torch.empty(rbi.decode_attn_workspace_size(ATT_B, HQ, D, LMAX, SPLIT),
                              dtype=torch.uint8, device=DEV)
        torch.cuda.synchronize()
        log(f"workload ready in {time.time() - t0:.1f}s: KV tokens {sum(self.lens)}, "
            f"cache {self.kv.k_cache.numel() * 4 / 1e9:.2f} GB")

    # the kernels of one step, by name, each a closure over buffer set i
    def calls(self, i):
        s = i % SETS
        return [
            ("rmsnorm_bi", lambda: rbi.rmsnorm_bi(self.x[s], self.w_ln, 1e-6, out=self.y[s])),
            ("matmul_bi_qkv", lambda: rbi.matmul_bi(self.a_qkv[s], self.w_qkv[s], out=self.c_qkv)),
            ("matmul_bi_oproj", lambda: rbi.matmul_bi(self.a_o[s], self.w_o[s], out=self.c_o)),
            ("kv_append", lambda: rbi.kv_append(self.k_new, self.v_new, self.slots,
                                                self.kv.k_cache, self.kv.v_cache)),
            ("decode_attn_bi", lambda: rbi.decode_attn_bi(
                self.q, self.kv.k_cache, self.kv.v_cache, self.kv.block_table, self.kv.kv_lens,
                LMAX, SPLIT, out=self.att_out, workspace=self.ws)),
        ]

    def work(self):
        return {
            "rmsnorm_bi": dict(bytes=rms_bytes(RMS_ROWS), bound="hbm"),
            "matmul_bi_qkv": dict(bytes=mm_bytes(MM_M, *QKV), flops=mm_flops(MM_M, *QKV),
                                  bound="mfma"),
            "matmul_bi_oproj": dict(bytes=mm_bytes(MM_M, *OPROJ), flops=mm_flops(MM_M, *OPROJ),
                                    bound="mfma"),
            "kv_append": dict(bytes=append_bytes(ATT_B), bound="hbm"),
            "decode_attn_bi": dict(bytes=attn_bytes(self.lens), bound="hbm"),
        }


# --------------------------------------------------------------------------------------
# timing helpers
# --------------------------------------------------------------------------------------

def time_fn(fn, reps=20, warm=3, inner=10):
    """Median device time (ms) of one call of fn, hipEvents on the current stream.
    Each sample queues `inner` calls back to back behind one untimed call, so the
    host's per-call cost (argument marshalling, launch) overlaps the device work
    instead of leaving the GPU idle between the events."""
    for _ in range(warm):
        fn()
    torch.cuda.synchronize()
    ts = []
    for _ in range(reps):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        fn()
        a.record()
        for _ in range(inner):
            fn()
        b.record()
        b.synchronize()
        ts.append(a.elapsed_time(b) / inner)
    return float(np.median(ts))


def graph_time_fn(fn, inner=20, reps=10):
    """Median device time (ms) of one call of fn: `inner` calls captured once as a
    HIP graph (through torch's capture of the current stream) and replayed between
    hipEvents, so neither the binding's host cost nor launch latency sits between
    the events, even for kernels of a few microseconds.  fn must allocate nothing
    on the device and copy nothing from the host."""
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for _ in range(2):
            fn()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for _ in range(inner):
            fn()
    g.replay()
    torch.cuda.synchronize()
    ts = []
    for _ in range(reps):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        g.replay()
        b.record()
        b.synchronize()
        ts.append(a.elapsed_time(b) / inner)
    del g
    return float(np.median(ts))


def vendor_gemm_us(wl: Workload):
    """Context only: the vendor GEMM (hipBLASLt, reached through torch.matmul) on the
    step's two projections with the same rotating operand sets, timed interleaved
    with matmul_bi (each sample: SETS calls queued back to back, one per operand
    set, behind an untimed call).  Median device us per call, {name: (bi_us, vendor_us)}."""
    out = {}
    for name, a_sets, w_sets, c in (("matmul_bi_qkv", wl.a_qkv, wl.w_qkv, wl.c_qkv),
                                    ("matmul_bi_oproj", wl.a_o, wl.w_o, wl.c_o)):
        fns = {"bi": lambda s: rbi.matmul_bi(a_sets[s], w_sets[s], out=c),
               "vendor": lambda s: torch.matmul(a_sets[s], w_sets[s].t(), out=c)}
        ts = {k: [] for k in fns}
        for i in range(3):
            for f in fns.values():
                f(i % SETS)
        torch.cuda.synchronize()
        for i in range(10):
            for k, f in fns.items():
                a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                f(SETS - 1)
                a.record()
                for s in range(SETS):
                    f(s)
                b.record()
                b.synchronize()
                ts[k].append(a.elapsed_time(b) * 1e3 / SETS)
        out[name] = (float(np.median(ts["bi"])), float(np.median(ts["vendor"])))
    return out


def ceilings(wl: Workload):
    """Read + write reference rates for RMSNorm on this device: the library's plain
    streaming copy (rbi_stream_copy, one 16-byte chunk per thread) over the same
    four rotating 64 MiB input / output sets the RMSNorm leg uses, with ordinary and
    with non-temporal stores, graph-replayed like the per-kernel graph_us."""
    out = {}
    nbytes = RMS_ROWS * H * 2
    for nt in (False, True):
        it = iter(range(1 << 30))

        def rot(nt=nt, it=it):
            i = next(it) % SETS
            rbi.stream_copy(wl.x[i], wl.y[i], nontemporal=nt)
        us = graph_time_fn(rot) * 1e3
        out["copy_64MiB_nt" if nt else "copy_64MiB"] = {
            "us": round(us, 2), "GB/s": round(2 * nbytes / us / 1e3, 1),
            "frac_hbm_peak": round(2 * nbytes / us / 1e3 / HBM_PEAK_GBS, 4)}
    return out


def twin_points(wl: Workload):
    """(name, bi_fn, tuned_fn) at the slowdown points: RMSNorm batch sizes, matmul M
    for both projections, attention batch sizes."""
    pts = []
    for B in (1, 64, 512, 4096, 8192):
        x = wl.x[0][:B]
        y = wl.y[0][:B]
        pts.append((f"rmsnorm B={B}",
                    lambda x=x, y=y: rbi.rmsnorm_bi(x, wl.w_ln, 1e-6, out=y),
                    lambda x=x, y=y: rbi.rmsnorm_tuned(x, wl.w_ln, 1e-6, out=y),
                    B < 1024))  # the twin's workgroup-per-row tree below 1024 rows
    for nm, A, W, C, K in (("qkv", wl.a_qkv[0], wl.w_qkv[0], wl.c_qkv, QKV[1]),
                           ("oproj", wl.a_o[0], wl.w_o[0], wl.c_o, OPROJ[1])):
        for M in (1, 7, 64, 127, 160, 256, 509, 1024, 2039, 4096):
            ws = torch.empty(max(16, rbi.matmul_tuned_workspace_size(M, W.shape[0], K)),
                             dtype=torch.uint8, device=DEV)
            pts.append((f"matmul {nm} M={M}",
                        lambda A=A[:M], W=W, C=C[:M]: rbi.matmul_bi(A, W, out=C),
                        lambda A=A[:M], W=W, C=C[:M], ws=ws: rbi.matmul_tuned(A, W, out=C,
                                                                              workspace=ws),
                        rbi.matmul_tuned_differs(M, W.shape[0], K)))
    kv = wl.kv
    for B in (1, 16, 64, 256):
        bt, ln, q = kv.block_table[:B], kv.kv_lens[:B], wl.q[:B]
        out = wl.att_out[:B]
        host = wl.lens[:B]
        split_t = rbi.decode_attn_tuned_split_size(B, HKV, LMAX, host)
        ws_t = torch.empty(rbi.decode_attn_workspace_size(B, HQ, D, LMAX, split_t),
                           dtype=torch.uint8, device=DEV)
        pts.append((f"decode_attn batch={B}",
                    lambda bt=bt, ln=ln, q=q, out=out: rbi.decode_attn_bi(
                        q, kv.k_cache, kv.v_cache, bt, ln, LMAX, SPLIT, out=out, workspace=wl.ws),
                    lambda bt=bt, ln=ln, q=q, out=out, host=host, ws_t=ws_t: rbi.decode_attn_tuned(
                        q, kv.k_cache, kv.v_cache, bt, ln, LMAX, kv_lens_host=host, out=out,
                        workspace=ws_t),
                    split_t != SPLIT))
    return pts


def layer_points():
    """End-to-end decode step of the dense layer (hidden 4096, 64/4 heads of 128,
    SwiGLU 12288, lm_head 151936, greedy argmax) built from the bi kernels versus
    the same layer built from the tuned twins, at batch sizes 1, 16, 64 and 128;
    each request has its own pages and a KV length ~ U{1..32768} (the decode-layer
    workload's lengths; the cache holds seeded random K/V, shared by the two layers).
    Wall clock per step (host scheduling included), median of 10 after 3 warmup
    steps, eager and replayed as a captured HIP graph (same kernels, no per-launch
    host cost); the graphed pair prices determinism on the device work, the eager
    pair includes each side's host cost."""
    from invariant_rmsnorm_bi_amd.layer import DecodeLayer, GraphedStep, LayerConfig
    cfg = LayerConfig()
    w = synth.dense_layer_weights(cfg.hidden, cfg.num_q_heads, cfg.num_kv_heads, cfg.head_dim,
                                  cfg.intermediate, cfg.vocab, device=DEV)
    rng = np.random.default_rng(synth.SEED_BATCH)
    Bmax, lmax = 128, cfg.max_kv_len
    pages_per = lmax // cfg.page_size
    layers = {False: DecodeLayer(cfg, w, num_pages=Bmax * pages_per, device=DEV),
              True: DecodeLayer(cfg, w, num_pages=1, device=DEV, tuned=True)}
    for seed, c in ((60, layers[False].k_cache), (61, layers[False].v_cache)):
        for i in range(0, c.shape[0], 8192):  # seeded N(0,1) K/V, drawn in slices
            c[i:i + 8192].copy_(synth.normal(tuple(c[i:i + 8192].shape),
                                             seed=seed * 1000003 + i, device=DEV))
    layers[True].k_cache, layers[True].v_cache = layers[False].k_cache, layers[False].v_cache
    table = np.zeros((Bmax, cfg.max_kv_len // cfg.page_size), dtype=np.int32)
    for r in range(Bmax):
        table[r, :pages_per] = np.arange(r * pages_per, (r + 1) * pages_per)
    pos = rng.integers(0, lmax, size=Bmax)
    toks = rng.integers(0, cfg.vocab, size=Bmax)
    pts = []
    for B in (1, 16, 64, 128):
        t = {}
        for tuned in (False, True):
            ly = layers[tuned]
            for _ in range(3):
                ly.step(toks[:B], table[:B], pos[:B])
            torch.cuda.synchronize()
            ts = []
            for _ in range(10):
                t0 = time.perf_counter()
                ly.step(toks[:B], table[:B], pos[:B])
                torch.cuda.synchronize()
                ts.append(time.perf_counter() - t0)
            t[tuned] = float(np.median(ts)) * 1e6
        # each step captured as a HIP graph: same kernels, no per-launch host cost
        tg = {}
        for tuned in (False, True):
            g = GraphedStep(layers[tuned], table[:B], pos[:B], toks[:B])
            for _ in range(3):
                g.step(toks[:B], pos[:B])
            torch.cuda.synchronize()
            ts = []
            for _ in range(10):
                t0 = time.perf_counter()
                g.step(toks[:B], pos[:B])
                torch.cuda.synchronize()
                ts.append(time.perf_counter() - t0)
            tg[tuned] = float(np.median(ts)) * 1e6
            del g
        pts.append({"point": f"layer step B={B}", "bi_us": round(t[False], 1),
                    "tuned_us": round(t[True], 1),
                    "slowdown_pct": round((t[False] / t[True] - 1) * 100, 2),
                    "bi_graph_us": round(tg[False], 1), "tuned_graph_us": round(tg[True], 1),
                    "graph_slowdown_pct": round((tg[False] / tg[True] - 1) * 100, 2)})
    del layers, w
    torch.cuda.empty_cache()
    return pts


PREFILL_POINTS = ((0, 4096), (2048, 2048), (0, 1024), (8000, 64))


def prefill_points():
    """prefill_attn_bi on one request's prompt chunk (64 query / 4 kv heads of 128,
    page 16, split 256; the chunk's K/V already in the cache, pages placed by a
    seeded permutation) against the same tokens run as decode_attn_bi rows
    (kv_len = position + 1): device time (median of 20), the algorithmic MFMA
    work 4 * Hq * D * sum(L_t) as TFLOP/s and its fraction of the bf16 peak, and
    whether every output bit agrees."""
    pts = []
    for start, T in PREFILL_POINTS:
        total = start + T
        npages = -(-total // PAGE)
        pages = synth.page_ids(npages + 8, seed=70)[:npages].to(torch.int32).to(DEV)
        kc = synth.normal((npages + 8, HKV, PAGE, D), seed=71, device=DEV)
        vc = synth.normal((npages + 8, HKV, D, PAGE), seed=72, device=DEV)
        q = synth.normal((T, HQ, D), seed=73, device=DEV)
        need = rbi.prefill_attn_workspace_size(T, HQ, HKV, D, start, SPLIT)
        ws = torch.empty(max(need, 16), dtype=torch.uint8, device=DEV)
        out_p = torch.empty_like(q)
        t_p = time_fn(lambda: rbi.prefill_attn_bi(q, kc, vc, pages, start, SPLIT, out=out_p,
                                                  workspace=ws))
        bt = pages[None].repeat(T, 1).contiguous()
        lens = torch.arange(start + 1, total + 1, dtype=torch.int32, device=DEV)
        ws_d = torch.empty(rbi.decode_attn_workspace_size(T, HQ, D, total, SPLIT),
                           dtype=torch.uint8, device=DEV)
        out_d = torch.empty_like(q)
        t_d = time_fn(lambda: rbi.decode_attn_bi(q, kc, vc, bt, lens, total, SPLIT, out=out_d,
                                                 workspace=ws_d))
        flops = 4 * HQ * D * (T * start + T * (T + 1) // 2)
        tf = flops / (t_p * 1e-3) / 1e12
        pts.append({"point": f"prefill start={start} tokens={T}",
                    "schedule": "fused" if need == 0 else "split",
                    "prefill_us": round(t_p * 1e3, 1), "decode_rows_us": round(t_d * 1e3, 1),
                    "speedup": round(t_d / t_p, 2), "flops": flops, "TFLOP/s": round(tf, 1),
                    "frac_mfma_peak": round(tf / MFMA_BF16_PEAK_TFS, 4),
                    "bitwise_equal_to_decode_rows": bool(torch.equal(out_p, out_d))})
        del kc, vc, q, ws, ws_d, out_p, out_d, bt
        torch.cuda.empty_cache()
    return pts


def sampling_points():
    """sample_gumbel over the decode layer's lm_head logits (fp32 [rows, 151936],
    N(0, 2) values, per-row seeds and positions, temperature 0.8) at 1 and 128
    rows, against the greedy rbi_argmax_rows over the same logits: device time of
    graph-replayed calls (the binding's host cost is not in it), the logits' read
    rate, and the rate of calls queued from Python for comparison."""
    pts = []
    V = 151936
    for rows in (1, 128):
        x = synth.normal((rows, V), std=2.0, seed=74, dtype=torch.float32, device=DEV)
        seeds = torch.arange(rows, dtype=torch.int64, device=DEV) * 7919 + 5
        pos = torch.arange(rows, dtype=torch.int64, device=DEV) + 1000
        temps = torch.full((rows,), 0.8, device=DEV)
        ws = torch.empty(rbi.sample_gumbel_workspace_size(rows, V), dtype=torch.uint8, device=DEV)
        tok = torch.empty(rows, dtype=torch.int32, device=DEV)
        tok_g = torch.empty(rows, dtype=torch.int32, device=DEV)
        f_s = lambda: rbi.sample_gumbel(x, seeds, pos, temps, out=tok, workspace=ws)  # noqa: E731
        f_g = lambda: rbi.argmax_rows(x, out=tok_g)  # noqa: E731
        q_s, q_g = time_fn(f_s), time_fn(f_g)
        t_s, t_g = graph_time_fn(f_s), graph_time_fn(f_g)
        nbytes = rows * V * 4
        pts.append({"point": f"sample_gumbel rows={rows} vocab={V}", "us": round(t_s * 1e3, 2),
                    "GB/s": round(nbytes / (t_s * 1e-3) / 1e9, 1),
                    "greedy_argmax_us": round(t_g * 1e3, 2),
                    "queued_us": round(q_s * 1e3, 2), "greedy_queued_us": round(q_g * 1e3, 2)})
        del x, ws
    return pts


# --------------------------------------------------------------------------------------
# CPU oracle baseline (bounded sample of the same workload)
# --------------------------------------------------------------------------------------

CPU_RMS_ROWS, CPU_MM_ROWS, CPU_ATT_ROWS = 8192, 768, 256


def cpu_baseline(wl: Workload, step_bytes: float):
    import oracle
    t_start = time.time()
    samples = {}
    # RMSNorm: CPU_RMS_ROWS of the 8192 rows
    xs = synth.bf16_bits(wl.x[0][:CPU_RMS_ROWS])
    wln = synth.bf16_bits(wl.w_ln)
    t = time.perf_counter()
    oracle.rmsnorm(xs, wln, 1e-6)
    samples["rmsnorm"] = (time.perf_counter() - t) * (RMS_ROWS / CPU_RMS_ROWS)
    # matmul: rows of A against the full weight (the oracle's cost is linear in M)
    for nm, A, W in (("qkv", wl.a_qkv[0], wl.w_qkv[0]), ("oproj", wl.a_o[0], wl.w_o[0])):
        m = CPU_MM_ROWS
        a, w = synth.bf16_bits(A[:m]), synth.bf16_bits(W)
        t = time.perf_counter()
        oracle.matmul(a, w)
        samples["matmul_" + nm] = (time.perf_counter() - t) * (MM_M / m)
    # attention: CPU_ATT_ROWS requests (cost linear in their total length)
    rows = list(range(CPU_ATT_ROWS))
    kc, vc = synth.bf16_bits(wl.kv.k_cache), synth.bf16_bits(wl.kv.v_cache)
    bt = wl.kv.block_table.cpu().numpy()[rows]
    lens = np.array([wl.lens[r] for r in rows], dtype=np.int32)
    q = synth.bf16_bits(wl.q[rows])
    t = time.perf_counter()
    oracle.decode_attn(q, kc, vc, bt, lens, 1 / math.sqrt(D))
    samples["decode_attn"] = (time.perf_counter() - t) * (sum(wl.lens) / lens.sum())
    t_step = sum(samples.values())
    return {
        "value": round(step_bytes / t_step / 1e9, 4),
        "unit": "GB/s",
        "cores": oracle.num_threads(),
        "kind": "oracle",
        "sample": (f"fp64 C oracle (OpenMP) on {CPU_RMS_ROWS} of 8192 RMSNorm rows, "
                   f"{CPU_MM_ROWS} of 4096 rows of each projection, {CPU_ATT_ROWS} of 256 "
                   f"attention requests ({int(lens.sum())} KV tokens); each scaled linearly "
                   "to the full step"),
        "seconds_per_step_extrapolated": round(t_step, 2),
        "sample_wall_s": round(time.time() - t_start, 1),
    }


TRAFFIC_FILE = os.path.join(ROOT, "profiles", "decode_attn_bi_b256_traffic.txt")
ATTN_SRCS = [os.path.join(ROOT, "invariant_rmsnorm_bi_amd", "csrc", f)
             for f in ("attention.hip", "device.h", "launch.h")]


def attn_source_sha():
    """sha256 over the sources the decode attention kernels are compiled from."""
    import hashlib
    h = hashlib.sha256()
    for p in ATTN_SRCS:
        with open(p, "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def measured_traffic():
    """HBM bytes per decode_attn_bi call from the committed FETCH_SIZE / WRITE_SIZE
    summary (copy-calibrated), or None when that summary is missing or was taken on
    a different attention source than the one built now."""
    try:
        kv = {}
        with open(TRAFFIC_FILE) as f:
            for line in f:
                if ":" in line and not line.startswith("#"):
                    k, v = line.split(":", 1)
                    kv[k.strip()] = v.strip()
        if kv.get("kernel_source_sha256") != attn_source_sha():
            return None
        return int(float(kv["traffic_bytes_per_launch"]))
    except (OSError, KeyError, ValueError):
        return None


def copy_probe():
    """A plain 1 GiB device-to-device copy, run 3 times: the known-size reference the
    FETCH_SIZE / WRITE_SIZE counters are calibrated against."""
    src = torch.empty(1 << 29, dtype=torch.bfloat16, device=DEV).fill_(1.0)
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()


def fingerprint():
    p = torch.cuda.get_device_properties(0)
    build = rbi.build_info()  # stamped into librbi.so when it was built
    cpu = ""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    cpu = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return {"gpu": p.name, "arch": getattr(p, "gcnArchName", ""), "cus": p.multi_processor_count,
            "torch": torch.__version__, "hip": torch.version.hip, "build": build, "host_cpu": cpu,
            "host_threads": os.cpu_count(), "python": platform.python_version(),
            "seeds": {"data": synth.SEED_DATA, "weights": synth.SEED_WEIGHTS,
                      "batch": synth.SEED_BATCH, "pages": synth.SEED_PAGES}}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--no-twins", action="store_true", help="skip the tuned-twin comparison")
    ap.add_argument("--no-layer", action="store_true",
                    help="skip the end-to-end decode-layer comparison")
    ap.add_argument("--no-prefill", action="store_true",
                    help="skip the prefill-attention and sampling legs")
    ap.add_argument("--copy-probe", action="store_true",
                    help="also run a plain 1 GiB copy (counter calibration for profiles/)")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures one GPU only: there is no multi-GPU path. The kernels "
              "work on one GPU's share (rows for RMSNorm, weight columns or K ranges for the "
              "matmul, KV heads or splits for attention), so a sharded deployment runs "
              "them per GPU.",
              file=sys.stderr)
        sys.exit(2)
    torch.cuda.set_device(0)
    rbi.lib()
    wl = Workload()

    # warmup
    for i in range(args.warmup):
        for _, fn in wl.calls(i):
            fn()
    torch.cuda.synchronize()

    # timed region: K steps; hipEvents around every kernel call, on the launch stream
    names = [n for n, _ in wl.calls(0)]
    ev = {n: [] for n in names}
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        for n, fn in wl.calls(i):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            fn()
            b.record()
            ev[n].append((a, b))
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_step = wall * 1e3 / args.steps
    work = wl.work()
    kernels = {}
    for n in names:
        us = float(np.mean([a.elapsed_time(b) for a, b in ev[n]])) * 1e3
        w = work[n]
        k = {"us": round(us, 2), "bytes": w["bytes"],
             "GB/s": round(w["bytes"] / us / 1e3, 1)}
        if w["bound"] == "mfma":
            tf = w["flops"] / us / 1e6
            k.update({"flops": w["flops"], "TFLOP/s": round(tf, 1),
                      "frac_mfma_peak": round(tf / MFMA_BF16_PEAK_TFS, 4)})
        else:
            k["frac_hbm_peak"] = round(w["bytes"] / us / 1e3 / HBM_PEAK_GBS, 4)
        kernels[n] = k
    step_bytes = sum(w["bytes"] for w in work.values())
    value = step_bytes / (ms_step / 1e3) / 1e9

    # the same calls' device time without the per-call events: each kernel's calls
    # over the rotating buffer sets, 20 of them replayed as one HIP graph (context:
    # a failure here is logged and leaves the field null)
    for idx, n in enumerate(names):
        fns = [wl.calls(i)[idx][1] for i in range(SETS)]

        def rotate(fns=fns, it=iter(range(1 << 30))):
            fns[next(it) % SETS]()
        w = work[n]
        k = kernels[n]
        try:
            us = graph_time_fn(rotate) * 1e3
        except Exception as e:  # noqa: BLE001 - context only
            log(f"graph timing of {n} failed: {e}")
            k["graph_us"] = None
            continue
        k["graph_us"] = round(us, 2)
        if w["bound"] == "mfma":
            k["graph_TFLOP/s"] = round(w["flops"] / us / 1e6, 1)
            k["graph_frac_mfma_peak"] = round(w["flops"] / us / 1e6 / MFMA_BF16_PEAK_TFS, 4)
        else:
            k["graph_GB/s"] = round(w["bytes"] / us / 1e3, 1)
            k["graph_frac_hbm_peak"] = round(w["bytes"] / us / 1e3 / HBM_PEAK_GBS, 4)

    dom = kernels["decode_attn_bi"]
    roofline = {"bound": "hbm",
                "kernel": "decode_attn_bi (plan, whole-row split kernel, ordered merge)",
                "achieved": dom["GB/s"], "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(dom["GB/s"] / HBM_PEAK_GBS, 4), "traffic": measured_traffic(),
                "algorithmic_bytes_per_launch": dom["bytes"], "avg_launch_us": dom["us"]}

    if args.copy_probe:
        copy_probe()
    log("timing the streaming-copy reference")
    ceil = ceilings(wl)

    twins = None
    if not args.no_twins:
        log("timing the vendor GEMM on the step's projections (context)")
        try:
            for n, (tb, tv) in vendor_gemm_us(wl).items():
                kernels[n].update({"interleaved_us": round(tb, 2),
                                   "vendor_gemm_us": round(tv, 2)})
        except Exception as e:  # noqa: BLE001 - context only
            log(f"vendor GEMM timing failed: {e}")
        log("timing the tuned twins")
        pts = []
        for name, fbi, ftu, differs in twin_points(wl):
            tb, tt = graph_time_fn(fbi), graph_time_fn(ftu)
            pts.append({"point": name, "bi_us": round(tb * 1e3, 2), "tuned_us": round(tt * 1e3, 2),
                        "slowdown_pct": round((tb / tt - 1) * 100, 2),
                        "schedule_differs": bool(differs)})
        mean = float(np.mean([p["slowdown_pct"] for p in pts]))
        diff = [p["slowdown_pct"] for p in pts if p["schedule_differs"]]
        twins = {"points": pts, "mean_slowdown_pct": round(mean, 2),
                 "mean_slowdown_pct_where_schedules_differ": (round(float(np.mean(diff)), 2)
                                                              if diff else None),
                 "points_where_schedules_differ": len(diff),
                 "unit": "time increase of bi over tuned, percent",
                 "timing": "device time per call: 20 calls replayed as one HIP graph, median of 10",
                 "pages_context": PAGES_COST_CONTEXT}
        if not args.no_layer:
            log("timing the decode layer, bi against tuned")
            lp = layer_points()
            twins["layer"] = {"points": lp, "mean_slowdown_pct": round(
                float(np.mean([p["slowdown_pct"] for p in lp])), 2),
                "mean_graph_slowdown_pct": round(
                float(np.mean([p["graph_slowdown_pct"] for p in lp])), 2)}

    prefill = None
    if not args.no_prefill:
        log("timing prefill attention against decode rows")
        prefill = {"points": prefill_points(),
                   "unit": "device us; TFLOP/s of the algorithmic 4*Hq*D*sum(L) MFMA work"}

    sampling = None
    if not args.no_prefill:
        log("timing seeded sampling")
        sampling = {"points": sampling_points()}

    cpu = None
    if not args.no_cpu:
        log("timing the CPU oracle on a bounded sample")
        cpu = cpu_baseline(wl, step_bytes)

    rec = {
        "metric": METRIC, "value": round(value, 2), "unit": "GB/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": ("qwen3-235b-a22b-shaped batch-invariant step: rmsnorm_bi "
                                "[8192,4096] + matmul_bi QKV [4096,4096]x[9216,4096]^T + o_proj "
                                "[4096,8192]x[4096,8192]^T + kv_append + decode_attn_bi batch 256 "
                                "(64q/4kv heads, d128, page 16, split 256, L~U{1..32768})"),
                   "step_bytes": step_bytes, "buffer_sets": SETS},
        "roofline": roofline, "cpu_baseline": cpu, "kernels": kernels, "ceilings": ceil,
        "twins": twins,
        "prefill": prefill, "sampling": sampling,
        "fingerprint": fingerprint(),
    }
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
