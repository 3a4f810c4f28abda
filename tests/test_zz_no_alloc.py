"""decode_attn_bi_noalloc, the entry point for callers that cannot allocate: its
split partials (and, for large batches, the work plan) live in the library's
static device scratch instead of a caller's workspace.  Checked bit for bit
against decode_attn_bi (the same kernels with a caller's workspace) on three calls
in a row, each with a smaller input than the one before, and its size limit.
Collected last (the name sorts last), so a failure here cannot hide the other GPU
tests.
"""
import pytest
import torch

import invariant_rmsnorm_bi_amd as rbi
import synth

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _case(lens, hq, hkv, d, lmax, seed):
    # block tables as wide as max_kv_len needs (ceil(max_kv_len / 16) entries)
    kv = synth.paged_kv(lens, hkv, d, 16, seed=seed, device=DEV, max_pages=-(-lmax // 16))
    q = synth.normal((len(lens), hq, d), seed=seed + 100, device=DEV)
    return q, kv


def test_noalloc_equals_decode_attn_bi_on_successive_calls():
    # call 1: 120 requests of U{1..8192} tokens, enough (row, kv head) units for whole
    # rows per workgroup from a plan kept in the scratch; call 2: 64 such requests
    # (64 x 64 heads x 8 groups of 4 splits x 132 floats, 17 MB of the 128 MiB scratch),
    # every group through the partials; call 3, smaller: 5 requests at head_dim 64
    # whose partials overwrite only the start of what the earlier calls left there
    cases = [(synth.uniform_lengths(120, 1, 8192, seed=42), 64, 4, 128, 8192, 256),
             (synth.uniform_lengths(64, 1, 8192, seed=41), 64, 4, 128, 8192, 256),
             ([1, 17, 300, 1000, 2500], 32, 4, 64, 2500, 128)]
    outs = []
    for lens, hq, hkv, d, lmax, split in cases:
        print(f"noalloc case rows={len(lens)} hq={hq} hkv={hkv} d={d} max_kv_len={lmax} "
              f"split={split}", flush=True)
        q, kv = _case(lens, hq, hkv, d, lmax, seed=len(lens))
        need = rbi.decode_attn_workspace_size(len(lens), hq, d, lmax, split)
        assert need <= rbi.NOALLOC_SCRATCH_BYTES
        ref = rbi.decode_attn_bi(q, kv.k_cache, kv.v_cache, kv.block_table, kv.kv_lens, lmax,
                                 split)
        out = torch.full_like(ref, float("nan"))
        rbi.decode_attn_bi_noalloc(q, kv.k_cache, kv.v_cache, kv.block_table, kv.kv_lens, lmax,
                                   split, out=out)
        torch.cuda.synchronize()
        assert torch.equal(out, ref)
        outs.append((out, ref))
    for out, ref in outs:  # neither output was touched by the later call
        assert torch.equal(out, ref)
