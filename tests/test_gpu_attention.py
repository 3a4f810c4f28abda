"""GPU tests of decode_attn_bi / decode_attn_tuned / kv_append: parity with the
CPU oracle (per row, max|out - RNE_bf16(ref)| <= 2e-2 * RMS(ref row); see
tests.conftest.attn_tol) and bitwise invariance across
batch size, neighbours, order, page placement, grid extent (max_kv_len), KV
growth across split boundaries and chunked versus unchunked prefill.
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


def _to(kv: synth.PagedKV) -> synth.PagedKV:
    return synth.PagedKV(kv.k_cache.to(DEV), kv.v_cache.to(DEV), kv.block_table.to(DEV),
                         kv.kv_lens.to(DEV), kv.page_size, kv.num_kv_heads, kv.head_dim,
                         kv.extra)


def _oracle(q, kv, scale, rows=None):
    bt = kv.block_table.cpu().numpy()
    lens = kv.kv_lens.cpu().numpy()
    qb = synth.bf16_bits(q.cpu())
    if rows is not None:
        bt, lens, qb = bt[rows], lens[rows], qb[rows]
    return oracle.decode_attn(qb, synth.bf16_bits(kv.k_cache.cpu()),
                              synth.bf16_bits(kv.v_cache.cpu()), bt, lens, scale)


def _run(fn, q, kv, max_len, **kw):
    return fn(q, kv.k_cache, kv.v_cache, kv.block_table, kv.kv_lens, max_len, **kw)


def test_c1_tiny_parity_and_rows_bitwise():
    # 4 query heads over 1 kv head, head_dim 64, lengths {5, 17, 63}, page 16, split 16
    lens = [5, 17, 63]
    kv = _to(synth.paged_kv(lens, 1, 64, 16))
    q = synth.normal((3, 4, 64), seed=100).to(DEV)
    scale = 1 / 8
    out = _run(rbi.decode_attn_bi, q, kv, 63, split_size=16, scale=scale)
    ok, ratio, row = attn_tol(out, _oracle(q, kv, scale), name="c1")
    assert ok, (ratio, row)
    assert not torch.isnan(out.float()).any()
    for r in range(3):
        sub = synth.PagedKV(kv.k_cache, kv.v_cache, kv.block_table[r:r + 1].contiguous(),
                            kv.kv_lens[r:r + 1].contiguous(), 16, 1, 64)
        alone = _run(rbi.decode_attn_bi, q[r:r + 1].contiguous(), sub, 63, split_size=16,
                     scale=scale)
        assert torch.equal(alone[0], out[r])
    perm = [2, 0, 1]
    sub = synth.PagedKV(kv.k_cache, kv.v_cache, kv.block_table[perm].contiguous(),
                        kv.kv_lens[perm].contiguous(), 16, 1, 64)
    shuf = _run(rbi.decode_attn_bi, q[perm].contiguous(), sub, 63, split_size=16, scale=scale)
    assert torch.equal(shuf, out[perm])


@pytest.mark.parametrize("lens", [[1], [255, 256, 257, 512, 513], [1, 2, 15, 16, 17, 31, 33],
                                  [1999, 700, 64, 1040]])
def test_c4_heads_parity(lens):
    # 64 query heads over 4 kv heads, head_dim 128, page 16, split 256
    kv = _to(synth.paged_kv(lens, 4, 128, 16))
    q = synth.normal((len(lens), 64, 128), seed=3).to(DEV)
    scale = 1 / math.sqrt(128)
    ref = _oracle(q, kv, scale)
    for fn, kw in ((rbi.decode_attn_bi, dict(split_size=256)), (rbi.decode_attn_tuned, {})):
        out = _run(fn, q, kv, max(lens), scale=scale, **kw)
        ok, ratio, row = attn_tol(out, ref, name=f"{fn.__name__} {lens}")
        assert ok, (fn.__name__, ratio, row)


@pytest.mark.parametrize("d,hq,hkv,split", [(64, 8, 1, 1024), (128, 16, 2, 512), (64, 32, 4, 64),
                                             (128, 4, 4, 16), (128, 64, 8, 1024)])
def test_shapes_and_split_sizes(d, hq, hkv, split):
    # head_dim 64 and 128, groups of 1, 2, 8 and 16 query heads, split sizes from one
    # page to 1024 tokens (up to 16 page pairs per wave); lengths straddle split and
    # page boundaries and reach max_kv_len exactly.  Parity per row, and every row
    # alone equals its row in the batch.
    lens = [1, split - 1, split, split + 1, 3 * split + 7, 2500]
    kv = _to(synth.paged_kv(lens, hkv, d, 16, seed=7))
    q = synth.normal((len(lens), hq, d), seed=8).to(DEV)
    scale = 1 / math.sqrt(d)
    L = max(lens)
    out = _run(rbi.decode_attn_bi, q, kv, L, split_size=split, scale=scale)
    ok, ratio, row = attn_tol(out, _oracle(q, kv, scale), name=f"d{d} hq{hq} hkv{hkv} S{split}")
    assert ok, (ratio, row)
    for r in (0, 2, 5):
        sub = synth.PagedKV(kv.k_cache, kv.v_cache, kv.block_table[r:r + 1].contiguous(),
                            kv.kv_lens[r:r + 1].contiguous(), 16, hkv, d)
        alone = _run(rbi.decode_attn_bi, q[r:r + 1].contiguous(), sub, L, split_size=split,
                     scale=scale)
        assert torch.equal(alone[0], out[r]), r


def test_single_token_is_exact():
    # L = 1: the softmax weight is exactly 1, so the output is v_0 bit for bit
    kv = _to(synth.paged_kv([1, 1, 1], 4, 128, 16))
    q = synth.normal((3, 64, 128), seed=4).to(DEV)
    out = _run(rbi.decode_attn_bi, q, kv, 1)
    for r in range(3):
        p = int(kv.block_table[r, 0])
        v0 = kv.v_cache[p, :, :, 0]                       # [4, 128]
        assert torch.equal(out[r], v0.repeat_interleave(16, 0))


def test_c4_full_batch_sampled_parity_and_batch_invariance():
    # batch 256 with lengths ~ U{1..32768}, split 256; oracle on sampled rows
    lens = synth.uniform_lengths(256, 1, 32768)
    kv = synth.paged_kv(lens, 4, 128, 16, max_pages=2048, device=DEV)
    q = synth.normal((256, 64, 128), seed=5).to(DEV)
    scale = 1 / math.sqrt(128)
    out = _run(rbi.decode_attn_bi, q, kv, 32768)
    rows = [0, 17, 100, 255]
    ok, ratio, row = attn_tol(out[rows], _oracle(q, kv, scale, rows=rows), name="c4 batch 256")
    assert ok, (ratio, row)
    # every batch size 1..256: a seeded random subset of the requests in random order
    # (so each row sits at a random position among random neighbours) gives every
    # row the bits it has in the full batch
    rng = np.random.default_rng(synth.SEED_BATCH)
    bad = torch.zeros((), dtype=torch.int64, device=DEV)
    o = torch.empty_like(out)
    ws = torch.empty(rbi.decode_attn_workspace_size(256, 64, 128, 32768, 256), dtype=torch.uint8,
                     device=DEV)
    first_bad = None
    for B in range(1, 257):
        members = synth.batch_members(256, B, seed=int(rng.integers(1 << 30)))
        idx = torch.tensor(members, device=DEV)
        sub = synth.PagedKV(kv.k_cache, kv.v_cache, kv.block_table[idx].contiguous(),
                            kv.kv_lens[idx].contiguous(), 16, 4, 128)
        _run(rbi.decode_attn_bi, q[idx].contiguous(), sub, 32768, out=o[:B], workspace=ws)
        bad += (o[:B] != out[idx]).sum()
        if B % 64 == 0:
            if first_bad is None and int(bad):
                first_bad = B
            print(f"batch sizes 1..{B}: {int(bad)} differing elements", flush=True)
    assert int(bad) == 0, f"first seen by batch {first_bad}"


def test_plan_mode_long_rows_in_chunks():
    # A large batch (200 rows x 4 kv heads, at least two (row, kv head) units per
    # compute unit) runs whole rows per workgroup, longest first.  Ten rows here are
    # far longer than a compute unit's share of the batch, so they are cut into
    # chunks of whole groups whose partials go through the merge, while the other
    # rows are folded and written by one workgroup each.  Every row keeps the bits
    # it has alone (grid mode), and the schedule, built with atomics, never changes
    # the output from one call to the next.
    rng = np.random.default_rng(31)
    lens = [int(x) for x in rng.integers(1, 600, size=200)]
    for i in range(0, 200, 20):
        lens[i] = 32768 - 7 * i
    kv = synth.paged_kv(lens, 4, 128, 16, max_pages=2048, device=DEV)
    q = synth.normal((200, 64, 128), seed=32).to(DEV)
    scale = 1 / math.sqrt(128)
    out = _run(rbi.decode_attn_bi, q, kv, 32768)
    rows = [0, 1, 20, 199]
    ok, ratio, row = attn_tol(out[rows], _oracle(q, kv, scale, rows=rows), name="plan chunks")
    assert ok, (ratio, row)
    alone = torch.empty_like(out)
    for r in range(200):
        sub = synth.PagedKV(kv.k_cache, kv.v_cache, kv.block_table[r:r + 1].contiguous(),
                            kv.kv_lens[r:r + 1].contiguous(), 16, 4, 128)
        _run(rbi.decode_attn_bi, q[r:r + 1].contiguous(), sub, 32768, out=alone[r:r + 1])
    assert torch.equal(alone, out)
    again = torch.empty_like(out)
    ws = torch.empty(rbi.decode_attn_workspace_size(200, 64, 128, 32768, 256),
                     dtype=torch.uint8, device=DEV)
    diff = torch.zeros((), dtype=torch.int64, device=DEV)
    for _ in range(50):
        _run(rbi.decode_attn_bi, q, kv, 32768, out=again, workspace=ws)
        diff += (again != out).sum()
    assert int(diff) == 0


@pytest.mark.parametrize("d,hq,hkv,rows,split", [(64, 32, 4, 120, 256), (128, 16, 2, 200, 256),
                                                 (128, 64, 8, 60, 256), (64, 8, 1, 400, 256),
                                                 (64, 8, 1, 1500, 256), (128, 16, 2, 200, 64),
                                                 (64, 4, 1, 400, 16)])
def test_plan_mode_shapes(d, hq, hkv, rows, split):
    # large batches of other head shapes (rows * kv heads >= 384, so whole rows per
    # workgroup on a 256-unit device; 1500 rows: more rows than the plan kernel has
    # threads): every row equals the same row alone, and sampled rows match the oracle
    rng = np.random.default_rng(40 + d + hkv)
    lens = [int(x) for x in rng.integers(1, 5000 if rows <= 400 else 2000, size=rows)]
    lens[3] = 1
    lens[5] = 8192
    kv = synth.paged_kv(lens, hkv, d, 16, max_pages=8192 // 16, device=DEV)
    q = synth.normal((rows, hq, d), seed=41).to(DEV)
    scale = 1 / math.sqrt(d)
    out = _run(rbi.decode_attn_bi, q, kv, 8192, split_size=split, scale=scale)
    sample = [0, 3, 5, rows - 1]
    ok, ratio, row = attn_tol(out[sample], _oracle(q, kv, scale, rows=sample),
                              name=f"plan d{d} {hq}/{hkv} split {split}")
    assert ok, (ratio, row)
    alone = torch.empty_like(out)
    for r in range(rows):
        sub = synth.PagedKV(kv.k_cache, kv.v_cache, kv.block_table[r:r + 1].contiguous(),
                            kv.kv_lens[r:r + 1].contiguous(), 16, hkv, d)
        _run(rbi.decode_attn_bi, q[r:r + 1].contiguous(), sub, 8192, split_size=split,
             out=alone[r:r + 1], scale=scale)
    assert torch.equal(alone, out)


def test_plan_mode_in_a_graph_follows_new_lengths():
    # decode_attn_bi at batch 160 (the large-batch schedule) captured once as a HIP
    # graph and replayed while the lengths change in place between replays, as a
    # captured decode step's do: the plan is rebuilt on the device from the lengths
    # at every replay, so each replay equals an eager call with those lengths
    rows, lmax = 160, 8192
    rng = np.random.default_rng(51)
    lens0 = [int(x) for x in rng.integers(1, lmax - 600, size=rows)]
    kv = synth.paged_kv([lmax] * rows, 4, 128, 16, max_pages=lmax // 16, device=DEV)
    kv_lens = torch.tensor(lens0, dtype=torch.int32, device=DEV)
    q = synth.normal((rows, 64, 128), seed=52).to(DEV)
    out = torch.empty((rows, 64, 128), dtype=torch.bfloat16, device=DEV)
    ws = torch.empty(rbi.decode_attn_workspace_size(rows, 64, 128, lmax, 256),
                     dtype=torch.uint8, device=DEV)

    def call(o):
        rbi.decode_attn_bi(q, kv.k_cache, kv.v_cache, kv.block_table, kv_lens, lmax, 256,
                           out=o, workspace=ws)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        call(out)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call(out)
    eager = torch.empty_like(out)
    for step in range(6):
        # every row grows, a few by whole splits, and the longest rows change
        grow = rng.integers(1, 120, size=rows) * (1 + (step % 3 == 2) * 4)
        lens = [min(lmax, L + int(d)) for L, d in zip(kv_lens.tolist(), grow)]
        lens[step * 7] = lmax
        kv_lens.copy_(torch.tensor(lens, dtype=torch.int32))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        call(eager)
        torch.cuda.synchronize()
        assert torch.equal(out, eager), step


def test_grid_extent_and_page_placement_do_not_matter():
    lens = [300, 1000, 77]
    a = synth.paged_kv(lens, 4, 128, 16, seed=0, page_seed=3)
    b = synth.paged_kv(lens, 4, 128, 16, seed=0, page_seed=99)
    for r, L in enumerate(lens):       # same logical content, other physical pages
        for j in range(-(-L // 16)):
            b.k_cache[int(b.block_table[r, j])] = a.k_cache[int(a.block_table[r, j])]
            b.v_cache[int(b.block_table[r, j])] = a.v_cache[int(a.block_table[r, j])]
    a, b = _to(a), _to(b)
    q = synth.normal((3, 64, 128), seed=6).to(DEV)
    o1 = _run(rbi.decode_attn_bi, q, a, 1000)
    o2 = _run(rbi.decode_attn_bi, q, b, 1000)
    assert torch.equal(o1, o2)
    wide = torch.full((3, 2048), int(a.extra["poison_page"]), dtype=torch.int32, device=DEV)
    wide[:, : a.block_table.shape[1]] = a.block_table
    a2 = synth.PagedKV(a.k_cache, a.v_cache, wide, a.kv_lens, 16, 4, 128)
    o3 = _run(rbi.decode_attn_bi, q, a2, 32768)       # larger grid and workspace
    assert torch.equal(o1, o3)


def test_kv_growth_across_split_boundaries():
    # one request grows by one token per step from 240 to 2100 tokens, crossing the
    # split boundaries 256, 512, ..., 2048; at every length its output in a random
    # batch equals its output alone, and the workspace partials of completed groups
    # of four splits (1024 tokens) never change
    D, HKV, HQ, S, LMAX = 128, 4, 64, 256, 4096
    pool_lens = synth.uniform_lengths(32, 1, LMAX, seed=77)
    others = synth.paged_kv(pool_lens, HKV, D, 16, seed=7)
    probe = synth.paged_kv([2100], HKV, D, 16, seed=8, page_seed=9)
    q = synth.normal((1, HQ, D), seed=10).to(DEV)
    qo = synth.normal((32, HQ, D), seed=11).to(DEV)
    # one cache holding both: probe pages appended after the others'
    n_o = others.k_cache.shape[0]
    kc = torch.cat([others.k_cache, probe.k_cache]).to(DEV)
    vc = torch.cat([others.v_cache, probe.v_cache]).to(DEV)
    bt_p = probe.block_table + n_o
    maxp = LMAX // 16
    bt_o = torch.full((32, maxp), int(others.extra["poison_page"]), dtype=torch.int32)
    bt_o[:, : others.block_table.shape[1]] = others.block_table
    bt_pp = torch.full((1, maxp), n_o + int(probe.extra["poison_page"]), dtype=torch.int32)
    bt_pp[:, : bt_p.shape[1]] = bt_p
    bt_pp_d = bt_pp.to(DEV)
    rng = np.random.default_rng(12)
    GS = 4                              # splits per workspace partial
    npmax = -(-LMAX // (S * GS))
    ws1 = torch.zeros(rbi.decode_attn_workspace_size(1, HQ, D, LMAX, S), dtype=torch.uint8,
                      device=DEV)
    done = {}
    for L in range(240, 2101):
        lens1 = torch.tensor([L], dtype=torch.int32, device=DEV)
        alone = rbi.decode_attn_bi(q, kc, vc, bt_pp_d, lens1, LMAX, S, workspace=ws1)
        # the row's partials: [kv head, group, query head of the kv group, acc | m | l | pad]
        # (the work plan of large batches follows them in the workspace)
        slots = ws1.view(torch.float32)[: HKV * npmax * (HQ // HKV) * (D + 4)].view(
            HKV, npmax, HQ // HKV, D + 4)
        for k in range(L // (S * GS)):
            if k in done:
                assert torch.equal(slots[:, k], done[k]), (L, k)
            else:
                done[k] = slots[:, k].clone()
        B = int(rng.integers(2, 33))
        pos = int(rng.integers(0, B))
        mem = rng.choice(32, size=B - 1, replace=False)
        qb = torch.cat([qo[mem[:pos]], q, qo[mem[pos:]]])
        btb = torch.cat([bt_o[mem[:pos]], bt_pp, bt_o[mem[pos:]]]).to(DEV)
        lb = torch.tensor([pool_lens[i] for i in mem[:pos]] + [L] +
                          [pool_lens[i] for i in mem[pos:]], dtype=torch.int32, device=DEV)
        ob = rbi.decode_attn_bi(qb, kc, vc, btb, lb, LMAX, S)
        assert torch.equal(ob[pos], alone[0]), L
    assert sorted(done) == list(range(2))


def test_chunked_prefill_equals_unchunked():
    # a 700-token prompt: append all K/V then attend every token (row p sees p+1
    # tokens), versus seeded random chunks, each appended before its rows attend
    T, HKV, HQ, D = 700, 4, 64, 128
    npages = -(-T // 16)
    pages = synth.page_ids(npages + 8, seed=13)[:npages].to(DEV)
    k_new = synth.normal((T, HKV, D), seed=14).to(DEV)
    v_new = synth.normal((T, HKV, D), seed=15).to(DEV)
    q = synth.normal((T, HQ, D), seed=16).to(DEV)
    slots = (pages[torch.arange(T, device=DEV) // 16] * 16 +
             torch.arange(T, device=DEV) % 16).to(torch.int32)
    bt = pages[None].repeat(T, 1).to(torch.int32).contiguous()

    def fresh():
        return (torch.full((npages + 8, HKV, 16, D), float("nan"), dtype=torch.bfloat16, device=DEV),
                torch.full((npages + 8, HKV, D, 16), float("nan"), dtype=torch.bfloat16, device=DEV))

    kc, vc = fresh()
    rbi.kv_append(k_new, v_new, slots, kc, vc)
    lens = torch.arange(1, T + 1, dtype=torch.int32, device=DEV)
    full = rbi.decode_attn_bi(q, kc, vc, bt, lens, T, 256)
    kc2, vc2 = fresh()
    rng = np.random.default_rng(17)
    cuts = sorted(set(rng.integers(1, T, size=9).tolist()))
    bounds = [0] + cuts + [T]
    chunked = torch.empty_like(full)
    for a, b in zip(bounds[:-1], bounds[1:]):
        rbi.kv_append(k_new[a:b], v_new[a:b], slots[a:b].contiguous(), kc2, vc2)
        chunked[a:b] = rbi.decode_attn_bi(q[a:b].contiguous(), kc2, vc2, bt[a:b].contiguous(),
                                          lens[a:b].contiguous(), T, 256)
    assert torch.equal(full, chunked)
    assert not torch.isnan(full.float()).any()


def test_kv_append_exact_placement():
    T, HKV, D = 37, 4, 128
    kc = torch.zeros((20, HKV, 16, D), dtype=torch.bfloat16, device=DEV)
    vc = torch.zeros((20, HKV, D, 16), dtype=torch.bfloat16, device=DEV)
    k_new = synth.normal((T, HKV * D), seed=18).to(DEV)
    v_new = synth.normal((T, HKV * D), seed=19).to(DEV)
    slots = torch.randperm(20 * 16, generator=synth.gen(20))[:T].to(torch.int32)
    slots[5] = -1                      # skipped
    slots[6] = 20 * 16                 # out of range: skipped
    rbi.kv_append(k_new, v_new, slots.to(DEV), kc, vc)
    kc_h, vc_h = kc.cpu(), vc.cpu()
    kn, vn = k_new.cpu().view(T, HKV, D), v_new.cpu().view(T, HKV, D)
    written = torch.zeros(20 * 16, dtype=torch.bool)
    for t in range(T):
        s = int(slots[t])
        if 0 <= s < 320:
            assert torch.equal(kc_h[s // 16, :, s % 16], kn[t])
            assert torch.equal(vc_h[s // 16, :, :, s % 16], vn[t])
            written[s] = True
    flat = kc_h.permute(0, 2, 1, 3).reshape(320, -1)
    assert float(flat[~written].abs().max()) == 0
    vflat = vc_h.permute(0, 3, 1, 2).reshape(320, -1)
    assert float(vflat[~written].abs().max()) == 0


@pytest.mark.parametrize("d,page", [(128, 16), (64, 16), (96, 16), (128, 8)])
def test_kv_append_whole_pages_and_scattered(d, page):
    # 48 tokens filling three pages in order (the whole-page path at page 16), five
    # scattered, 17 from the middle of a page on, one out of range: every value at its
    # slot, nothing else written
    hkv, npages = 3, 24
    kc = torch.zeros((npages, hkv, page, d), dtype=torch.bfloat16, device=DEV)
    vc = torch.zeros((npages, hkv, d, page), dtype=torch.bfloat16, device=DEV)
    slot_list = [pg * page + i for pg in (3, 7, 1, 5, 9, 2) for i in range(page)][:48]
    slot_list = slot_list + [n * page + page - 1 for n in (10, 11, 12, 13, 14)]
    start = 20 * page + page // 2
    slot_list += list(range(start, start + 17))
    slot_list[50] = npages * page            # out of range: skipped
    T = len(slot_list)
    slots = torch.tensor(slot_list, dtype=torch.int32)
    k_new = synth.normal((T, hkv * d), seed=61).to(DEV)
    v_new = synth.normal((T, hkv * d), seed=62).to(DEV)
    rbi.kv_append(k_new, v_new, slots.to(DEV), kc, vc)
    kc_h, vc_h = kc.cpu(), vc.cpu()
    kn, vn = k_new.cpu().view(T, hkv, d), v_new.cpu().view(T, hkv, d)
    written = torch.zeros(npages * page, dtype=torch.bool)
    for t in range(T):
        s_ = int(slots[t])
        if 0 <= s_ < npages * page:
            assert torch.equal(kc_h[s_ // page, :, s_ % page], kn[t]), t
            assert torch.equal(vc_h[s_ // page, :, :, s_ % page], vn[t]), t
            written[s_] = True
    assert float(kc_h.permute(0, 2, 1, 3).reshape(npages * page, -1)[~written].abs().max()) == 0
    assert float(vc_h.permute(0, 3, 1, 2).reshape(npages * page, -1)[~written].abs().max()) == 0


def test_tuned_twin_sensitivity():
    # the balanced twin picks a different split size for a lone long request than
    # for a full batch, so the probe's bits move
    lens = synth.uniform_lengths(256, 1, 32768, seed=21)
    lens[0] = 20000
    kv = synth.paged_kv(lens, 4, 128, 16, max_pages=2048, device=DEV)
    q = synth.normal((256, 64, 128), seed=22).to(DEV)
    full = rbi.decode_attn_tuned(q, kv.k_cache, kv.v_cache, kv.block_table, kv.kv_lens, 32768,
                                 kv_lens_host=lens)
    one = rbi.decode_attn_tuned(q[:1], kv.k_cache, kv.v_cache, kv.block_table[:1].contiguous(),
                                kv.kv_lens[:1].contiguous(), 32768, kv_lens_host=lens[:1])
    assert rbi.decode_attn_tuned_split_size(1, 4, 32768, lens[:1]) != \
        rbi.decode_attn_tuned_split_size(256, 4, 32768, lens)
    assert not torch.equal(full[0], one[0])


def test_run_to_run_1000():
    # hidekazu-konishi.com sections 4.2 and 6.3: the same call 1000 times, every bit equal
    lens = synth.uniform_lengths(64, 1, 8192, seed=23)
    kv = _to(synth.paged_kv(lens, 4, 128, 16, max_pages=8192 // 16))
    q = synth.normal((64, 64, 128), seed=24).to(DEV)
    ref = _run(rbi.decode_attn_bi, q, kv, 8192)
    out = torch.empty_like(ref)
    ws = torch.empty(rbi.decode_attn_workspace_size(64, 64, 128, 8192, 256), dtype=torch.uint8,
                     device=DEV)
    diff = torch.zeros((), dtype=torch.int64, device=DEV)
    for _ in range(1000):
        _run(rbi.decode_attn_bi, q, kv, 8192, out=out, workspace=ws)
        diff += (out != ref).sum()
    assert int(diff) == 0
