"""Host-side tests of the C ABI (no GPU needed): the library loads, exports every
symbol include/rbi.h declares, and rejects bad arguments with the documented
status before anything would be enqueued.  Only invalid calls are made here, so
no kernel is ever launched.
"""
import ctypes
import os
import re

import pytest

import invariant_rmsnorm_bi_amd as rbi

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "rbi.h")

OK, EINVAL, EUNSUPPORTED, EWORKSPACE = 0, -1, -2, -3
NULL = None
FAKE = 0x10000  # a 16-byte aligned, never-dereferenced stand-in pointer


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?(?:int|size_t|char\s*\*|const char\s*\*)\s*\*?\s*(\w+)\s*\(",
                       src, flags=re.M)
    return sorted(set(names))


def test_header_and_binding_agree():
    assert set(declared_functions()) == set(rbi.EXPORTS)


def test_library_exports_every_declared_symbol():
    L = rbi.lib()
    for name in declared_functions():
        assert hasattr(L, name), name
        assert ctypes.cast(getattr(L, name), ctypes.c_void_p).value


def test_status_strings_and_version():
    L = rbi.lib()
    for st in (OK, EINVAL, EUNSUPPORTED, EWORKSPACE, -4, 7):
        assert L.rbi_status_string(st)
    assert L.rbi_status_string(EINVAL).startswith(b"RBI_EINVAL")
    assert L.rbi_abi_version() == 1


def test_rmsnorm_validation():
    f = rbi.lib().rmsnorm_bi
    assert f(FAKE, 8, FAKE, FAKE, 8, 0, 8, 1e-6, 1, NULL) == OK          # zero rows: no-op
    assert f(FAKE, 8, FAKE, FAKE, 8, 4, 8, 1e-6, 7, NULL) == EUNSUPPORTED
    assert f(NULL, 8, FAKE, FAKE, 8, 4, 8, 1e-6, 1, NULL) == EINVAL
    assert f(FAKE + 2, 8, FAKE, FAKE, 8, 4, 8, 1e-6, 1, NULL) == EINVAL  # misaligned
    assert f(FAKE, 12, FAKE, FAKE, 16, 4, 8, 1e-6, 1, NULL) == EINVAL    # stride not 16 B
    assert f(FAKE, 8, FAKE, FAKE, 8, 4, 16, 1e-6, 1, NULL) == EINVAL     # stride < hidden
    assert f(FAKE, 8, FAKE, FAKE, 8, -1, 8, 1e-6, 1, NULL) == EINVAL
    assert f(FAKE, 8, FAKE, FAKE, 8, 4, 0, 1e-6, 1, NULL) == EINVAL
    assert rbi.lib().rmsnorm_tuned(NULL, 8, FAKE, FAKE, 8, 4, 8, 1e-6, 1, NULL) == EINVAL


def test_matmul_validation():
    f = rbi.lib().matmul_bi
    assert f(FAKE, 64, FAKE, 64, FAKE, 64, 1, 0, 64, 64, NULL) == OK
    assert f(FAKE, 64, FAKE, 64, FAKE, 64, 5, 4, 64, 64, NULL) == EUNSUPPORTED
    assert f(FAKE, 64, FAKE, 64, FAKE, 64, 1, 4, 64, 60, NULL) == EINVAL   # K % 8
    assert f(FAKE, 64, FAKE, 64, FAKE, 64, 1, 4, 62, 64, NULL) == EINVAL   # N % 4
    assert f(FAKE, 60, FAKE, 64, FAKE, 64, 1, 4, 64, 64, NULL) == EINVAL   # lda < K
    assert f(FAKE, 64, NULL, 64, FAKE, 64, 1, 4, 64, 64, NULL) == EINVAL
    assert f(FAKE, 64, FAKE, 64, FAKE + 8, 64, 1, 4, 64, 64, NULL) == EINVAL
    assert f(FAKE, 64, FAKE, 64, FAKE, 32, 1, 4, 64, 64, NULL) == EINVAL  # ldc < N
    g = rbi.lib().matmul_tuned
    need = rbi.matmul_tuned_workspace_size(64, 4096, 8192)
    assert need == 4 * 64 * 4096 * 4                    # four K ranges of fp32 partials
    assert g(FAKE, 8192, FAKE, 8192, FAKE, 4096, 1, 64, 4096, 8192, NULL, need, NULL) == EWORKSPACE
    assert g(FAKE, 8192, FAKE, 8192, FAKE, 4096, 1, 64, 4096, 8192, FAKE, need - 1, NULL) == EWORKSPACE


def test_matmul_tuned_workspace_shape_dependence():
    # the twin's measured table: long-K projections split K from M = 9 to 256 (and the
    # longest K, 12288 and up, to 768), QKV-wide N in 2 ranges at M = 129 .. 192, very
    # wide N in 2 ranges up to M = 32; elsewhere matmul_bi's plan (no workspace, same
    # schedule)
    for M, N, K, splits in ((1, 4096, 8192, 1), (8, 4096, 8192, 1), (9, 4096, 8192, 2),
                            (32, 4096, 8192, 2), (64, 4096, 8192, 4), (160, 4096, 8192, 4),
                            (161, 4096, 8192, 2), (256, 4096, 8192, 2), (257, 4096, 8192, 1),
                            (509, 4096, 14336, 4), (768, 4096, 14336, 4),
                            (769, 4096, 14336, 1), (127, 4096, 12288, 4),
                            (127, 9216, 4096, 1), (129, 9216, 4096, 2), (192, 9216, 4096, 2),
                            (193, 9216, 4096, 1), (64, 9216, 4096, 1), (4096, 9216, 4096, 1),
                            (32, 24576, 4096, 2), (33, 24576, 4096, 1), (1, 9216, 4096, 1)):
        assert rbi.matmul_tuned_workspace_size(M, N, K) == (splits * M * N * 4 if splits > 1
                                                            else 0), (M, N, K)
        assert rbi.matmul_tuned_differs(M, N, K) == (splits > 1), (M, N, K)
    assert rbi.matmul_tuned_workspace_size(0, 9216, 4096) == 0


def _attn(**kw):
    a = dict(q=FAKE, qs=64 * 128, kc=FAKE, vc=FAKE, bt=FAKE, bts=2048, lens=FAKE, out=FAKE,
             os=64 * 128, rows=4, hq=64, hkv=4, d=128, page=16, split=256, maxlen=32768,
             scale=0.088, ws=FAKE, wsb=1 << 40)
    a.update(kw)
    return rbi.lib().decode_attn_bi(a["q"], a["qs"], a["kc"], a["vc"], a["bt"], a["bts"],
                                    a["lens"], a["out"], a["os"], a["rows"], a["hq"], a["hkv"],
                                    a["d"], a["page"], a["split"], a["maxlen"], a["scale"],
                                    a["ws"], a["wsb"], NULL)


def test_decode_attn_validation():
    assert _attn(rows=0) == OK
    assert _attn(d=96) == EUNSUPPORTED
    assert _attn(page=32) == EUNSUPPORTED
    assert _attn(split=250) == EUNSUPPORTED        # not a multiple of the page
    assert _attn(split=2048) == EUNSUPPORTED       # longer than 1024 tokens
    assert _attn(hq=64, hkv=2) == EUNSUPPORTED      # group of 32 query heads
    assert _attn(hq=63) == EINVAL                   # not a multiple of hkv
    assert _attn(maxlen=0) == EINVAL
    assert _attn(bts=100) == EINVAL                 # table too narrow for max_kv_len
    assert _attn(q=NULL) == EINVAL
    assert _attn(lens=NULL) == EINVAL
    assert _attn(out=FAKE + 4) == EINVAL
    assert _attn(qs=64 * 128 - 8) == EINVAL
    assert _attn(ws=NULL) == EWORKSPACE
    need = rbi.decode_attn_workspace_size(4, 64, 128, 32768, 256)
    # 128 splits of 256 in 32 groups, 132-float slots; then the large-batch work plan:
    # 4 header words, chunk counts per row, (row, chunk) per item for rows + 1024 items
    assert need == 4 * 64 * 32 * 132 * 4 + plan_bytes(4)
    assert _attn(wsb=need - 1) == EWORKSPACE
    # bounds: lengths up to 2^30, rows <= 65535, (splits per row) * kv heads < 2^22
    # (512 threads each), rows * query heads < 2^25 (the merge's 64 threads each)
    assert _attn(rows=65536) == EUNSUPPORTED
    assert _attn(maxlen=(1 << 30) + 1, bts=1 << 27) == EUNSUPPORTED
    assert _attn(maxlen=(1 << 31) - 1, bts=1 << 27) == EUNSUPPORTED
    big = dict(maxlen=1 << 26, split=32, bts=1 << 22)   # 2^21 splits per row
    assert _attn(hq=32, hkv=2, **big) == EUNSUPPORTED
    assert _attn(hq=16, hkv=1, wsb=1 << 20, **big) == EWORKSPACE  # 2^30 threads: in bounds
    wide = dict(hq=1024, hkv=64, qs=1024 * 128, os=1024 * 128)
    assert _attn(rows=32768, **wide) == EUNSUPPORTED
    assert _attn(rows=32767, wsb=1 << 20, **wide) == EWORKSPACE
    # the size query takes any int length without overflowing
    assert (rbi.decode_attn_workspace_size(1, 16, 64, (1 << 31) - 1, 16)
            == 16 * (1 << 25) * 68 * 4 + plan_bytes(1))


def plan_bytes(rows):
    """The large-batch work plan after the group partials: 4 header words, chunks per
    row, and a (row, chunk) pair for each of up to rows + 1024 items."""
    return (4 + rows + 2 * (rows + 1024)) * 4


def test_decode_attn_workspace_depends_only_on_bounds():
    a = rbi.decode_attn_workspace_size(256, 64, 128, 32768, 256)
    assert a == 256 * 64 * 32 * (128 + 4) * 4 + plan_bytes(256)  # groups of 4 splits of 256
    assert rbi.decode_attn_workspace_size(5, 4, 64, 63, 16) == 5 * 4 * 1 * 68 * 4 + plan_bytes(5)
    assert rbi.decode_attn_workspace_size(5, 4, 64, 65, 16) == 5 * 4 * 2 * 68 * 4 + plan_bytes(5)
    # splits longer than 256 tokens: no groups, no plan
    assert rbi.decode_attn_workspace_size(5, 4, 64, 4096, 512) == 5 * 4 * 8 * 68 * 4


def test_tuned_split_size_follows_the_batch():
    # the twin's split size moves with the batch (the fixed-size kernel would use
    # 256 for every batch)
    one = rbi.decode_attn_tuned_split_size(1, 4, 32768, [20000])
    many = rbi.decode_attn_tuned_split_size(256, 4, 32768, [32768] * 256)
    assert one == 512 and many == 256
    # work units of 256-token splits: 4 x 127 = 508 < 512 -> 512; 4 x 128 = 512 -> 256
    assert rbi.decode_attn_tuned_split_size(1, 4, 32768, [127 * 256]) == 512
    assert rbi.decode_attn_tuned_split_size(1, 4, 32768, [127 * 256 + 1]) == 256
    assert rbi.decode_attn_tuned_split_size(3, 4, 32768, [100, 20000, 9000]) == 512
    assert rbi.decode_attn_tuned_split_size(2, 4, 32768, None) == 256   # estimate 4 x 128
    assert rbi.decode_attn_tuned_split_size(1, 4, 32768, None) == 512
    # capped near short maximum lengths, always a multiple of the page
    short = rbi.decode_attn_tuned_split_size(1, 4, 100, None)
    assert short % 16 == 0 and 16 <= short <= 128


def test_kv_append_and_glue_validation():
    L = rbi.lib()
    assert L.kv_append(FAKE, 512, FAKE, 512, FAKE, 0, FAKE, FAKE, 10, 4, 128, 16, NULL) == OK
    assert L.kv_append(FAKE, 512, FAKE, 512, NULL, 3, FAKE, FAKE, 10, 4, 128, 16, NULL) == EINVAL
    assert L.kv_append(FAKE, 500, FAKE, 512, FAKE, 3, FAKE, FAKE, 10, 4, 128, 16, NULL) == EINVAL
    assert L.rbi_embed(FAKE, 100, 64, NULL, 3, FAKE, 64, NULL) == EINVAL
    assert L.rbi_embed(FAKE, 100, 60, FAKE, 3, FAKE, 64, NULL) == EINVAL
    assert L.rbi_residual_add(FAKE, FAKE, FAKE, 0, NULL) == OK
    assert L.rbi_residual_add(NULL, FAKE, FAKE, 8, NULL) == EINVAL
    assert L.rbi_swiglu(FAKE, 10, FAKE, 5, 3, 6, NULL) == EINVAL
    assert L.rbi_argmax_rows(FAKE, 10, 3, 20, FAKE, NULL) == EINVAL
    assert L.rbi_argmax_rows(NULL, 10, 3, 10, FAKE, NULL) == EINVAL


def test_grid_thread_bounds():
    # sizes that would put 2^31 or more threads along a grid dimension are refused
    # before anything is launched (fake pointers: nothing here may reach a kernel)
    L = rbi.lib()
    for f in (L.rmsnorm_bi, L.rmsnorm_tuned):
        assert f(FAKE, 8, FAKE, FAKE, 8, 1 << 23, 8, 1e-6, 1, NULL) == EUNSUPPORTED
    big = 1 << 28
    assert L.kv_append(FAKE, 512, FAKE, 512, FAKE, big, FAKE, FAKE, 10, 4, 128, 16, NULL) == EUNSUPPORTED
    assert L.rbi_embed(FAKE, 100, 64, FAKE, big, FAKE, 64, NULL) == EUNSUPPORTED
    assert L.rbi_residual_add(FAKE, FAKE, FAKE, 1 << 34, NULL) == EUNSUPPORTED
    assert L.rbi_swiglu(FAKE, 128, FAKE, 64, big, 64, NULL) == EUNSUPPORTED
    assert L.rbi_argmax_rows(FAKE, 16, 1 << 21, 16, FAKE, NULL) == EUNSUPPORTED
    assert L.rbi_stream_copy(FAKE, FAKE, 1 << 35, 0, NULL) == EUNSUPPORTED
    assert _prefill(tokens=1 << 22) == EUNSUPPORTED


def test_binding_refuses_cpu_tensors():
    import torch
    x = torch.zeros(2, 8, dtype=torch.bfloat16)
    with pytest.raises(rbi.RbiError):
        rbi.rmsnorm_bi(x, torch.ones(8, dtype=torch.bfloat16))


def _prefill(**kw):
    a = dict(q=FAKE, qs=64 * 128, kc=FAKE, vc=FAKE, bt=FAKE, start=0, tokens=700, out=FAKE,
             os=64 * 128, hq=64, hkv=4, d=128, page=16, split=256, scale=0.088, ws=NULL, wsb=0)
    a.update(kw)
    return rbi.lib().prefill_attn_bi(a["q"], a["qs"], a["kc"], a["vc"], a["bt"], a["start"],
                                     a["tokens"], a["out"], a["os"], a["hq"], a["hkv"], a["d"],
                                     a["page"], a["split"], a["scale"], a["ws"], a["wsb"], NULL)


def test_prefill_attn_validation():
    assert _prefill(tokens=0) == OK
    assert _prefill(tokens=-1) == EINVAL
    assert _prefill(start=-1) == EINVAL
    assert _prefill(d=96) == EUNSUPPORTED
    assert _prefill(split=512) == EUNSUPPORTED     # more than one page pair per wave
    assert _prefill(split=200) == EUNSUPPORTED     # not a multiple of the page
    assert _prefill(page=32) == EUNSUPPORTED
    assert _prefill(hq=64, hkv=2) == EUNSUPPORTED   # group of 32
    assert _prefill(hq=63) == EINVAL
    assert _prefill(q=NULL) == EINVAL
    assert _prefill(bt=NULL) == EINVAL
    assert _prefill(out=FAKE + 4) == EINVAL
    assert _prefill(qs=64 * 128 - 8) == EINVAL
    assert _prefill(start=1 << 30) == EUNSUPPORTED
    # a short chunk after a long prefix runs the split schedule and needs a workspace
    need = rbi.prefill_attn_workspace_size(40, 64, 4, 128, 1000, 256)
    assert need == 40 * 64 * 2 * 132 * 4     # ceil(1040 / 256) = 5 splits in 2 groups
    assert _prefill(tokens=40, start=1000) == EWORKSPACE
    assert _prefill(tokens=40, start=1000, ws=FAKE, wsb=need - 1) == EWORKSPACE


def test_prefill_workspace_follows_the_schedule():
    # fused (no workspace) once ceil(tokens / 8) * num_kv_heads token blocks reach 256
    # (8 tokens per workgroup, one per wave)
    assert rbi.prefill_attn_workspace_size(512, 64, 4, 128, 0, 256) == 0
    assert rbi.prefill_attn_workspace_size(505, 64, 4, 128, 0, 256) == 0
    assert rbi.prefill_attn_workspace_size(504, 64, 4, 128, 0, 256) > 0
    assert rbi.prefill_attn_workspace_size(512, 32, 4, 64, 0, 256) == 0
    assert rbi.prefill_attn_workspace_size(504, 32, 4, 64, 0, 256) > 0
    assert rbi.prefill_attn_workspace_size(2048, 8, 1, 64, 100, 16) == 0
    assert rbi.prefill_attn_workspace_size(0, 64, 4, 128, 0, 256) == 0


def test_sample_gumbel_validation():
    f = rbi.lib().sample_gumbel
    need = rbi.sample_gumbel_workspace_size(4, 151936)
    assert need == 4 * 38 * 8                      # ceil(151936 / 4096) chunks of (score, index)
    assert f(FAKE, 151936, 0, 151936, FAKE, FAKE, FAKE, FAKE, FAKE, need, NULL) == OK
    assert f(FAKE, 151934, 4, 151936, FAKE, FAKE, FAKE, FAKE, FAKE, need, NULL) == EINVAL  # ld < vocab
    assert f(FAKE, 151938, 4, 151936, FAKE, FAKE, FAKE, FAKE, FAKE, need, NULL) == EINVAL  # ld % 4
    assert f(FAKE + 4, 151936, 4, 151936, FAKE, FAKE, FAKE, FAKE, FAKE, need, NULL) == EINVAL
    assert f(FAKE, 151936, 4, 151936, NULL, FAKE, FAKE, FAKE, FAKE, need, NULL) == EINVAL
    assert f(FAKE, 151936, 4, 151936, FAKE, FAKE, FAKE, NULL, FAKE, need, NULL) == EINVAL
    assert f(FAKE, 151936, 4, 0, FAKE, FAKE, FAKE, FAKE, FAKE, need, NULL) == EINVAL
    assert f(FAKE, 151936, -1, 151936, FAKE, FAKE, FAKE, FAKE, FAKE, need, NULL) == EINVAL
    assert f(FAKE, 151936, 4, 151936, FAKE, FAKE, FAKE, FAKE, NULL, need, NULL) == EWORKSPACE
    assert f(FAKE, 151936, 4, 151936, FAKE, FAKE, FAKE, FAKE, FAKE, need - 1, NULL) == EWORKSPACE


def test_exact_matmul_cases_reach_every_tile_shape():
    # the integer-exact GPU cases must run every tile shape matmul_bi can launch
    # (the plan is a host-side choice, so this needs no GPU)
    from tests.test_gpu_matmul import BIG_EXACT_CASES, SMALL_EXACT_CASES
    seen = set()
    for mnk in SMALL_EXACT_CASES + [c for c, _ in BIG_EXACT_CASES]:
        p = rbi.matmul_bi_plan(*mnk)
        seen.add(p["first"])
        if p["second"]:
            seen.add(p["second"])
    every = {(256, 256, 0), (256, 128, 0), (128, 128, 0), (128, 64, 0), (64, 64, 0), (64, 32, 0),
             (32, 32, 0), (32, 16, 0), (16, 16, 0), (16, 16, 1), (128, 128, 2)}
    assert seen == every, every ^ seen
    # every LDS-pipelined shape runs in both of its kernels: 64-k stages (K % 64 == 0)
    # and 32-k stages (K % 64 == 32)
    lds = {t for t in every if t[2] == 0}
    kinds = set()
    for mnk in SMALL_EXACT_CASES + [c for c, _ in BIG_EXACT_CASES]:
        p = rbi.matmul_bi_plan(*mnk)
        for t in (p["first"], p["second"]):
            if t in lds and mnk[2] % 32 == 0:
                kinds.add((t, mnk[2] % 64))
    assert kinds == {(t, r) for t in lds for r in (0, 32)}, {(t, r) for t in lds for r in (0, 32)} ^ kinds
    for mnk, plan in BIG_EXACT_CASES:
        p = rbi.matmul_bi_plan(*mnk)
        assert (p["first"], p["n1"], p["second"]) == plan, mnk


def test_matmul_grid_bound():
    # more 16 x 16 tiles than one launch's threads can cover: refused before any launch
    L = rbi.lib()
    p = ctypes.c_void_p(16)
    st = L.matmul_bi(p, 1 << 20, p, 1 << 20, p, 1 << 17, 1, 1 << 17, 1 << 17, 1 << 20, None)
    assert st == -2
    buf = (ctypes.c_int64 * 7)()
    assert L.matmul_bi_plan(4096, 9216, 4096, buf) == 0 and buf[3] == 8192
    assert L.matmul_bi_plan(0, 9216, 4096, buf) == -1


def test_decode_attn_noalloc_limit():
    # more partials than the static scratch holds (256 rows of 64 heads at 32768
    # tokens: 545 MB > 128 MiB): refused on the host before the device is touched
    L = rbi.lib()
    f = ctypes.c_void_p(FAKE)
    assert rbi.decode_attn_workspace_size(256, 64, 128, 32768, 256) > rbi.NOALLOC_SCRATCH_BYTES
    st = L.decode_attn_bi_noalloc(f, 64 * 128, f, f, f, 2048, f, f, 64 * 128, 256, 64, 4, 128, 16,
                                  256, 32768, 0.1, None)
    assert st == EWORKSPACE
    # the usual argument checks come first
    st = L.decode_attn_bi_noalloc(f, 64 * 128, f, f, f, 2047, f, f, 64 * 128, 256, 64, 4, 128, 16,
                                  256, 32768, 0.1, None)
    assert st == EINVAL
    assert L.decode_attn_bi_noalloc(f, 64 * 128, f, f, f, 2048, f, f, 64 * 128, 0, 64, 4, 128, 16,
                                    256, 32768, 0.1, None) == OK
