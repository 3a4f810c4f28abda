"""Batch-invariant forward reductions for AMD MI355X (gfx950).

Thin Python binding over ``librbi.so`` (the C ABI declared in ``include/rbi.h``):
each function checks dtypes and devices, allocates outputs and workspaces with
torch (device memory and the current stream are all torch provides), and calls
the entry point of the same name.  Every step of the computation runs in the
library's HIP kernels; there is no fallback.  If ``librbi.so`` is missing or
cannot be loaded, every call raises ``RbiError``.

Entry points (see include/rbi.h for the exact contracts):
  rmsnorm_bi / rmsnorm_tuned
  matmul_bi / matmul_tuned
  decode_attn_bi / decode_attn_tuned
  prefill_attn_bi
  sample_gumbel
  kv_append, embed, residual_add, swiglu, argmax_rows
"""
from __future__ import annotations

import ctypes
import math
import os

import torch

__all__ = [
    "RbiError", "lib", "lib_path", "build_info", "rmsnorm_bi", "rmsnorm_tuned", "matmul_bi", "matmul_tuned",
    "matmul_tuned_workspace_size", "matmul_bi_plan", "matmul_tuned_differs", "decode_attn_bi", "decode_attn_tuned",
    "decode_attn_workspace_size", "decode_attn_tuned_split_size", "decode_attn_bi_noalloc",
    "NOALLOC_SCRATCH_BYTES", "prefill_attn_bi",
    "prefill_attn_workspace_size", "sample_gumbel", "sample_gumbel_workspace_size",
    "kv_append", "embed",
    "residual_add", "swiglu", "argmax_rows", "stream_copy", "EXPORTS",
]

_HERE = os.path.dirname(os.path.abspath(__file__))
lib_path = os.path.join(_HERE, "librbi.so")

RBI_F32, RBI_BF16 = 0, 1

# every symbol include/rbi.h declares
EXPORTS = (
    "rbi_status_string", "rbi_abi_version", "rbi_build_info", "rmsnorm_bi", "rmsnorm_tuned", "matmul_bi",
    "matmul_tuned", "matmul_tuned_workspace_size", "matmul_bi_plan", "matmul_tuned_differs",
    "decode_attn_workspace_size",
    "decode_attn_bi", "decode_attn_bi_noalloc", "decode_attn_tuned_split_size", "decode_attn_tuned",
    "prefill_attn_workspace_size", "prefill_attn_bi", "sample_gumbel_workspace_size",
    "sample_gumbel", "kv_append",
    "rbi_embed", "rbi_residual_add", "rbi_swiglu", "rbi_argmax_rows", "rbi_stream_copy",
)


class RbiError(RuntimeError):
    def __init__(self, msg: str, status: int | None = None):
        super().__init__(msg)
        self.status = status


_lib = None


def lib() -> ctypes.CDLL:
    """Load librbi.so (once).  Raises RbiError when it is absent: the library has
    no CPU fallback."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(lib_path):
        raise RbiError(f"{lib_path} is not built; run `python -m invariant_rmsnorm_bi_amd.build`")
    try:
        L = ctypes.CDLL(lib_path)
    except OSError as e:  # pragma: no cover - depends on the host
        raise RbiError(f"cannot load {lib_path}: {e}") from e
    p, i64, i32, f32, sz = (ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_float,
                            ctypes.c_size_t)
    sig = {
        "rbi_status_string": ([i32], ctypes.c_char_p),
        "rbi_abi_version": ([], i32),
        "rbi_build_info": ([], ctypes.c_char_p),
        "rmsnorm_bi": ([p, i64, p, p, i64, i64, i64, f32, i32, p], i32),
        "rmsnorm_tuned": ([p, i64, p, p, i64, i64, i64, f32, i32, p], i32),
        "matmul_bi": ([p, i64, p, i64, p, i64, i32, i64, i64, i64, p], i32),
        "matmul_tuned_workspace_size": ([i64, i64, i64], sz),
        "matmul_bi_plan": ([i64, i64, i64, p], i32),
        "matmul_tuned_differs": ([i64, i64, i64], i32),
        "matmul_tuned": ([p, i64, p, i64, p, i64, i32, i64, i64, i64, p, sz, p], i32),
        "decode_attn_workspace_size": ([i64, i32, i32, i32, i32], sz),
        "decode_attn_bi": ([p, i64, p, p, p, i64, p, p, i64, i64, i32, i32, i32, i32, i32, i32,
                            f32, p, sz, p], i32),
        "decode_attn_bi_noalloc": ([p, i64, p, p, p, i64, p, p, i64, i64, i32, i32, i32, i32,
                                    i32, i32, f32, p], i32),
        "decode_attn_tuned_split_size": ([i64, i32, i32, p], i32),
        "decode_attn_tuned": ([p, i64, p, p, p, i64, p, p, p, i64, i64, i32, i32, i32, i32, i32,
                               f32, p, sz, p], i32),
        "prefill_attn_workspace_size": ([i64, i32, i32, i32, i64, i32], sz),
        "prefill_attn_bi": ([p, i64, p, p, p, i64, i64, p, i64, i32, i32, i32, i32, i32, f32, p,
                             sz, p], i32),
        "sample_gumbel_workspace_size": ([i64, i64], sz),
        "sample_gumbel": ([p, i64, i64, i64, p, p, p, p, p, sz, p], i32),
        "kv_append": ([p, i64, p, i64, p, i64, p, p, i64, i32, i32, i32, p], i32),
        "rbi_embed": ([p, i64, i64, p, i64, p, i64, p], i32),
        "rbi_residual_add": ([p, p, p, i64, p], i32),
        "rbi_swiglu": ([p, i64, p, i64, i64, i64, p], i32),
        "rbi_argmax_rows": ([p, i64, i64, i64, p, p], i32),
        "rbi_stream_copy": ([p, p, i64, i32, p], i32),
    }
    for name, (args, res) in sig.items():
        fn = getattr(L, name)
        fn.argtypes = args
        fn.restype = res
    _lib = L
    return L


def build_info() -> str:
    """The commit and source hash librbi.so was built from (rbi_build_info)."""
    return lib().rbi_build_info().decode()


def _check(status: int, what: str) -> None:
    if status != 0:
        msg = lib().rbi_status_string(status).decode()
        raise RbiError(f"{what}: {msg}", status)


def _stream(t: torch.Tensor | None = None):
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _ptr(t: torch.Tensor | None):
    return ctypes.c_void_p(0 if t is None else t.data_ptr())


def _need_cuda(*ts: torch.Tensor) -> None:
    for t in ts:
        if not t.is_cuda:
            raise RbiError("librbi works on GPU tensors only (got a CPU tensor)")


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return RBI_BF16
    if t.dtype == torch.float32:
        return RBI_F32
    raise RbiError(f"unsupported dtype {t.dtype}")


def _row_stride(t: torch.Tensor) -> int:
    if t.dim() < 2 or t.stride(-1) != 1:
        raise RbiError("expected a 2-D view with unit stride in the last dimension")
    return _lead_stride(t)


def _lead_stride(t: torch.Tensor) -> int:
    """Stride of dimension 0 in elements.  A size-1 leading dimension may carry any
    stride (numpy's newaxis gives 0); only row 0 is read then, so report the packed
    row length instead."""
    if t.shape[0] > 1:
        return t.stride(0)
    n = 1
    for s in t.shape[1:]:
        n *= s
    return max(n, 1)


# -------------------------------------------------------------------------------------
# RMSNorm
# -------------------------------------------------------------------------------------

def _rmsnorm(fn: str, x: torch.Tensor, w: torch.Tensor, eps: float, out):
    _need_cuda(x, w)
    if w.dtype != x.dtype or w.dim() != 1 or w.shape[0] != x.shape[-1] or not w.is_contiguous():
        raise RbiError("w must be a contiguous [hidden] tensor of x's dtype")
    if out is None:
        out = torch.empty_like(x)
    st = getattr(lib(), fn)(_ptr(x), _row_stride(x), _ptr(w), _ptr(out), _row_stride(out),
                            x.shape[0], x.shape[1], float(eps), _dtype_code(x), _stream())
    _check(st, fn)
    return out


def rmsnorm_bi(x: torch.Tensor, w: torch.Tensor, eps: float = 1e-6, out=None) -> torch.Tensor:
    """Batch-invariant RMSNorm of the rows of x [rows, hidden] (fp32 or bf16)."""
    return _rmsnorm("rmsnorm_bi", x, w, eps, out)


def rmsnorm_tuned(x: torch.Tensor, w: torch.Tensor, eps: float = 1e-6, out=None) -> torch.Tensor:
    """Shape-tuned (not batch-invariant) twin of rmsnorm_bi."""
    return _rmsnorm("rmsnorm_tuned", x, w, eps, out)


# -------------------------------------------------------------------------------------
# Matmul
# -------------------------------------------------------------------------------------

def _mm_prep(A, W, out_dtype, out):
    _need_cuda(A, W)
    if A.dtype != torch.bfloat16 or W.dtype != torch.bfloat16:
        raise RbiError("matmul inputs must be bf16")
    M, K = A.shape
    N, K2 = W.shape
    if K != K2:
        raise RbiError(f"K mismatch: A has {K}, W has {K2}")
    if out is None:
        out = torch.empty((M, N), dtype=out_dtype, device=A.device)
    return M, N, K, out


def matmul_bi(A: torch.Tensor, W: torch.Tensor, out_dtype=torch.bfloat16, out=None) -> torch.Tensor:
    """C = A @ W.T, A [M, K] bf16, W [N, K] bf16, fp32 accumulation."""
    M, N, K, out = _mm_prep(A, W, out_dtype, out)
    st = lib().matmul_bi(_ptr(A), _row_stride(A), _ptr(W), _row_stride(W), _ptr(out),
                         _row_stride(out), _dtype_code(out), M, N, K, _stream())
    _check(st, "matmul_bi")
    return out


def matmul_bi_plan(M: int, N: int, K: int) -> dict:
    """The launches matmul_bi makes for (M, N, K): {"first": (rows, cols, kind),
    "n1": columns of the first launch, "second": (rows, cols, kind) or None};
    kind 0 LDS-pipelined, 1 register streaming, 2 register-staged.  Host only."""
    buf = (ctypes.c_int64 * 7)()
    _check(lib().matmul_bi_plan(M, N, K, buf), "matmul_bi_plan")
    v = list(buf)
    return {"first": tuple(v[0:3]), "n1": v[3], "second": tuple(v[4:7]) if v[4] else None}


def matmul_tuned_differs(M: int, N: int, K: int) -> bool:
    """Whether matmul_tuned runs another schedule than matmul_bi for (M, N, K)."""
    return bool(lib().matmul_tuned_differs(M, N, K))


def matmul_tuned_workspace_size(M: int, N: int, K: int) -> int:
    return int(lib().matmul_tuned_workspace_size(M, N, K))


def matmul_tuned(A: torch.Tensor, W: torch.Tensor, out_dtype=torch.bfloat16, out=None,
                 workspace: torch.Tensor | None = None) -> torch.Tensor:
    """Split-K twin of matmul_bi (not batch-invariant)."""
    M, N, K, out = _mm_prep(A, W, out_dtype, out)
    need = matmul_tuned_workspace_size(M, N, K)
    if need and (workspace is None or workspace.numel() * workspace.element_size() < need):
        workspace = torch.empty(need, dtype=torch.uint8, device=A.device)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    st = lib().matmul_tuned(_ptr(A), _row_stride(A), _ptr(W), _row_stride(W), _ptr(out),
                            _row_stride(out), _dtype_code(out), M, N, K, _ptr(workspace),
                            ws_bytes, _stream())
    _check(st, "matmul_tuned")
    return out


# -------------------------------------------------------------------------------------
# Decode attention
# -------------------------------------------------------------------------------------

def decode_attn_workspace_size(rows: int, num_q_heads: int, head_dim: int, max_kv_len: int,
                               split_size: int) -> int:
    return int(lib().decode_attn_workspace_size(rows, num_q_heads, head_dim, max_kv_len,
                                                split_size))


def decode_attn_tuned_split_size(rows: int, num_kv_heads: int, max_kv_len: int,
                                 kv_lens_host=None) -> int:
    arr = None
    if kv_lens_host is not None:
        arr = torch.as_tensor(kv_lens_host, dtype=torch.int32).contiguous()
    return int(lib().decode_attn_tuned_split_size(rows, num_kv_heads, max_kv_len, _ptr(arr)))


def _attn_prep(q, k_cache, v_cache, block_table, kv_lens, out):
    _need_cuda(q, k_cache, v_cache, block_table, kv_lens)
    if q.dtype != torch.bfloat16 or k_cache.dtype != torch.bfloat16 or v_cache.dtype != torch.bfloat16:
        raise RbiError("q and the KV cache must be bf16")
    if block_table.dtype != torch.int32 or kv_lens.dtype != torch.int32:
        raise RbiError("block_table and kv_lens must be int32")
    if not (k_cache.is_contiguous() and v_cache.is_contiguous() and kv_lens.is_contiguous()):
        raise RbiError("caches and kv_lens must be contiguous")
    if k_cache.dim() != 4 or v_cache.shape != (k_cache.shape[0], k_cache.shape[1],
                                               k_cache.shape[3], k_cache.shape[2]):
        raise RbiError("caches must be K [num_pages, num_kv_heads, page_size, head_dim] and "
                       "V [num_pages, num_kv_heads, head_dim, page_size]")
    rows, hq, d = q.shape
    if q.stride(2) != 1 or q.stride(1) != d:
        raise RbiError("q must be [rows, heads, head_dim] with packed heads")
    _, hkv, page, d2 = k_cache.shape
    if d2 != d:
        raise RbiError("head_dim mismatch between q and the cache")
    if block_table.dim() != 2 or block_table.stride(1) != 1 or block_table.shape[0] != rows:
        raise RbiError("block_table must be [rows, max_pages] with unit inner stride")
    if out is None:
        out = torch.empty((rows, hq, d), dtype=torch.bfloat16, device=q.device)
    if out.stride(2) != 1 or out.stride(1) != d:
        raise RbiError("out must be [rows, heads, head_dim] with packed heads")
    return rows, hq, hkv, d, page, out


def decode_attn_bi(q, k_cache, v_cache, block_table, kv_lens, max_kv_len: int,
                   split_size: int = 256, scale: float | None = None, out=None,
                   workspace: torch.Tensor | None = None) -> torch.Tensor:
    """Fixed-split-size paged decode attention (batch-invariant)."""
    rows, hq, hkv, d, page, out = _attn_prep(q, k_cache, v_cache, block_table, kv_lens, out)
    scale = 1.0 / math.sqrt(d) if scale is None else scale
    need = decode_attn_workspace_size(rows, hq, d, max_kv_len, split_size)
    if workspace is None or workspace.numel() * workspace.element_size() < need:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=q.device)
    st = lib().decode_attn_bi(_ptr(q), _lead_stride(q), _ptr(k_cache), _ptr(v_cache),
                              _ptr(block_table), _lead_stride(block_table), _ptr(kv_lens),
                              _ptr(out), _lead_stride(out), rows, hq, hkv, d, page, split_size, max_kv_len,
                              float(scale), _ptr(workspace),
                              workspace.numel() * workspace.element_size(), _stream())
    _check(st, "decode_attn_bi")
    return out


NOALLOC_SCRATCH_BYTES = 128 << 20  # RBI_NOALLOC_SCRATCH_BYTES


def decode_attn_bi_noalloc(q, k_cache, v_cache, block_table, kv_lens, max_kv_len: int,
                           split_size: int = 256, scale: float | None = None,
                           out=None) -> torch.Tensor:
    """decode_attn_bi with its split partials in the library's static device scratch
    (no workspace, nothing allocated by the library; pass `out` to allocate nothing
    here either).  Same bits as decode_attn_bi.  Calls that overlap on one device
    race on the shared scratch."""
    rows, hq, hkv, d, page, out = _attn_prep(q, k_cache, v_cache, block_table, kv_lens, out)
    scale = 1.0 / math.sqrt(d) if scale is None else scale
    st = lib().decode_attn_bi_noalloc(_ptr(q), _lead_stride(q), _ptr(k_cache), _ptr(v_cache),
                                      _ptr(block_table), _lead_stride(block_table), _ptr(kv_lens),
                                      _ptr(out), _lead_stride(out), rows, hq, hkv, d, page,
                                      split_size, max_kv_len, float(scale), _stream())
    _check(st, "decode_attn_bi_noalloc")
    return out


def decode_attn_tuned(q, k_cache, v_cache, block_table, kv_lens, max_kv_len: int,
                      kv_lens_host=None, scale: float | None = None, out=None,
                      workspace: torch.Tensor | None = None) -> torch.Tensor:
    """Balanced-split twin of decode_attn_bi (split size from the batch shape)."""
    rows, hq, hkv, d, page, out = _attn_prep(q, k_cache, v_cache, block_table, kv_lens, out)
    scale = 1.0 / math.sqrt(d) if scale is None else scale
    host = None
    if kv_lens_host is not None:
        host = torch.as_tensor(kv_lens_host, dtype=torch.int32).contiguous()
    split = decode_attn_tuned_split_size(rows, hkv, max_kv_len, host)
    need = decode_attn_workspace_size(rows, hq, d, max_kv_len, split)
    if workspace is None or workspace.numel() * workspace.element_size() < need:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=q.device)
    st = lib().decode_attn_tuned(_ptr(q), _lead_stride(q), _ptr(k_cache), _ptr(v_cache),
                                 _ptr(block_table), _lead_stride(block_table), _ptr(kv_lens),
                                 _ptr(host), _ptr(out), _lead_stride(out), rows, hq, hkv, d, page,
                                 max_kv_len, float(scale), _ptr(workspace),
                                 workspace.numel() * workspace.element_size(), _stream())
    _check(st, "decode_attn_tuned")
    return out


def prefill_attn_workspace_size(tokens: int, num_q_heads: int, num_kv_heads: int,
                                head_dim: int, start_pos: int, split_size: int) -> int:
    return int(lib().prefill_attn_workspace_size(tokens, num_q_heads, num_kv_heads, head_dim,
                                                 start_pos, split_size))


def prefill_attn_bi(q, k_cache, v_cache, block_table_row, start_pos: int,
                    split_size: int = 256, scale: float | None = None, out=None,
                    workspace: torch.Tensor | None = None) -> torch.Tensor:
    """Attention of consecutive prompt tokens start_pos .. start_pos + len(q) - 1 of one
    request (causal), bit-identical per token to the decode_attn_bi row with
    kv_len = position + 1.  The chunk's K/V must already be in the cache."""
    _need_cuda(q, k_cache, v_cache, block_table_row)
    if q.dtype != torch.bfloat16 or k_cache.dtype != torch.bfloat16 or v_cache.dtype != torch.bfloat16:
        raise RbiError("q and the KV cache must be bf16")
    if block_table_row.dtype != torch.int32 or block_table_row.dim() != 1 or \
            not block_table_row.is_contiguous():
        raise RbiError("block_table_row must be a contiguous int32 vector")
    if not (k_cache.is_contiguous() and v_cache.is_contiguous()) or k_cache.dim() != 4 or \
            v_cache.shape != (k_cache.shape[0], k_cache.shape[1], k_cache.shape[3],
                              k_cache.shape[2]):
        raise RbiError("caches must be K [num_pages, num_kv_heads, page_size, head_dim] and "
                       "V [num_pages, num_kv_heads, head_dim, page_size], contiguous")
    tokens, hq, d = q.shape
    if q.stride(2) != 1 or q.stride(1) != d:
        raise RbiError("q must be [tokens, heads, head_dim] with packed heads")
    _, hkv, page, d2 = k_cache.shape
    if d2 != d:
        raise RbiError("head_dim mismatch between q and the cache")
    if block_table_row.shape[0] * page < start_pos + tokens:
        raise RbiError("block_table_row does not cover start_pos + tokens")
    if out is None:
        out = torch.empty((tokens, hq, d), dtype=torch.bfloat16, device=q.device)
    if out.stride(2) != 1 or out.stride(1) != d:
        raise RbiError("out must be [tokens, heads, head_dim] with packed heads")
    scale = 1.0 / math.sqrt(d) if scale is None else scale
    need = prefill_attn_workspace_size(tokens, hq, hkv, d, start_pos, split_size)
    if need and (workspace is None or workspace.numel() * workspace.element_size() < need):
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    st = lib().prefill_attn_bi(_ptr(q), _lead_stride(q), _ptr(k_cache), _ptr(v_cache),
                               _ptr(block_table_row), start_pos, tokens, _ptr(out),
                               _lead_stride(out), hq, hkv, d, page, split_size, float(scale),
                               _ptr(workspace), ws_bytes, _stream())
    _check(st, "prefill_attn_bi")
    return out


def sample_gumbel_workspace_size(rows: int, vocab: int) -> int:
    return int(lib().sample_gumbel_workspace_size(rows, vocab))


def sample_gumbel(logits: torch.Tensor, seeds, positions, temperatures, out=None,
                  workspace: torch.Tensor | None = None) -> torch.Tensor:
    """Seeded Gumbel-max sampling of fp32 logits [rows, vocab]: per row,
    argmax(logit / T + Gumbel noise of (seed, position, vocab id)); greedy when
    T <= 0.  seeds (uint64 values), positions and temperatures are per-row device
    tensors or sequences.  Returns int32 tokens [rows]."""
    _need_cuda(logits)
    if logits.dtype != torch.float32 or logits.dim() != 2 or logits.stride(1) != 1:
        raise RbiError("logits must be fp32 [rows, vocab] with unit inner stride")
    rows, vocab = logits.shape
    dev = logits.device

    def dev_tensor(v, dtype):
        t = v if isinstance(v, torch.Tensor) else torch.as_tensor(v)
        return t.to(device=dev, dtype=dtype).contiguous().reshape(rows)

    s = seeds if isinstance(seeds, torch.Tensor) else torch.as_tensor(
        [int(x) - (1 << 64) if int(x) >= (1 << 63) else int(x) for x in seeds], dtype=torch.int64)
    s = dev_tensor(s, torch.int64)          # uint64 bits carried in int64
    p = dev_tensor(positions, torch.int64)
    t = dev_tensor(temperatures, torch.float32)
    if out is None:
        out = torch.empty(rows, dtype=torch.int32, device=dev)
    need = sample_gumbel_workspace_size(rows, vocab)
    if workspace is None or workspace.numel() * workspace.element_size() < need:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=dev)
    st = lib().sample_gumbel(_ptr(logits), _lead_stride(logits), rows, vocab, _ptr(s), _ptr(p),
                             _ptr(t), _ptr(out), _ptr(workspace),
                             workspace.numel() * workspace.element_size(), _stream())
    _check(st, "sample_gumbel")
    return out


def kv_append(k_new, v_new, slot_mapping, k_cache, v_cache) -> None:
    """Write k_new/v_new [tokens, Hkv, D] (or [tokens, Hkv*D] row views) into the cache
    slots given by slot_mapping [tokens] int32 (page * page_size + offset); K pages
    token-major [pages, Hkv, page, D], V pages head-dim-major [pages, Hkv, D, page]."""
    _need_cuda(k_new, v_new, slot_mapping, k_cache, v_cache)
    num_pages, hkv, page, d = k_cache.shape
    tokens = k_new.shape[0]
    if slot_mapping.dtype != torch.int32 or slot_mapping.shape[0] != tokens:
        raise RbiError("slot_mapping must be int32 [tokens]")
    st = lib().kv_append(_ptr(k_new), _lead_stride(k_new), _ptr(v_new), _lead_stride(v_new),
                         _ptr(slot_mapping), tokens, _ptr(k_cache), _ptr(v_cache), num_pages, hkv,
                         d, page, _stream())
    _check(st, "kv_append")


# -------------------------------------------------------------------------------------
# glue
# -------------------------------------------------------------------------------------

def embed(table: torch.Tensor, ids: torch.Tensor, out=None) -> torch.Tensor:
    _need_cuda(table, ids)
    vocab, hidden = table.shape
    if out is None:
        out = torch.empty((ids.shape[0], hidden), dtype=table.dtype, device=table.device)
    st = lib().rbi_embed(_ptr(table), vocab, hidden, _ptr(ids), ids.shape[0], _ptr(out),
                         _row_stride(out), _stream())
    _check(st, "rbi_embed")
    return out


def residual_add(a: torch.Tensor, b: torch.Tensor, out=None) -> torch.Tensor:
    _need_cuda(a, b)
    if not (a.is_contiguous() and b.is_contiguous()) or a.shape != b.shape:
        raise RbiError("residual_add needs two contiguous tensors of one shape")
    if out is None:
        out = torch.empty_like(a)
    st = lib().rbi_residual_add(_ptr(a), _ptr(b), _ptr(out), a.numel(), _stream())
    _check(st, "rbi_residual_add")
    return out


def swiglu(gu: torch.Tensor, out=None) -> torch.Tensor:
    _need_cuda(gu)
    rows, two_i = gu.shape
    inter = two_i // 2
    if out is None:
        out = torch.empty((rows, inter), dtype=gu.dtype, device=gu.device)
    st = lib().rbi_swiglu(_ptr(gu), _row_stride(gu), _ptr(out), _row_stride(out), rows, inter,
                          _stream())
    _check(st, "rbi_swiglu")
    return out


def argmax_rows(x: torch.Tensor, out=None) -> torch.Tensor:
    _need_cuda(x)
    if x.dtype != torch.float32:
        raise RbiError("argmax_rows takes fp32 rows")
    rows, n = x.shape
    if out is None:
        out = torch.empty((rows,), dtype=torch.int32, device=x.device)
    st = lib().rbi_argmax_rows(_ptr(x), _row_stride(x), rows, n, _ptr(out), _stream())
    _check(st, "rbi_argmax_rows")
    return out


def stream_copy(src: torch.Tensor, dst: torch.Tensor, nontemporal: bool = False) -> None:
    """dst <- src (same byte size, contiguous) by the library's plain streaming copy
    kernel: the read + write reference rate for RMSNorm (a measurement aid)."""
    _need_cuda(src, dst)
    nbytes = src.numel() * src.element_size()
    if not (src.is_contiguous() and dst.is_contiguous()) or dst.numel() * dst.element_size() != nbytes:
        raise RbiError("stream_copy needs two contiguous tensors of one byte size")
    _check(lib().rbi_stream_copy(_ptr(src), _ptr(dst), nbytes, int(nontemporal), _stream()),
           "rbi_stream_copy")
