// capi.hip -- the extern "C" boundary of librbi (declared in include/rbi.h):
// argument validation, workspace sizing and dispatch to the kernel launchers.
// Every check runs before anything is enqueued, so an error leaves no trace.
#include "../../include/rbi.h"

#include <hip/hip_runtime.h>

#include <mutex>

#include "launch.h"

// Device scratch of decode_attn_bi_noalloc: its split partials, for callers that
// cannot allocate.  Each device the library runs on holds one copy until the
// process ends.  In host code `scratch` names a host-side stand-in, not device
// memory: kernels get the address hipGetSymbolAddress returns for it.
static __device__ __align__(256) unsigned char scratch[RBI_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::mutex scratch_mu;
void *scratch_dev[kMaxDevices];  // device address of `scratch`, per device, once looked up

// The device address of `scratch` on the calling thread's current device: looked
// up once per device (with that device current) and kept; allocates nothing.
int scratch_for_current_device(void **ptr)
{
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices)
        return RBI_ELAUNCH;
    std::lock_guard<std::mutex> lock(scratch_mu);
    if (!scratch_dev[dev]) {
        void *p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p)
            return RBI_ELAUNCH;
        scratch_dev[dev] = p;
    }
    *ptr = scratch_dev[dev];
    return RBI_OK;
}

inline bool aligned16(const void *p)
{
    return (reinterpret_cast<uintptr_t>(p) & 15u) == 0;
}

inline int launched(hipError_t e)
{
    return e == hipSuccess ? RBI_OK : RBI_ELAUNCH;
}

inline hipStream_t stream_of(void *s)
{
    return reinterpret_cast<hipStream_t>(s);
}

constexpr int64_t kGridYZ = 65535;  // maximum grid extent in y and z
// Every launch keeps fewer than kMaxThreadsX threads along the grid's x dimension
// (blocks x threads per block), the range the dispatch packet's 32-bit grid size
// holds with a margin; the checks below bound the sizes that feed each launch.
constexpr int64_t kMaxThreadsX = (int64_t)1 << 31;

int check_rmsnorm(const void *x, int64_t xs, const void *w, void *y, int64_t ys, int64_t rows,
                  int64_t hidden, int dtype)
{
    if (dtype != RBI_F32 && dtype != RBI_BF16)
        return RBI_EUNSUPPORTED;
    if (rows < 0 || hidden < 1)
        return RBI_EINVAL;
    if (rows == 0)
        return RBI_OK;
    if (!x || !w || !y || !aligned16(x) || !aligned16(w) || !aligned16(y))
        return RBI_EINVAL;
    const int64_t vec = dtype == RBI_BF16 ? 8 : 4;
    if (xs < hidden || ys < hidden || xs % vec || ys % vec)
        return RBI_EINVAL;
    if (rows * 256 >= kMaxThreadsX)  // 256 threads per row beyond 1024 rows (512 below)
        return RBI_EUNSUPPORTED;
    return RBI_OK;
}

int check_matmul(const void *A, int64_t lda, const void *W, int64_t ldw, void *C, int64_t ldc,
                 int c_dtype, int64_t M, int64_t N, int64_t K)
{
    if (c_dtype != RBI_F32 && c_dtype != RBI_BF16)
        return RBI_EUNSUPPORTED;
    if (M < 0 || N < 1 || K < 8 || K % 8 || N % 4)
        return RBI_EINVAL;
    if (M == 0)
        return RBI_OK;
    if (!A || !W || !C || !aligned16(A) || !aligned16(W) || !aligned16(C))
        return RBI_EINVAL;
    if (lda < K || ldw < K || lda % 8 || ldw % 8 || ldc < N || ldc % 4)
        return RBI_EINVAL;
    if (M > (int64_t)0x3fffffff || N > (int64_t)0x3fffffff || K > (int64_t)0x3fffffff)
        return RBI_EUNSUPPORTED;
    // grid bound: the smallest tile is 16 x 16 on one 64-lane wave, and every other
    // tile shape has fewer threads per output element
    if (((M + 15) / 16) * ((N + 15) / 16) * 64 >= kMaxThreadsX)
        return RBI_EUNSUPPORTED;
    return RBI_OK;
}

int check_attn(const void *q, int64_t qs, const void *kc, const void *vc, const int32_t *bt,
               int64_t bts, const int32_t *lens, void *out, int64_t os, int64_t rows, int hq,
               int hkv, int d, int page, int split, int max_kv_len)
{
    if (rows < 0 || hq < 1 || hkv < 1 || max_kv_len < 1 || split < 1 || page < 1)
        return RBI_EINVAL;
    if (hq % hkv)
        return RBI_EINVAL;
    if (d != 64 && d != 128)
        return RBI_EUNSUPPORTED;
    if (page != 16 || split % page || split > 1024)
        return RBI_EUNSUPPORTED;
    if (hq / hkv > 16)
        return RBI_EUNSUPPORTED;
    if (rows == 0)
        return RBI_OK;
    if (!q || !kc || !vc || !bt || !lens || !out)
        return RBI_EINVAL;
    if (!aligned16(q) || !aligned16(kc) || !aligned16(vc) || !aligned16(out))
        return RBI_EINVAL;
    if (qs < (int64_t)hq * d || os < (int64_t)hq * d || qs % 8 || os % 8)
        return RBI_EINVAL;
    const int64_t pages_needed = ((int64_t)max_kv_len + page - 1) / page;
    if (bts < pages_needed)
        return RBI_EINVAL;
    const int64_t nsmax = ((int64_t)max_kv_len + split - 1) / split;
    // lengths up to 2^30 keep every token index the kernels form (a split's end, a
    // length rounded up to the page or split) inside int
    if (max_kv_len > (1 << 30) || rows > kGridYZ || nsmax * hkv * 512 >= kMaxThreadsX ||
        rows * hq * 64 >= kMaxThreadsX)
        return RBI_EUNSUPPORTED;
    return RBI_OK;
}

}  // namespace

extern "C" {

const char *rbi_status_string(int status)
{
    switch (status) {
    case RBI_OK: return "RBI_OK";
    case RBI_EINVAL: return "RBI_EINVAL: invalid argument";
    case RBI_EUNSUPPORTED: return "RBI_EUNSUPPORTED: valid but not implemented";
    case RBI_EWORKSPACE: return "RBI_EWORKSPACE: workspace missing or too small";
    case RBI_ELAUNCH: return "RBI_ELAUNCH: kernel launch failed";
    default: return "RBI: unknown status";
    }
}

int rbi_abi_version(void)
{
    return 1;
}

#ifndef RBI_BUILD_INFO
#define RBI_BUILD_INFO "git=unknown src_sha256=unknown"
#endif

const char *rbi_build_info(void)
{
    return RBI_BUILD_INFO;
}

int rmsnorm_bi(const void *x, int64_t x_row_stride, const void *w, void *y, int64_t y_row_stride,
               int64_t rows, int64_t hidden, float eps, int dtype, void *stream)
{
    const int st = check_rmsnorm(x, x_row_stride, w, y, y_row_stride, rows, hidden, dtype);
    if (st != RBI_OK || rows == 0)
        return st;
    return launched(rbi::launch_rmsnorm_wave(x, x_row_stride, w, y, y_row_stride, rows, hidden,
                                             eps, dtype == RBI_BF16, stream_of(stream)));
}

int rmsnorm_tuned(const void *x, int64_t x_row_stride, const void *w, void *y,
                  int64_t y_row_stride, int64_t rows, int64_t hidden, float eps, int dtype,
                  void *stream)
{
    const int st = check_rmsnorm(x, x_row_stride, w, y, y_row_stride, rows, hidden, dtype);
    if (st != RBI_OK || rows == 0)
        return st;
    // fewer rows than wave slots of one wave per SIMD (256 CUs x 4): give each row a workgroup
    if (rows < 1024)
        return launched(rbi::launch_rmsnorm_block(x, x_row_stride, w, y, y_row_stride, rows,
                                                  hidden, eps, dtype == RBI_BF16,
                                                  stream_of(stream)));
    return launched(rbi::launch_rmsnorm_wave(x, x_row_stride, w, y, y_row_stride, rows, hidden,
                                             eps, dtype == RBI_BF16, stream_of(stream)));
}

int matmul_bi(const void *A, int64_t lda, const void *W, int64_t ldw, void *C, int64_t ldc,
              int c_dtype, int64_t M, int64_t N, int64_t K, void *stream)
{
    const int st = check_matmul(A, lda, W, ldw, C, ldc, c_dtype, M, N, K);
    if (st != RBI_OK || M == 0)
        return st;
    const rbi::MatmulArgs a{(const uint16_t *)A, lda, (const uint16_t *)W, ldw, C, ldc,
                            c_dtype == RBI_BF16, M, N, K};
    return launched(rbi::launch_matmul_bi(a, stream_of(stream)));
}

int matmul_bi_plan(int64_t M, int64_t N, int64_t K, int64_t *plan)
{
    if (!plan || M < 1 || N < 1 || K < 8 || K % 8 || N % 4)
        return RBI_EINVAL;
    rbi::describe_matmul_plan(rbi::plan_matmul_bi(M, N, K), plan);
    return RBI_OK;
}

int matmul_tuned_differs(int64_t M, int64_t N, int64_t K)
{
    if (M < 1 || N < 1 || K < 8 || K % 8 || N % 4)
        return 0;
    return rbi::matmul_tuned_splits(M, N, K) > 1 ? 1 : 0;
}

size_t matmul_tuned_workspace_size(int64_t M, int64_t N, int64_t K)
{
    if (M <= 0 || N <= 0 || K <= 0)
        return 0;
    const int splits = rbi::matmul_tuned_splits(M, N, K);
    return splits > 1 ? (size_t)splits * (size_t)M * (size_t)N * sizeof(float) : 0;
}

int matmul_tuned(const void *A, int64_t lda, const void *W, int64_t ldw, void *C, int64_t ldc,
                 int c_dtype, int64_t M, int64_t N, int64_t K, void *workspace,
                 size_t workspace_bytes, void *stream)
{
    const int st = check_matmul(A, lda, W, ldw, C, ldc, c_dtype, M, N, K);
    if (st != RBI_OK || M == 0)
        return st;
    const size_t need = matmul_tuned_workspace_size(M, N, K);
    if (need && (!workspace || workspace_bytes < need || !aligned16(workspace)))
        return RBI_EWORKSPACE;
    const rbi::MatmulArgs a{(const uint16_t *)A, lda, (const uint16_t *)W, ldw, C, ldc,
                            c_dtype == RBI_BF16, M, N, K};
    const int splits = rbi::matmul_tuned_splits(M, N, K);
    if (splits == 1)
        return launched(rbi::launch_matmul_bi(a, stream_of(stream)));
    return launched(rbi::launch_matmul_splitk(a, splits, (float *)workspace, stream_of(stream)));
}

size_t decode_attn_workspace_size(int64_t rows, int num_q_heads, int head_dim, int max_kv_len,
                                  int split_size)
{
    if (rows <= 0 || num_q_heads <= 0 || head_dim <= 0 || max_kv_len <= 0 || split_size <= 0)
        return 0;
    return rbi::attn_workspace_bytes(rows, num_q_heads, head_dim, max_kv_len, split_size);
}

static int attn_common(const void *q, int64_t qs, const void *kc, const void *vc,
                       const int32_t *bt, int64_t bts, const int32_t *lens, void *out, int64_t os,
                       int64_t rows, int hq, int hkv, int d, int page, int split, int max_kv_len,
                       float scale, void *ws, size_t ws_bytes, void *stream)
{
    const int st = check_attn(q, qs, kc, vc, bt, bts, lens, out, os, rows, hq, hkv, d, page, split,
                              max_kv_len);
    if (st != RBI_OK || rows == 0)
        return st;
    const size_t need = rbi::attn_workspace_bytes(rows, hq, d, max_kv_len, split);
    if (!ws || ws_bytes < need || !aligned16(ws))
        return RBI_EWORKSPACE;
    const rbi::AttnArgs a{(const uint16_t *)q, qs, (const uint16_t *)kc, (const uint16_t *)vc,
                          bt, bts, lens, (uint16_t *)out, os, rows, hq, hkv, d, page, split,
                          max_kv_len, scale, (float *)ws};
    return launched(rbi::launch_decode_attn(a, stream_of(stream)));
}

int decode_attn_bi(const void *q, int64_t q_row_stride, const void *k_cache, const void *v_cache,
                   const int32_t *block_table, int64_t bt_stride, const int32_t *kv_lens,
                   void *out, int64_t out_row_stride, int64_t rows, int num_q_heads,
                   int num_kv_heads, int head_dim, int page_size, int split_size, int max_kv_len,
                   float scale, void *workspace, size_t workspace_bytes, void *stream)
{
    return attn_common(q, q_row_stride, k_cache, v_cache, block_table, bt_stride, kv_lens, out,
                       out_row_stride, rows, num_q_heads, num_kv_heads, head_dim, page_size,
                       split_size, max_kv_len, scale, workspace, workspace_bytes, stream);
}

int decode_attn_bi_noalloc(const void *q, int64_t q_row_stride, const void *k_cache,
                           const void *v_cache, const int32_t *block_table, int64_t bt_stride,
                           const int32_t *kv_lens, void *out, int64_t out_row_stride, int64_t rows,
                           int num_q_heads, int num_kv_heads, int head_dim, int page_size,
                           int split_size, int max_kv_len, float scale, void *stream)
{
    const int st = check_attn(q, q_row_stride, k_cache, v_cache, block_table, bt_stride, kv_lens,
                              out, out_row_stride, rows, num_q_heads, num_kv_heads, head_dim,
                              page_size, split_size, max_kv_len);
    if (st != RBI_OK || rows == 0)
        return st;
    // every partial the merge reads, and the work plan, are written by the same call
    // first, so nothing in the scratch has to start at zero
    if (rbi::attn_workspace_bytes(rows, num_q_heads, head_dim, max_kv_len, split_size) >
        (size_t)RBI_NOALLOC_SCRATCH_BYTES)
        return RBI_EWORKSPACE;
    void *ws = nullptr;
    const int sp = scratch_for_current_device(&ws);
    if (sp != RBI_OK)
        return sp;
    const rbi::AttnArgs a{(const uint16_t *)q, q_row_stride, (const uint16_t *)k_cache,
                          (const uint16_t *)v_cache, block_table, bt_stride, kv_lens,
                          (uint16_t *)out, out_row_stride, rows, num_q_heads, num_kv_heads,
                          head_dim, page_size, split_size, max_kv_len, scale, (float *)ws};
    return launched(rbi::launch_decode_attn(a, stream_of(stream)));
}

size_t prefill_attn_workspace_size(int64_t tokens, int num_q_heads, int num_kv_heads,
                                   int head_dim, int64_t start_pos, int split_size)
{
    if (tokens <= 0 || num_q_heads <= 0 || num_kv_heads <= 0 || head_dim <= 0 ||
        start_pos < 0 || split_size <= 0)
        return 0;
    return rbi::prefill_workspace_bytes(tokens, num_q_heads, num_kv_heads, head_dim, start_pos,
                                        split_size);
}

int prefill_attn_bi(const void *q, int64_t q_row_stride, const void *k_cache, const void *v_cache,
                    const int32_t *block_table_row, int64_t start_pos, int64_t tokens, void *out,
                    int64_t out_row_stride, int num_q_heads, int num_kv_heads, int head_dim,
                    int page_size, int split_size, float scale, void *workspace,
                    size_t workspace_bytes, void *stream)
{
    const int hq = num_q_heads, hkv = num_kv_heads, d = head_dim;
    if (tokens < 0 || start_pos < 0 || hq < 1 || hkv < 1 || split_size < 1 || page_size < 1)
        return RBI_EINVAL;
    if (hq % hkv)
        return RBI_EINVAL;
    if (d != 64 && d != 128)
        return RBI_EUNSUPPORTED;
    if (page_size != 16 || split_size % page_size || split_size > 256)
        return RBI_EUNSUPPORTED;
    if (hq / hkv > 16)
        return RBI_EUNSUPPORTED;
    if (tokens == 0)
        return RBI_OK;
    if (!q || !k_cache || !v_cache || !block_table_row || !out)
        return RBI_EINVAL;
    if (!aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache) || !aligned16(out))
        return RBI_EINVAL;
    if (q_row_stride < (int64_t)hq * d || out_row_stride < (int64_t)hq * d || q_row_stride % 8 ||
        out_row_stride % 8)
        return RBI_EINVAL;
    // fused: 512 threads per (block of up to 8 tokens, kv head) in one grid dimension;
    // split schedule: 512 per group of four splits, and the merge's 64 per (token, head)
    const int64_t groups = (start_pos + tokens + 4 * (int64_t)split_size - 1) /
                           (4 * (int64_t)split_size);
    if (start_pos + tokens > ((int64_t)1 << 30) || hkv > kGridYZ || tokens * 512 >= kMaxThreadsX ||
        (tokens + 7) / 8 * hkv * 512 >= kMaxThreadsX || groups * 512 >= kMaxThreadsX ||
        tokens * hq * 64 >= kMaxThreadsX)
        return RBI_EUNSUPPORTED;
    const size_t need =
        rbi::prefill_workspace_bytes(tokens, hq, hkv, d, start_pos, split_size);
    if (need && (!workspace || workspace_bytes < need || !aligned16(workspace)))
        return RBI_EWORKSPACE;
    const rbi::PrefillArgs a{(const uint16_t *)q, q_row_stride, (const uint16_t *)k_cache,
                             (const uint16_t *)v_cache, block_table_row, start_pos, tokens,
                             (uint16_t *)out, out_row_stride, hq, hkv, d, page_size, split_size,
                             scale, (float *)workspace};
    return launched(rbi::launch_prefill_attn(a, stream_of(stream)));
}

size_t sample_gumbel_workspace_size(int64_t rows, int64_t vocab)
{
    if (rows <= 0 || vocab <= 0)
        return 0;
    return rbi::sample_workspace_bytes(rows, vocab);
}

int sample_gumbel(const float *logits, int64_t logits_row_stride, int64_t rows, int64_t vocab,
                  const uint64_t *seeds, const int64_t *positions, const float *temperatures,
                  int32_t *tokens, void *workspace, size_t workspace_bytes, void *stream)
{
    if (rows < 0 || vocab < 1 || logits_row_stride < vocab || logits_row_stride % 4)
        return RBI_EINVAL;
    if (rows == 0)
        return RBI_OK;
    if (!logits || !seeds || !positions || !temperatures || !tokens || !aligned16(logits))
        return RBI_EINVAL;
    if (vocab > (int64_t)0x7ffffff0 || rows > kGridYZ)
        return RBI_EUNSUPPORTED;
    const size_t need = rbi::sample_workspace_bytes(rows, vocab);
    if (!workspace || workspace_bytes < need || !aligned16(workspace))
        return RBI_EWORKSPACE;
    return launched(rbi::launch_sample_gumbel(logits, logits_row_stride, rows, vocab, seeds,
                                              positions, temperatures, tokens, workspace,
                                              stream_of(stream)));
}

// Split size of the twin, tuned to the batch: the fastest size measured on MI355X
// for these kernels (decode batches of 64 query / 4 kv heads, d128, lengths up to
// 32768, split sizes 64 .. 1024 at batch 1 .. 256): 256-token splits from batch
// 4 up (batch 8: 59.1 us against 60.8 at 512; batch 256: 1.78 ms against 1.85 at
// 1024), 512-token splits when the batch is so small that 256-token splits give
// fewer than two (split, kv head) work units per compute unit (batch 1, 23.7 k
// tokens: 17.9 against 22.1 us) -- fewer, longer splits leave fewer partials to
// fold.  The work units are counted from the host lengths when given, else
// estimated as half of rows * ceil(max_kv_len / 256) per kv head.  Capped near
// max_kv_len (rounded up to the page).
int decode_attn_tuned_split_size(int64_t rows, int num_kv_heads, int max_kv_len,
                                 const int32_t *kv_lens_host)
{
    if (rows <= 0 || max_kv_len <= 0)
        return 16;
    const int64_t hkv = num_kv_heads > 0 ? num_kv_heads : 1;
    int64_t units = 0;
    if (kv_lens_host) {
        for (int64_t r = 0; r < rows; ++r) {
            const int64_t L = kv_lens_host[r] < 1 ? 1 : (kv_lens_host[r] > max_kv_len ? max_kv_len
                                                                                   : kv_lens_host[r]);
            units += (L + 255) / 256 * hkv;
        }
    } else {
        units = rows * (((int64_t)max_kv_len + 255) / 256) * hkv / 2;
    }
    int S = units < 2 * 256 ? 512 : 256;
    const int64_t cap = ((int64_t)max_kv_len + 15) / 16 * 16;
    while (S > 16 && S / 2 >= cap)
        S /= 2;
    return S;
}

int decode_attn_tuned(const void *q, int64_t q_row_stride, const void *k_cache,
                      const void *v_cache, const int32_t *block_table, int64_t bt_stride,
                      const int32_t *kv_lens, const int32_t *kv_lens_host, void *out,
                      int64_t out_row_stride, int64_t rows, int num_q_heads, int num_kv_heads,
                      int head_dim, int page_size, int max_kv_len, float scale, void *workspace,
                      size_t workspace_bytes, void *stream)
{
    const int split = decode_attn_tuned_split_size(rows, num_kv_heads, max_kv_len, kv_lens_host);
    return attn_common(q, q_row_stride, k_cache, v_cache, block_table, bt_stride, kv_lens, out,
                       out_row_stride, rows, num_q_heads, num_kv_heads, head_dim, page_size, split,
                       max_kv_len, scale, workspace, workspace_bytes, stream);
}

int kv_append(const void *k_new, int64_t k_row_stride, const void *v_new, int64_t v_row_stride,
              const int32_t *slot_mapping, int64_t tokens, void *k_cache, void *v_cache,
              int64_t num_pages, int num_kv_heads, int head_dim, int page_size, void *stream)
{
    if (tokens < 0 || num_pages < 1 || num_kv_heads < 1 || head_dim < 8 || head_dim % 8 ||
        page_size < 1)
        return RBI_EINVAL;
    if (tokens == 0)
        return RBI_OK;
    if (!k_new || !v_new || !slot_mapping || !k_cache || !v_cache)
        return RBI_EINVAL;
    if (!aligned16(k_new) || !aligned16(v_new) || !aligned16(k_cache) || !aligned16(v_cache))
        return RBI_EINVAL;
    if (k_row_stride % 8 || v_row_stride % 8 || k_row_stride < (int64_t)num_kv_heads * head_dim ||
        v_row_stride < (int64_t)num_kv_heads * head_dim)
        return RBI_EINVAL;
    if (tokens * num_kv_heads * (head_dim / 8) >= kMaxThreadsX)  // a thread per 16 bytes
        return RBI_EUNSUPPORTED;
    return launched(rbi::launch_kv_append((const uint16_t *)k_new, k_row_stride,
                                          (const uint16_t *)v_new, v_row_stride, slot_mapping,
                                          tokens, (uint16_t *)k_cache, (uint16_t *)v_cache,
                                          num_pages, num_kv_heads, head_dim, page_size,
                                          stream_of(stream)));
}

int rbi_embed(const void *table, int64_t vocab, int64_t hidden, const int32_t *ids, int64_t rows,
              void *out, int64_t out_row_stride, void *stream)
{
    if (rows < 0 || vocab < 1 || hidden < 8 || hidden % 8)
        return RBI_EINVAL;
    if (rows == 0)
        return RBI_OK;
    if (!table || !ids || !out || !aligned16(table) || !aligned16(out) ||
        out_row_stride < hidden || out_row_stride % 8)
        return RBI_EINVAL;
    if (rows * (hidden / 8) >= kMaxThreadsX)
        return RBI_EUNSUPPORTED;
    return launched(rbi::launch_embed((const uint16_t *)table, vocab, hidden, ids, rows,
                                      (uint16_t *)out, out_row_stride, stream_of(stream)));
}

int rbi_residual_add(const void *a, const void *b, void *out, int64_t n, void *stream)
{
    if (n < 0)
        return RBI_EINVAL;
    if (n == 0)
        return RBI_OK;
    if (!a || !b || !out)
        return RBI_EINVAL;
    if ((n + 7) / 8 >= kMaxThreadsX)
        return RBI_EUNSUPPORTED;
    return launched(rbi::launch_residual_add((const uint16_t *)a, (const uint16_t *)b,
                                             (uint16_t *)out, n, stream_of(stream)));
}

int rbi_swiglu(const void *gu, int64_t gu_row_stride, void *out, int64_t out_row_stride,
               int64_t rows, int64_t inter, void *stream)
{
    if (rows < 0 || inter < 1)
        return RBI_EINVAL;
    if (rows == 0)
        return RBI_OK;
    if (!gu || !out || gu_row_stride < 2 * inter || out_row_stride < inter)
        return RBI_EINVAL;
    if (rows * ((inter + 7) / 8) >= kMaxThreadsX)
        return RBI_EUNSUPPORTED;
    return launched(rbi::launch_swiglu((const uint16_t *)gu, gu_row_stride, (uint16_t *)out,
                                       out_row_stride, rows, inter, stream_of(stream)));
}

int rbi_argmax_rows(const float *x, int64_t x_row_stride, int64_t rows, int64_t n, int32_t *out,
                    void *stream)
{
    if (rows < 0 || n < 1 || n > (int64_t)0x7ffffffe)
        return RBI_EINVAL;
    if (rows == 0)
        return RBI_OK;
    if (!x || !out || x_row_stride < n)
        return RBI_EINVAL;
    if (rows * 1024 >= kMaxThreadsX)  // a 1024-thread workgroup per row
        return RBI_EUNSUPPORTED;
    return launched(rbi::launch_argmax(x, x_row_stride, rows, n, out, stream_of(stream)));
}

int rbi_stream_copy(const void *src, void *dst, int64_t bytes, int nontemporal, void *stream)
{
    if (bytes < 0 || bytes % 16)
        return RBI_EINVAL;
    if (bytes == 0)
        return RBI_OK;
    if (!src || !dst || !aligned16(src) || !aligned16(dst))
        return RBI_EINVAL;
    if (bytes / 16 >= kMaxThreadsX)
        return RBI_EUNSUPPORTED;
    return launched(rbi::launch_stream_copy(src, dst, bytes, nontemporal != 0, stream_of(stream)));
}

}  // extern "C"
