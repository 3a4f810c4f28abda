/*
 * rbi.h -- C ABI of the batch-invariant forward-reduction library for AMD
 * MI355X (gfx950): librbi.so.
 *
 * Property delivered by every *_bi entry point ("batch invariance"): the bits
 * of each output row depend only on that row's own inputs (and, for attention,
 * on its own KV length and cache contents), never on how many other rows are in
 * the call, where the row sits in the batch, what its neighbours hold, or how a
 * sequence was cut into prefill chunks.  Sources (web pages, by title/section):
 *   [P1] "Reproducible LLM Inference - Batch Invariance, the Cost of
 *        Determinism, and Where Bitwise Identity Is Actually Required"
 *        (hidekazu-konishi.com), sections 5.1-5.5.
 *   [P3] "Your Answer Depends on Who Else Is in the Batch" (praveentn.live),
 *        "Where the reductions are", "The attention detail that gets missed".
 * Each *_tuned entry point is a deliberately shape-tuned twin that computes the
 * same function but picks its reduction split from the shape, so it is
 * run-to-run deterministic but NOT batch-invariant; it exists to price
 * determinism.
 *
 * Conventions shared by every entry point
 *  - All tensor pointers are DEVICE pointers (hipMalloc'd or from a framework
 *    allocator) unless an argument says "host".  The caller owns all memory.
 *    The library never allocates, frees or synchronises, and keeps no mutable
 *    global state other than the device scratch of decode_attn_bi_noalloc.
 *  - `stream` is a hipStream_t passed as void* (NULL = the null stream).  Work is
 *    enqueued asynchronously on it; results are ready when the stream is.
 *  - Return value: RBI_OK (0) or a negative status.  Arguments are validated
 *    before anything is enqueued; on error nothing is enqueued and no memory is
 *    touched.  A zero-sized problem (rows == 0, M == 0, tokens == 0) is a no-op
 *    that returns RBI_OK.  No C++ exception crosses this boundary.
 *  - Layouts are row-major; strides are in ELEMENTS.  bf16 is IEEE bfloat16
 *    stored as 16-bit words; every rounding to bf16 is round-to-nearest-even.
 *  - No kernel uses atomics: repeated calls on the same inputs give the same
 *    bits (run-to-run determinism, [P1] sections 4.2-4.3).
 *  - Sizes that would need 2^31 or more threads along one grid dimension of a
 *    launch give RBI_EUNSUPPORTED; each entry point states its bound.
 */
#ifndef RBI_H
#define RBI_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* element types */
enum { RBI_F32 = 0, RBI_BF16 = 1 };

/* status codes */
enum {
    RBI_OK = 0,
    RBI_EINVAL = -1,       /* null pointer, negative size, bad stride or alignment */
    RBI_EUNSUPPORTED = -2, /* valid but outside what the kernels implement        */
    RBI_EWORKSPACE = -3,   /* workspace pointer null or smaller than required      */
    RBI_ELAUNCH = -4       /* the HIP runtime refused a kernel launch               */
};

/* Human-readable name of a status code (static string, never NULL). */
const char *rbi_status_string(int status);

/* Library ABI version, incremented on any signature change. */
int rbi_abi_version(void);

/* What the library was built from (static string, never NULL): "git=<commit>"
 * (suffixed "-dirty" when the checkout had uncommitted changes) and
 * "src_sha256=<first 16 hex digits>" over the kernel and ABI sources. */
const char *rbi_build_info(void);

/* -------------------------------------------------------------------------- */
/* RMSNorm                                                                     */
/* -------------------------------------------------------------------------- */
/*
 * rmsnorm_bi: y[r,i] = x[r,i] * (1 / sqrt(sum_j x[r,j]^2 / hidden + eps)) * w[i]
 * ([P1] section 5.4 "The Three Operations That Involve a Reduction", first
 * operation; [P3] "A Concrete Example").  Each row is reduced by ONE wavefront
 * in an order fixed by `hidden` alone ([P1] section 5.3: one row per core, so
 * the order is the same at any batch size): lane-strided fp32 partial sums over
 * 16-byte chunks, then a fixed xor-butterfly across the 64 lanes.  The scale and
 * product are formed in fp32, (x * r) * w, and rounded once to the output type.
 *
 *  x      [rows, hidden], row stride x_row_stride; dtype RBI_F32 or RBI_BF16
 *  w      [hidden], same dtype as x
 *  y      [rows, hidden], row stride y_row_stride, same dtype; may alias x when
 *         the strides are equal (each row is read fully before it is written)
 *  eps    added to the mean of squares, inside the root
 * Requirements: x, y, w 16-byte aligned; row strides multiples of 16 bytes
 * (8 bf16 / 4 fp32 elements) and >= hidden; hidden >= 1.  Otherwise RBI_EINVAL.
 * rows >= 2^23 gives RBI_EUNSUPPORTED.
 */
int rmsnorm_bi(const void *x, int64_t x_row_stride, const void *w, void *y,
               int64_t y_row_stride, int64_t rows, int64_t hidden, float eps, int dtype,
               void *stream);

/*
 * rmsnorm_tuned: same function and arguments.  When rows are too few to fill
 * the chip it spreads each row over a whole 256-thread workgroup (a different
 * reduction tree), otherwise it uses the one-wavefront-per-row layout; the bits
 * of a row therefore depend on the batch size ([P1] section 5.3, the
 * small-batch split that breaks invariance).
 */
int rmsnorm_tuned(const void *x, int64_t x_row_stride, const void *w, void *y,
                  int64_t y_row_stride, int64_t rows, int64_t hidden, float eps, int dtype,
                  void *stream);

/* -------------------------------------------------------------------------- */
/* Matmul                                                                      */
/* -------------------------------------------------------------------------- */
/*
 * matmul_bi: C[m,n] = sum_k A[m,k] * W[n,k]   (C = A . W^T, W stored [N, K] as a
 * linear layer's weight).  bf16 inputs, fp32 accumulation, one rounding to
 * c_dtype (RBI_BF16 or RBI_F32).  [P1] section 5.4, second operation: one
 * kernel configuration for every shape -- no split-K and no change of matrix
 * instruction with M.  Every output element is accumulated by the same
 * sequence of v_mfma_f32_16x16x32_bf16 steps over K in ascending 32-wide
 * blocks, starting from zero, whatever M, N or its position in the tile.
 *
 *  A  [M, K] bf16, row stride lda;  W [N, K] bf16, row stride ldw;
 *  C  [M, N] c_dtype, row stride ldc.
 * Requirements: A, W 16-byte aligned, lda and ldw multiples of 8, K a positive
 * multiple of 8, lda >= K, ldw >= K; C 16-byte aligned, ldc a multiple of 4,
 * ldc >= N, N a multiple of 4.  Otherwise RBI_EINVAL.  Sizes with
 * ceil(M/16) * ceil(N/16) >= 2^25 (the 16 x 16 tile's 64 threads each) give
 * RBI_EUNSUPPORTED.
 */
int matmul_bi(const void *A, int64_t lda, const void *W, int64_t ldw, void *C, int64_t ldc,
              int c_dtype, int64_t M, int64_t N, int64_t K, void *stream);

/*
 * matmul_bi_plan: which launches matmul_bi makes for (M, N, K), for tests that
 * must reach every tile shape and for tuning.  The choice only decides which
 * wave computes an element, never the element's arithmetic.  Fills plan[7]
 * (host memory): {tile rows, tile columns, kind} of the first launch, the
 * number of columns it covers (N when there is one launch), then {tile rows,
 * tile columns, kind} of the launch over the remaining columns (zeros when
 * there is none).  kind: 0 LDS-pipelined tile, 1 register-streaming tile,
 * 2 register-staged tile (K % 32 != 0).  Returns RBI_EINVAL for sizes matmul_bi
 * would reject; needs no GPU.
 */
int matmul_bi_plan(int64_t M, int64_t N, int64_t K, int64_t *plan);

/*
 * matmul_tuned: same function, shape-tuned.  Chooses a tile shape and a split-K
 * count from (M, N, K) by a table measured on MI355X ([P1] section 5.4, "split
 * reduction, also known as split-K"): where splitting K into 2 or 4 equal ranges
 * beat matmul_bi's plan (long-K projections from M = 9 to 768, QKV-wide N near
 * M = 128, very wide N at M <= 16) the ranges' fp32 partials are added in
 * ascending order by a second kernel; elsewhere it runs matmul_bi's plan.  Run to
 * run deterministic, but the K partition -- and so the bits -- changes with M.
 * Needs `workspace` of matmul_tuned_workspace_size(M, N, K) bytes (0 means none
 * is needed; NULL is then allowed).
 */
size_t matmul_tuned_workspace_size(int64_t M, int64_t N, int64_t K);
/* 1 when matmul_tuned runs a different schedule (and so, in general, different
 * bits) than matmul_bi for (M, N, K), else 0; host only. */
int matmul_tuned_differs(int64_t M, int64_t N, int64_t K);
int matmul_tuned(const void *A, int64_t lda, const void *W, int64_t ldw, void *C, int64_t ldc,
                 int c_dtype, int64_t M, int64_t N, int64_t K, void *workspace,
                 size_t workspace_bytes, void *stream);

/* -------------------------------------------------------------------------- */
/* Paged split-KV decode attention                                             */
/* -------------------------------------------------------------------------- */
/*
 * decode_attn_bi: one query token per row, grouped-query heads, over a paged
 * KV cache, split along the KV length at a FIXED SPLIT SIZE ([P1] section 5.5
 * "Why Attention Is the Hardest Case"; [P3] "The attention detail that gets
 * missed").  For row r with length L = kv_lens[r] and query head h (kv head
 * g = h / (num_q_heads / num_kv_heads)):
 *     out[r,h] = sum_{j<L} softmax_j(scale * <q[r,h], k_j>) v_j
 * where k_j and v_j sit in page block_table[r][j / page_size], slot
 * j % page_size.  Split s covers tokens [s*split_size, min((s+1)*split_size, L));
 * the boundaries depend on nothing but L.  Per split the kernel forms a partial
 * (max m, sum l, accumulator acc) with bf16 MFMA products and fp32 softmax;
 * partials are folded in ascending split order with log-sum-exp rescaling
 * (running maximum M; a partial (m, l_s, acc_s) makes M' = max(M, m),
 * l = l 2^(M - M') + 2^(m - M') l_s, acc likewise): for split sizes up to 256
 * first within each group of 4 consecutive splits (splits 4k .. 4k+3), then the
 * groups' partials by a second kernel; longer splits are each their own group.
 * acc / l is rounded to bf16 once.  The whole reduction tree is a function of L
 * alone.
 *
 *  q            [rows, num_q_heads, head_dim] bf16, row stride q_row_stride
 *               (head stride head_dim)
 *  k_cache      [num_pages, num_kv_heads, page_size, head_dim] bf16 (token-major
 *               pages: element (t, d) of a page at t * head_dim + d)
 *  v_cache      [num_pages, num_kv_heads, head_dim, page_size] bf16 (head-dim-major
 *               pages: element (t, d) at d * page_size + t).  Stored this way, a
 *               16-byte run of a V page is the 8 consecutive tokens one matrix-core
 *               operand lane needs for the P.V product, so V is read straight into
 *               the operand with no transposition.
 *  block_table  [rows, bt_stride] int32 physical page ids; only the first
 *               ceil(kv_lens[r] / page_size) entries of a row are read
 *  kv_lens      [rows] int32 (device), each in [1, max_kv_len]
 *  out          [rows, num_q_heads, head_dim] bf16, row stride out_row_stride
 *  max_kv_len   an upper bound on every kv_lens[r]; it sizes the grid and the
 *               workspace only -- results do not depend on it
 *  workspace    >= decode_attn_workspace_size(rows, num_q_heads, head_dim,
 *               max_kv_len, split_size) bytes, 16-byte aligned.  It starts with
 *               the group partials: with GS = 4 splits per group when split_size
 *               <= 256 (else 1), np = ceil(ceil(max_kv_len / split_size) / GS),
 *               G = num_q_heads / num_kv_heads and query head h = g * G + hh, the
 *               partial of (row r, head h, group s) is the (D + 4)-float slot
 *               (((r * num_kv_heads + g) * np + s) * G + hh): fp32 acc[0 .. D),
 *               then m (log2 units: scale * log2(e) * <q, k>), l (the sum of the
 *               weights 2^(score - m) as the P.V product takes them: each weight
 *               split into two bf16 parts, so 16 significant bits) and two zeros.
 *               One group's G slots are one contiguous block.  Groups past
 *               the row's last split are not written.  When GS = 4, a work plan
 *               of 4 + rows + 2 * (rows + 1024) int32 words follows the partials.
 *               Large batches (rows * num_kv_heads at least 1.5 times the
 *               device's compute units) use it: the call builds it on the device
 *               from kv_lens, and each row whose split count is at most the
 *               batch's work per compute unit is computed by one workgroup per
 *               kv head, longest rows first, which folds the row's groups in the
 *               same ascending order and writes out directly; that row's slots
 *               are then not written.  Longer rows, and every row of a smaller
 *               batch, go through the slots as above.  Either way every output
 *               bit is the same
 * Supported: head_dim 64 or 128; page_size 16; split_size a positive multiple of
 * page_size, at most 1024; num_q_heads % num_kv_heads == 0 with a group of 1..16
 * query heads; max_kv_len <= 2^30; rows <= 65535, rows * num_q_heads < 2^25
 * and ceil(max_kv_len / split_size) * num_kv_heads < 2^22;
 * q, out 16-byte aligned with row strides multiples of 8.  A kv_lens entry
 * outside [1, max_kv_len] is clamped into that range on the device (it cannot
 * be reported from there); keep lengths valid.
 */
size_t decode_attn_workspace_size(int64_t rows, int num_q_heads, int head_dim, int max_kv_len,
                                  int split_size);
int decode_attn_bi(const void *q, int64_t q_row_stride, const void *k_cache, const void *v_cache,
                   const int32_t *block_table, int64_t bt_stride, const int32_t *kv_lens,
                   void *out, int64_t out_row_stride, int64_t rows, int num_q_heads,
                   int num_kv_heads, int head_dim, int page_size, int split_size, int max_kv_len,
                   float scale, void *workspace, size_t workspace_bytes, void *stream);

/*
 * decode_attn_bi_noalloc: decode_attn_bi for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc).  Same function, kernels and bits as decode_attn_bi; the
 * split partials go to a static device array of the library instead of a
 * caller's workspace.  The caller still passes inputs and outputs.
 *  - Limit: decode_attn_workspace_size(rows, num_q_heads, head_dim, max_kv_len,
 *    split_size) <= RBI_NOALLOC_SCRATCH_BYTES (128 MiB), else RBI_EWORKSPACE with
 *    nothing enqueued (e.g. 64 query heads of 128 at split 256: rows *
 *    ceil(max_kv_len / 1024) up to about 3970, so 124 rows at 32768 tokens).
 *  - The array is held by every device the library runs on until the process
 *    ends.  The first call on a device looks up its address there (no
 *    allocation); make that first call outside a graph capture.
 *  - Every call on one device shares that device's array, which keeps the last
 *    call's partials and plan.  Calls that overlap on one device (two streams at once)
 *    race and give undefined results; calls in one stream are ordered.
 *  - Nothing in the array needs to start at zero.  No hipMalloc, hipFree or
 *    other allocating routine is called.
 * Other arguments, requirements and errors as decode_attn_bi.
 */
#define RBI_NOALLOC_SCRATCH_BYTES (128u << 20)
int decode_attn_bi_noalloc(const void *q, int64_t q_row_stride, const void *k_cache,
                           const void *v_cache, const int32_t *block_table, int64_t bt_stride,
                           const int32_t *kv_lens, void *out, int64_t out_row_stride, int64_t rows,
                           int num_q_heads, int num_kv_heads, int head_dim, int page_size,
                           int split_size, int max_kv_len, float scale, void *stream);

/*
 * decode_attn_tuned: same function, but the split size is chosen from the
 * batch shape -- the per-batch scheduling of [P1] section 5.5 that the page
 * names as not batch-invariant: a row's split boundaries, and so its bits, move
 * with the batch.  The rule is the fastest split size measured on MI355X for
 * these kernels: 512 tokens when 256-token splits would give fewer than two
 * (split, kv head) work units per compute unit (counted from kv_lens_host, the
 * lengths on the host, when given, else estimated from rows and max_kv_len), 256
 * otherwise (capped near max_kv_len) -- so from a few rows on it coincides with
 * decode_attn_bi's usual configuration.  decode_attn_tuned_split_size() returns
 * the size it will use; the workspace is sized with decode_attn_workspace_size(...,
 * that split size).  Other arguments as decode_attn_bi.
 */
int decode_attn_tuned_split_size(int64_t rows, int num_kv_heads, int max_kv_len,
                                 const int32_t *kv_lens_host);
int decode_attn_tuned(const void *q, int64_t q_row_stride, const void *k_cache,
                      const void *v_cache, const int32_t *block_table, int64_t bt_stride,
                      const int32_t *kv_lens, const int32_t *kv_lens_host, void *out,
                      int64_t out_row_stride, int64_t rows, int num_q_heads, int num_kv_heads,
                      int head_dim, int page_size, int max_kv_len, float scale, void *workspace,
                      size_t workspace_bytes, void *stream);

/*
 * prefill_attn_bi: attention of a run of consecutive prompt tokens of ONE
 * request -- positions start_pos .. start_pos + tokens - 1, token t attending
 * causally to the L_t = start_pos + t + 1 cache entries 0 .. start_pos + t --
 * over the request's block-table row.  Chunked prefill and prefix caching
 * ([P1] section 5.5 "Why Attention Is the Hardest Case", section 6.4 "A Single
 * Request Can Break It Too"; [P3] "Where It Breaks", on prefix caching
 * reintroducing shape dependence) need a token's reduction order not to depend on how many tokens
 * of its sequence are processed together.  Here each (token, query head) is
 * reduced exactly as decode_attn_bi reduces a row with that query and
 * kv_len = L_t (same absolute split boundaries, same per-split partial, same
 * ascending merge), so the output of token t is bit-identical to the
 * decode_attn_bi row for it, whatever start_pos, tokens and the chunking are.
 * Only the schedule differs: a workgroup copies each split's K/V pages of one kv
 * head into LDS once and serves a block of 8 prompt tokens from them.
 * The chunk's K and V must already be in the cache (kv_append first).
 *  q              [tokens, num_q_heads, head_dim] bf16, row stride q_row_stride
 *  k_cache, v_cache  as for decode_attn_bi
 *  block_table_row  int32 physical page ids of the request, at least
 *                 ceil((start_pos + tokens) / page_size) entries (device)
 *  out            [tokens, num_q_heads, head_dim] bf16, row stride out_row_stride
 *  workspace      >= prefill_attn_workspace_size(...) bytes, 16-byte aligned; that
 *                 size is 0 (no workspace; NULL allowed) when the chunk has enough
 *                 tokens to fill the GPU with token blocks, otherwise the split
 *                 group partials are staged there as in decode_attn_bi (slot
 *                 layout with rows = tokens and max_kv_len = start_pos + tokens)
 * Supported: head_dim 64 or 128; page_size 16; split_size a positive multiple of
 * page_size, at most 256 (one page pair per wave); a group of 1..16 query heads
 * per kv head; start_pos + tokens <= 2^30, tokens < 2^22, tokens * num_q_heads
 * < 2^25, ceil(tokens / 8) * num_kv_heads < 2^22 and ceil((start_pos + tokens) /
 * (4 * split_size)) < 2^22; 16-byte
 * aligned q, out and caches, row strides multiples of 8.  tokens == 0 is a no-op.
 */
size_t prefill_attn_workspace_size(int64_t tokens, int num_q_heads, int num_kv_heads,
                                   int head_dim, int64_t start_pos, int split_size);
int prefill_attn_bi(const void *q, int64_t q_row_stride, const void *k_cache, const void *v_cache,
                    const int32_t *block_table_row, int64_t start_pos, int64_t tokens, void *out,
                    int64_t out_row_stride, int num_q_heads, int num_kv_heads, int head_dim,
                    int page_size, int split_size, float scale, void *workspace,
                    size_t workspace_bytes, void *stream);

/*
 * sample_gumbel: seeded Gumbel-max sampling, one token per row ([P1] section 9.3
 * "Non-Greedy Sampling Can Be Deterministic Too").  A counter-based hash of
 * (seed, position, vocabulary id) supplies Gumbel noise that is added to the
 * scaled logits, so a sample is a pure function of the logits and the seed at
 * any temperature.  For row r with T = temperatures[r] > 0:
 *     tokens[r] = argmax_i (logits[r,i] / T + g_i),   g_i = -ln(-ln u_i),
 * u_i = (floor(w / 2^9) + 1/2) / 2^23, w = word (i mod 4) of Philox4x32-10
 * (Salmon et al., "Parallel Random Numbers: As Easy as 1, 2, 3", SC 2011) with
 * counter (i / 4, positions[r] mod 2^32, positions[r] / 2^32, 0) and key
 * (seeds[r] mod 2^32, seeds[r] / 2^32).  T <= 0 is greedy (argmax of the
 * logits).  NaN logits are never chosen; among equal scores the lowest index
 * wins; a row of NaNs gives 0.  The noise depends only on (seed, position,
 * vocabulary id) and the argmax is exact, so a row's token depends on nothing
 * but its own logits and parameters: batch-invariant whenever the logits are.
 * To vary samples across requests, give each request its own seed.
 *  logits        [rows, vocab] fp32, row stride logits_row_stride (a multiple of
 *                4, >= vocab), 16-byte aligned
 *  seeds         [rows] uint64 (device)
 *  positions     [rows] int64 (device), the token position being sampled
 *  temperatures  [rows] fp32 (device)
 *  tokens        [rows] int32 (device), written
 *  workspace     >= sample_gumbel_workspace_size(rows, vocab) bytes, 16-byte
 *                aligned: per-chunk partials
 * Limits: vocab < 2^31 - 16, rows <= 65535.  rows == 0 is a no-op.
 */
size_t sample_gumbel_workspace_size(int64_t rows, int64_t vocab);
int sample_gumbel(const float *logits, int64_t logits_row_stride, int64_t rows, int64_t vocab,
                  const uint64_t *seeds, const int64_t *positions, const float *temperatures,
                  int32_t *tokens, void *workspace, size_t workspace_bytes, void *stream);

/*
 * kv_append: write new tokens' K and V into their cache slots BEFORE attention
 * runs, so cached and fresh tokens are reduced as one sequence with the same
 * split boundaries ([P1] section 5.5: update the KV cache and page table before
 * the attention kernel).  Token t goes to page slot_mapping[t] / page_size, slot
 * slot_mapping[t] % page_size, for every kv head.
 *  k_new, v_new  [tokens, num_kv_heads, head_dim] bf16, row strides
 *                k_row_stride / v_row_stride (head stride head_dim)
 *  slot_mapping  [tokens] int32 (device); an entry < 0 or >= num_pages*page_size
 *                is skipped (no write)
 *  k_cache, v_cache  in the layouts decode_attn_bi documents (token-major K pages,
 *                head-dim-major V pages)
 * Requirements: 16-byte aligned pointers, head_dim a multiple of 8, row strides
 * multiples of 8.  tokens * num_kv_heads * head_dim / 8 >= 2^31 gives
 * RBI_EUNSUPPORTED.
 */
int kv_append(const void *k_new, int64_t k_row_stride, const void *v_new, int64_t v_row_stride,
              const int32_t *slot_mapping, int64_t tokens, void *k_cache, void *v_cache,
              int64_t num_pages, int num_kv_heads, int head_dim, int page_size, void *stream);

/* -------------------------------------------------------------------------- */
/* Element-wise glue of a decode step (invariant by construction: no reduction */
/* crosses rows; [P1] section 5.4)                                             */
/* -------------------------------------------------------------------------- */
/* out[r,:] = table[ids[r], :]; bf16, table [vocab, hidden]; an id outside
 * [0, vocab) yields a zero row.  hidden a multiple of 8, 16-byte aligned.
 * Each glue op runs one thread per 8 elements (argmax: a 1024-thread workgroup
 * per row); sizes needing 2^31 threads or more give RBI_EUNSUPPORTED. */
int rbi_embed(const void *table, int64_t vocab, int64_t hidden, const int32_t *ids, int64_t rows,
              void *out, int64_t out_row_stride, void *stream);

/* out = bf16(float(a) + float(b)) over n contiguous bf16 elements (may alias). */
int rbi_residual_add(const void *a, const void *b, void *out, int64_t n, void *stream);

/* out[r,i] = bf16(silu(g) * u), g = gu[r, i], u = gu[r, inter + i], in fp32;
 * silu(g) = g / (1 + exp(-g)).  gu [rows, 2*inter] bf16, out [rows, inter]. */
int rbi_swiglu(const void *gu, int64_t gu_row_stride, void *out, int64_t out_row_stride,
               int64_t rows, int64_t inter, void *stream);

/* out[r] = index of the largest x[r, :] (fp32), the lowest index on ties; NaN
 * entries are skipped (a row of only NaN yields 0). */
int rbi_argmax_rows(const float *x, int64_t x_row_stride, int64_t rows, int64_t n,
                    int32_t *out, void *stream);

/* -------------------------------------------------------------------------- */
/* Measurement aid                                                             */
/* -------------------------------------------------------------------------- */
/* rbi_stream_copy: dst[0, bytes) = src[0, bytes), one 16-byte chunk per thread,
 * with ordinary or (nontemporal != 0) non-temporal stores: the read + write rate
 * a read-once write-once kernel such as rmsnorm_bi is judged against.  bytes a
 * multiple of 16 and below 2^35, both pointers 16-byte aligned, the ranges must
 * not overlap. */
int rbi_stream_copy(const void *src, void *dst, int64_t bytes, int nontemporal, void *stream);

#ifdef __cplusplus
}
#endif
#endif /* RBI_H */
