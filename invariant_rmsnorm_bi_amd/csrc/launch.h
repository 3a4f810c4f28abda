// launch.h -- host-side launchers of the librbi kernels (internal; the public
// boundary is include/rbi.h).  Arguments reaching these functions have already
// been validated by capi.cpp; each returns hipSuccess or the launch error.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace rbi {

// rmsnorm.hip
hipError_t launch_rmsnorm_wave(const void *x, int64_t xs, const void *w, void *y, int64_t ys,
                               int64_t rows, int64_t hidden, float eps, bool bf16,
                               hipStream_t s);
hipError_t launch_rmsnorm_block(const void *x, int64_t xs, const void *w, void *y, int64_t ys,
                                int64_t rows, int64_t hidden, float eps, bool bf16,
                                hipStream_t s);

// matmul.hip
struct MatmulArgs {
    const uint16_t *A;
    int64_t lda;
    const uint16_t *W;
    int64_t ldw;
    void *C;
    int64_t ldc;
    bool c_bf16;
    int64_t M, N, K;
};
// The launches matmul_bi makes for a problem size: tile shape t1 over the first n1
// columns, then tile shape t2 over the rest (t2 < 0: one launch over all N); t1 < 0
// is the register-staged 128 x 128 kernel for K % 32 != 0.  Shapes index the tile
// table of matmul.hip.
struct MatmulPlan {
    int t1;
    int64_t n1;
    int t2;
};
MatmulPlan plan_matmul_bi(int64_t M, int64_t N, int64_t K);
void describe_matmul_plan(const MatmulPlan &p, int64_t out[7]);
hipError_t launch_matmul_bi(const MatmulArgs &a, hipStream_t s);
// split-K twin: `splits` partial products over equal K ranges into fp32 workspace
// [splits, M, N], then an ascending-order reduction into C.
hipError_t launch_matmul_splitk(const MatmulArgs &a, int splits, float *ws, hipStream_t s);
// The twin's tile shape (an index of the tile table; -1: matmul_bi's own choice)
// and split-K count (1: matmul_bi's plan unchanged).
struct TwinPlan {
    int tile;
    int split;
};
TwinPlan plan_matmul_tuned(int64_t M, int64_t N, int64_t K);
int matmul_tuned_splits(int64_t M, int64_t N, int64_t K);

// attention.hip
struct AttnArgs {
    const uint16_t *q;
    int64_t q_row_stride;
    const uint16_t *k_cache, *v_cache;
    const int32_t *block_table;
    int64_t bt_stride;
    const int32_t *kv_lens;
    uint16_t *out;
    int64_t out_row_stride;
    int64_t rows;
    int hq, hkv, d, page, split, max_kv_len;
    float scale;
    float *ws;  // group partials: [rows, hkv, groups_max, hq / hkv] x (D + 4) floats
};
size_t attn_workspace_bytes(int64_t rows, int hq, int d, int max_kv_len, int split);
hipError_t launch_decode_attn(const AttnArgs &a, hipStream_t s);
struct PrefillArgs {
    const uint16_t *q;
    int64_t q_row_stride;
    const uint16_t *k_cache, *v_cache;
    const int32_t *block_table_row;
    int64_t start, tokens;  // prompt positions start .. start + tokens - 1
    uint16_t *out;
    int64_t out_row_stride;
    int hq, hkv, d, page, split;
    float scale;
    float *ws;  // split schedule only: [tokens, hkv, groups_max, hq / hkv] x (D + 4) floats
};
size_t prefill_workspace_bytes(int64_t tokens, int hq, int hkv, int d, int64_t start, int split);
hipError_t launch_prefill_attn(const PrefillArgs &a, hipStream_t s);
hipError_t launch_kv_append(const uint16_t *k_new, int64_t ks, const uint16_t *v_new, int64_t vs,
                            const int32_t *slots, int64_t tokens, uint16_t *k_cache,
                            uint16_t *v_cache, int64_t num_pages, int hkv, int d, int page,
                            hipStream_t s);

// sampling.hip
int sample_chunks(int64_t vocab);
size_t sample_workspace_bytes(int64_t rows, int64_t vocab);
hipError_t launch_sample_gumbel(const float *logits, int64_t ld, int64_t rows, int64_t vocab,
                                const uint64_t *seeds, const int64_t *positions,
                                const float *temps, int32_t *tokens, void *ws, hipStream_t s);

// glue.hip
hipError_t launch_embed(const uint16_t *table, int64_t vocab, int64_t hidden, const int32_t *ids,
                        int64_t rows, uint16_t *out, int64_t os, hipStream_t s);
hipError_t launch_residual_add(const uint16_t *a, const uint16_t *b, uint16_t *out, int64_t n,
                               hipStream_t s);
hipError_t launch_swiglu(const uint16_t *gu, int64_t gs, uint16_t *out, int64_t os, int64_t rows,
                         int64_t inter, hipStream_t s);
hipError_t launch_stream_copy(const void *src, void *dst, int64_t bytes, bool nt, hipStream_t s);
hipError_t launch_argmax(const float *x, int64_t xs, int64_t rows, int64_t n, int32_t *out,
                         hipStream_t s);

}  // namespace rbi
