// attention.hip -- paged split-KV decode attention for gfx950.
//
// Batch invariance of attention ("Reproducible LLM Inference ...",
// hidekazu-konishi.com, section 5.5; "Your Answer Depends on Who Else Is in the
// Batch", praveentn.live, "The attention detail that gets missed"): the KV
// length is cut at a FIXED split SIZE S, so split s always covers tokens
// [s*S, min((s+1)*S, L)) whatever else is in the batch, and only the number of
// splits grows with L.  The per-token reduction order is therefore a function
// of the request's own length.
//
// Kernel 1 (one workgroup of 4 waves per (row, kv head, split)):
//   * the 16-token pages of the split are dealt to the waves round robin
//     (wave w takes split-relative pages w, w+4, w+8, ...), four pages per step;
//   * scores S^T[token][head] = K . q^T with v_mfma_f32_16x16x32_bf16 (K rows are
//     operand A, the group's query heads operand B; head_dim is the k dimension,
//     lane group q = lane/16 carrying d = q*D/4 + 8c .. +7 in step c);
//   * log2-domain softmax in fp32: s2 = score * (scale * log2 e), masked to -inf
//     past the split end; per wave a running max m and, per lane, a running sum
//     of the bf16-rounded p = 2^(s2 - m) (the same p that feeds the product);
//   * acc[head][d] += P . V with the same MFMA (P operand A, V operand B; V is
//     staged through LDS to read it token-major);
//   * the four waves' (m, l, acc) are combined in wave order 0, 1, 2, 3.
//   The split's partial (m, l, acc) goes to the fp32 workspace.
// Kernel 2 (one wave per (row, query head)): M = max_s m_s, then
//   l = sum_s 2^(m_s - M) l_s and acc = sum_s 2^(m_s - M) acc_s in ascending s,
//   and out = bf16(acc / l).  It always runs, even for a single split.
// No atomics: the final combine is a separate ordered clean-up pass.
//
// The twin (decode_attn_tuned) runs the same kernels with a split size picked
// from the batch shape -- the largest that still gives every compute unit work
// -- which moves the split boundaries with the batch.
#include "device.h"
#include "launch.h"

namespace rbi {
namespace {

constexpr int PAGE = 16;
constexpr int WAVES = 4;
constexpr int GPAGES = 4;  // pages a wave handles per step

template <int D>
struct AttnK {
    static constexpr int KCH = D / 32;      // 16-byte chunks per lane per token row
    static constexpr int DPL = D / 4;       // head_dim elements per lane group
    static constexpr int DB = D / 16;       // 16-wide d blocks of the PV product
    static constexpr int VROW = D + 8;      // LDS row stride (elements), 16-byte pad
};

__device__ __forceinline__ int clamp_len(int L, int max_len)
{
    return L < 1 ? 1 : (L > max_len ? max_len : L);
}

template <int D>
__global__ __launch_bounds__(256, 2) void attn_split_kernel(
    const uint16_t *__restrict__ q, int64_t q_row_stride, const uint16_t *__restrict__ k_cache,
    const uint16_t *__restrict__ v_cache, const int32_t *__restrict__ block_table,
    int64_t bt_stride, const int32_t *__restrict__ kv_lens, int hq, int hkv, int S,
    int max_kv_len, int nsmax, float scale_log2, float *__restrict__ ws_acc,
    float *__restrict__ ws_ml)
{
    using P = AttnK<D>;
    __shared__ __attribute__((aligned(16))) uint16_t vlds[WAVES][2][PAGE][P::VROW];
    __shared__ float c_m[WAVES][16], c_l[WAVES][16];
    __shared__ __attribute__((aligned(16))) float c_acc[WAVES][16][D];

    const int s = blockIdx.x, g = blockIdx.y;
    const int64_t r = blockIdx.z;
    const int L = clamp_len(kv_lens[r], max_kv_len);
    const int nsplit = (L + S - 1) / S;
    if (s >= nsplit)
        return;
    const int t0 = s * S;
    const int t1 = min(t0 + S, L);
    const int valid_pages = (t1 - t0 + PAGE - 1) / PAGE;
    const int split_pages = S / PAGE;
    const int G = hq / hkv;

    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int lr = lane & 15, lg = lane >> 4;

    // query fragment: column = head lr of the group, k = head_dim slice of lane group lg
    bf16x8_t qf[P::KCH];
    {
        const uint16_t *qp = q + r * q_row_stride + (int64_t)(g * G + lr) * D + lg * P::DPL;
#pragma unroll
        for (int c = 0; c < P::KCH; ++c)
            qf[c] = as_bf16x8(lr < G ? *reinterpret_cast<const uint4 *>(qp + 8 * c)
                                     : make_uint4(0, 0, 0, 0));
    }

    float m_run = -INFINITY;  // running max of head lr (log2 domain)
    float l_run = 0.f;        // this lane's share of the running sum for head lr
    f32x4_t acc[P::DB];       // acc[db][j]: head 4*lg + j, d = 16*db + lr
#pragma unroll
    for (int db = 0; db < P::DB; ++db)
        acc[db] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    const int pages_per_wave = (split_pages + WAVES - 1) / WAVES;
    const int nsteps = (pages_per_wave + GPAGES - 1) / GPAGES;
    const int32_t *bt = block_table + r * bt_stride + t0 / PAGE;

    for (int step = 0; step < nsteps; ++step) {
        uint4 kr[GPAGES][P::KCH], vr[GPAGES][P::KCH];
        int pbase[GPAGES];  // absolute index of the page's first token, or -1 if absent
#pragma unroll
        for (int c = 0; c < GPAGES; ++c) {
            const int j = wave + WAVES * (step * GPAGES + c);
            pbase[c] = (j < valid_pages) ? t0 + j * PAGE : -1;
            if (pbase[c] >= 0) {
                const int64_t phys = bt[j];
                const int64_t off = ((phys * hkv + g) * PAGE + lr) * D + lg * P::DPL;
                const bool tok_ok = pbase[c] + lr < t1;
#pragma unroll
                for (int cc = 0; cc < P::KCH; ++cc) {
                    kr[c][cc] = *reinterpret_cast<const uint4 *>(k_cache + off + 8 * cc);
                    vr[c][cc] = tok_ok ? *reinterpret_cast<const uint4 *>(v_cache + off + 8 * cc)
                                       : make_uint4(0, 0, 0, 0);
                }
            } else {
#pragma unroll
                for (int cc = 0; cc < P::KCH; ++cc) {
                    kr[c][cc] = make_uint4(0, 0, 0, 0);
                    vr[c][cc] = make_uint4(0, 0, 0, 0);
                }
            }
        }

        // scores: lane holds head lr, tokens 4*lg + j of each page slot c
        float sv[GPAGES][4];
        float mloc = -INFINITY;
#pragma unroll
        for (int c = 0; c < GPAGES; ++c) {
            f32x4_t sc = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int cc = 0; cc < P::KCH; ++cc)
                sc = mfma_16x16x32_bf16(as_bf16x8(kr[c][cc]), qf[cc], sc);
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int tok = pbase[c] + 4 * lg + j;
                const float v = (pbase[c] >= 0 && tok < t1) ? sc[j] * scale_log2 : -INFINITY;
                sv[c][j] = v;
                mloc = fmaxf(mloc, v);
            }
        }
        mloc = fmaxf(mloc, __shfl_xor(mloc, 16, kWave));
        mloc = fmaxf(mloc, __shfl_xor(mloc, 32, kWave));
        const float m_new = fmaxf(m_run, mloc);
        const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
        const float alpha = exp2f(m_run - m_use);

        uint32_t pw[GPAGES][2];  // bf16 p, two per word, token order within the page slot
        float psum = 0.f;
#pragma unroll
        for (int c = 0; c < GPAGES; ++c) {
            uint32_t b[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                b[j] = f32_to_bf16(exp2f(sv[c][j] - m_use));
                psum += bf16_to_f32(b[j]);
            }
            pw[c][0] = b[0] | (b[1] << 16);
            pw[c][1] = b[2] | (b[3] << 16);
        }
        l_run = l_run * alpha + psum;
        m_run = m_new;

#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const float aj = __shfl(alpha, 4 * lg + j, kWave);
#pragma unroll
            for (int db = 0; db < P::DB; ++db)
                acc[db][j] *= aj;
        }

        // P . V, two pages per MFMA k-step
#pragma unroll
        for (int kk = 0; kk < GPAGES / 2; ++kk) {
            __syncthreads();
#pragma unroll
            for (int h = 0; h < 2; ++h)
#pragma unroll
                for (int cc = 0; cc < P::KCH; ++cc)
                    *reinterpret_cast<uint4 *>(&vlds[wave][h][lr][lg * P::DPL + 8 * cc]) =
                        vr[2 * kk + h][cc];
            __syncthreads();
            const uint4 pu = make_uint4(pw[2 * kk][0], pw[2 * kk][1], pw[2 * kk + 1][0],
                                        pw[2 * kk + 1][1]);
            const bf16x8_t pf = as_bf16x8(pu);
#pragma unroll
            for (int db = 0; db < P::DB; ++db) {
                const int d = 16 * db + lr;
                uint32_t e[8];
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    e[j] = vlds[wave][0][4 * lg + j][d];
                    e[4 + j] = vlds[wave][1][4 * lg + j][d];
                }
                const uint4 vu = make_uint4(e[0] | (e[1] << 16), e[2] | (e[3] << 16),
                                            e[4] | (e[5] << 16), e[6] | (e[7] << 16));
                acc[db] = mfma_16x16x32_bf16(pf, as_bf16x8(vu), acc[db]);
            }
        }
    }

    // this wave's sum for head lr: the four lane groups in butterfly order
    float l_w = l_run;
    l_w += __shfl_xor(l_w, 16, kWave);
    l_w += __shfl_xor(l_w, 32, kWave);
    if (lg == 0) {
        c_m[wave][lr] = m_run;
        c_l[wave][lr] = l_w;
    }
#pragma unroll
    for (int db = 0; db < P::DB; ++db)
#pragma unroll
        for (int j = 0; j < 4; ++j)
            c_acc[wave][4 * lg + j][16 * db + lr] = acc[db][j];
    __syncthreads();

    // combine the waves in order 0..3; thread t: head t/16, d slice (t%16)*(D/16)
    const int h = threadIdx.x >> 4;
    const int dq = (threadIdx.x & 15) * (D / 16);
    float mw[WAVES], M = -INFINITY;
#pragma unroll
    for (int w = 0; w < WAVES; ++w) {
        mw[w] = c_m[w][h];
        M = fmaxf(M, mw[w]);
    }
    float cw[WAVES];
#pragma unroll
    for (int w = 0; w < WAVES; ++w)
        cw[w] = (mw[w] == -INFINITY) ? 0.f : exp2f(mw[w] - M);
    float l = 0.f;
#pragma unroll
    for (int w = 0; w < WAVES; ++w)
        l = l + cw[w] * c_l[w][h];
    if (h < G) {
        const int64_t item = (r * hq + g * G + h) * nsmax + s;
        float *dst = ws_acc + item * D + dq;
#pragma unroll
        for (int i = 0; i < D / 16; i += 4) {
            float o[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                float a = 0.f;
#pragma unroll
                for (int w = 0; w < WAVES; ++w)
                    a = a + cw[w] * c_acc[w][h][dq + i + e];
                o[e] = a;
            }
            *reinterpret_cast<float4 *>(dst + i) = make_float4(o[0], o[1], o[2], o[3]);
        }
        if ((threadIdx.x & 15) == 0) {
            ws_ml[item * 2] = M;
            ws_ml[item * 2 + 1] = l;
        }
    }
}

// One wave per (row, query head): ordered combine of the row's split partials.
template <int D>
__global__ __launch_bounds__(256) void attn_merge_kernel(
    const float *__restrict__ ws_acc, const float *__restrict__ ws_ml,
    const int32_t *__restrict__ kv_lens, int64_t rows, int hq, int S, int max_kv_len, int nsmax,
    uint16_t *__restrict__ out, int64_t out_row_stride)
{
    constexpr int EPL = D / 64;  // elements per lane
    const int lane = threadIdx.x & 63;
    const int64_t item = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (item >= rows * hq)
        return;
    const int64_t r = item / hq;
    const int h = (int)(item % hq);
    const int L = clamp_len(kv_lens[r], max_kv_len);
    const int n = (L + S - 1) / S;
    const float *ml = ws_ml + item * nsmax * 2;
    const float *ac = ws_acc + item * nsmax * D + lane * EPL;
    float M = -INFINITY;
    for (int s = 0; s < n; ++s)
        M = fmaxf(M, ml[2 * s]);
    float l = 0.f, o[EPL];
#pragma unroll
    for (int e = 0; e < EPL; ++e)
        o[e] = 0.f;
    for (int s = 0; s < n; ++s) {
        const float c = exp2f(ml[2 * s] - M);
        l = l + c * ml[2 * s + 1];
#pragma unroll
        for (int e = 0; e < EPL; ++e)
            o[e] = o[e] + c * ac[(int64_t)s * D + e];
    }
    uint16_t *dst = out + r * out_row_stride + (int64_t)h * D + lane * EPL;
    if constexpr (EPL == 2) {
        *reinterpret_cast<uint32_t *>(dst) = pack_bf16x2(o[0] / l, o[1] / l);
    } else {
        dst[0] = (uint16_t)f32_to_bf16(o[0] / l);
    }
}

// One thread per 16-byte chunk of a (token, kv head) row.
__global__ __launch_bounds__(256) void kv_append_kernel(
    const uint16_t *__restrict__ k_new, int64_t ks, const uint16_t *__restrict__ v_new, int64_t vs,
    const int32_t *__restrict__ slots, int64_t tokens, uint16_t *__restrict__ k_cache,
    uint16_t *__restrict__ v_cache, int64_t num_pages, int hkv, int d, int page)
{
    const int cpr = d / 8;  // chunks per head row
    const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (idx >= tokens * hkv * cpr)
        return;
    const int64_t t = idx / (hkv * cpr);
    const int h = (int)((idx / cpr) % hkv);
    const int c = (int)(idx % cpr);
    const int64_t slot = slots[t];
    if (slot < 0 || slot >= num_pages * page)
        return;
    const int64_t dst = (((slot / page) * hkv + h) * page + slot % page) * d + 8 * c;
    *reinterpret_cast<uint4 *>(k_cache + dst) =
        *reinterpret_cast<const uint4 *>(k_new + t * ks + (int64_t)h * d + 8 * c);
    *reinterpret_cast<uint4 *>(v_cache + dst) =
        *reinterpret_cast<const uint4 *>(v_new + t * vs + (int64_t)h * d + 8 * c);
}

template <int D>
hipError_t launch_attn_d(const AttnArgs &a, hipStream_t s)
{
    const int nsmax = (a.max_kv_len + a.split - 1) / a.split;
    float *ws_acc = a.ws;
    float *ws_ml = a.ws + a.rows * a.hq * (int64_t)nsmax * D;
    const float scale_log2 = (float)((double)a.scale * 1.4426950408889634);
    const dim3 g1((unsigned)nsmax, (unsigned)a.hkv, (unsigned)a.rows), b1(256);
    attn_split_kernel<D><<<g1, b1, 0, s>>>(a.q, a.q_row_stride, a.k_cache, a.v_cache,
                                           a.block_table, a.bt_stride, a.kv_lens, a.hq, a.hkv,
                                           a.split, a.max_kv_len, nsmax, scale_log2, ws_acc, ws_ml);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess)
        return e;
    const int64_t items = a.rows * a.hq;
    const dim3 g2((unsigned)((items + 3) / 4)), b2(256);
    attn_merge_kernel<D><<<g2, b2, 0, s>>>(ws_acc, ws_ml, a.kv_lens, a.rows, a.hq, a.split,
                                           a.max_kv_len, nsmax, a.out, a.out_row_stride);
    return hipGetLastError();
}

}  // namespace

size_t attn_workspace_bytes(int64_t rows, int hq, int d, int max_kv_len, int split)
{
    const int64_t nsmax = (max_kv_len + split - 1) / split;
    return (size_t)(rows * hq * nsmax) * (size_t)(d + 2) * sizeof(float);
}

hipError_t launch_decode_attn(const AttnArgs &a, hipStream_t s)
{
    return a.d == 128 ? launch_attn_d<128>(a, s) : launch_attn_d<64>(a, s);
}

hipError_t launch_kv_append(const uint16_t *k_new, int64_t ks, const uint16_t *v_new, int64_t vs,
                            const int32_t *slots, int64_t tokens, uint16_t *k_cache,
                            uint16_t *v_cache, int64_t num_pages, int hkv, int d, int page,
                            hipStream_t s)
{
    const int64_t n = tokens * hkv * (d / 8);
    const dim3 grid((unsigned)((n + 255) / 256)), block(256);
    kv_append_kernel<<<grid, block, 0, s>>>(k_new, ks, v_new, vs, slots, tokens, k_cache, v_cache,
                                            num_pages, hkv, d, page);
    return hipGetLastError();
}

}  // namespace rbi
