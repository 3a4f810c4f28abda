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
// Kernel 1 (one workgroup of 8 waves per (row, kv head, split)):
//   * the split's 16-token pages are dealt to the waves in pairs (wave w takes
//     pages 2w and 2w+1, then 2w+16, 2w+17, ... when the split is longer), each
//     pair loaded in one burst;
//   * scores S^T[token][head] = K . q^T with v_mfma_f32_16x16x32_bf16 (K rows are
//     operand A, the group's query heads operand B; head_dim is the k dimension,
//     lane group q = lane/16 carrying d = q*D/4 + 8c .. +7 in step c);
//   * log2-domain softmax in fp32: s2 = score * (scale * log2 e), masked to -inf
//     past the split end; per wave a running max m and, per lane, a running sum
//     of the bf16-rounded p = 2^(s2 - m) (the same p that feeds the product);
//   * acc[head][d] += P . V with the same MFMA (P operand A, V operand B).  V pages
//     are stored head-dim-major ([d][token]), so one 16-byte load of a V page row is
//     exactly the operand fragment (8 consecutive tokens at one d): no staging;
//   * the eight waves' (m, l, acc) are combined in wave order 0 .. 7
//     (M = max m, l = sum 2^(m_w - M) l_w, acc = sum 2^(m_w - M) acc_w), and the
//     split's partial goes to the fp32 workspace.
// Kernel 2 (one wave per (row, query head)): the same combine over the row's
//   splits in ascending order, then out = bf16(acc / l).  It always runs, even
//   for a single split.  The whole reduction tree is a function of L alone.
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
constexpr int WAVES = 8;   // waves per split workgroup

template <int D>
struct AttnK {
    static constexpr int KCH = D / 32;      // 16-byte chunks per lane per token row
    static constexpr int DPL = D / 4;       // head_dim elements per lane group
    static constexpr int DB = D / 16;       // 16-wide d blocks of the PV product
};

__device__ __forceinline__ int clamp_len(int L, int max_len)
{
    return L < 1 ? 1 : (L > max_len ? max_len : L);
}



template <int D>
__global__ __launch_bounds__(512, 4) void attn_split_kernel(
    const uint16_t *__restrict__ q, int64_t q_row_stride, const uint16_t *__restrict__ k_cache,
    const uint16_t *__restrict__ v_cache, const int32_t *__restrict__ block_table,
    int64_t bt_stride, const int32_t *__restrict__ kv_lens, int hq, int hkv, int S,
    int max_kv_len, int nsmax, float scale_log2, float *__restrict__ ws_acc,
    float *__restrict__ ws_ml)
{
    using P = AttnK<D>;
    __shared__ __attribute__((aligned(16))) uint16_t q_lds[16][D];
    __shared__ float c_m[WAVES][16], c_l[WAVES][16];
    __shared__ __attribute__((aligned(16))) float c_acc[WAVES][16][D];

    const int s = blockIdx.x, g = blockIdx.y;
    const int64_t r = blockIdx.z;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int lr = lane & 15, lg = lane >> 4;
    // The split's block-table entries (up to 64, one per lane) are read before the
    // length is known, so that this read and the length read overlap; the index is
    // clamped into the table row (ceil(max_kv_len / 16) entries, checked by the
    // caller), and entries past the row's last page are never used.
    const int split_pages = S / PAGE;
    const int row_pages = (max_kv_len + PAGE - 1) / PAGE;
    const int32_t *btrow = block_table + r * bt_stride;
    const int my_page = btrow[min(s * split_pages + min(lane, split_pages - 1), row_pages - 1)];
    const int L = clamp_len(kv_lens[r], max_kv_len);
    const int nsplit = (L + S - 1) / S;
    if (s >= nsplit)
        return;
    const int G = hq / hkv;
    const int t0 = s * S;
    const int t1 = min(t0 + S, L);
    const int valid_pages = (t1 - t0 + PAGE - 1) / PAGE;

    float m_run = -INFINITY;  // running max of head lr (log2 domain)
    float l_run = 0.f;        // this lane's share of the running sum for head lr
    f32x4_t acc[P::DB];       // acc[db][j]: head 4*lg + j, d = 16*db + lr
#pragma unroll
    for (int db = 0; db < P::DB; ++db)
        acc[db] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    // Wave w takes the page pairs 2w, 2w+1 (+ 2*WAVES*i for splits longer than
    // 2*WAVES pages), one pair per step.  Within a step:
    //   * lane group lg owns the 8-token run lg: page slot lg/2, in-page tokens
    //     8*(lg%2) .. +7 -- its scores, its P values and its V loads;
    //   * score block b (one MFMA, b = 0, 1) has K row i = in-page token
    //     8*((i/4)%2) + 4b + i%4 of slot i/8, so output rows 4*lg + j land in lane
    //     group lg as token 4b + j of its run;
    //   * the P.V k-step then takes each lane group's run: the lane's P values in
    //     token order, and one 16-byte run of the head-dim-major V page per d.
    // A page slot past the split's last page reads that last page again and is
    // masked afterwards, so no load is conditional.
    const int kslot = lr >> 3;                              // K row's page slot
    const int krow = 8 * ((lr >> 2) & 1) + (lr & 3);        // K row's in-page token (b = 0)
    const int vslot = lg >> 1, vrun = 8 * (lg & 1);         // this lane group's run
    const int pairs = (valid_pages + 1) / 2;

    struct StepData {
        uint4 k[2][P::KCH];
        uint4 v[P::DB];
    };
    auto load_step = [&](int pr, StepData &sd) {
        const int64_t kphys = __shfl(my_page, min(2 * pr + kslot, valid_pages - 1), kWave);
        const int64_t vphys = __shfl(my_page, min(2 * pr + vslot, valid_pages - 1), kWave);
        const uint16_t *kp = k_cache + ((kphys * hkv + g) * PAGE + krow) * D + lg * P::DPL;
#pragma unroll
        for (int b = 0; b < 2; ++b)
#pragma unroll
            for (int cc = 0; cc < P::KCH; ++cc)
                sd.k[b][cc] = *reinterpret_cast<const uint4 *>(kp + 4 * b * D + 8 * cc);
        const uint16_t *vp = v_cache + ((vphys * hkv + g) * D + lr) * PAGE + vrun;
#pragma unroll
        for (int db = 0; db < P::DB; ++db)
            sd.v[db] = *reinterpret_cast<const uint4 *>(vp + 16 * db * PAGE);
    };
    // first step's loads go out before the query is staged
    StepData sd;
    if (wave < pairs)
        load_step(wave, sd);

    // the group's query rows, staged once in LDS (rows past the group are zero)
    for (int i = threadIdx.x; i < 16 * D / 8; i += WAVES * 64) {
        const int h = i / (D / 8), c = i % (D / 8);
        *reinterpret_cast<uint4 *>(&q_lds[h][8 * c]) =
            h < G ? *reinterpret_cast<const uint4 *>(q + r * q_row_stride + (int64_t)(g * G + h) * D + 8 * c)
                  : make_uint4(0, 0, 0, 0);
    }
    __syncthreads();  // q_lds ready

    for (int pr = wave; pr < pairs; pr += WAVES) {
        if (pr != wave)
            load_step(pr, sd);
        uint4(&kd)[2][P::KCH] = sd.k;
        uint4(&vd)[P::DB] = sd.v;

        // live tokens of this lane group's run; the others get weight 0 and their V
        // entries exact zeros (a stale non-finite value times 0 would not be 0)
        const int first = t0 + (2 * pr + vslot) * PAGE + vrun;
        const int keep = (2 * pr + vslot < valid_pages) ? max(0, min(8, t1 - first)) : 0;
        uint32_t vmask[4];
#pragma unroll
        for (int i = 0; i < 4; ++i)
            vmask[i] = (2 * i < keep ? 0x0000ffffu : 0u) | (2 * i + 1 < keep ? 0xffff0000u : 0u);
#pragma unroll
        for (int db = 0; db < P::DB; ++db)
            vd[db] = make_uint4(vd[db].x & vmask[0], vd[db].y & vmask[1], vd[db].z & vmask[2],
                                vd[db].w & vmask[3]);

        // scores: lane holds head lr, token 4b + j of its run
        float sv[2][4];
        float mloc = -INFINITY;
#pragma unroll
        for (int b = 0; b < 2; ++b) {
            f32x4_t sc = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int cc = 0; cc < P::KCH; ++cc) {
                const bf16x8_t qf = as_bf16x8(
                    *reinterpret_cast<const uint4 *>(&q_lds[lr][lg * P::DPL + 8 * cc]));
                sc = mfma_16x16x32_bf16(as_bf16x8(kd[b][cc]), qf, sc);
            }
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const float v = (4 * b + j < keep) ? sc[j] * scale_log2 : -INFINITY;
                sv[b][j] = v;
                mloc = fmaxf(mloc, v);
            }
        }
        mloc = fmaxf(mloc, __shfl_xor(mloc, 16, kWave));
        mloc = fmaxf(mloc, __shfl_xor(mloc, 32, kWave));
        const float m_new = fmaxf(m_run, mloc);
        const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
        const float alpha = exp2f(m_run - m_use);

        uint32_t pw[2][2];  // bf16 p, two per word, token order within the run
        float psum = 0.f;
#pragma unroll
        for (int b = 0; b < 2; ++b) {
            uint32_t e[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                e[j] = f32_to_bf16(exp2f(sv[b][j] - m_use));
                psum += bf16_to_f32(e[j]);
            }
            pw[b][0] = e[0] | (e[1] << 16);
            pw[b][1] = e[2] | (e[3] << 16);
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
        const bf16x8_t pf = as_bf16x8(make_uint4(pw[0][0], pw[0][1], pw[1][0], pw[1][1]));
#pragma unroll
        for (int db = 0; db < P::DB; ++db)
            acc[db] = mfma_16x16x32_bf16(pf, as_bf16x8(vd[db]), acc[db]);
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

    // combine the waves in order 0 .. WAVES-1; thread t: head t / 32, d slice
    const int h = threadIdx.x >> 5;
    const int dq = (threadIdx.x & 31) * (D / 32);
    static_assert(D == 64 || D == 128, "head_dim 64 or 128");
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
        constexpr int EPT = D / 32;  // elements of the head row this thread owns
        float o[EPT];
#pragma unroll
        for (int e = 0; e < EPT; ++e) {
            float a = 0.f;
#pragma unroll
            for (int w = 0; w < WAVES; ++w)
                a = a + cw[w] * c_acc[w][h][dq + e];
            o[e] = a;
        }
        float *dst = ws_acc + item * D + dq;
        if constexpr (EPT == 4)
            *reinterpret_cast<float4 *>(dst) = make_float4(o[0], o[1], o[2], o[3]);
        else
            *reinterpret_cast<float2 *>(dst) = make_float2(o[0], o[1]);
        if ((threadIdx.x & 31) == 0) {
            ws_ml[item * 2] = M;
            ws_ml[item * 2 + 1] = l;
        }
    }
}

// One wave per (row, query head): ordered combine of the row's split partials.
// The maximum is taken lane-parallel (exact, so order-free); the scale factors
// 2^(m_s - M) are formed lane-parallel, one split per lane; the sums over splits
// run in ascending split order in every lane.
template <int D>
__global__ __launch_bounds__(256) void attn_merge_kernel(
    const float *__restrict__ ws_acc, const float *__restrict__ ws_ml,
    const int32_t *__restrict__ kv_lens, int64_t rows, int hq, int S, int max_kv_len, int nsmax,
    uint16_t *__restrict__ out, int64_t out_row_stride)
{
    constexpr int EPL = D / 64;  // elements per lane
    constexpr int UNROLL = 8;
    const int lane = threadIdx.x & 63;
    const int64_t item = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (item >= rows * hq)
        return;
    const int64_t r = item / hq;
    const int h = (int)(item % hq);
    const int L = clamp_len(kv_lens[r], max_kv_len);
    const int n = (L + S - 1) / S;  // splits of this row
    const float *ml = ws_ml + item * nsmax * 2;
    const float *ac = ws_acc + item * nsmax * D + lane * EPL;
    float M = -INFINITY;
    for (int s = lane; s < n; s += 64)
        M = fmaxf(M, ml[2 * s]);
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1)
        M = fmaxf(M, __shfl_xor(M, off, kWave));
    float l = 0.f, o[EPL];
#pragma unroll
    for (int e = 0; e < EPL; ++e)
        o[e] = 0.f;
    for (int s0 = 0; s0 < n; s0 += 64) {
        const int sl = s0 + lane;
        const float c_l = sl < n ? exp2f(ml[2 * sl] - M) : 0.f;
        const float l_l = sl < n ? ml[2 * sl + 1] : 0.f;
        const int cnt = min(64, n - s0);
        for (int j0 = 0; j0 < cnt; j0 += UNROLL) {
            float a[UNROLL][EPL];
#pragma unroll
            for (int u = 0; u < UNROLL; ++u)
#pragma unroll
                for (int e = 0; e < EPL; ++e)
                    a[u][e] = (j0 + u < cnt) ? ac[(int64_t)(s0 + j0 + u) * D + e] : 0.f;
#pragma unroll
            for (int u = 0; u < UNROLL; ++u) {
                if (j0 + u < cnt) {
                    const float c = __shfl(c_l, j0 + u, kWave);
                    l = l + c * __shfl(l_l, j0 + u, kWave);
#pragma unroll
                    for (int e = 0; e < EPL; ++e)
                        o[e] = o[e] + c * a[u][e];
                }
            }
        }
    }
    uint16_t *dst = out + r * out_row_stride + (int64_t)h * D + lane * EPL;
    if constexpr (EPL == 2) {
        *reinterpret_cast<uint32_t *>(dst) = pack_bf16x2(o[0] / l, o[1] / l);
    } else {
        dst[0] = (uint16_t)f32_to_bf16(o[0] / l);
    }
}

// One thread per 16-byte chunk of a (token, kv head) row.  K rows are stored
// token-major ([token][d]), V head-dim-major ([d][token]): the K chunk is copied
// whole, the V chunk's 8 values go to 8 rows of the page.
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
    const int64_t pg = slot / page, off = slot % page;
    *reinterpret_cast<uint4 *>(k_cache + ((pg * hkv + h) * page + off) * d + 8 * c) =
        *reinterpret_cast<const uint4 *>(k_new + t * ks + (int64_t)h * d + 8 * c);
    const uint4 v = *reinterpret_cast<const uint4 *>(v_new + t * vs + (int64_t)h * d + 8 * c);
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
    uint16_t *vd = v_cache + ((pg * hkv + h) * d + 8 * c) * page + off;
#pragma unroll
    for (int e = 0; e < 8; ++e)
        vd[(int64_t)e * page] = (uint16_t)((e & 1) ? (w[e >> 1] >> 16) : (w[e >> 1] & 0xffffu));
}

template <int D>
hipError_t launch_attn_d(const AttnArgs &a, hipStream_t s)
{
    const int nsmax = (a.max_kv_len + a.split - 1) / a.split;
    float *ws_acc = a.ws;
    float *ws_ml = a.ws + a.rows * a.hq * (int64_t)nsmax * D;
    const float scale_log2 = (float)((double)a.scale * 1.4426950408889634);
    const dim3 g1((unsigned)nsmax, (unsigned)a.hkv, (unsigned)a.rows), b1(WAVES * 64);
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
