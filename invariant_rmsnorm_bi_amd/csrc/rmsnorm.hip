// rmsnorm.hip -- row-local RMSNorm for gfx950.
//
//   y[r,i] = (x[r,i] * rsq) * w[i],  rsq = 1 / sqrt(sum_j x[r,j]^2 / H + eps)
//
// Batch invariance ("Reproducible LLM Inference ...", hidekazu-konishi.com,
// section 5.3: give each batch element its own core so its reduction never
// splits): every row is reduced in one order that is a function of H alone --
// that of a single wavefront, below -- whether one wave or several share the
// row's loads and stores.
//
// Reduction order of one row (the contract of rmsnorm_bi):
//   * the row is cut into 16-byte chunks (8 bf16 or 4 fp32 elements);
//   * lane l owns chunks l, l+64, l+128, ... and keeps one fp32 partial per
//     element slot e of a chunk, updated with fmaf(x, x, partial) over its
//     chunks in ascending order;
//   * the slot partials of a lane are added by a fixed pairwise tree;
//   * the 64 lane sums are added by the xor butterfly (32, 16, ..., 1).
// Keeping one partial per slot gives every lane several short chains, so a
// large square cannot absorb a long run of small ones the way a single
// sequential accumulator does (the failure worked through on the
// praveentn.live page, "A Concrete Example").
//
// The twin (rmsnorm_tuned) spreads a row over a 256-thread workgroup when the
// batch is too small to fill the chip: a different tree, hence different bits.
#include "device.h"
#include "launch.h"

namespace rbi {
namespace {

template <bool BF16>
struct Elt {
    static constexpr int VEC = BF16 ? 8 : 4;    // elements per 16-byte chunk
    static constexpr int SIZE = BF16 ? 2 : 4;   // bytes per element
};

// Chunk c of a row with H elements, widened to fp32; elements at or past H read as 0.
template <bool BF16>
__device__ __forceinline__ void load_chunk(const char *row, int64_t c, int64_t H, float *v)
{
    constexpr int VEC = Elt<BF16>::VEC;
    const int64_t e0 = c * VEC;
    if (e0 + VEC <= H) {
        const uint4 q = *reinterpret_cast<const uint4 *>(row + e0 * Elt<BF16>::SIZE);
        if constexpr (BF16) {
            unpack8(q, v);
        } else {
            v[0] = __uint_as_float(q.x);
            v[1] = __uint_as_float(q.y);
            v[2] = __uint_as_float(q.z);
            v[3] = __uint_as_float(q.w);
        }
    } else {
#pragma unroll
        for (int e = 0; e < VEC; ++e) {
            const int64_t i = e0 + e;
            if (i < H) {
                if constexpr (BF16)
                    v[e] = bf16_to_f32(reinterpret_cast<const uint16_t *>(row)[i]);
                else
                    v[e] = reinterpret_cast<const float *>(row)[i];
            } else {
                v[e] = 0.f;
            }
        }
    }
}

// y chunk = round((x * rsq) * w), elements past H are not written.
template <bool BF16>
__device__ __forceinline__ void store_chunk(char *row, const char *wrow, int64_t c, int64_t H,
                                            const float *v, float rsq)
{
    constexpr int VEC = Elt<BF16>::VEC;
    float w[VEC];
    load_chunk<BF16>(wrow, c, H, w);
    float o[VEC];
#pragma unroll
    for (int e = 0; e < VEC; ++e)
        o[e] = (v[e] * rsq) * w[e];
    const int64_t e0 = c * VEC;
    if (e0 + VEC <= H) {
        uint4 q;
        if constexpr (BF16) {
            q.x = pack_bf16x2(o[0], o[1]);
            q.y = pack_bf16x2(o[2], o[3]);
            q.z = pack_bf16x2(o[4], o[5]);
            q.w = pack_bf16x2(o[6], o[7]);
        } else {
            q.x = __float_as_uint(o[0]);
            q.y = __float_as_uint(o[1]);
            q.z = __float_as_uint(o[2]);
            q.w = __float_as_uint(o[3]);
        }
        *reinterpret_cast<uint4 *>(row + e0 * Elt<BF16>::SIZE) = q;
    } else {
#pragma unroll
        for (int e = 0; e < VEC; ++e) {
            const int64_t i = e0 + e;
            if (i < H) {
                if constexpr (BF16)
                    reinterpret_cast<uint16_t *>(row)[i] = (uint16_t)f32_to_bf16(o[e]);
                else
                    reinterpret_cast<float *>(row)[i] = o[e];
            }
        }
    }
}

// The VEC elements of a full 16-byte chunk, widened to fp32.
template <bool BF16>
__device__ __forceinline__ void unpack_chunk(const uint4 &q, float *v)
{
    if constexpr (BF16) {
        unpack8(q, v);
    } else {
        v[0] = __uint_as_float(q.x);
        v[1] = __uint_as_float(q.y);
        v[2] = __uint_as_float(q.z);
        v[3] = __uint_as_float(q.w);
    }
}

// A full chunk of y = round((x * rsq) * w), with w already loaded.  NT: a
// non-temporal store (y is written once and not read back by this kernel).
template <bool BF16, bool NT = false>
__device__ __forceinline__ void store_full_chunk(char *row, int64_t c, const float *v,
                                                 const float *w, float rsq)
{
    constexpr int VEC = Elt<BF16>::VEC;
    float o[VEC];
#pragma unroll
    for (int e = 0; e < VEC; ++e)
        o[e] = (v[e] * rsq) * w[e];
    uint4 q;
    if constexpr (BF16) {
        q.x = pack_bf16x2(o[0], o[1]);
        q.y = pack_bf16x2(o[2], o[3]);
        q.z = pack_bf16x2(o[4], o[5]);
        q.w = pack_bf16x2(o[6], o[7]);
    } else {
        q.x = __float_as_uint(o[0]);
        q.y = __float_as_uint(o[1]);
        q.z = __float_as_uint(o[2]);
        q.w = __float_as_uint(o[3]);
    }
    if constexpr (NT) {
        typedef unsigned u32x4_t __attribute__((ext_vector_type(4)));
        __builtin_nontemporal_store(u32x4_t{q.x, q.y, q.z, q.w},
                                    reinterpret_cast<u32x4_t *>(row + c * 16));
    } else {
        *reinterpret_cast<uint4 *>(row + c * 16) = q;
    }
}

// Fixed pairwise tree over the per-slot partials of one lane.
template <int VEC>
__device__ __forceinline__ float slot_tree(const float *p)
{
    if constexpr (VEC == 8)
        return ((p[0] + p[1]) + (p[2] + p[3])) + ((p[4] + p[5]) + (p[6] + p[7]));
    else
        return (p[0] + p[1]) + (p[2] + p[3]);
}

__device__ __forceinline__ float inv_rms(float sumsq, int64_t H, float eps)
{
    const float ms = sumsq / (float)H;
    return 1.0f / sqrtf(ms + eps);
}

// One wavefront per row, RPW rows per workgroup, for rows too long to hold in
// registers (more than 64 * 8 chunks): the row is read twice, once for the sum of
// squares and once for the store.  This is the reference form of the reduction
// order above; rmsnorm_split_kernel reproduces it for shorter rows.
template <bool BF16, int RPW>
__global__ __launch_bounds__(64 * RPW) void rmsnorm_wave_kernel(const char *x, int64_t xs,
                                                                const char *__restrict__ w,
                                                                char *y, int64_t ys,
                                                                int64_t rows, int64_t H,
                                                                float eps)
{
    constexpr int VEC = Elt<BF16>::VEC;
    constexpr int SZ = Elt<BF16>::SIZE;
    const int lane = threadIdx.x & 63;
    const int64_t row = (int64_t)blockIdx.x * RPW + (threadIdx.x >> 6);
    if (row >= rows)
        return;
    const char *xr = x + row * xs * SZ;
    char *yr = y + row * ys * SZ;
    const int64_t nchunks = (H + VEC - 1) / VEC;
    float part[VEC];
#pragma unroll
    for (int e = 0; e < VEC; ++e)
        part[e] = 0.f;
    for (int64_t c = lane; c < nchunks; c += 64) {
        float v[VEC];
        load_chunk<BF16>(xr, c, H, v);
#pragma unroll
        for (int e = 0; e < VEC; ++e)
            part[e] = fmaf(v[e], v[e], part[e]);
    }
    const float rsq = inv_rms(wave_sum_butterfly(slot_tree<VEC>(part)), H, eps);
    for (int64_t c = lane; c < nchunks; c += 64) {
        float v[VEC];
        load_chunk<BF16>(xr, c, H, v);
        store_chunk<BF16>(yr, w, c, H, v, rsq);
    }
}

// The wave-per-row arithmetic with the row's memory traffic spread over NWV waves,
// one row per workgroup, for rows of at most 64 * CPL chunks: a single wave issuing
// every load and store of its row was slower at every batch size measured.  Here
// wave v loads and stores the chunks of steps i = v*CPL/NWV ..
// of every lane (lane l, step i: chunk l + 64 i, as in rmsnorm_wave_kernel), parks
// their fp32 values in LDS, and after one barrier wave 0 reduces the whole row
// exactly as the single wave does: lane l's slot partials over its chunks in
// ascending step order, the slot tree and the butterfly.  After a second barrier
// every wave writes its own chunks with that rsq (letting every wave repeat the
// reduction instead read the row from LDS NWV times and was 6-14 % slower).
// Rows of at most 64 * CPL chunks.  NT: y is stored non-temporally (large batches).
template <bool BF16, int CPL, int NWV, bool NT>
__global__ __launch_bounds__(64 * NWV) void rmsnorm_split_kernel(const char *x, int64_t xs,
                                                                 const char *__restrict__ w,
                                                                 char *y, int64_t ys,
                                                                 int64_t rows, int64_t H,
                                                                 float eps)
{
    constexpr int VEC = Elt<BF16>::VEC;
    constexpr int SZ = Elt<BF16>::SIZE;
    constexpr int SPW = CPL / NWV;  // steps per wave
    static_assert(CPL % NWV == 0, "steps per wave");
    __shared__ float vs[CPL * VEC][64];
    const int lane = threadIdx.x & 63;
    const int wv = threadIdx.x >> 6;
    const int64_t row = blockIdx.x;
    const char *xr = x + row * xs * SZ;
    char *yr = y + row * ys * SZ;
    const int64_t nchunks = (H + VEC - 1) / VEC;
    const int64_t nfull = H / VEC;
    const bool tail = nfull < nchunks;

    uint4 xq[SPW], wq[SPW];
    if (nfull > 0) {
#pragma unroll
        for (int j = 0; j < SPW; ++j) {
            const int64_t c = min((int64_t)lane + 64 * (wv * SPW + j), nfull - 1);
            xq[j] = *reinterpret_cast<const uint4 *>(xr + c * 16);
        }
#pragma unroll
        for (int j = 0; j < SPW; ++j) {
            const int64_t c = min((int64_t)lane + 64 * (wv * SPW + j), nfull - 1);
            wq[j] = *reinterpret_cast<const uint4 *>(w + c * 16);
        }
    }
    float v[SPW][VEC];
#pragma unroll
    for (int j = 0; j < SPW; ++j) {
        const int i = wv * SPW + j;
        const int64_t c = lane + 64 * i;
        float t[VEC];
        unpack_chunk<BF16>(xq[j], t);
#pragma unroll
        for (int e = 0; e < VEC; ++e)
            v[j][e] = c < nfull ? t[e] : 0.f;
        if (tail && c == nfull)
            load_chunk<BF16>(xr, c, H, v[j]);
#pragma unroll
        for (int e = 0; e < VEC; ++e)
            vs[i * VEC + e][lane] = v[j][e];
    }
    __syncthreads();

    // wave 0 reduces the row; the other waves take its rsq from LDS
    __shared__ float rsq_lds;
    if (wv == 0) {
        float part[VEC];
#pragma unroll
        for (int e = 0; e < VEC; ++e)
            part[e] = 0.f;
#pragma unroll
        for (int i = 0; i < CPL; ++i)
#pragma unroll
            for (int e = 0; e < VEC; ++e) {
                const float a = vs[i * VEC + e][lane];
                part[e] = fmaf(a, a, part[e]);
            }
        const float r = inv_rms(wave_sum_butterfly(slot_tree<VEC>(part)), H, eps);
        if (lane == 0)
            rsq_lds = r;
    }
    __syncthreads();
    const float rsq = rsq_lds;
#pragma unroll
    for (int j = 0; j < SPW; ++j) {
        const int64_t c = lane + 64 * (wv * SPW + j);
        if (c < nfull) {
            float wv8[VEC];
            unpack_chunk<BF16>(wq[j], wv8);
            store_full_chunk<BF16, NT>(yr, c, v[j], wv8, rsq);
        } else if (tail && c == nfull) {
            store_chunk<BF16>(yr, w, c, H, v[j], rsq);
        }
    }
}

// Twin: one 256-thread workgroup per row.  Thread t owns chunks t, t+256, ...;
// slot tree, wave butterfly, then the four wave sums ((w0 + w1) + (w2 + w3)).
template <bool BF16>
__global__ __launch_bounds__(256) void rmsnorm_block_kernel(const char *x, int64_t xs,
                                                            const char *__restrict__ w, char *y,
                                                            int64_t ys, int64_t rows, int64_t H,
                                                            float eps)
{
    constexpr int VEC = Elt<BF16>::VEC;
    constexpr int SZ = Elt<BF16>::SIZE;
    __shared__ float wsum[4];
    const int t = threadIdx.x;
    const int64_t row = blockIdx.x;
    const char *xr = x + row * xs * SZ;
    char *yr = y + row * ys * SZ;
    const int64_t nchunks = (H + VEC - 1) / VEC;
    float part[VEC];
#pragma unroll
    for (int e = 0; e < VEC; ++e)
        part[e] = 0.f;
    constexpr int CPT = 4;  // chunks per thread held in registers (rows up to 1024 chunks)
    const int64_t nfull = H / VEC;
    if (nchunks <= 256 * CPT && nfull == nchunks) {
        // every chunk full: x and w requested up front (clamped, unconditional
        // 16-byte loads), one memory latency per row
        uint4 xq[CPT], wq[CPT];
#pragma unroll
        for (int i = 0; i < CPT; ++i) {
            const int64_t c = min((int64_t)t + 256 * i, nfull - 1);
            xq[i] = *reinterpret_cast<const uint4 *>(xr + c * 16);
            wq[i] = *reinterpret_cast<const uint4 *>(w + c * 16);
        }
        float v[CPT][VEC];
#pragma unroll
        for (int i = 0; i < CPT; ++i) {
            float tmp[VEC];
            unpack_chunk<BF16>(xq[i], tmp);
#pragma unroll
            for (int e = 0; e < VEC; ++e)
                v[i][e] = t + 256 * i < nfull ? tmp[e] : 0.f;
#pragma unroll
            for (int e = 0; e < VEC; ++e)
                part[e] = fmaf(v[i][e], v[i][e], part[e]);
        }
        const float s = wave_sum_butterfly(slot_tree<VEC>(part));
        if ((t & 63) == 0)
            wsum[t >> 6] = s;
        __syncthreads();
        const float rsq = inv_rms((wsum[0] + wsum[1]) + (wsum[2] + wsum[3]), H, eps);
#pragma unroll
        for (int i = 0; i < CPT; ++i) {
            const int64_t c = t + 256 * i;
            if (c < nfull) {
                float wv[VEC];
                unpack_chunk<BF16>(wq[i], wv);
                store_full_chunk<BF16>(yr, c, v[i], wv, rsq);
            }
        }
        return;
    }
    for (int64_t c = t; c < nchunks; c += 256) {
        float v[VEC];
        load_chunk<BF16>(xr, c, H, v);
#pragma unroll
        for (int e = 0; e < VEC; ++e)
            part[e] = fmaf(v[e], v[e], part[e]);
    }
    const float s = wave_sum_butterfly(slot_tree<VEC>(part));
    if ((t & 63) == 0)
        wsum[t >> 6] = s;
    __syncthreads();
    const float rsq = inv_rms((wsum[0] + wsum[1]) + (wsum[2] + wsum[3]), H, eps);
    for (int64_t c = t; c < nchunks; c += 256) {
        float v[VEC];
        load_chunk<BF16>(xr, c, H, v);
        store_chunk<BF16>(yr, w, c, H, v, rsq);
    }
}

}  // namespace

hipError_t launch_rmsnorm_wave(const void *x, int64_t xs, const void *w, void *y, int64_t ys,
                               int64_t rows, int64_t hidden, float eps, bool bf16,
                               hipStream_t s)
{
    // The workgroup shape changes with the batch, never a row's arithmetic.
    // Measured on MI355X with H = 4096 bf16 (device time of graph-replayed calls
    // over four input sets): up to 1024 rows, eight waves per row (1 row 2.8 us,
    // 512 rows 4.0 us, 1024 rows 5.9 us; four waves 3.3, 4.3, 6.1 us); beyond,
    // four waves per row (1536 rows 7.5 vs 8.2 us with eight, 4096 rows 13.3 vs
    // 14.8, 8192 rows 26.2 vs 28.9; one wave per row, four rows per workgroup:
    // 28.6 us at 8192 rows).  Rows longer than 64 * 8 chunks take the two-pass
    // wave kernel, four rows per workgroup from 4096 rows on.
    // Beyond 1024 rows y is stored non-temporally: back-to-back calls over four
    // 8192-row sets 28.1 -> 23.3 us (4.8 -> 5.8 TB/s), 4096 rows 14.0 -> 12.7 us;
    // same bits.  (Right after a 1 GiB copy has left the caches full of dirty
    // lines, one call is slower that way, 29.4 -> 32.0 us at 8192 rows; at up to
    // 1024 rows, the batch sizes whose output the next kernel reads at once,
    // the stores stay ordinary.)
    const int64_t vec = bf16 ? 8 : 4;
    const bool in_regs = (hidden + vec - 1) / vec <= 64 * 8;
    if (!in_regs && rows >= 4096) {
        const dim3 grid((unsigned)((rows + 3) / 4)), block(256);
        if (bf16)
            rmsnorm_wave_kernel<true, 4><<<grid, block, 0, s>>>(
                (const char *)x, xs, (const char *)w, (char *)y, ys, rows, hidden, eps);
        else
            rmsnorm_wave_kernel<false, 4><<<grid, block, 0, s>>>(
                (const char *)x, xs, (const char *)w, (char *)y, ys, rows, hidden, eps);
    } else if (!in_regs) {
        const dim3 grid((unsigned)rows), block(64);
        if (bf16)
            rmsnorm_wave_kernel<true, 1><<<grid, block, 0, s>>>(
                (const char *)x, xs, (const char *)w, (char *)y, ys, rows, hidden, eps);
        else
            rmsnorm_wave_kernel<false, 1><<<grid, block, 0, s>>>(
                (const char *)x, xs, (const char *)w, (char *)y, ys, rows, hidden, eps);
    } else if (rows <= 1024) {
        const dim3 grid((unsigned)rows), block(512);
        if (bf16)
            rmsnorm_split_kernel<true, 8, 8, false><<<grid, block, 0, s>>>(
                (const char *)x, xs, (const char *)w, (char *)y, ys, rows, hidden, eps);
        else
            rmsnorm_split_kernel<false, 8, 8, false><<<grid, block, 0, s>>>(
                (const char *)x, xs, (const char *)w, (char *)y, ys, rows, hidden, eps);
    } else {
        const dim3 grid((unsigned)rows), block(256);
        if (bf16)
            rmsnorm_split_kernel<true, 8, 4, true><<<grid, block, 0, s>>>(
                (const char *)x, xs, (const char *)w, (char *)y, ys, rows, hidden, eps);
        else
            rmsnorm_split_kernel<false, 8, 4, true><<<grid, block, 0, s>>>(
                (const char *)x, xs, (const char *)w, (char *)y, ys, rows, hidden, eps);
    }
    return hipGetLastError();
}

hipError_t launch_rmsnorm_block(const void *x, int64_t xs, const void *w, void *y, int64_t ys,
                                int64_t rows, int64_t hidden, float eps, bool bf16,
                                hipStream_t s)
{
    const dim3 grid((unsigned)rows), block(256);
    if (bf16)
        rmsnorm_block_kernel<true><<<grid, block, 0, s>>>(
            (const char *)x, xs, (const char *)w, (char *)y, ys, rows, hidden, eps);
    else
        rmsnorm_block_kernel<false><<<grid, block, 0, s>>>(
            (const char *)x, xs, (const char *)w, (char *)y, ys, rows, hidden, eps);
    return hipGetLastError();
}

}  // namespace rbi
