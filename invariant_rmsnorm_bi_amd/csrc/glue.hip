// glue.hip -- element-wise pieces of a decode step: embedding gather, residual
// add, SwiGLU and the greedy row argmax.  None of them reduces across rows, so
// they are batch-invariant by construction ("Reproducible LLM Inference ...",
// hidekazu-konishi.com, section 5.4: element-wise operations involve no
// reduction).  The argmax reduces within a row but its result (the maximum and
// the lowest index holding it) is exact, so any reduction order gives the same
// answer.
#include "device.h"
#include "launch.h"

namespace rbi {
namespace {

__global__ __launch_bounds__(256) void embed_kernel(const uint16_t *__restrict__ table,
                                                    int64_t vocab, int64_t hidden,
                                                    const int32_t *__restrict__ ids, int64_t rows,
                                                    uint16_t *__restrict__ out, int64_t os)
{
    const int64_t cpr = hidden / 8;
    const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (idx >= rows * cpr)
        return;
    const int64_t r = idx / cpr, c = idx % cpr;
    const int64_t id = ids[r];
    uint4 v = make_uint4(0, 0, 0, 0);
    if (id >= 0 && id < vocab)
        v = *reinterpret_cast<const uint4 *>(table + id * hidden + 8 * c);
    *reinterpret_cast<uint4 *>(out + r * os + 8 * c) = v;
}

__device__ __forceinline__ uint32_t add_bf16x2(uint32_t a, uint32_t b)
{
    const float lo = __uint_as_float(a << 16) + __uint_as_float(b << 16);
    const float hi = __uint_as_float(a & 0xffff0000u) + __uint_as_float(b & 0xffff0000u);
    return pack_bf16x2(lo, hi);
}

__global__ __launch_bounds__(256) void residual_kernel(const uint16_t *a, const uint16_t *b,
                                                       uint16_t *out, int64_t n)
{
    const int64_t i8 = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 8;
    if (i8 >= n)
        return;
    if (i8 + 8 <= n && ((reinterpret_cast<uintptr_t>(a) | reinterpret_cast<uintptr_t>(b) |
                         reinterpret_cast<uintptr_t>(out)) & 15) == 0) {
        const uint4 x = *reinterpret_cast<const uint4 *>(a + i8);
        const uint4 y = *reinterpret_cast<const uint4 *>(b + i8);
        *reinterpret_cast<uint4 *>(out + i8) = make_uint4(add_bf16x2(x.x, y.x), add_bf16x2(x.y, y.y),
                                                          add_bf16x2(x.z, y.z), add_bf16x2(x.w, y.w));
    } else {
        for (int64_t i = i8; i < n && i < i8 + 8; ++i)
            out[i] = (uint16_t)f32_to_bf16(bf16_to_f32(a[i]) + bf16_to_f32(b[i]));
    }
}

__device__ __forceinline__ float silu_mul(float g, float u)
{
    return g / (1.0f + expf(-g)) * u;
}

__global__ __launch_bounds__(256) void swiglu_kernel(const uint16_t *__restrict__ gu, int64_t gs,
                                                     uint16_t *__restrict__ out, int64_t os,
                                                     int64_t rows, int64_t inter)
{
    const int64_t cpr = (inter + 7) / 8;
    const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (idx >= rows * cpr)
        return;
    const int64_t r = idx / cpr, i0 = (idx % cpr) * 8;
    const uint16_t *g = gu + r * gs;
    const uint16_t *u = g + inter;
    uint16_t *o = out + r * os;
    for (int64_t i = i0; i < i0 + 8 && i < inter; ++i)
        o[i] = (uint16_t)f32_to_bf16(silu_mul(bf16_to_f32(g[i]), bf16_to_f32(u[i])));
}

// (value, index) pair ordering: larger value wins, the lower index wins a tie.
__device__ __forceinline__ bool better(float v, int i, float bv, int bi)
{
    return v > bv || (v == bv && i < bi);
}

// One 1024-thread workgroup per row.
// VEC4: the row is 16-byte aligned, so its full 4-element chunks are read as
// float4, four per thread per step, all requested before any is compared (a
// thread past the last chunk re-reads it and ignores the value); the elements
// after the last full chunk are read one by one.
template <bool VEC4>
__global__ __launch_bounds__(1024) void argmax_kernel(const float *x, int64_t xs, int64_t n,
                                                      int32_t *__restrict__ out)
{
    __shared__ float sv[16];
    __shared__ int si[16];
    const int64_t r = blockIdx.x;
    const float *row = x + r * xs;
    float bv = -INFINITY;
    int bi = 0x7fffffff;
    int64_t scalar_from = 0;
    if constexpr (VEC4) {
        const int64_t n4 = n / 4;
        const float4 *row4 = reinterpret_cast<const float4 *>(row);
        for (int64_t base = 0; base < n4; base += 4 * 1024) {
            float4 v[4];
#pragma unroll
            for (int k = 0; k < 4; ++k)
                v[k] = row4[min(base + k * 1024 + threadIdx.x, n4 - 1)];
            asm volatile("" ::: "memory");  // all four loads in flight before the compares
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                const int64_t c = base + k * 1024 + threadIdx.x;
                if (c < n4) {
                    const float e[4] = {v[k].x, v[k].y, v[k].z, v[k].w};
#pragma unroll
                    for (int j = 0; j < 4; ++j)
                        if (e[j] == e[j] && better(e[j], (int)(4 * c + j), bv, bi)) {
                            bv = e[j];
                            bi = (int)(4 * c + j);
                        }
                }
            }
        }
        scalar_from = 4 * n4;
    }
    for (int64_t i = scalar_from + threadIdx.x; i < n; i += 1024) {
        const float v = row[i];
        if (v == v && better(v, (int)i, bv, bi)) {
            bv = v;
            bi = (int)i;
        }
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
        const float ov = __shfl_xor(bv, off, kWave);
        const int oi = __shfl_xor(bi, off, kWave);
        if (better(ov, oi, bv, bi)) {
            bv = ov;
            bi = oi;
        }
    }
    const int wave = threadIdx.x >> 6;
    if ((threadIdx.x & 63) == 0) {
        sv[wave] = bv;
        si[wave] = bi;
    }
    __syncthreads();
    if (threadIdx.x == 0) {
        for (int w = 1; w < 16; ++w)
            if (better(sv[w], si[w], bv, bi)) {
                bv = sv[w];
                bi = si[w];
            }
        out[r] = bi == 0x7fffffff ? 0 : bi;
    }
}

// Plain streaming copy, one 16-byte chunk per thread: the read + write reference
// a read-once write-once kernel such as RMSNorm is measured against.
template <bool NT>
__global__ __launch_bounds__(256) void stream_copy_kernel(const uint4 *__restrict__ src,
                                                          uint4 *__restrict__ dst, int64_t n)
{
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= n)
        return;
    const uint4 v = src[i];
    if constexpr (NT) {
        typedef unsigned u32x4_t __attribute__((ext_vector_type(4)));
        __builtin_nontemporal_store(u32x4_t{v.x, v.y, v.z, v.w},
                                    reinterpret_cast<u32x4_t *>(dst + i));
    } else {
        dst[i] = v;
    }
}

}  // namespace

hipError_t launch_embed(const uint16_t *table, int64_t vocab, int64_t hidden, const int32_t *ids,
                        int64_t rows, uint16_t *out, int64_t os, hipStream_t s)
{
    const int64_t n = rows * (hidden / 8);
    embed_kernel<<<dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s>>>(table, vocab, hidden, ids,
                                                                         rows, out, os);
    return hipGetLastError();
}

hipError_t launch_residual_add(const uint16_t *a, const uint16_t *b, uint16_t *out, int64_t n,
                               hipStream_t s)
{
    const int64_t t = (n + 7) / 8;
    residual_kernel<<<dim3((unsigned)((t + 255) / 256)), dim3(256), 0, s>>>(a, b, out, n);
    return hipGetLastError();
}

hipError_t launch_swiglu(const uint16_t *gu, int64_t gs, uint16_t *out, int64_t os, int64_t rows,
                         int64_t inter, hipStream_t s)
{
    const int64_t n = rows * ((inter + 7) / 8);
    swiglu_kernel<<<dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s>>>(gu, gs, out, os, rows,
                                                                          inter);
    return hipGetLastError();
}

hipError_t launch_argmax(const float *x, int64_t xs, int64_t rows, int64_t n, int32_t *out,
                         hipStream_t s)
{
    if ((reinterpret_cast<uintptr_t>(x) & 15) == 0 && xs % 4 == 0)
        argmax_kernel<true><<<dim3((unsigned)rows), dim3(1024), 0, s>>>(x, xs, n, out);
    else
        argmax_kernel<false><<<dim3((unsigned)rows), dim3(1024), 0, s>>>(x, xs, n, out);
    return hipGetLastError();
}

}  // namespace rbi

namespace rbi {

hipError_t launch_stream_copy(const void *src, void *dst, int64_t bytes, bool nt, hipStream_t s)
{
    const int64_t n = bytes / 16;
    const dim3 grid((unsigned)((n + 255) / 256)), block(256);
    if (nt)
        stream_copy_kernel<true><<<grid, block, 0, s>>>((const uint4 *)src, (uint4 *)dst, n);
    else
        stream_copy_kernel<false><<<grid, block, 0, s>>>((const uint4 *)src, (uint4 *)dst, n);
    return hipGetLastError();
}

}  // namespace rbi
