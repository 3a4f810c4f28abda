// device.h -- small device-side helpers shared by the HIP kernels of librbi.
// CDNA4 (gfx950) only: 64-lane wavefronts, MFMA bf16 matrix cores.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace rbi {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;

__device__ __forceinline__ float bf16_to_f32(uint32_t bits16)
{
    return __uint_as_float(bits16 << 16);
}

// fp32 -> bf16 bits, round to nearest, ties to even; NaN stays a quiet NaN.
__device__ __forceinline__ uint32_t f32_to_bf16(float f)
{
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7fffffffu) > 0x7f800000u)
        return ((u >> 16) | 0x40u) & 0xffffu;
    u += 0x7fffu + ((u >> 16) & 1u);
    return u >> 16;
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi)
{
    return f32_to_bf16(lo) | (f32_to_bf16(hi) << 16);
}

// The 8 bf16 values held in a 16-byte chunk, widened to fp32 in element order.
__device__ __forceinline__ void unpack8(const uint4 &c, float *v)
{
    const uint32_t w[4] = {c.x, c.y, c.z, c.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        v[2 * i] = __uint_as_float(w[i] << 16);
        v[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
    }
}

__device__ __forceinline__ bf16x8_t as_bf16x8(const uint4 &c)
{
    return __builtin_bit_cast(bf16x8_t, c);
}

// Sum across the 64 lanes of a wavefront by a fixed xor butterfly (offsets 32,
// 16, ..., 1).  Every lane ends with the same value: at each step the two lanes
// of a pair add the same two operands (fp32 addition commutes).
__device__ __forceinline__ float wave_sum_butterfly(float v)
{
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1)
        v += __shfl_xor(v, off, kWave);
    return v;
}

__device__ __forceinline__ f32x4_t mfma_16x16x32_bf16(const bf16x8_t &a, const bf16x8_t &b,
                                                      const f32x4_t &c)
{
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

}  // namespace rbi
