// sampling.hip -- seeded Gumbel-max sampling for gfx950.
//
// Non-greedy decoding that stays reproducible ("Reproducible LLM Inference ...",
// hidekazu-konishi.com, section 9.3 "Non-Greedy Sampling Can Be Deterministic
// Too"): every logit is perturbed by Gumbel noise drawn from a seeded
// counter-based hash instead of a stateful generator, and the token is the
// argmax.  For row r with seed s, position p and temperature T > 0:
//     token = argmax_i (logit_i / T + g_i),   g_i = -ln(-ln u_i),
// u_i = (floor(w_i / 2^9) + 1/2) / 2^23 from word i mod 4 of Philox4x32-10
// (Salmon et al., "Parallel Random Numbers: As Easy as 1, 2, 3", SC 2011) with
// counter (i / 4, p mod 2^32, p / 2^32, 0) and key (s mod 2^32, s / 2^32).
// T <= 0 is greedy.  The noise depends on nothing but (seed, position, i), and
// the argmax (the maximum score, the lowest index holding it; NaN never chosen)
// is exact, so any reduction order gives the same token: the result is a
// function of the row alone -- batch-invariant when the logits are.
//
// Pass 1: grid (chunks of 4096 entries, rows), 256 threads, each thread 4
// consecutive entries per step (one Philox call, one 16-byte load); the chunk's
// best (score, index) goes to the workspace.  Pass 2: one wave per row reduces
// the chunks' partials.
#include "device.h"
#include "launch.h"

namespace rbi {
namespace {

constexpr int kSampleThreads = 256;
constexpr int kSampleSteps = 4;
constexpr int kSampleChunk = kSampleThreads * 4 * kSampleSteps;  // entries per workgroup

// Philox4x32-10: ten rounds of two 32x32->64-bit products, the key advancing by
// the Weyl constants between rounds.
__device__ __forceinline__ uint4 philox4x32_10(uint4 c, uint32_t k0, uint32_t k1)
{
#pragma unroll
    for (int round = 0; round < 10; ++round) {
        if (round > 0) {
            k0 += 0x9E3779B9u;
            k1 += 0xBB67AE85u;
        }
        const uint32_t lo0 = 0xD2511F53u * c.x, hi0 = __umulhi(0xD2511F53u, c.x);
        const uint32_t lo1 = 0xCD9E8D57u * c.z, hi1 = __umulhi(0xCD9E8D57u, c.z);
        c = make_uint4(hi1 ^ c.y ^ k0, lo1, hi0 ^ c.w ^ k1, lo0);
    }
    return c;
}

__device__ __forceinline__ float gumbel_of_word(uint32_t w)
{
    const float u = ((float)(w >> 9) + 0.5f) * 0x1p-23f;  // exact: 24 significant bits
    return -logf(-logf(u));
}

// (v, i) beats (bv, bi): larger score, or the same score at a lower index.
__device__ __forceinline__ bool beats(float v, int i, float bv, int bi)
{
    return v > bv || (v == bv && i < bi);
}

__device__ __forceinline__ void wave_best(float &bv, int &bi)
{
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
        const float ov = __shfl_xor(bv, off, kWave);
        const int oi = __shfl_xor(bi, off, kWave);
        if (beats(ov, oi, bv, bi)) {
            bv = ov;
            bi = oi;
        }
    }
}

__global__ __launch_bounds__(kSampleThreads) void sample_chunk_kernel(
    const float *__restrict__ logits, int64_t ld, int64_t vocab,
    const uint64_t *__restrict__ seeds, const int64_t *__restrict__ positions,
    const float *__restrict__ temps, int nchunks, float *__restrict__ ws_score,
    int32_t *__restrict__ ws_index)
{
    __shared__ float s_v[kSampleThreads / kWave];
    __shared__ int s_i[kSampleThreads / kWave];
    const int64_t r = blockIdx.y;
    const float T = temps[r];
    const bool noisy = T > 0.f;
    const uint64_t seed = seeds[r];
    const uint64_t pos = (uint64_t)positions[r];
    const uint32_t k0 = (uint32_t)seed, k1 = (uint32_t)(seed >> 32);
    const float *row = logits + r * ld;
    float bv = -INFINITY;
    int bi = 0x7fffffff;
#pragma unroll
    for (int step = 0; step < kSampleSteps; ++step) {
        const int64_t i0 = (int64_t)blockIdx.x * kSampleChunk +
                           ((int64_t)step * kSampleThreads + threadIdx.x) * 4;
        if (i0 >= vocab)
            continue;
        float x[4];
        if (i0 + 4 <= vocab) {
            const float4 v4 = *reinterpret_cast<const float4 *>(row + i0);
            x[0] = v4.x;
            x[1] = v4.y;
            x[2] = v4.z;
            x[3] = v4.w;
        } else {
#pragma unroll
            for (int j = 0; j < 4; ++j)
                x[j] = i0 + j < vocab ? row[i0 + j] : __uint_as_float(0x7fc00000u);
        }
        float s[4];
        if (noisy) {
            const uint4 w = philox4x32_10(
                make_uint4((uint32_t)(i0 >> 2), (uint32_t)pos, (uint32_t)(pos >> 32), 0u), k0, k1);
            s[0] = x[0] / T + gumbel_of_word(w.x);
            s[1] = x[1] / T + gumbel_of_word(w.y);
            s[2] = x[2] / T + gumbel_of_word(w.z);
            s[3] = x[3] / T + gumbel_of_word(w.w);
        } else {
#pragma unroll
            for (int j = 0; j < 4; ++j)
                s[j] = x[j];
        }
#pragma unroll
        for (int j = 0; j < 4; ++j)
            if (x[j] == x[j] && beats(s[j], (int)(i0 + j), bv, bi)) {  // NaN logits never win
                bv = s[j];
                bi = (int)(i0 + j);
            }
    }
    wave_best(bv, bi);
    const int wave = threadIdx.x >> 6;
    if ((threadIdx.x & 63) == 0) {
        s_v[wave] = bv;
        s_i[wave] = bi;
    }
    __syncthreads();
    if (threadIdx.x == 0) {
        for (int w = 1; w < kSampleThreads / kWave; ++w)
            if (beats(s_v[w], s_i[w], bv, bi)) {
                bv = s_v[w];
                bi = s_i[w];
            }
        ws_score[r * nchunks + blockIdx.x] = bv;
        ws_index[r * nchunks + blockIdx.x] = bi;
    }
}

// One wave per row: the best of the row's chunk partials.
__global__ __launch_bounds__(256) void sample_reduce_kernel(const float *__restrict__ ws_score,
                                                            const int32_t *__restrict__ ws_index,
                                                            int64_t rows, int nchunks,
                                                            int32_t *__restrict__ tokens)
{
    const int64_t r = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (r >= rows)
        return;
    const int lane = threadIdx.x & 63;
    float bv = -INFINITY;
    int bi = 0x7fffffff;
    for (int c = lane; c < nchunks; c += kWave) {
        const float v = ws_score[r * nchunks + c];
        const int i = ws_index[r * nchunks + c];
        if (beats(v, i, bv, bi)) {
            bv = v;
            bi = i;
        }
    }
    wave_best(bv, bi);
    if (lane == 0)
        tokens[r] = bi == 0x7fffffff ? 0 : bi;
}

}  // namespace

int sample_chunks(int64_t vocab)
{
    return (int)((vocab + kSampleChunk - 1) / kSampleChunk);
}

size_t sample_workspace_bytes(int64_t rows, int64_t vocab)
{
    return (size_t)rows * (size_t)sample_chunks(vocab) * (sizeof(float) + sizeof(int32_t));
}

hipError_t launch_sample_gumbel(const float *logits, int64_t ld, int64_t rows, int64_t vocab,
                                const uint64_t *seeds, const int64_t *positions,
                                const float *temps, int32_t *tokens, void *ws, hipStream_t s)
{
    const int nchunks = sample_chunks(vocab);
    float *ws_score = static_cast<float *>(ws);
    int32_t *ws_index = reinterpret_cast<int32_t *>(ws_score + rows * nchunks);
    sample_chunk_kernel<<<dim3((unsigned)nchunks, (unsigned)rows), dim3(kSampleThreads), 0, s>>>(
        logits, ld, vocab, seeds, positions, temps, nchunks, ws_score, ws_index);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess)
        return e;
    sample_reduce_kernel<<<dim3((unsigned)((rows + 3) / 4)), dim3(256), 0, s>>>(
        ws_score, ws_index, rows, nchunks, tokens);
    return hipGetLastError();
}

}  // namespace rbi
