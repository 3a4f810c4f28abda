// matmul.hip -- C = A . W^T on gfx950 MFMA, bf16 in, fp32 accumulate.
//
// Batch invariance of the matmul ("Reproducible LLM Inference ...",
// hidekazu-konishi.com, section 5.4, second operation): the reduction over K of
// an output element must not depend on M.  The two things that break it are
// split-K and a change of matrix instruction at small batch; both are absent
// from matmul_bi.  Its per-element contract:
//   * one instruction, v_mfma_f32_16x16x32_bf16, for every shape;
//   * acc starts at +0 and takes ceil(K/64)*2 MFMA steps of 32 k each, in
//     ascending k, with k >= K zero-filled;
//   * inside a step, lane group q = lane/16 carries k = 8q .. 8q+7 of the row it
//     serves (the same mapping for both operands);
//   * the W row (output feature n) is operand A, the activation row (batch row m)
//     operand B; the result is rounded once to the output type.
// Which workgroup, wave or MFMA slot computes an element never enters its
// arithmetic, so the tile grid may cover any M.
//
// The twin (split-K) cuts K into equal ranges when the output tiles are too few
// to fill 256 compute units, computes each range with the same tile kernel into
// an fp32 workspace, and adds the ranges in ascending order: deterministic run
// to run, but the K partition -- and so the bits -- changes with M.
#include "device.h"
#include "launch.h"

namespace rbi {
namespace {

constexpr int BM = 128, BN = 128, BK = 64;
constexpr int GROUP_M = 8;

// LDS tile [rows][BK] bf16; 16-byte chunk q of row r lives at chunk slot q ^ (r & 7)
// so that the 16 rows read by one MFMA fragment spread over the banks.
__device__ __forceinline__ int lds_off(int r, int q)
{
    return r * BK + ((q ^ (r & 7)) << 3);
}

template <bool OUT_BF16>
__global__ __launch_bounds__(256, 2) void mm_tile_kernel(
    const uint16_t *__restrict__ A, int64_t lda, const uint16_t *__restrict__ W, int64_t ldw,
    void *__restrict__ C, int64_t ldc, int M, int N, int K, int tiles_m, int tiles_n,
    int64_t k_split, int64_t c_split_stride)
{
    __shared__ __attribute__((aligned(16))) uint16_t smem[2][2][BM * BK];

    // split-K offsets (blockIdx.y = split; a single split for the invariant path)
    const int64_t kb0 = (int64_t)blockIdx.y * k_split;
    A += kb0;
    W += kb0;
    const int Kl = (int)((K - kb0) < k_split ? (K - kb0) : k_split);

    // grouped tile order: GROUP_M row-tiles share each column sweep (L2 reuse of W)
    const int pid = blockIdx.x;
    const int in_group = GROUP_M * tiles_n;
    const int first_m = (pid / in_group) * GROUP_M;
    const int gsz = min(tiles_m - first_m, GROUP_M);
    const int tm = first_m + (pid % in_group) % gsz;
    const int tn = (pid % in_group) / gsz;
    const int m0 = tm * BM, n0 = tn * BN;

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave & 1, wn = wave >> 1;
    const int lr = lane & 15, lq = lane >> 4;

    uint4 ra[4], rw[4];
    auto gload = [&](int kt) {
        const int kb = kt * BK;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int q = tid + 256 * i;
            const int r = q >> 3, cc = q & 7;
            const int k = kb + cc * 8;
            const int m = m0 + r, n = n0 + r;
            ra[i] = (m < M && k < Kl) ? *reinterpret_cast<const uint4 *>(A + (int64_t)m * lda + k)
                                      : make_uint4(0, 0, 0, 0);
            rw[i] = (n < N && k < Kl) ? *reinterpret_cast<const uint4 *>(W + (int64_t)n * ldw + k)
                                      : make_uint4(0, 0, 0, 0);
        }
    };
    auto sstore = [&](int buf) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int q = tid + 256 * i;
            const int r = q >> 3, cc = q & 7;
            *reinterpret_cast<uint4 *>(&smem[buf][0][lds_off(r, cc)]) = ra[i];
            *reinterpret_cast<uint4 *>(&smem[buf][1][lds_off(r, cc)]) = rw[i];
        }
    };

    f32x4_t acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
            acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    const int nk = (Kl + BK - 1) / BK;
    gload(0);
    sstore(0);
    __syncthreads();
    for (int kt = 0; kt < nk; ++kt) {
        const int buf = kt & 1;
        if (kt + 1 < nk)
            gload(kt + 1);
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
            const int q = ks * 4 + lq;
            bf16x8_t af[4], wf[4];
#pragma unroll
            for (int b = 0; b < 4; ++b) {
                af[b] = as_bf16x8(*reinterpret_cast<const uint4 *>(
                    &smem[buf][0][lds_off(wm * 64 + b * 16 + lr, q)]));
                wf[b] = as_bf16x8(*reinterpret_cast<const uint4 *>(
                    &smem[buf][1][lds_off(wn * 64 + b * 16 + lr, q)]));
            }
#pragma unroll
            for (int bm = 0; bm < 4; ++bm)
#pragma unroll
                for (int bn = 0; bn < 4; ++bn)
                    acc[bm][bn] = mfma_16x16x32_bf16(wf[bn], af[bm], acc[bm][bn]);
        }
        if (kt + 1 < nk)
            sstore(buf ^ 1);
        __syncthreads();
    }

    // lane holds batch row m = lane % 16 of each block and features n = 4*(lane/16) + j
    char *Cb = reinterpret_cast<char *>(C) + (int64_t)blockIdx.y * c_split_stride;
#pragma unroll
    for (int bm = 0; bm < 4; ++bm) {
        const int m = m0 + wm * 64 + bm * 16 + lr;
        if (m >= M)
            continue;
#pragma unroll
        for (int bn = 0; bn < 4; ++bn) {
            const int n = n0 + wn * 64 + bn * 16 + 4 * lq;
            if (n >= N)
                continue;
            const f32x4_t v = acc[bm][bn];
            if constexpr (OUT_BF16) {
                uint2 o;
                o.x = pack_bf16x2(v[0], v[1]);
                o.y = pack_bf16x2(v[2], v[3]);
                *reinterpret_cast<uint2 *>(Cb + ((int64_t)m * ldc + n) * 2) = o;
            } else {
                *reinterpret_cast<float4 *>(Cb + ((int64_t)m * ldc + n) * 4) =
                    make_float4(v[0], v[1], v[2], v[3]);
            }
        }
    }
}

// C[m, n..n+3] = sum over splits (ascending) of ws[split][m][n..n+3]
template <bool OUT_BF16>
__global__ __launch_bounds__(256) void splitk_reduce_kernel(const float *__restrict__ ws, int splits,
                                                            int64_t M, int64_t N, void *C,
                                                            int64_t ldc)
{
    const int64_t nv = N / 4;
    const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (idx >= M * nv)
        return;
    const int64_t m = idx / nv, n = (idx % nv) * 4;
    const int64_t mn = M * N;
    float4 s = *reinterpret_cast<const float4 *>(ws + m * N + n);
    for (int sp = 1; sp < splits; ++sp) {
        const float4 t = *reinterpret_cast<const float4 *>(ws + sp * mn + m * N + n);
        s.x += t.x;
        s.y += t.y;
        s.z += t.z;
        s.w += t.w;
    }
    if constexpr (OUT_BF16) {
        uint2 o;
        o.x = pack_bf16x2(s.x, s.y);
        o.y = pack_bf16x2(s.z, s.w);
        *reinterpret_cast<uint2 *>(reinterpret_cast<uint16_t *>(C) + m * ldc + n) = o;
    } else {
        *reinterpret_cast<float4 *>(reinterpret_cast<float *>(C) + m * ldc + n) = s;
    }
}

hipError_t launch_tiles(const MatmulArgs &a, int splits, int64_t k_split, void *C, int64_t ldc,
                        bool out_bf16, int64_t c_split_stride, hipStream_t s)
{
    const int tiles_m = (int)((a.M + BM - 1) / BM), tiles_n = (int)((a.N + BN - 1) / BN);
    const dim3 grid((unsigned)(tiles_m * tiles_n), (unsigned)splits), block(256);
    if (out_bf16)
        mm_tile_kernel<true><<<grid, block, 0, s>>>(a.A, a.lda, a.W, a.ldw, C, ldc, (int)a.M,
                                                    (int)a.N, (int)a.K, tiles_m, tiles_n, k_split,
                                                    c_split_stride);
    else
        mm_tile_kernel<false><<<grid, block, 0, s>>>(a.A, a.lda, a.W, a.ldw, C, ldc, (int)a.M,
                                                     (int)a.N, (int)a.K, tiles_m, tiles_n, k_split,
                                                     c_split_stride);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_matmul_bi(const MatmulArgs &a, hipStream_t s)
{
    return launch_tiles(a, 1, a.K, a.C, a.ldc, a.c_bf16, 0, s);
}

// Split count of the twin: enough K ranges that the tiles fill ~2 workgroups per
// compute unit, each range at least 256 deep, at most 16 ranges.
int matmul_tuned_splits(int64_t M, int64_t N, int64_t K)
{
    const int64_t tiles = ((M + BM - 1) / BM) * ((N + BN - 1) / BN);
    int splits = 1;
    while (splits < 16 && tiles * splits * 2 <= 512 && K / (splits * 2) >= 256)
        splits *= 2;
    return splits;
}

hipError_t launch_matmul_splitk(const MatmulArgs &a, int splits, float *ws, hipStream_t s)
{
    // equal ranges, each a multiple of BK
    int64_t k_split = (a.K + splits - 1) / splits;
    k_split = (k_split + BK - 1) / BK * BK;
    splits = (int)((a.K + k_split - 1) / k_split);
    hipError_t e = launch_tiles(a, splits, k_split, ws, a.N, false, a.M * a.N * 4, s);
    if (e != hipSuccess)
        return e;
    const int64_t nvec = a.M * (a.N / 4);
    const dim3 grid((unsigned)((nvec + 255) / 256)), block(256);
    if (a.c_bf16)
        splitk_reduce_kernel<true><<<grid, block, 0, s>>>(ws, splits, a.M, a.N, a.C, a.ldc);
    else
        splitk_reduce_kernel<false><<<grid, block, 0, s>>>(ws, splits, a.M, a.N, a.C, a.ldc);
    return hipGetLastError();
}

}  // namespace rbi
