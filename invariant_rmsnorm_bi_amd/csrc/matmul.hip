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
#include <cmath>

#include "device.h"
#include "launch.h"

namespace rbi {
namespace {

constexpr int BM = 128, BN = 128, BK = 64;
constexpr int GROUP_M = 8;
constexpr int BIG_GROUP_M = 4;
constexpr int NUM_XCD = 8;

// Output tile of workgroup `pid`.  Workgroups are dealt to the eight XCDs (each with
// its own L2) round robin, so pid -> XCD is pid % 8; first give each XCD a contiguous
// run of logical tile ids, then order tiles in groups of `group_m` tile rows that
// sweep the columns together.  The workgroups resident on one XCD then cover a compact
// block of C and share their A rows and W rows in that XCD's L2.  The map is a
// bijection on [0, tiles_m * tiles_n) whatever the placement; only speed depends on it.
__device__ __forceinline__ void tile_coords(int pid, int tiles_m, int tiles_n, int group_m,
                                            int &tm, int &tn)
{
    const int total = tiles_m * tiles_n;
    const int per = total / NUM_XCD, extra = total % NUM_XCD;
    const int xcd = pid % NUM_XCD, local = pid / NUM_XCD;
    const int t = xcd * per + min(xcd, extra) + local;
    const int in_group = group_m * tiles_n;
    const int first_m = (t / in_group) * group_m;
    const int gsz = min(tiles_m - first_m, group_m);
    tm = first_m + (t % in_group) % gsz;
    tn = (t % in_group) / gsz;
}

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

    int tm, tn;
    tile_coords(blockIdx.x, tiles_m, tiles_n, GROUP_M, tm, tn);
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

// Pipelined tile kernel for K a multiple of 32 (mm_pipe64_kernel below takes over when
// every K range is a multiple of 64, so this one serves K = 32 mod 64): a TBM x TBN
// output tile per workgroup of WM*WN waves in a WM x WN grid, each wave owning (TBM/WM) batch rows x
// (TBN/WN) features.  K advances one MFMA step (32 k) per stage; P stages of
// operand tiles are in flight at once, copied from global memory straight into LDS
// (global_load_lds_dwordx4: no register staging), so a load has P-1 stages of MFMA
// work to arrive in.  Operand fragments are double buffered in registers: the next
// stage's are read from LDS while this stage's MFMAs run.  The MFMA instruction, its
// operand roles, the k fragment mapping and the ascending k order are those of
// mm_tile_kernel, so each element gets the same bits from either kernel (a K that is
// 32 mod 64 only drops the tile kernel's trailing all-zero step, an exact no-op).
//
// LDS stage layout: TBM activation rows then TBN weight rows, each 32 k (64 bytes,
// four 16-byte chunks); chunk c of stage row r sits in slot c ^ pswz(r).  One load
// instruction fills 16 consecutive rows (lane l -> row l/4, slot l%4) and each lane
// fetches the global chunk that belongs in its slot.  A fragment read is 16
// consecutive rows (16 lanes per chunk, four chunks).  Measured on gfx950 with the
// LDS bank-conflict counter over all 256 swizzles that XOR the slot with a linear
// function of the four row bits: whether the read conflicts depends only on the
// offsets c2, c3 that row bits 2 and 3 (byte-address bits 8 and 9) contribute, and
// it is conflict free exactly when c2 != c3 and neither is 1 (an offset of 1 keeps
// a chunk inside its 32-byte half of the row).  The swizzle below has c2 = 2,
// c3 = 3; the earlier ((r >> 1) ^ (r >> 3)) & 3 (c2 = 2, c3 = 1) measured two-way
// conflicts.  The layout only moves data within LDS, so no result changes.
constexpr int PK = 32;

__device__ __forceinline__ int pswz(int r)
{
    return (((r >> 2) & 1) * 2) ^ (((r >> 3) & 1) * 3);
}

// Wait until at most N of this wave's global loads are outstanding and all of its LDS
// reads have returned, then meet the other waves.  s_waitcnt immediate (gfx9):
// vmcnt bits [3:0] and [15:14], expcnt [6:4], lgkmcnt [11:8].  The empty asm
// statements keep the compiler from moving memory accesses across the barrier.
template <int N>
__device__ __forceinline__ void wait_loads_and_barrier()
{
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (0 << 8) | ((N >> 4) << 14));
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

template <int TBM, int TBN, int WM, int WN, int P, bool OUT_BF16>
__global__ __launch_bounds__(64 * WM * WN, 1) void mm_pipe_kernel(
    const uint16_t *__restrict__ A, int64_t lda, const uint16_t *__restrict__ W, int64_t ldw,
    void *__restrict__ C, int64_t ldc, int M, int N, int K, int tiles_m, int tiles_n,
    int64_t k_split, int64_t c_split_stride)
{
    // split-K (blockIdx.y = range; the invariant path always has one range)
    {
        const int64_t kb0 = (int64_t)blockIdx.y * k_split;
        A += kb0;
        W += kb0;
        K = (int)((K - kb0) < k_split ? (K - kb0) : k_split);
        C = reinterpret_cast<char *>(C) + (int64_t)blockIdx.y * c_split_stride;
    }
    constexpr int NW = WM * WN;                   // waves
    constexpr int WTM = TBM / WM, WTN = TBN / WN; // wave tile
    constexpr int FM = WTM / 16, FN = WTN / 16;  // MFMA blocks per wave
    constexpr int ROWS = TBM + TBN;
    constexpr int STAGE = ROWS * PK;             // bf16 elements per stage
    constexpr int LPW = ROWS / (16 * NW);        // 16-row load instructions per wave per stage
    static_assert(ROWS % (16 * NW) == 0 && TBM % 16 == 0 && WTN % 16 == 0 && WTM % 16 == 0,
                  "tile shape");
    static_assert(P >= 3, "pipeline depth");
    extern __shared__ __attribute__((aligned(16))) uint16_t smem_dyn[];

    int tm, tn;
    tile_coords(blockIdx.x, tiles_m, tiles_n, BIG_GROUP_M, tm, tn);
    const int m0 = tm * TBM, n0 = tn * TBN;

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int wm = wave % WM, wn = wave / WM;
    const int lr = lane & 15, lq = lane >> 4;

    // source of this lane's 16 bytes in load instruction i of a stage (k = 0); rows
    // past M or N read a valid row whose results are never stored
    const uint16_t *src[LPW];
#pragma unroll
    for (int i = 0; i < LPW; ++i) {
        const int R = (i * NW + wave) * 16 + (lane >> 2);
        const int c = (lane & 3) ^ pswz(R);
        if ((i * NW + wave) * 16 < TBM)
            src[i] = A + (int64_t)min(m0 + R, M - 1) * lda + 8 * c;
        else
            src[i] = W + (int64_t)min(n0 + R - TBM, N - 1) * ldw + 8 * c;
    }
    auto issue = [&](int stage, int buf) {
        uint16_t *base = smem_dyn + buf * STAGE;
#pragma unroll
        for (int i = 0; i < LPW; ++i)
            __builtin_amdgcn_global_load_lds(
                (const void *)(src[i] + stage * PK),
                (void __attribute__((address_space(3))) *)(base + (i * NW + wave) * 16 * PK), 16,
                0, 0);
    };
    auto read_frags = [&](int buf, bf16x8_t (&fa)[FM], bf16x8_t (&fw)[FN]) {
        const uint16_t *base = smem_dyn + buf * STAGE;
#pragma unroll
        for (int b = 0; b < FN; ++b) {
            const int R = TBM + wn * WTN + b * 16 + lr;
            fw[b] = as_bf16x8(*reinterpret_cast<const uint4 *>(base + R * PK + 8 * (lq ^ pswz(R))));
        }
#pragma unroll
        for (int b = 0; b < FM; ++b) {
            const int R = wm * WTM + b * 16 + lr;
            fa[b] = as_bf16x8(*reinterpret_cast<const uint4 *>(base + R * PK + 8 * (lq ^ pswz(R))));
        }
    };

    f32x4_t acc[FM][FN];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
            acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    auto mfmas = [&](const bf16x8_t (&fa)[FM], const bf16x8_t (&fw)[FN]) {
#pragma unroll
        for (int bm = 0; bm < FM; ++bm)
#pragma unroll
            for (int bn = 0; bn < FN; ++bn)
                acc[bm][bn] = mfma_16x16x32_bf16(fw[bn], fa[bm], acc[bm][bn]);
    };

    const int nk = K / PK;
    // stage s lives in buffer s % P; stages 0 .. P-1 are issued up front and stage
    // s + P is issued once every wave has read stage s's fragments.  Before step kt
    // waits, stages 0 .. kt+P-1 have been issued (loads complete in issue order).
#pragma unroll
    for (int st = 0; st < P; ++st)
        if (st < nk)
            issue(st, st);
    if (nk >= P)
        wait_loads_and_barrier<(P - 1) * LPW>();
    else
        wait_loads_and_barrier<0>();
    bf16x8_t fa0[FM], fw0[FN], fa1[FM], fw1[FN];
    read_frags(0, fa0, fw0);

    // one k step: make stage kt+1 resident, refill the buffer stage kt vacated, read
    // stage kt+1's fragments, run stage kt's MFMAs.  The steady-state step is branch
    // free so that its LDS reads can be interleaved with its MFMAs, which hides LDS
    // latency under matrix work (instruction classes: 0x8 MFMA, 0x100 LDS read).
    auto steady = [&](int kt, const bf16x8_t (&fa)[FM], const bf16x8_t (&fw)[FN],
                      bf16x8_t (&na)[FM], bf16x8_t (&nw)[FN]) {
        wait_loads_and_barrier<(P - 2) * LPW>();
        issue(kt + P, kt % P);
        read_frags((kt + 1) % P, na, nw);
        mfmas(fa, fw);
        constexpr int NR = FM + FN, MPR = FM * FN / NR;
#pragma unroll
        for (int i = 0; i < NR; ++i) {
            __builtin_amdgcn_sched_group_barrier(0x008, MPR, 0);
            __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        }
        __builtin_amdgcn_sched_group_barrier(0x008, FM * FN - NR * MPR, 0);
    };
    // the last P steps: fewer stages left to issue and to wait for
    auto drain = [&](int kt, const bf16x8_t (&fa)[FM], const bf16x8_t (&fw)[FN],
                     bf16x8_t (&na)[FM], bf16x8_t (&nw)[FN]) {
        if (kt + 1 < nk) {
            if (kt + P - 1 < nk)
                wait_loads_and_barrier<(P - 2) * LPW>();
            else
                wait_loads_and_barrier<0>();
            if (kt + P < nk)
                issue(kt + P, kt % P);
            read_frags((kt + 1) % P, na, nw);
        }
        mfmas(fa, fw);
    };
    int kt = 0;
    for (; kt + P + 1 < nk; kt += 2) {
        steady(kt, fa0, fw0, fa1, fw1);
        steady(kt + 1, fa1, fw1, fa0, fw0);
    }
    for (; kt + 1 < nk; kt += 2) {
        drain(kt, fa0, fw0, fa1, fw1);
        drain(kt + 1, fa1, fw1, fa0, fw0);
    }
    if (kt < nk)
        drain(kt, fa0, fw0, fa1, fw1);

    // lane holds batch row m = lane % 16 of each block and features n = 4*(lane/16) + j
#pragma unroll
    for (int bm = 0; bm < FM; ++bm) {
        const int m = m0 + wm * WTM + bm * 16 + lr;
        if (m >= M)
            continue;
#pragma unroll
        for (int bn = 0; bn < FN; ++bn) {
            const int n = n0 + wn * WTN + bn * 16 + 4 * lq;
            if (n >= N)
                continue;
            const f32x4_t v = acc[bm][bn];
            if constexpr (OUT_BF16) {
                uint2 o;
                o.x = pack_bf16x2(v[0], v[1]);
                o.y = pack_bf16x2(v[2], v[3]);
                *reinterpret_cast<uint2 *>(reinterpret_cast<uint16_t *>(C) + (int64_t)m * ldc + n) = o;
            } else {
                *reinterpret_cast<float4 *>(reinterpret_cast<float *>(C) + (int64_t)m * ldc + n) =
                    make_float4(v[0], v[1], v[2], v[3]);
            }
        }
    }
}

template <int TBM, int TBN, int WM, int WN, int P>
hipError_t launch_pipe(const MatmulArgs &a, hipStream_t s, int splits = 1, int64_t k_split = 0,
                       int64_t c_split_stride = 0)
{
    if (splits == 1)
        k_split = a.K;
    const int tiles_m = (int)((a.M + TBM - 1) / TBM), tiles_n = (int)((a.N + TBN - 1) / TBN);
    const size_t lds = (size_t)P * (TBM + TBN) * PK * sizeof(uint16_t);
    const void *fn = a.c_bf16 ? (const void *)mm_pipe_kernel<TBM, TBN, WM, WN, P, true>
                              : (const void *)mm_pipe_kernel<TBM, TBN, WM, WN, P, false>;
    hipError_t e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess)
        return e;
    const dim3 grid((unsigned)(tiles_m * tiles_n), (unsigned)splits), block(64 * WM * WN);
    if (a.c_bf16)
        mm_pipe_kernel<TBM, TBN, WM, WN, P, true><<<grid, block, lds, s>>>(
            a.A, a.lda, a.W, a.ldw, a.C, a.ldc, (int)a.M, (int)a.N, (int)a.K, tiles_m, tiles_n,
            k_split, c_split_stride);
    else
        mm_pipe_kernel<TBM, TBN, WM, WN, P, false><<<grid, block, lds, s>>>(
            a.A, a.lda, a.W, a.ldw, a.C, a.ldc, (int)a.M, (int)a.N, (int)a.K, tiles_m, tiles_n,
            k_split, c_split_stride);
    return hipGetLastError();
}

// Two-step stages (K a multiple of 64): the same waves, fragment reads and MFMA sequence
// as mm_pipe_kernel, but a stage holds 64 k, so a stage row is one whole 128-byte line
// of its operand row.  One load instruction fills 8 rows (lane l -> row l/8, slot l%8,
// fetching the global chunk that belongs in its slot), so every line the L1 fetches from
// L2 is used in full by one instruction; with 64-byte rows the two halves of a line were
// fetched by different stages, too far apart for the line to stay in the L1, and each
// line crossed from L2 twice (the L1-to-L2 read requests of the 256 x 256 tile measured
// half as many).  P stages are resident and one barrier serves 64 k:
//   step 2s   : read step 2s+1's fragments (stage s) while step 2s's MFMAs run;
//   barrier   : stage s+1 has landed for every wave, and every wave has read stage s;
//               refill stage s's buffer with stage s+P;
//   step 2s+1 : read step 2s+2's fragments (stage s+1) while step 2s+1's MFMAs run.
// A load thus has 2P-2 steps of MFMA work to arrive in.  Chunk c of stage row r sits in
// slot c ^ swz8(r).  Measured on gfx950 with the LDS bank-conflict counter over every
// swizzle that XORs the slot with a linear function of the four row bits (a one-wave
// probe of this read pattern): a fragment read is conflict free exactly when the offsets
// that row bits 1 and 2 contribute differ from each other and from zero in slot bits
// 1..2 (byte-address bits 5..6); row bits 0 and 3 may contribute anything.  swz8 takes
// 4 for row bit 1 and 2 for row bit 2.  It depends on r % 16 only, so every fragment
// read of a wave shares one lane-dependent address part and differs by a constant.
constexpr int SK = 64;

__device__ __forceinline__ int swz8(int r)
{
    return ((r & 2) << 1) | ((r & 4) >> 1);
}

template <int TBM, int TBN, int WM, int WN, int P, bool OUT_BF16>
__global__ __launch_bounds__(64 * WM * WN, 1) void mm_pipe64_kernel(
    const uint16_t *__restrict__ A, int64_t lda, const uint16_t *__restrict__ W, int64_t ldw,
    void *__restrict__ C, int64_t ldc, int M, int N, int K, int tiles_m, int tiles_n,
    int64_t k_split, int64_t c_split_stride)
{
    {
        const int64_t kb0 = (int64_t)blockIdx.y * k_split;
        A += kb0;
        W += kb0;
        K = (int)((K - kb0) < k_split ? (K - kb0) : k_split);
        C = reinterpret_cast<char *>(C) + (int64_t)blockIdx.y * c_split_stride;
    }
    constexpr int NW = WM * WN;
    constexpr int WTM = TBM / WM, WTN = TBN / WN;
    constexpr int FM = WTM / 16, FN = WTN / 16;
    constexpr int ROWS = TBM + TBN;
    constexpr int STAGE = ROWS * SK;             // bf16 elements per stage
    constexpr int LPW = ROWS / (8 * NW);         // 8-row load instructions per wave per stage
    constexpr int LA = TBM / (8 * NW);           // of which fill activation rows
    static_assert(TBM % (8 * NW) == 0 && TBN % (8 * NW) == 0 && WTM % 16 == 0 && WTN % 16 == 0,
                  "tile shape");
    static_assert(P >= 2, "pipeline depth");
    extern __shared__ __attribute__((aligned(16))) uint16_t smem_dyn[];

    int tm, tn;
    tile_coords(blockIdx.x, tiles_m, tiles_n, BIG_GROUP_M, tm, tn);
    const int m0 = tm * TBM, n0 = tn * TBN;

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int wm = wave % WM, wn = wave / WM;
    const int lr = lane & 15, lq = lane >> 4;

    // byte offset of this lane's 16 bytes in load instruction i of a stage, from its
    // operand's base; rows past M or N read a valid row whose results are never stored
    uint32_t off[LPW];
#pragma unroll
    for (int i = 0; i < LPW; ++i) {
        const int R = (i * NW + wave) * 8 + (lane >> 3);
        const int c = (lane & 7) ^ swz8(R);
        if (i < LA)
            off[i] = (uint32_t)(((int64_t)min(m0 + R, M - 1) * lda + 8 * c) * 2);
        else
            off[i] = (uint32_t)(((int64_t)min(n0 + R - TBM, N - 1) * ldw + 8 * c) * 2);
    }
    // Buffer loads to LDS: a descriptor per operand (base, no range limit below 4 GiB,
    // the gfx9 raw 32-bit data format), the lane's 32-bit offset and the stage's byte
    // offset as a scalar, so advancing a stage costs no vector instruction (measured
    // 1.5-5 % faster than 64-bit per-lane global addresses over the decode-layer
    // shapes, e.g. o_proj M = 4096 199.5 -> 191.9 us).  The host pass never runs this
    // body, and it drops the kernel's launch stub when it meets the buffer builtin
    // inside the lambda, so the loop is compiled for the device only.
    auto issue = [&](int stage, int buf) {
        uint16_t *base = smem_dyn + buf * STAGE;
#if defined(__HIP_DEVICE_COMPILE__)
#pragma unroll
        for (int i = 0; i < LPW; ++i)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                __builtin_amdgcn_make_buffer_rsrc((void *)(i < LA ? A : W), (short)0, -1,
                                                  0x00020000),
                (void __attribute__((address_space(3))) *)(base + (i * NW + wave) * 8 * SK), 16,
                off[i], stage * SK * 2, 0, 0);
#else
        (void)base, (void)stage, (void)A, (void)W;
#endif
    };
    auto read_frags = [&](int buf, int sub, bf16x8_t (&fa)[FM], bf16x8_t (&fw)[FN]) {
        const uint16_t *base = smem_dyn + buf * STAGE;
        const int q = sub * 4 + lq;
#pragma unroll
        for (int b = 0; b < FN; ++b) {
            const int R = TBM + wn * WTN + b * 16 + lr;
            fw[b] = as_bf16x8(*reinterpret_cast<const uint4 *>(base + R * SK + 8 * (q ^ swz8(R))));
        }
#pragma unroll
        for (int b = 0; b < FM; ++b) {
            const int R = wm * WTM + b * 16 + lr;
            fa[b] = as_bf16x8(*reinterpret_cast<const uint4 *>(base + R * SK + 8 * (q ^ swz8(R))));
        }
    };

    f32x4_t acc[FM][FN];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
            acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    // this step's MFMAs with the next step's fragment reads between them (instruction
    // classes: 0x8 MFMA, 0x100 LDS read), so LDS latency hides under matrix work
    auto step = [&](const bf16x8_t (&fa)[FM], const bf16x8_t (&fw)[FN]) {
#pragma unroll
        for (int bm = 0; bm < FM; ++bm)
#pragma unroll
            for (int bn = 0; bn < FN; ++bn)
                acc[bm][bn] = mfma_16x16x32_bf16(fw[bn], fa[bm], acc[bm][bn]);
        constexpr int NR = FM + FN, MPR = FM * FN / NR;
#pragma unroll
        for (int i = 0; i < NR; ++i) {
            __builtin_amdgcn_sched_group_barrier(0x008, MPR, 0);
            __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        }
        __builtin_amdgcn_sched_group_barrier(0x008, FM * FN - NR * MPR, 0);
    };

    const int ns = K / SK;  // an empty K range leaves acc at zero
    bf16x8_t fa0[FM], fw0[FN], fa1[FM], fw1[FN];
    // stages 0 .. P-1 up front; stage 0 must land before the first fragment read
#pragma unroll
    for (int st = 0; st < P; ++st)
        if (st < ns)
            issue(st, st);
    if (ns >= P)
        wait_loads_and_barrier<(P - 1) * LPW>();
    else
        wait_loads_and_barrier<0>();
    if (ns > 0)
        read_frags(0, 0, fa0, fw0);
    // stage s in buffer s % P.  In the steady state (stage s+P exists) stages up to
    // s+P-1 have been issued when stage s waits for s+1, so P-2 stages may still be in
    // flight; the last P stages wait for everything.
    auto stage = [&](int s, int buf, bool more, bool refill, bool all) {
        read_frags(buf, 1, fa1, fw1);
        step(fa0, fw0);
        if (more) {
            if (all)
                wait_loads_and_barrier<0>();
            else
                wait_loads_and_barrier<(P - 2) * LPW>();
            if (refill)
                issue(s + P, buf);
            read_frags(buf + 1 == P ? 0 : buf + 1, 0, fa0, fw0);
        }
        step(fa1, fw1);
    };
    // The buffer index stays a run-time value: with constant buffers the compiler's
    // own LDS-DMA tracking adds a wait for the loads just issued before each fragment
    // read, which serialises the pipeline.  The waits above already order every read
    // after the loads it depends on.
    int s = 0, buf = 0;
    for (; s + P < ns; ++s) {
        stage(s, buf, true, true, false);
        buf = buf + 1 == P ? 0 : buf + 1;
    }
    for (; s < ns; ++s) {
        stage(s, buf, s + 1 < ns, false, true);
        buf = buf + 1 == P ? 0 : buf + 1;
    }

#pragma unroll
    for (int bm = 0; bm < FM; ++bm) {
        const int m = m0 + wm * WTM + bm * 16 + lr;
        if (m >= M)
            continue;
#pragma unroll
        for (int bn = 0; bn < FN; ++bn) {
            const int n = n0 + wn * WTN + bn * 16 + 4 * lq;
            if (n >= N)
                continue;
            const f32x4_t v = acc[bm][bn];
            if constexpr (OUT_BF16) {
                uint2 o;
                o.x = pack_bf16x2(v[0], v[1]);
                o.y = pack_bf16x2(v[2], v[3]);
                *reinterpret_cast<uint2 *>(reinterpret_cast<uint16_t *>(C) + (int64_t)m * ldc + n) = o;
            } else {
                *reinterpret_cast<float4 *>(reinterpret_cast<float *>(C) + (int64_t)m * ldc + n) =
                    make_float4(v[0], v[1], v[2], v[3]);
            }
        }
    }
}

// mm_pipe64_kernel serves a launch when every K range is whole 64-k stages and every
// operand byte it reads lies within 4 GiB of its operand's base (32-bit lane offsets)
bool pipe64_fits(const MatmulArgs &a, int splits, int64_t k_split)
{
    const int64_t kr = splits == 1 ? a.K : k_split;
    if (a.K % SK != 0 || kr % SK != 0)
        return false;
    const int64_t lim = (int64_t)1 << 32;
    return ((a.M - 1) * a.lda + kr) * 2 < lim && ((a.N - 1) * a.ldw + kr) * 2 < lim;
}

template <int TBM, int TBN, int WM, int WN, int P>
hipError_t launch_pipe64(const MatmulArgs &a, hipStream_t s, int splits, int64_t k_split,
                         int64_t c_split_stride)
{
    if (splits == 1)
        k_split = a.K;
    const int tiles_m = (int)((a.M + TBM - 1) / TBM), tiles_n = (int)((a.N + TBN - 1) / TBN);
    const size_t lds = (size_t)P * (TBM + TBN) * SK * sizeof(uint16_t);
    const void *fn = a.c_bf16 ? (const void *)mm_pipe64_kernel<TBM, TBN, WM, WN, P, true>
                              : (const void *)mm_pipe64_kernel<TBM, TBN, WM, WN, P, false>;
    hipError_t e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess)
        return e;
    const dim3 grid((unsigned)(tiles_m * tiles_n), (unsigned)splits), block(64 * WM * WN);
    if (a.c_bf16)
        mm_pipe64_kernel<TBM, TBN, WM, WN, P, true><<<grid, block, lds, s>>>(
            a.A, a.lda, a.W, a.ldw, a.C, a.ldc, (int)a.M, (int)a.N, (int)a.K, tiles_m, tiles_n,
            k_split, c_split_stride);
    else
        mm_pipe64_kernel<TBM, TBN, WM, WN, P, false><<<grid, block, lds, s>>>(
            a.A, a.lda, a.W, a.ldw, a.C, a.ldc, (int)a.M, (int)a.N, (int)a.K, tiles_m, tiles_n,
            k_split, c_split_stride);
    return hipGetLastError();
}

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

// One-wave weight-streaming tile for small M (K a multiple of 32): TBM batch rows x
// 16 features per wave, one wave per workgroup.  A single wave shares nothing through
// LDS, so the operand fragments go straight from global memory into a register ring
// of P steps: each lane loads exactly the 16 bytes it feeds to the MFMA (row lane % 16,
// k = 8 * (lane / 16) .. +7 of the step), P steps ahead of their use.  A step is then
// one MFMA per 16-row block and one load per operand, with no barrier and no LDS round
// trip.  Instruction, operand roles, k fragment mapping and the ascending step order
// are those of mm_tile_kernel and mm_pipe_kernel, so every element gets the same bits.
// Rows past M or N read a valid row whose results are never stored; the ring's refills
// past the last step re-read that step (in bounds) and are never used.
template <int TBM, int P, bool OUT_BF16>
__global__ __launch_bounds__(64) void mm_stream_kernel(
    const uint16_t *__restrict__ A, int64_t lda, const uint16_t *__restrict__ W, int64_t ldw,
    void *__restrict__ C, int64_t ldc, int M, int N, int K, int tiles_m, int tiles_n,
    int64_t k_split, int64_t c_split_stride)
{
    {  // split-K (blockIdx.y = range; the invariant path always has one range)
        const int64_t kb0 = (int64_t)blockIdx.y * k_split;
        A += kb0;
        W += kb0;
        K = (int)((K - kb0) < k_split ? (K - kb0) : k_split);
        C = reinterpret_cast<char *>(C) + (int64_t)blockIdx.y * c_split_stride;
    }
    constexpr int FM = TBM / 16;
    int tm, tn;
    tile_coords(blockIdx.x, tiles_m, tiles_n, BIG_GROUP_M, tm, tn);
    const int m0 = tm * TBM, n0 = tn * 16;
    const int lane = threadIdx.x & 63, lr = lane & 15, lq = lane >> 4;

    const uint16_t *wp = W + (int64_t)min(n0 + lr, N - 1) * ldw + 8 * lq;
    const uint16_t *ap[FM];
#pragma unroll
    for (int b = 0; b < FM; ++b)
        ap[b] = A + (int64_t)min(m0 + b * 16 + lr, M - 1) * lda + 8 * lq;

    const int nk = K / PK;
    uint4 rw[P], ra[P][FM];
    auto load = [&](int slot, int step) {
        const int st = min(step, nk - 1);
        rw[slot] = *reinterpret_cast<const uint4 *>(wp + (int64_t)st * PK);
#pragma unroll
        for (int b = 0; b < FM; ++b)
            ra[slot][b] = *reinterpret_cast<const uint4 *>(ap[b] + (int64_t)st * PK);
    };
    f32x4_t acc[FM];
#pragma unroll
    for (int b = 0; b < FM; ++b)
        acc[b] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    auto step = [&](int slot) {
#pragma unroll
        for (int b = 0; b < FM; ++b)
            acc[b] = mfma_16x16x32_bf16(as_bf16x8(rw[slot]), as_bf16x8(ra[slot][b]), acc[b]);
    };
#pragma unroll
    for (int j = 0; j < P; ++j)
        load(j, j);
    // Steady rounds are branch free, so the compiler's load-counter waits stay exact
    // (each step waits only for its own slot); the last partial round has no refills.
    int kt = 0;
    for (; kt + P <= nk; kt += P) {
#pragma unroll
        for (int j = 0; j < P; ++j) {
            step(j);
            load(j, kt + j + P);
        }
        // keep each refill right behind the MFMAs that free its slot (instruction
        // classes: 0x8 MFMA, 0x20 global load), rather than batched at the round's end
#pragma unroll
        for (int j = 0; j < P; ++j) {
            __builtin_amdgcn_sched_group_barrier(0x008, FM, 0);
            __builtin_amdgcn_sched_group_barrier(0x020, 1 + FM, 0);
        }
    }
#pragma unroll
    for (int j = 0; j < P; ++j)
        if (kt + j < nk)
            step(j);

    // lane holds batch row m = lane % 16 of each block and features n = 4*(lane/16) + j
    const int n = n0 + 4 * lq;
    if (n >= N)
        return;
#pragma unroll
    for (int b = 0; b < FM; ++b) {
        const int m = m0 + b * 16 + lr;
        if (m >= M)
            continue;
        const f32x4_t v = acc[b];
        if constexpr (OUT_BF16) {
            uint2 o;
            o.x = pack_bf16x2(v[0], v[1]);
            o.y = pack_bf16x2(v[2], v[3]);
            *reinterpret_cast<uint2 *>(reinterpret_cast<uint16_t *>(C) + (int64_t)m * ldc + n) = o;
        } else {
            *reinterpret_cast<float4 *>(reinterpret_cast<float *>(C) + (int64_t)m * ldc + n) =
                make_float4(v[0], v[1], v[2], v[3]);
        }
    }
}

template <int TBM, int P>
hipError_t launch_stream(const MatmulArgs &a, hipStream_t s, int splits = 1, int64_t k_split = 0,
                         int64_t c_split_stride = 0)
{
    if (splits == 1)
        k_split = a.K;
    const int tiles_m = (int)((a.M + TBM - 1) / TBM), tiles_n = (int)((a.N + 15) / 16);
    const dim3 grid((unsigned)(tiles_m * tiles_n), (unsigned)splits), block(64);
    if (a.c_bf16)
        mm_stream_kernel<TBM, P, true><<<grid, block, 0, s>>>(
            a.A, a.lda, a.W, a.ldw, a.C, a.ldc, (int)a.M, (int)a.N, (int)a.K, tiles_m, tiles_n,
            k_split, c_split_stride);
    else
        mm_stream_kernel<TBM, P, false><<<grid, block, 0, s>>>(
            a.A, a.lda, a.W, a.ldw, a.C, a.ldc, (int)a.M, (int)a.N, (int)a.K, tiles_m, tiles_n,
            k_split, c_split_stride);
    return hipGetLastError();
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

// Pipelined tile shapes and their measured throughput per unit of tile area (the
// fraction of MFMA peak one full round of 256 workgroups reached on MI355X).
struct TileCand {
    int tbm, tbn;
    double eff;
};
constexpr TileCand kTiles[] = {{256, 256, 0.56}, {256, 128, 0.42}, {128, 128, 0.39},
                               {128, 64, 0.20},  {64, 64, 0.15},   {64, 32, 0.10},
                               {16, 16, 0.0},    {32, 16, 0.0},    {16, 16, 0.0},
                               {32, 32, 0.0}};
constexpr int kNumTiles = 6;  // priced by the cost model; the rest are weight-streaming
                              // tiles for small M (rule below): 16 x 16 and 32 x 16
                              // through LDS, 16 x 16 in registers, two-wave 32 x 32

// (rounds of 256 workgroups) x (tile area) / (throughput per unit area)
double tile_cost(int i, int64_t M, int64_t N)
{
    const TileCand &c = kTiles[i];
    const int64_t tiles = ((M + c.tbm - 1) / c.tbm) * ((N + c.tbn - 1) / c.tbn);
    return (double)((tiles + 255) / 256) * c.tbm * c.tbn / c.eff;
}

int best_tile(int64_t M, int64_t N, double *cost)
{
    // Small M is a weight stream: one-wave 16-row tiles give every compute unit
    // several independent streams.  Measured on MI355X (decode-layer weights):
    //  * at most one 16 x 16 tile per compute unit (N <= 4096): a wave's stream is
    //    latency bound, and the register-streaming kernel, free of the LDS round
    //    trip and barrier of every step, is faster up to M = 16 (o_proj M = 1:
    //    20.6 -> 14.0 us, down projection 28.4 -> 18.7 us); with more tiles per
    //    unit the LDS kernels are as fast or faster (QKV M = 1: 16.9 vs 18.7 us);
    //  * from M = 33 with N <= 4096, two-wave 32 x 32 tiles (o_proj M = 48:
    //    31.2 -> 23.7 us, down projection M = 48: 52.2 -> 35.2 us; M = 64: 28.6 ->
    //    24.7 and 49.2 -> 39.8 us): twice the workgroups of the 64-row tiles, more
    //    rows per wave than 16 x 16;
    //  * otherwise 16 x 16 through LDS while there are at most 1024 of them, and
    //    for vocabulary-sized N up to M = 8 (lm_head M = 1: 217.9 -> 204.8 us);
    //  * else 32 x 16 up to M = 32.
    if (M <= 64) {
        const int64_t t16 = ((M + 15) / 16) * ((N + 15) / 16);
        if (M <= 16 && t16 <= 256) {
            *cost = 0;
            return 8;
        }
        if (M > 32 && N <= 4096) {
            *cost = 0;
            return 9;
        }
        if (t16 <= 1024 || (M <= 8 && t16 > 2048)) {
            *cost = 0;
            return 6;
        }
        if (M <= 32) {
            *cost = 0;
            return 7;
        }
    }
    int best = 0;
    double bc = tile_cost(0, M, N);
    for (int i = 1; i < kNumTiles; ++i) {
        const double c = tile_cost(i, M, N);
        if (c < bc) {
            best = i;
            bc = c;
        }
    }
    // With N <= 4096 (the long-K o_proj and down projection shapes), a single
    // partial round of 256 x 128 tiles is slower than one round of 128 x 128 tiles,
    // which the per-round pricing above does not see (graph-replayed, o_proj M =
    // 1024: 103.6 -> 75.6 us; down projection: 175.0 -> 122.8 us).  From 1.5 rounds
    // of 128 x 128 tiles on, the 256 x 128 round is the faster (o_proj M = 1536: 128.6
    // vs 106.1 us; down: 215.8 vs 176.2 us), and with a full round (M = 2048) or a
    // wide N (QKV, gate/up) the priced choice stands.
    if (best == 1 && N <= 4096) {
        const int64_t t1 = ((M + 255) / 256) * ((N + 127) / 128);
        const int64_t t2 = ((M + 127) / 128) * ((N + 127) / 128);
        if (t1 < 256 && t2 <= 256) {
            *cost = tile_cost(2, M, N);
            return 2;
        }
    }
    *cost = bc;
    return best;
}

// An LDS-pipelined tile: P64 stages of 64 k when every K range is whole 64-k stages,
// else P32 stages of 32 k.  Both kernels give every element the same bits.
template <int TBM, int TBN, int WM, int WN, int P64, int P32>
hipError_t launch_lds_tile(const MatmulArgs &a, hipStream_t s, int splits, int64_t k_split,
                           int64_t c_split_stride)
{
    if (pipe64_fits(a, splits, k_split))
        return launch_pipe64<TBM, TBN, WM, WN, P64>(a, s, splits, k_split, c_split_stride);
    return launch_pipe<TBM, TBN, WM, WN, P32>(a, s, splits, k_split, c_split_stride);
}

hipError_t launch_tile_shape(int i, const MatmulArgs &a, hipStream_t s, int splits = 1,
                             int64_t k_split = 0, int64_t c_split_stride = 0)
{
    // Stage counts, measured with graph-replayed device time on the decode-layer
    // projection shapes at M = 16 .. 4096: the 64-k kernel keeps the 32-k kernel's LDS
    // budget except for the 128-row tiles, which need three 64-k stages (two left loads
    // too little MFMA work to arrive in: o_proj M = 512 on 128 x 64 tiles 48.7 us in
    // 32-k stages, 59.2 in two 64-k stages, 43.9 in three; down M = 1024 on 128 x 128
    // tiles 131.9 / 140.5 / 124.4 us).
    switch (i) {
    case 0: return launch_lds_tile<256, 256, 2, 4, 2, 4>(a, s, splits, k_split, c_split_stride);
    case 1: return launch_lds_tile<256, 128, 2, 2, 3, 6>(a, s, splits, k_split, c_split_stride);
    // 32-k stages: four, i.e. 64 or 48 KiB of LDS, two or three workgroups per compute
    // unit (measured as fast or faster than 8 and 12 stages at every M from 48 to 4096
    // on the decode-layer shapes, e.g. QKV M = 4096 as one 128 x 128 launch 427 -> 358
    // us)
    case 2: return launch_lds_tile<128, 128, 2, 2, 3, 4>(a, s, splits, k_split, c_split_stride);
    case 3: return launch_lds_tile<128, 64, 2, 2, 3, 4>(a, s, splits, k_split, c_split_stride);
    case 4: return launch_lds_tile<64, 64, 2, 2, 4, 8>(a, s, splits, k_split, c_split_stride);
    case 5: return launch_lds_tile<64, 32, 2, 1, 8, 16>(a, s, splits, k_split, c_split_stride);
    case 6: return launch_lds_tile<16, 16, 1, 1, 8, 16>(a, s, splits, k_split, c_split_stride);
    case 7: return launch_lds_tile<32, 16, 1, 1, 8, 16>(a, s, splits, k_split, c_split_stride);
    case 8: return launch_stream<16, 12>(a, s, splits, k_split, c_split_stride);
    default: return launch_lds_tile<32, 32, 2, 1, 8, 16>(a, s, splits, k_split, c_split_stride);
    }
}

MatmulPlan plan_matmul_bi(int64_t M, int64_t N, int64_t K)
{
    // The tile shape is picked from the problem size; that changes which wave
    // computes an element, never the element's arithmetic.  Big tiles are efficient
    // once there are enough of them, small tiles keep all 256 compute units
    // streaming weights when M is small.  When the best single shape would leave a
    // last round of workgroups mostly empty, the columns are cut in two: the first
    // N1 columns in full rounds of a big tile, the rest with the shape that suits
    // them, as two launches on the same stream.
    MatmulPlan p{-1, N, -1};
    if (K % PK != 0)
        return p;  // the register-staged 128 x 128 tile kernel
    double c1;
    const int t1 = best_tile(M, N, &c1);
    if (t1 <= 1) {
        // a partly filled last round of big tiles runs faster than a full one
        // (less contention); price it at sqrt(fill) of a round for this choice
        const TileCand &c = kTiles[t1];
        const int64_t tiles = ((M + c.tbm - 1) / c.tbm) * ((N + c.tbn - 1) / c.tbn);
        const int64_t full = tiles / 256, rem = tiles % 256;
        c1 = ((double)full + (rem ? std::sqrt(rem / 256.0) : 0.0)) * c.tbm * c.tbn / c.eff;
    }
    p.t1 = t1;
    double best = c1;
    for (int i = 0; i < 2; ++i) {  // the big shapes as the first part
        const int64_t tbn = kTiles[i].tbn;
        for (int64_t n1 = (N / tbn) * tbn; n1 >= tbn && n1 * 2 >= N; n1 -= tbn) {
            if (n1 == N)
                continue;
            double c2;
            const int r = best_tile(M, N - n1, &c2);
            if (r >= kNumTiles)
                continue;  // small-M tiles are not priced; keep one launch
            const double c = tile_cost(i, M, n1) + c2;
            if (c < best * 0.95) {  // a clear win only: two launches cost a little
                best = c;
                p = MatmulPlan{i, n1, r};
            }
        }
    }
    return p;
}

void describe_matmul_plan(const MatmulPlan &p, int64_t out[7])
{
    // tile rows, tile columns and kind (0 LDS-pipelined, 1 register streaming,
    // 2 register-staged for K % 32 != 0) of each launch, and the first launch's
    // column count
    auto put = [&](int t, int64_t *o) {
        if (t < 0) {
            o[0] = BM, o[1] = BN, o[2] = 2;
        } else {
            o[0] = kTiles[t].tbm, o[1] = kTiles[t].tbn, o[2] = t == 8 ? 1 : 0;
        }
    };
    put(p.t1, out);
    out[3] = p.n1;
    if (p.t2 >= 0) {
        put(p.t2, out + 4);
    } else {
        out[4] = out[5] = out[6] = 0;
    }
}

hipError_t launch_matmul_bi(const MatmulArgs &a, hipStream_t s)
{
    const MatmulPlan p = plan_matmul_bi(a.M, a.N, a.K);
    if (p.t1 < 0)
        return launch_tiles(a, 1, a.K, a.C, a.ldc, a.c_bf16, 0, s);
    if (p.t2 < 0)
        return launch_tile_shape(p.t1, a, s);
    MatmulArgs left = a, right = a;
    left.N = p.n1;
    right.N = a.N - p.n1;
    right.W = a.W + p.n1 * a.ldw;
    right.C = a.c_bf16 ? (void *)((uint16_t *)a.C + p.n1) : (void *)((float *)a.C + p.n1);
    hipError_t e = launch_tile_shape(p.t1, left, s);
    if (e != hipSuccess)
        return e;
    return launch_tile_shape(p.t2, right, s);
}

// The twin's schedule: a tile shape and a split-K count, picked from (M, N, K) by a
// table measured on MI355X (graph-replayed device time on the decode layer's
// projection shapes, every pipelined tile shape x 2 and 4 equal K ranges, M = 9 ..
// 1024): wherever a split beat matmul_bi's own plan by a clear margin it is taken,
// and everywhere else the twin runs matmul_bi's plan unchanged.  Winning splits:
//  * long K with few output columns (N <= 4096, K >= 8192: o_proj, the down
//    projection) from M = 9: 16 x 16 tiles in 2 ranges up to M = 16, 32 x 32 in 2
//    up to 32, 64 x 64 in 4 up to 64, 128 x 64 in 4 up to 160 and in 2 up to 256
//    (o_proj M = 16: 16.7 -> 14.8 us; M = 64: 19.9 -> 16.3; M = 127: 26.1 -> 19.0;
//    M = 256: 29.6 -> 26.6; down M = 127: 43.1 -> 27.9; M = 256: 49.9 -> 41.7).
//    Beyond M = 256 only the longest K gains: with K >= 12288, 256 x 128 tiles in 4
//    ranges up to M = 512 and 256 x 256 in 4 up to 768 (down M = 509: 72.7 ->
//    65.5 us; M = 768: 110.3 -> 91.8); o_proj there runs bi's plan (M = 384: 38.6
//    us, no split under 38.7);
//  * QKV-wide N (8192 < N <= 12288, K <= 4096) at 129 <= M <= 192: 64 x 64 tiles in
//    2 ranges (M = 160: 35.4 -> 29.0 us; M = 192: 35.6 -> 30.8);
//  * very wide N (N >= 16384: gate/up) up to M = 32: 64 x 64 tiles in 2 ranges
//    (M = 16: 42.8 -> 37.0 us; M = 32: 44.6 -> 38.8).
// The partition is a function of M, so the bits move with M.  With K % 32 != 0 the
// 128 x 128 register-staged kernel splits K until its tiles fill the chip.
TwinPlan plan_matmul_tuned(int64_t M, int64_t N, int64_t K)
{
    if (K % PK != 0) {
        const int64_t tiles = ((M + BM - 1) / BM) * ((N + BN - 1) / BN);
        int splits = 1;
        while (splits < 16 && tiles * splits < 256 && K / (splits * 2) >= 256)
            splits *= 2;
        return TwinPlan{-1, splits};
    }
    if (N <= 4096 && K >= 8192 && M > 8) {
        if (M <= 16)
            return TwinPlan{6, 2};   // 16 x 16
        if (M <= 32)
            return TwinPlan{9, 2};   // 32 x 32
        if (M <= 64)
            return TwinPlan{4, 4};   // 64 x 64
        if (M <= 160)
            return TwinPlan{3, 4};   // 128 x 64
        if (M <= 256)
            return TwinPlan{3, 2};
        if (K >= 12288 && M <= 512)
            return TwinPlan{1, 4};   // 256 x 128
        if (K >= 12288 && M <= 768)
            return TwinPlan{0, 4};   // 256 x 256
    }
    if (N > 8192 && N <= 12288 && K <= 4096 && M > 128 && M <= 192)
        return TwinPlan{4, 2};
    if (N >= 16384 && K <= 4096 && M <= 32)
        return TwinPlan{4, 2};
    return TwinPlan{-1, 1};  // matmul_bi's plan
}

int matmul_tuned_splits(int64_t M, int64_t N, int64_t K)
{
    return plan_matmul_tuned(M, N, K).split;
}

hipError_t launch_matmul_splitk(const MatmulArgs &a, int splits, float *ws, hipStream_t s)
{
    if (splits <= 1)
        return launch_matmul_bi(a, s);
    // equal ranges, each a multiple of the kernel's k step
    const int64_t step = (a.K % PK == 0) ? PK : BK;
    int64_t k_split = (a.K + splits - 1) / splits;
    k_split = (k_split + step - 1) / step * step;
    splits = (int)((a.K + k_split - 1) / k_split);
    hipError_t e;
    if (a.K % PK == 0) {
        double c;
        const int pt = plan_matmul_tuned(a.M, a.N, a.K).tile;
        const int t = pt >= 0 ? pt : best_tile(a.M, a.N, &c);
        MatmulArgs w = a;
        w.C = ws;
        w.ldc = a.N;
        w.c_bf16 = false;
        e = launch_tile_shape(t, w, s, splits, k_split, a.M * a.N * 4);
    } else {
        e = launch_tiles(a, splits, k_split, ws, a.N, false, a.M * a.N * 4, s);
    }
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
