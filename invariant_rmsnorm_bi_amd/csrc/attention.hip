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
// Kernel 1 (a workgroup of 8 waves per run of consecutive splits of one (row,
// kv head), for split sizes up to 256 tokens: a group of GROUP = 4 splits, or,
// for large batches, a whole row or a chunk of whole groups of it, taken longest
// first from a plan that a one-workgroup kernel builds from the lengths):
//   * each split's 16-token pages are dealt to the waves in pairs (wave w takes
//     pages 2w and 2w+1), each pair loaded in one burst; the next split's pair is
//     requested as soon as the current one's update is done;
//   * scores S^T[token][head] = K . q^T with v_mfma_f32_16x16x32_bf16 (K rows are
//     operand A, the group's query heads operand B; head_dim is the k dimension,
//     lane group q = lane/16 carrying d = q*D/4 + 8c .. +7 in step c);
//   * log2-domain softmax in fp32: s2 = score * (scale * log2 e), masked to -inf
//     past the split end; per wave a running max m and, per lane, a running sum
//     of p = 2^(s2 - m) as the product sees it: p is split into two bf16 parts,
//     hi = bf16(p) and lo = bf16(p - hi), so it keeps 16 significant bits;
//   * acc^T[d][head] += V^T . HI + V^T . LO with the same MFMA (V operand A, P
//     operand B; two MFMAs into one accumulator), so a lane holds four consecutive
//     d of its own head, the head of its scores.  V pages
//     are stored head-dim-major ([d][token]), so one 16-byte load of a V page row is
//     exactly the operand fragment (8 consecutive tokens at one d): no staging;
//   * the eight waves' (m, l, acc) are combined in wave order 0 .. 7
//     (M = max m, l = sum 2^(m_w - M) l_w, acc = sum 2^(m_w - M) acc_w) into the
//     split's partial, and the group's splits are folded in ascending order (the
//     fold below); the group's partial goes to the fp32 workspace -- unless the
//     workgroup holds the whole row, which folds its groups in ascending order
//     itself, exactly as kernel 2 would, and writes the output.
//   Longer splits (up to 1024 tokens): one workgroup per (row, kv head, split),
//   each wave walking several pairs; a group is then one split.
// Kernel 2 (one wave per (row, query head)): the same ascending fold over the
//   row's group partials, then out = bf16(acc / l), for every row not written
//   whole by kernel 1 (even one with a single group).  The whole reduction tree
//   -- pairs, waves, splits, groups -- is a function of L alone; which workgroup
//   computes which part of it is the only thing the batch decides.
// No atomics in any reduction (the plan's LDS atomics only order the work).
//
// The twin (decode_attn_tuned) runs the same kernels with a split size picked
// from the batch shape, which moves the split boundaries with the batch.
#include <atomic>
#include <type_traits>

#include "device.h"
#include "launch.h"

namespace rbi {
namespace {

constexpr int PAGE = 16;
constexpr int WAVES = 8;   // waves per split workgroup
// Splits per workgroup (and per workspace partial) for split sizes up to
// 2 * PAGE * WAVES tokens.  Measured at the bench shape (batch 256, 64q/4kv, d128,
// lengths U{1..32768}, split 256): one split per workgroup with its partial stored
// 1.95 ms; groups of 4 at one workgroup per compute unit 1.80 ms (groups of 2:
// 1.92, of 8: 1.85), with the next split's loads behind the current split's
// pair update.  A workgroup's partial store costs far more than its bytes: the
// same kernel with its stores removed ran 1.43 instead of 1.82 ms.
constexpr int GROUP = 4;

// Splits folded into one workspace partial: GROUP for splits of at most one page
// pair per wave, else 1.  A function of the split size alone.
constexpr int splits_per_partial(int split)
{
    return split <= 2 * PAGE * WAVES ? GROUP : 1;
}
// Row padding of the LDS stash of the waves' accumulators, in floats: lane l of a
// wave writes its head l % 16 at d = 16 * db + 4 * (l / 16) .. +3 (16 bytes), so
// with rows of D + 4 floats the heads of eight consecutive lanes start 16 bytes
// apart modulo 128 and a write is free of bank conflicts.
constexpr int CPAD = 4;
// Row length of the LDS query tile, in bf16: a score MFMA reads 16 bytes of head
// row lane % 16 per lane, so rows of D elements (a multiple of 256 bytes) put the
// 16 lanes of a lane group on the same banks; 8 more elements shift each row by
// four banks and make the read conflict free.
template <int D>
constexpr int QROW = D + 8;

// Workspace of split partials.  For each (row, kv head, split) one block holds the
// G query heads' partials, IST = D + 4 floats each: acc[0 .. D), then m, l and two
// zero pads.  A split workgroup writes its block as one contiguous run of whole
// 128-byte lines (the block is G * IST * 4 bytes, a multiple of 128 for G a multiple
// of 8 at D 128).  Writing each head's acc and its (m, l) pair to separate arrays
// instead -- 512-byte and 8-byte pieces scattered over the workspace -- cost 22 %
// of the call at the bench shape (measured without the stores: 2.01 -> 1.56 ms).
template <int D>
constexpr int IST = D + 4;

__device__ __forceinline__ int64_t part_off(int64_t r, int g, int s, int hh, int hkv, int nsmax,
                                            int G, int ist)
{
    return (((r * hkv + g) * (int64_t)nsmax + s) * G + hh) * (int64_t)ist;
}

template <int D>
struct AttnK {
    static constexpr int KCH = D / 32;      // 16-byte chunks per lane per token row
    static constexpr int DPL = D / 4;       // head_dim elements per lane group
    static constexpr int DB = D / 16;       // 16-wide d blocks of the PV product
};

// 2^x on the transcendental unit (v_exp_f32).  Results below the normal range
// may flush to zero; every use here is a softmax weight or a rescaling factor,
// where that is immaterial, and all attention paths share this one function.
__device__ __forceinline__ float exp2_hw(float x)
{
    return __builtin_amdgcn_exp2f(x);
}

typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

// Two fp32 values to packed bf16 (lo in bits 0..15), round to nearest even, by
// the conversion instruction.
__device__ __forceinline__ uint32_t cvt_pk_bf16(float lo, float hi)
{
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2_t{lo, hi}, bf16x2_t));
}

__device__ __forceinline__ int clamp_len(int L, int max_len)
{
    return L < 1 ? 1 : (L > max_len ? max_len : L);
}



// ---------------------------------------------------------------------------
// The per-(token, query head) arithmetic, shared by the decode and the prefill
// kernels so that a prompt token's result is the same bits as the decode row
// with the same query, cache and length.
// ---------------------------------------------------------------------------

// Register image of one page pair (32 tokens) of one kv head: K as operand A of
// the score product, V as operand B of the P.V product.
template <int D>
struct PairFrag {
    uint4 k[2][AttnK<D>::KCH];
    uint4 v[AttnK<D>::DB];
};

// Lane roles inside a wave (fixed):
//   * lane group lg = lane / 16 owns the 8-token run lg of the pair: page slot
//     lg / 2, in-page tokens 8 * (lg % 2) .. +7 -- its scores, P values and V loads;
//   * score block b (one MFMA, b = 0, 1) has K row i = in-page token
//     8 * ((i / 4) % 2) + 4b + i % 4 of slot i / 8, so output rows 4 * lg + j land
//     in lane group lg as token 4b + j of its run;
//   * the P.V k-step then takes each lane group's run: the lane's P values in
//     token order, and one 16-byte run of the head-dim-major V page per d.
struct PairLanes {
    int lane;
    __device__ __forceinline__ explicit PairLanes(int l) : lane(l) {}
    __device__ __forceinline__ int lr() const { return lane & 15; }
    __device__ __forceinline__ int lg() const { return lane >> 4; }
    __device__ __forceinline__ int kslot() const { return (lane & 15) >> 3; }     // K row's page slot
    __device__ __forceinline__ int krow() const { return 8 * ((lane >> 2) & 1) + (lane & 3); }
    __device__ __forceinline__ int vslot() const { return lane >> 5; }           // run's page slot
    __device__ __forceinline__ int vrun() const { return 8 * ((lane >> 4) & 1); }  // run's first token
};

// Loads page pair pr of a split whose first valid_pages pages have their
// physical ids in lanes 0 .. of my_page.  A page slot past the last valid page
// reads that page again (masked later), so no load is conditional.
template <int D>
__device__ __forceinline__ void load_pair(PairFrag<D> &f, int pr, int my_page, int valid_pages,
                                          const uint16_t *__restrict__ k_cache,
                                          const uint16_t *__restrict__ v_cache, int hkv, int g,
                                          const PairLanes &ln)
{
    using P = AttnK<D>;
    const int64_t kphys = __shfl(my_page, min(2 * pr + ln.kslot(), valid_pages - 1), kWave);
    const int64_t vphys = __shfl(my_page, min(2 * pr + ln.vslot(), valid_pages - 1), kWave);
    const uint16_t *kp = k_cache + ((kphys * hkv + g) * PAGE + ln.krow()) * D + ln.lg() * P::DPL;
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
        for (int cc = 0; cc < P::KCH; ++cc)
            f.k[b][cc] = *reinterpret_cast<const uint4 *>(kp + 4 * b * D + 8 * cc);
    const uint16_t *vp = v_cache + ((vphys * hkv + g) * D + ln.lr()) * PAGE + ln.vrun();
#pragma unroll
    for (int db = 0; db < P::DB; ++db)
        f.v[db] = *reinterpret_cast<const uint4 *>(vp + 16 * db * PAGE);
}

// Workgroups go to the eight XCDs round robin by linear id, which for a grid of
// (X, 1, rows) with X a multiple of 8 is x % 8.  A row's live workgroups are a
// prefix of its x range (its splits or groups, kv heads innermost), so with an
// unrotated x every row's prefix starts on XCD 0 and the XCDs at the start of the
// rotation get the rows' odd remainders: with 17 groups of 4 kv heads per row,
// XCDs 0..3 would take 9 of every 17 x 4 workgroups and XCDs 4..7 only 8.  Row r
// starts its prefix (r * hkv) mod 8 positions further round, which spreads the
// remainders evenly; the map is a bijection on [0, X) and only decides which
// workgroup computes a (split or group, kv head), never its arithmetic.
__device__ __forceinline__ int xcd_rotated_x(int hkv)
{
    const unsigned X = gridDim.x;
    const unsigned rot = ((unsigned)blockIdx.z * (unsigned)hkv) & 7u;
    return (int)((blockIdx.x + X - rot % X) % X);
}

// Live tokens of this lane group's run in page pair pr of the split [t0, t1)
// (valid_pages = ceil((t1 - t0) / PAGE)).
__device__ __forceinline__ int run_keep(int pr, int t0, int t1, int valid_pages,
                                        const PairLanes &ln)
{
    const int first = t0 + (2 * pr + ln.vslot()) * PAGE + ln.vrun();
    return (2 * pr + ln.vslot() < valid_pages) ? max(0, min(8, t1 - first)) : 0;
}

// V entries of tokens past `keep` in this lane group's run, set to exact zeros
// (their weights are 0, but a stale non-finite value times 0 would not be 0).
template <int D>
__device__ __forceinline__ void mask_runs(const uint4 (&src)[AttnK<D>::DB], int keep,
                                          uint4 (&dst)[AttnK<D>::DB])
{
    uint32_t vmask[4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
        vmask[i] = (2 * i < keep ? 0x0000ffffu : 0u) | (2 * i + 1 < keep ? 0xffff0000u : 0u);
#pragma unroll
    for (int db = 0; db < AttnK<D>::DB; ++db)
        dst[db] = make_uint4(src[db].x & vmask[0], src[db].y & vmask[1], src[db].z & vmask[2],
                             src[db].w & vmask[3]);
}

// The maximum of x over the four 16-lane rows of a wave, in the butterfly order
// (lane i with i ^ 16, then with i ^ 32); every lane ends with the same value.  LANES: the partner values come from
// v_permlane16_swap / v_permlane32_swap, which exchange the odd 16-lane rows of
// one operand with the even rows of the other (the upper 32 lanes of one with
// the lower 32 of the other), so with x in both operands a lane gets its own
// value in one result and its partner's in the other -- no LDS round trip.
// Otherwise the partner values come from LDS lane permutes (__shfl_xor).
template <bool LANES>
__device__ __forceinline__ float rows_max(float x)
{
    if constexpr (LANES) {
        const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x),
                                                        false, false);
        x = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
        const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x),
                                                        false, false);
        return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
    } else {
        x = fmaxf(x, __shfl_xor(x, 16, kWave));
        return fmaxf(x, __shfl_xor(x, 32, kWave));
    }
}

// One page pair folded into the wave's running (m, l, acc) for the 16 query rows
// whose fragments qfrag(cc) gives (head lr, d = lg * DPL + 8 * cc ..), with K from
// k and V from v (already masked by mask_runs unless the pair is full).  Tokens
// past `keep` in a run get weight 0.
//   scores  s2 = (K . q) * scale * log2(e), fp32, -inf when masked
//   m_new   = max(m_run, max_j s2_j)           (per head, over the 32 tokens)
//   e_j     = 2^(s2_j - m_new),  p_j = hi_j + lo_j with hi_j = bf16(e_j),
//             lo_j = bf16(e_j - hi_j)
//   l_run   = fma(l_run, 2^(m_run - m_new), HI . 1 + LO . 1)  (the pair's sum of p_j
//             per head, on MFMA against an operand of ones; the same in every lane)
//   acc     = acc * 2^(m_run - m_new) + HI . V + LO . V  (bf16 MFMA, fp32 accumulate)
// In two parts: pair_scores (s2 and the pair's maximum) and pair_pv (the rest).
// FRESH: the state is the initial (-inf, 0, 0), for which the rescaling is the
// identity on zeros and is skipped (same bits).  full: every token of the pair
// is live (keep = 8 in every run), so the score mask is all-pass and skipped.
template <int D, bool LANES = false, typename QFrag>
__device__ __forceinline__ float pair_scores(const uint4 (&k)[2][AttnK<D>::KCH], int keep,
                                             bool full, const QFrag &qfrag, float scale_log2,
                                             float (&sv)[2][4])
{
    using P = AttnK<D>;
    // scores: lane holds head lr, token 4b + j of its run
    float mloc = -INFINITY;
#pragma unroll
    for (int b = 0; b < 2; ++b) {
        f32x4_t sc = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int cc = 0; cc < P::KCH; ++cc)
            sc = mfma_16x16x32_bf16(as_bf16x8(k[b][cc]), qfrag(cc), sc);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const float v = (full || 4 * b + j < keep) ? sc[j] * scale_log2 : -INFINITY;
            sv[b][j] = v;
            mloc = fmaxf(mloc, v);
        }
    }
    return rows_max<LANES>(mloc);
}

// pair_scores for NP fully live pairs at once (keep = 8, full): the same MFMA chain
// per (pair, score block) and the same scaling, with the pairs' chains interleaved
// so that consecutive MFMAs are independent.
template <int D, int NP, typename QFrag>
__device__ __forceinline__ void full_pairs_scores(const uint4 (&k)[NP][2][AttnK<D>::KCH],
                                                  const QFrag &qfrag, float scale_log2,
                                                  float (&sv)[NP][2][4], float (&mloc)[NP])
{
    using P = AttnK<D>;
    f32x4_t sc[NP][2];
#pragma unroll
    for (int i = 0; i < NP; ++i)
#pragma unroll
        for (int b = 0; b < 2; ++b)
            sc[i][b] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int cc = 0; cc < P::KCH; ++cc) {
        const bf16x8_t qf = qfrag(cc);
#pragma unroll
        for (int i = 0; i < NP; ++i)
#pragma unroll
            for (int b = 0; b < 2; ++b)
                sc[i][b] = mfma_16x16x32_bf16(as_bf16x8(k[i][b][cc]), qf, sc[i][b]);
    }
#pragma unroll
    for (int i = 0; i < NP; ++i) {
        float m = -INFINITY;
#pragma unroll
        for (int b = 0; b < 2; ++b)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                sv[i][b][j] = sc[i][b][j] * scale_log2;
                m = fmaxf(m, sv[i][b][j]);
            }
        mloc[i] = rows_max<true>(m);
    }
}

template <int D, bool FRESH>
__device__ __forceinline__ void pair_pv(const float (&sv)[2][4], float mloc,
                                        const uint4 (&v)[AttnK<D>::DB], float &m_run,
                                        float &l_run, f32x4_t (&acc)[AttnK<D>::DB])
{
    using P = AttnK<D>;
    const float m_new = FRESH ? mloc : fmaxf(m_run, mloc);
    const float m_use = (m_new == -INFINITY) ? 0.f : m_new;

    // p enters the bf16 P.V product as two bf16 parts, p_hi = bf16(p) and
    // p_lo = bf16(p - p_hi) (two MFMAs into one accumulator), so the weights carry
    // 16 significant bits instead of 8; l sums the same two parts, by the same two
    // MFMAs against a V of ones, so every lane gets its head's sum over the pair's
    // 32 tokens without a lane exchange.
    uint32_t pw[2][2], pl[2][2];  // bf16 p_hi / p_lo, two per word, token order in the run
#pragma unroll
    for (int b = 0; b < 2; ++b) {
#pragma unroll
        for (int j = 0; j < 4; j += 2) {
            const float e0 = exp2_hw(sv[b][j] - m_use), e1 = exp2_hw(sv[b][j + 1] - m_use);
            const uint32_t w = cvt_pk_bf16(e0, e1);
            const float h0 = __uint_as_float(w << 16), h1 = __uint_as_float(w & 0xffff0000u);
            pw[b][j / 2] = w;
            pl[b][j / 2] = cvt_pk_bf16(e0 - h0, e1 - h1);
        }
    }
    const bf16x8_t pf = as_bf16x8(make_uint4(pw[0][0], pw[0][1], pw[1][0], pw[1][1]));
    const bf16x8_t pfl = as_bf16x8(make_uint4(pl[0][0], pl[0][1], pl[1][0], pl[1][1]));
    constexpr uint32_t kOnes = 0x3f803f80u;  // two bf16 1.0
    const bf16x8_t ones = as_bf16x8(make_uint4(kOnes, kOnes, kOnes, kOnes));
    f32x4_t ls = mfma_16x16x32_bf16(ones, pf, f32x4_t{0.f, 0.f, 0.f, 0.f});
    ls = mfma_16x16x32_bf16(ones, pfl, ls);
    if constexpr (FRESH) {
        l_run = ls[0];
    } else {
        const float alpha = exp2_hw(m_run - m_use);  // of head lr, which all of acc is
        l_run = fmaf(l_run, alpha, ls[0]);
#pragma unroll
        for (int db = 0; db < P::DB; ++db)
#pragma unroll
            for (int j = 0; j < 4; ++j)
                acc[db][j] *= alpha;
    }
    m_run = m_new;

    // V as operand A, P as operand B: acc[db][j] is d = 16 * db + 4 * lg + j of head lr.
    // A fresh state's accumulator is +0, given to the first MFMA as a constant.
#pragma unroll
    for (int db = 0; db < P::DB; ++db) {
        const f32x4_t c0 = FRESH ? f32x4_t{0.f, 0.f, 0.f, 0.f} : acc[db];
        acc[db] = mfma_16x16x32_bf16(as_bf16x8(v[db]), pf, c0);
        acc[db] = mfma_16x16x32_bf16(as_bf16x8(v[db]), pfl, acc[db]);
    }
}

// The decode form: K and V from the pair's registers, q rows from the LDS tile qt
// ([16][QROW]).
template <int D, bool FRESH>
__device__ __forceinline__ void pair_update(const PairFrag<D> &f, const uint4 (&v)[AttnK<D>::DB],
                                            int keep, bool full, const uint16_t *__restrict__ qt,
                                            float scale_log2, const PairLanes &ln, float &m_run,
                                            float &l_run, f32x4_t (&acc)[AttnK<D>::DB])
{
    using P = AttnK<D>;
    const uint16_t *qrow = qt + ln.lr() * QROW<D> + ln.lg() * P::DPL;
    float sv[2][4];
    const float mloc = pair_scores<D>(
        f.k, keep, full,
        [&](int cc) { return as_bf16x8(*reinterpret_cast<const uint4 *>(qrow + 8 * cc)); },
        scale_log2, sv);
    pair_pv<D, FRESH>(sv, mloc, v, m_run, l_run, acc);
}

// True when page pair pr of the split [t0, t1) is live in every token.
__device__ __forceinline__ bool pair_full(int pr, int t0, int t1)
{
    return t0 + (2 * pr + 2) * PAGE <= t1;
}

// A wave's (m, l, acc) into the workgroup's combine buffers ((m, l) head-major,
// [head][wave]); l_run, the wave's sum for head lr, is the same in every lane.
template <int D>
__device__ __forceinline__ void stash_wave(float m_run, float l_run,
                                           const f32x4_t (&acc)[AttnK<D>::DB], int wave,
                                           const PairLanes &ln, float (*c_m)[WAVES],
                                           float (*c_l)[WAVES], float (*c_acc)[16][D + CPAD])
{
    if (ln.lg() == 0) {
        c_m[ln.lr()][wave] = m_run;
        c_l[ln.lr()][wave] = l_run;
    }
#pragma unroll
    for (int db = 0; db < AttnK<D>::DB; ++db)
        *reinterpret_cast<float4 *>(&c_acc[wave][ln.lr()][16 * db + 4 * ln.lg()]) =
            make_float4(acc[db][0], acc[db][1], acc[db][2], acc[db][3]);
}

// The split's partial for head h from the waves' stashes, in wave order
// 0 .. WAVES-1:  M = max_w m_w, c_w = 2^(m_w - M) (0 for an idle wave),
// l = fma(c_w, l_w, l) and acc = fma(c_w, acc_w, acc) over w, starting from 0,
// for the EPT elements at dq.
template <int D>
__device__ __forceinline__ void combine_ml(const float (*c_m)[WAVES], const float (*c_l)[WAVES],
                                           int h, float &M, float &l, float (&cw)[WAVES])
{
    static_assert(WAVES % 4 == 0, "whole 16-byte reads");
    float mw[WAVES], lw[WAVES];
#pragma unroll
    for (int w = 0; w < WAVES; w += 4) {
        const float4 m4 = *reinterpret_cast<const float4 *>(&c_m[h][w]);
        const float4 l4 = *reinterpret_cast<const float4 *>(&c_l[h][w]);
        mw[w] = m4.x, mw[w + 1] = m4.y, mw[w + 2] = m4.z, mw[w + 3] = m4.w;
        lw[w] = l4.x, lw[w + 1] = l4.y, lw[w + 2] = l4.z, lw[w + 3] = l4.w;
    }
    M = -INFINITY;
#pragma unroll
    for (int w = 0; w < WAVES; ++w)
        M = fmaxf(M, mw[w]);
#pragma unroll
    for (int w = 0; w < WAVES; ++w)
        cw[w] = (mw[w] == -INFINITY) ? 0.f : exp2_hw(mw[w] - M);
    l = 0.f;
#pragma unroll
    for (int w = 0; w < WAVES; ++w)
        l = fmaf(cw[w], lw[w], l);
}

template <int D, int EPT>
__device__ __forceinline__ void combine_acc(const float (*c_acc)[16][D + CPAD],
                                            const float (&cw)[WAVES],
                                            int h, int dq, float (&o)[EPT])
{
#pragma unroll
    for (int e = 0; e < EPT; ++e) {
        float a = 0.f;
#pragma unroll
        for (int w = 0; w < WAVES; ++w)
            a = fmaf(cw[w], c_acc[w][h][dq + e], a);
        o[e] = a;
    }
}

// The value v holds in lane `src` (the same src in every lane), read into a scalar
// register: exact, and without the LDS round trip of a general lane permute.
__device__ __forceinline__ float lane_value(float v, int src)
{
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), src));
}

// Ascending fold of split partials (the merge): with M the largest partial
// maximum folded so far (-inf before the first), a new partial (m, l_s, a_s)
// gives M' = max(M, m), al = 2^(M - M'), be = 2^(m - M'),
// l = fma(be, l_s, l * al) and o = fma(be, a_s, o * al).
__device__ __forceinline__ float fold_step(float acc, float al, float be, float x)
{
    return fmaf(be, x, acc * al);
}

// One head's split partial (acc elements dq .. dq + EPT - 1 from this thread; the
// thread holding the last elements also writes m, l and the pads) to its IST slot.
template <int D, int EPT>
__device__ __forceinline__ void store_partial(float *dst, int dq, const float (&o)[EPT], float M,
                                              float l)
{
    // non-temporal: the partials are read once, by the merge (grid mode at the
    // bench's lengths: batch 256 1752 -> 1731 us, 64 482 -> 474, 16 105.2 -> 103.6)
    typedef float f4v __attribute__((ext_vector_type(4)));
    typedef float f2v __attribute__((ext_vector_type(2)));
    if constexpr (EPT == 4)
        __builtin_nontemporal_store(f4v{o[0], o[1], o[2], o[3]}, reinterpret_cast<f4v *>(dst + dq));
    else
        __builtin_nontemporal_store(f2v{o[0], o[1]}, reinterpret_cast<f2v *>(dst + dq));
    if (dq == D - EPT)
        __builtin_nontemporal_store(f4v{M, l, 0.f, 0.f}, reinterpret_cast<f4v *>(dst + D));
}

// Splits longer than 2 * PAGE * WAVES tokens: one workgroup per (row, kv head,
// split), wave w folding page pairs w, w + WAVES, ... with the running update.
// The loop keeps a pair, the accumulators and the loop state live at once, more
// than the 128 registers of two workgroups per compute unit at head_dim 128, so it
// runs one workgroup per unit (no spills).
template <int D>
__global__ __launch_bounds__(512, 2) void attn_split_kernel(
    const uint16_t *__restrict__ q, int64_t q_row_stride, const uint16_t *__restrict__ k_cache,
    const uint16_t *__restrict__ v_cache, const int32_t *__restrict__ block_table,
    int64_t bt_stride, const int32_t *__restrict__ kv_lens, int hq, int hkv, int S,
    int max_kv_len, int nsmax, float scale_log2, float *__restrict__ ws)
{
    using P = AttnK<D>;
    __shared__ __attribute__((aligned(16))) uint16_t q_lds[16][QROW<D>];
    __shared__ __attribute__((aligned(16))) float c_m[16][WAVES], c_l[16][WAVES];
    __shared__ __attribute__((aligned(16))) float c_acc[WAVES][16][D + CPAD];

    // grid x = split * hkv + kv head: the kv heads of one split are dispatched
    // back to back, so the head slices of each K and V page are read close together
    const int bx = xcd_rotated_x(hkv);
    const int s = bx / hkv, g = bx % hkv;
    const int64_t r = blockIdx.z;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const PairLanes ln(lane);
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
    float l_run = 0.f;        // the running sum for head lr (the same in every lane)
    f32x4_t acc[P::DB];       // acc[db][j]: d = 16*db + 4*lg + j of head lr
#pragma unroll
    for (int db = 0; db < P::DB; ++db)
        acc[db] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    const int pairs = (valid_pages + 1) / 2;
    // first step's loads go out before the query is staged
    PairFrag<D> f;
    if (wave < pairs)
        load_pair<D>(f, wave, my_page, valid_pages, k_cache, v_cache, hkv, g, ln);

    // the group's query rows, staged once in LDS (rows past the group are zero)
    for (int i = threadIdx.x; i < 16 * D / 8; i += WAVES * 64) {
        const int h = i / (D / 8), c = i % (D / 8);
        *reinterpret_cast<uint4 *>(&q_lds[h][8 * c]) =
            h < G ? *reinterpret_cast<const uint4 *>(q + r * q_row_stride + (int64_t)(g * G + h) * D + 8 * c)
                  : make_uint4(0, 0, 0, 0);
    }
    __syncthreads();  // q_lds ready

    // (register budget: the query fragments are re-read from LDS every pair -- the
    // empty asm keeps them from being hoisted out of the loop -- and the all-pass
    // mask of a full pair is applied anyway, which gives the same bits)
    for (int pr = wave; pr < pairs; pr += WAVES) {
        asm volatile("" ::: "memory");
        if (pr != wave)
            load_pair<D>(f, pr, my_page, valid_pages, k_cache, v_cache, hkv, g, ln);
        const int keep = run_keep(pr, t0, t1, valid_pages, ln);
        mask_runs<D>(f.v, keep, f.v);
        pair_update<D, false>(f, f.v, keep, false, &q_lds[0][0], scale_log2, ln, m_run, l_run,
                              acc);
    }

    stash_wave<D>(m_run, l_run, acc, wave, ln, c_m, c_l, c_acc);
    __syncthreads();

    // combine the waves; thread t: head t / 32, d slice
    static_assert(D == 64 || D == 128, "head_dim 64 or 128");
    constexpr int EPT = D / 32;  // elements of the head row this thread owns
    const int h = threadIdx.x >> 5;
    const int dq = (threadIdx.x & 31) * EPT;
    float M, l, cw[WAVES];
    combine_ml<D>(c_m, c_l, h, M, l, cw);
    if (h < G) {
        float o[EPT];
        combine_acc<D, EPT>(c_acc, cw, h, dq, o);
        store_partial<D, EPT>(ws + part_off(r, g, s, h, hkv, nsmax, G, IST<D>), dq, o, M, l);
    }
}

// Work plan of a decode call with a large batch (plan mode of attn_group_kernel),
// built on the device from the lengths by attn_plan_kernel, int32 words:
//   [0] items, [1] T (splits per chunk, a multiple of GROUP), [2..3] unused,
//   then chunks[rows] (chunks of each row) and item_row, item_chunk[rows + kPlanCuMax].
// Row r with n splits is cut into ceil(n / T) chunks of T consecutive splits (the
// last one shorter); the items, one per (row, chunk), are ordered by size,
// longest first.  T is 1.5 times the batch's work per compute unit, 1.5 W / CUs
// with W = hkv * sum of the rows' split counts, rounded up to whole groups, so
// the total count of items is at most rows + CUs / hkv.  (The call is bound by
// HBM, so a unit that runs past its share while others finish gets more of the
// bandwidth: whole rows up to 1.5 shares beat cutting them at one share, e.g.
// batch 112 at the bench's lengths 709 vs 736 us; 1.25 and 2 shares measured as
// 1.5.)  Only the schedule depends on the batch: a chunk's splits get exactly the
// arithmetic of the grid mode, whichever workgroup takes them.
constexpr int kPlanHdr = 4;
constexpr int kPlanCuMax = 1024;   // compute units a plan has room for
constexpr int kPlanKeys = 1024;    // size classes of the longest-first order
__host__ __device__ constexpr int64_t plan_words(int64_t rows)
{
    return kPlanHdr + rows + 2 * (rows + kPlanCuMax);
}

// One workgroup: the plan above.  The order among items of equal size (and among
// items of kPlanKeys - 1 splits or more) is whatever the LDS atomics give; it
// decides only which workgroup takes an item.
__global__ __launch_bounds__(1024) void attn_plan_kernel(const int32_t *__restrict__ kv_lens,
                                                         int rows, int hkv, int S, int max_kv_len,
                                                         int ncu, int32_t *__restrict__ plan)
{
    constexpr int kLdsRows = 4096;  // split counts kept in LDS for the first rows
    __shared__ int hist[kPlanKeys];
    __shared__ int nsp_lds[kLdsRows];
    __shared__ int wave_tot[16];
    __shared__ unsigned long long wsum;
    __shared__ int T_s;
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    int *chunks = plan + kPlanHdr;
    int *item_row = chunks + rows, *item_chunk = item_row + rows + kPlanCuMax;
    auto nsp_mem = [&](int r) { return (clamp_len(kv_lens[r], max_kv_len) + S - 1) / S; };
    auto nsp_of = [&](int r) { return r < kLdsRows ? nsp_lds[r] : nsp_mem(r); };
    hist[tid] = 0;
    if (tid == 0)
        wsum = 0;
    __syncthreads();
    unsigned long long part = 0;
    for (int r = tid; r < rows; r += 1024) {
        const int n = nsp_mem(r);
        if (r < kLdsRows)
            nsp_lds[r] = n;
        part += (unsigned)n;
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1)
        part += __shfl_xor(part, off, kWave);
    if (lane == 0)
        atomicAdd(&wsum, part);
    __syncthreads();
    if (tid == 0) {
        const unsigned long long W = wsum * (unsigned long long)hkv;
        unsigned long long t = (3 * W + 2ull * ncu - 1) / (2ull * ncu);
        t = (t + GROUP - 1) / GROUP * GROUP;
        T_s = (int)(t < GROUP ? GROUP : (t > (1u << 30) ? (1u << 30) : t));
        plan[1] = T_s;
    }
    __syncthreads();
    const int T = T_s;
    for (int r = tid; r < rows; r += 1024) {
        const int n = nsp_of(r), nc = (n + T - 1) / T;
        chunks[r] = nc;
        for (int c = 0; c < nc; ++c)
            atomicAdd(&hist[min(min(T, n - c * T), kPlanKeys - 1)], 1);
    }
    __syncthreads();
    // exclusive scan over the size classes, largest first: thread t holds class
    // kPlanKeys - 1 - t
    const int hv = hist[kPlanKeys - 1 - tid];
    int inc = hv;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const int u = __shfl_up(inc, off, kWave);
        if (lane >= off)
            inc += u;
    }
    if (lane == 63)
        wave_tot[wv] = inc;
    __syncthreads();
    int base = 0;
    for (int w = 0; w < wv; ++w)
        base += wave_tot[w];
    const int start = base + inc - hv;
    __syncthreads();
    hist[kPlanKeys - 1 - tid] = start;
    if (tid == 1023)
        plan[0] = base + inc;
    __syncthreads();
    for (int r = tid; r < rows; r += 1024) {
        const int n = nsp_of(r), nc = (n + T - 1) / T;
        for (int c = 0; c < nc; ++c) {
            const int pos = atomicAdd(&hist[min(min(T, n - c * T), kPlanKeys - 1)], 1);
            item_row[pos] = r;
            item_chunk[pos] = c;
        }
    }
}

// Splits of at most 2 * PAGE * WAVES tokens (one page pair per wave).  A workgroup
// takes a run of consecutive splits of one (row, kv head): in grid mode (plan
// null) one group of GROUP splits, grid (groups * hkv, 1, rows); in plan mode the
// plan's chunk blockIdx.x / hkv, grid (items bound * hkv).  Each split's partial is
// formed exactly as a split workgroup would (wave w's pair 2w, 2w + 1 with a fresh
// state, the wave combine in order) and folded into its group's running
// (M, l, acc) held by the combining threads.  A finished group goes to the
// workspace as the merge's partial -- or, when the chunk is the whole row, is
// folded at once into the row's total as the merge would fold it, and the row's
// output is written here (the merge then skips the row).  A wave requests its pair
// of split s + 1 as soon as its update of split s is done, so the loads run under
// the stash, the combine and the fold (requesting it before the update, into a
// second register buffer, measured slower: 1.85 vs 1.80 ms at the bench shape).
// The stash is double-buffered (split s uses buffer s % 2), so one barrier per
// split suffices.  One workgroup per compute unit.
//   Why whole rows: a workgroup cannot finish before its stores are written, and a
// group partial store at the end of every workgroup, with the loads of the other
// workgroups queued ahead of it, cost 14 % of the call at the bench shape (the
// same kernel without them: 1511 vs 1749 us); a whole row stores 16 output rows
// of bf16 once.  Longest chunks first keep the last compute units busy: in row
// order the same kernel took 1654 us, longest first 1467.
template <int D, bool PLAN>
__global__ __launch_bounds__(512, 2) void attn_group_kernel(
    const uint16_t *__restrict__ q, int64_t q_row_stride, const uint16_t *__restrict__ k_cache,
    const uint16_t *__restrict__ v_cache, const int32_t *__restrict__ block_table,
    int64_t bt_stride, const int32_t *__restrict__ kv_lens, int hq, int hkv, int S,
    int max_kv_len, int ngmax, int rows, const int32_t *__restrict__ plan, float scale_log2,
    float *__restrict__ ws, uint16_t *__restrict__ out, int64_t out_row_stride)
{
    using P = AttnK<D>;
    __shared__ __attribute__((aligned(16))) uint16_t q_lds[16][QROW<D>];
    __shared__ __attribute__((aligned(16))) float c_m[2][16][WAVES], c_l[2][16][WAVES];
    __shared__ __attribute__((aligned(16))) float c_acc[2][WAVES][16][D + CPAD];

    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const PairLanes ln(lane);
    const int split_pages = S / PAGE;
    const int grp_pages = GROUP * split_pages;  // <= 64: one block-table entry per lane
    const int row_pages = (max_kv_len + PAGE - 1) / PAGE;
    int64_t r;
    int g, s_begin, run;  // run: splits in this workgroup's chunk (a bound in grid mode)
    if constexpr (PLAN) {
        const int item = (int)blockIdx.x / hkv;
        g = (int)blockIdx.x % hkv;
        if (item >= plan[0])
            return;
        run = plan[1];
        r = plan[kPlanHdr + rows + item];
        s_begin = plan[kPlanHdr + 2 * rows + kPlanCuMax + item] * run;
    } else {
        // grid x = group * hkv + kv head (the kv heads of a group back to back)
        const int bx = xcd_rotated_x(hkv);
        g = bx % hkv;
        r = blockIdx.z;
        s_begin = bx / hkv * GROUP;
        run = GROUP;
    }
    const int32_t *btrow = block_table + r * bt_stride;
    // group grp's block-table entries, one per lane (clamped into the table row;
    // entries past the row's last page are never used)
    auto entries = [&](int grp) {
        return btrow[min(grp * grp_pages + min(lane, grp_pages - 1), row_pages - 1)];
    };
    int my_page = entries(s_begin / GROUP);  // read before the length
    const int L = clamp_len(kv_lens[r], max_kv_len);
    const int nsplit = (L + S - 1) / S;
    if (s_begin >= nsplit)
        return;
    const int s_end = min(s_begin + run, nsplit);
    const bool whole = PLAN && s_begin == 0 && s_end == nsplit;
    int next_page = PLAN && s_begin + GROUP < s_end ? entries(s_begin / GROUP + 1) : my_page;
    const int G = hq / hkv;

    // pages of split s: entries (s % GROUP) * split_pages .. of its group's entries
    auto vpages = [&](int s) { return (min(s * S + S, L) - s * S + PAGE - 1) / PAGE; };
    PairFrag<D> f;
    auto load = [&](int s, int pages) {
        if (wave < (vpages(s) + 1) / 2)
            load_pair<D>(f, wave, __shfl(pages, (lane + (s % GROUP) * split_pages) & 63, kWave),
                         vpages(s), k_cache, v_cache, hkv, g, ln);
    };

    load(s_begin, my_page);
    for (int i = threadIdx.x; i < 16 * D / 8; i += WAVES * 64) {
        const int h = i / (D / 8), c = i % (D / 8);
        *reinterpret_cast<uint4 *>(&q_lds[h][8 * c]) =
            h < G ? *reinterpret_cast<const uint4 *>(q + r * q_row_stride + (int64_t)(g * G + h) * D + 8 * c)
                  : make_uint4(0, 0, 0, 0);
    }
    __syncthreads();  // q_lds ready

    static_assert(D == 64 || D == 128, "head_dim 64 or 128");
    constexpr int EPT = D / 32;
    const int h = threadIdx.x >> 5;  // combining thread: head h, elements dq .. dq + EPT - 1
    const int dq = (threadIdx.x & 31) * EPT;
    float Mg = -INFINITY, lg = 0.f, og[EPT];  // the current group's fold
    float Mt = -INFINITY, lt = 0.f, ot[EPT];  // whole row: the fold of its groups
    // a finished group's partial when more groups follow in the chunk: stored one
    // split later, after that split's loads are requested
    float pM = 0.f, pl = 0.f, po[EPT];
    int pgrp = -1;
#pragma unroll
    for (int e = 0; e < EPT; ++e)
        og[e] = ot[e] = po[e] = 0.f;
    for (int s = s_begin; s < s_end; ++s) {
        const int buf = (s - s_begin) & 1;
        const int t0 = s * S, t1 = min(t0 + S, L);
        const int vp = vpages(s);
        float m_run = -INFINITY, l_run = 0.f;
        f32x4_t acc[P::DB];
#pragma unroll
        for (int db = 0; db < P::DB; ++db)
            acc[db] = f32x4_t{0.f, 0.f, 0.f, 0.f};
        if (wave < (vp + 1) / 2) {
            const int keep = run_keep(wave, t0, t1, vp, ln);
            const bool full = pair_full(wave, t0, t1);
            if (!full)
                mask_runs<D>(f.v, keep, f.v);
            pair_update<D, true>(f, f.v, keep, full, &q_lds[0][0], scale_log2, ln, m_run, l_run,
                                 acc);
        }
        const bool grp_end = s % GROUP == GROUP - 1 || s + 1 == s_end;
        if (s + 1 < s_end)
            load(s + 1, PLAN && grp_end ? next_page : my_page);
        if (PLAN && pgrp >= 0) {
            if (h < G)
                store_partial<D, EPT>(ws + part_off(r, g, pgrp, h, hkv, ngmax, G, IST<D>), dq, po,
                                      pM, pl);
            pgrp = -1;
        }
        stash_wave<D>(m_run, l_run, acc, wave, ln, c_m[buf], c_l[buf], c_acc[buf]);
        // the split's stash complete; every combine of split s - 1 (which read the
        // other buffer) done before split s + 1 writes it
        __syncthreads();
        float Ms, ls, cw[WAVES];
        combine_ml<D>(c_m[buf], c_l[buf], h, Ms, ls, cw);
        if (h < G) {
            float os[EPT];
            combine_acc<D, EPT>(c_acc[buf], cw, h, dq, os);
            const float Mn = fmaxf(Mg, Ms);
            const float al = exp2_hw(Mg - Mn), be = exp2_hw(Ms - Mn);
            lg = fold_step(lg, al, be, ls);
#pragma unroll
            for (int e = 0; e < EPT; ++e)
                og[e] = fold_step(og[e], al, be, os[e]);
            Mg = Mn;
        }
        if (grp_end) {
            if (PLAN && whole) {
                if (h < G) {  // the group into the row's total, as the merge folds it
                    const float Mn = fmaxf(Mt, Mg);
                    const float al = exp2_hw(Mt - Mn), be = exp2_hw(Mg - Mn);
                    lt = fold_step(lt, al, be, lg);
#pragma unroll
                    for (int e = 0; e < EPT; ++e)
                        ot[e] = fold_step(ot[e], al, be, og[e]);
                    Mt = Mn;
                }
            } else if (s + 1 == s_end) {
                if (h < G)
                    store_partial<D, EPT>(ws + part_off(r, g, s / GROUP, h, hkv, ngmax, G, IST<D>),
                                          dq, og, Mg, lg);
            } else if constexpr (PLAN) {
                pgrp = s / GROUP;
                pM = Mg;
                pl = lg;
#pragma unroll
                for (int e = 0; e < EPT; ++e)
                    po[e] = og[e];
            }
            Mg = -INFINITY;
            lg = 0.f;
#pragma unroll
            for (int e = 0; e < EPT; ++e)
                og[e] = 0.f;
            if (PLAN && s + 1 < s_end) {
                my_page = next_page;
                next_page = entries(s / GROUP + 2);
            }
        }
    }
    if (PLAN && whole && h < G) {
        uint16_t *dst = out + r * out_row_stride + (int64_t)(g * G + h) * D + dq;
        if constexpr (EPT == 4)
            *reinterpret_cast<uint2 *>(dst) = make_uint2(pack_bf16x2(ot[0] / lt, ot[1] / lt),
                                                         pack_bf16x2(ot[2] / lt, ot[3] / lt));
        else
            *reinterpret_cast<uint32_t *>(dst) = pack_bf16x2(ot[0] / lt, ot[1] / lt);
    }
}

// One wave per (row, query head): the ascending fold of the row's partials, each
// covering S tokens (a group of splits, or one long split).  The running maxima (prefix maxima over the splits, exact, so
// order-free) and the factors al, be of each split are formed lane-parallel,
// one split per lane; the fold itself runs in ascending split order in every
// lane.  Row r's length is kv_lens[r], or start + r + 1 when kv_lens is null
// (consecutive prompt tokens).
template <int D>
__global__ __launch_bounds__(256) void attn_merge_kernel(
    const float *ws, const int32_t *__restrict__ kv_lens, int start, int64_t rows, int hq,
    int hkv, int S, int max_kv_len, int nsmax, const int32_t *__restrict__ row_chunks,
    uint16_t *__restrict__ out, int64_t out_row_stride)
{
    constexpr int EPL = D / 64;  // elements per lane
    constexpr int UNROLL = 16;
    const int lane = threadIdx.x & 63;
    const int64_t item = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (item >= rows * hq)
        return;
    const int64_t r = item / hq;
    if (row_chunks && row_chunks[r] == 1)
        return;  // a whole-row workgroup has written this row
    const int h = (int)(item % hq);
    const int L = kv_lens ? clamp_len(kv_lens[r], max_kv_len) : start + (int)r + 1;
    const int n = (L + S - 1) / S;  // splits of this row
    const int G = hq / hkv;
    // split s of this (row, head) at base + s * sst: acc, then (m, l) at + D
    const float *base = ws + part_off(r, h / G, 0, h % G, hkv, nsmax, G, IST<D>);
    const int64_t sst = (int64_t)G * IST<D>;
    const float *ac = base + lane * EPL;
    float M = -INFINITY;  // running maximum, the same in every lane
    float l = 0.f, o[EPL];
#pragma unroll
    for (int e = 0; e < EPL; ++e)
        o[e] = 0.f;
    for (int s0 = 0; s0 < n; s0 += 64) {
        const int sl = s0 + lane;
        const int cnt = min(64, n - s0);
        // every load issued before its first use; past the row's last split a lane
        // re-reads that split (its value is never folded)
        float a[UNROLL][EPL];
        auto load_batch = [&](int j0) {
#pragma unroll
            for (int u = 0; u < UNROLL; ++u) {
                const float *src = ac + (int64_t)(s0 + min(j0 + u, cnt - 1)) * sst;
                if constexpr (EPL == 2) {
                    const float2 t = *reinterpret_cast<const float2 *>(src);
                    a[u][0] = t.x;
                    a[u][1] = t.y;
                } else {
                    a[u][0] = src[0];
                }
            }
        };
        // the group's (m, l), and with them its first batch of partials, so that the
        // scan below runs while they arrive (batch 1: 10.0 -> 8.9 us, same bits)
        const float2 ml_l = *reinterpret_cast<const float2 *>(base + min(sl, n - 1) * sst + D);
        load_batch(0);
        asm volatile("" ::: "memory");
        const float m_l = sl < n ? ml_l.x : -INFINITY;
        const float l_l = sl < n ? ml_l.y : 0.f;
        float Mi = m_l;  // max(M, m_s0 .. m_sl)
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
            const float t = __shfl_up(Mi, off, kWave);
            if (lane >= off)
                Mi = fmaxf(Mi, t);
        }
        Mi = fmaxf(Mi, M);
        float Mp = __shfl_up(Mi, 1, kWave);  // the maximum before split sl
        if (lane == 0)
            Mp = M;
        const float al_l = exp2_hw(Mp - Mi);
        const float be_l = exp2_hw(m_l - Mi);
        M = lane_value(Mi, 63);
        for (int j0 = 0; j0 < cnt; j0 += UNROLL) {
            if (j0 > 0) {
                load_batch(j0);
                asm volatile("" ::: "memory");  // keep the batch ahead of its folds
            }
#pragma unroll
            for (int u = 0; u < UNROLL; ++u) {
                if (j0 + u < cnt) {
                    // split j0 + u's factors from its lane: the lane index is the same in
                    // every lane, so a scalar read (v_readlane) rather than an LDS permute
                    const float al = lane_value(al_l, j0 + u);
                    const float be = lane_value(be_l, j0 + u);
                    l = fold_step(l, al, be, lane_value(l_l, j0 + u));
#pragma unroll
                    for (int e = 0; e < EPL; ++e)
                        o[e] = fold_step(o[e], al, be, a[u][e]);
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

// Prefill: one request's consecutive prompt tokens start .. start + tokens - 1,
// token t with causal length L_t = start + t + 1, over one block-table row.
// Each (token, query head) goes through exactly the decode arithmetic above --
// the same split boundaries, the same page pairs and per-pair step (pair_scores,
// pair_pv), the same combine of a split's pairs in pair order, the same fold of
// each group of GROUP splits and the same ascending fold of the groups -- so its
// bits are those of the decode row with that query and length.  What changes is
// the schedule: a workgroup of WAVES waves takes WAVES consecutive tokens of one
// kv head, one token per wave, and copies each split's K and V pages into LDS once
// (LDS DMA), from where every wave reads all of the split's page pairs for its
// token.  A wave holds its token's whole state, so the pairs of a split are
// combined in its registers: no stash and no barrier per token.  Per split:
//   barrier (K pages in; every wave done with the V pages) -> the split's V pages
//   requested -> pass 1: every pair's scores and maximum from K, kept in
//   registers, and the split's maximum M -> barrier (V pages in; every wave done
//   with K) -> the next split's K pages requested -> pass 2: per pair, the
//   softmax weights and P.V from V, folded with weight 2^(m_pair - M) into the
//   split's (l, acc) in pair order, as the decode folds its waves.
//   FUSED:  1-D grid over (token block, kv head); the workgroup walks the splits in
//           ascending order, folds each split into its group and each finished
//           group into the token's total, in registers; no workspace.
//   !FUSED: grid (groups, kv heads, token blocks); each workgroup writes its
//           tokens' group partials to the workspace (slot layout of the decode
//           kernel) and the merge kernel folds them.  For short chunks after a
//           long prefix, where token blocks alone cannot fill the chip.
// Split sizes up to 2 * PAGE * WAVES = 256 tokens (at most WAVES page pairs).
//
// LDS images.  A 16-byte LDS read (ds_read_b128) serves a wave in passes of 16
// lanes, lanes 0-7 with 16-23 and so on, over 64 four-byte banks: it is free of
// bank conflicts when those 16 lanes read 16 distinct 16-byte positions modulo 256
// bytes (the rule the matmul's measured fragment reads follow).  Page slot p of
// an image holds the split's page p of the kv head.  V pages keep the cache's
// head-dim-major layout: a V fragment read (rows d = 16 db + lr of 32 bytes, the
// run's half) is conflict free as stored.  A K fragment read takes 16-byte chunk
// lg * KCH + cc of token rows krow + 4 b, with rows of 2 D bytes; K row r stores
// its chunk c at position c ^ kswz(r), which sends the row bits that vary within a
// pass (0, 1 and 3) to distinct chunk bits other than the lane group's.  The
// query rows (one 16 x D tile per token, row r = head) store chunk c at
// c ^ qswz(r) for the same reason (row bits 0, 1, 2 vary within a pass).
template <int D>
__device__ __forceinline__ int kswz(int r)
{
    if constexpr (D == 128)
        return r & 11;                        // row bits 0, 1, 3 -> chunk bits 0, 1, 3
    else
        return ((r >> 1) & 1) | ((r >> 1) & 4);  // row bit 0 picks the 128-byte half;
                                                 // bits 1, 3 -> chunk bits 0, 2
}

template <int D>
__device__ __forceinline__ int qswz(int r)
{
    if constexpr (D == 128)
        return (r & 3) | ((r & 4) << 1);   // row bits 0, 1, 2 -> chunk bits 0, 1, 3
    else
        return ((r >> 1) & 1) | (r & 4);   // row bit 0 picks the half; 1, 2 -> 0, 2
}

// Wait for this wave's outstanding global loads (the LDS DMA) and LDS reads, then
// meet the other waves.  s_waitcnt immediate (gfx9): vmcnt bits [3:0] and [15:14],
// expcnt [6:4], lgkmcnt [11:8].  The empty asm statements keep the compiler from
// moving memory accesses across the barrier.
__device__ __forceinline__ void wait_dma_and_barrier()
{
    __builtin_amdgcn_s_waitcnt(7 << 4);
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

template <int D, bool FUSED>
__global__ __launch_bounds__(512, 1) void attn_prefill_kernel(
    const uint16_t *__restrict__ q, int64_t q_row_stride, const uint16_t *__restrict__ k_cache,
    const uint16_t *__restrict__ v_cache, const int32_t *__restrict__ btrow, int start, int tokens,
    int hq, int hkv, int S, float scale_log2, uint16_t *__restrict__ out, int64_t out_row_stride,
    int npmax, float *__restrict__ ws)
{
    using P = AttnK<D>;
    static_assert(D == 64 || D == 128, "head_dim 64 or 128");
    constexpr int PG = PAGE * D;              // bf16 per page of one kv head
    constexpr int CPR = D / 8;                // 16-byte chunks per K row or query row
    constexpr int QPP = PG * 2 / 1024;        // 1 KiB DMA pieces per page
    static_assert(WAVES % QPP == 0, "a wave copies the same piece of every page");
    __shared__ __attribute__((aligned(16))) uint16_t k_img[2 * WAVES * PG];
    __shared__ __attribute__((aligned(16))) uint16_t v_img[2 * WAVES * PG];
    __shared__ __attribute__((aligned(16))) uint16_t q_img[WAVES][16 * D];

    const int nblk = (tokens + WAVES - 1) / WAVES;
    int rank, g;
    if constexpr (FUSED) {
        // kv heads innermost: with hkv dividing 8, the XCD of a workgroup (linear id
        // mod 8) serves the same kv heads throughout, whose pages then share its L2
        rank = (int)blockIdx.x / hkv;
        g = (int)blockIdx.x % hkv;
    } else {
        rank = (int)blockIdx.z;
        g = (int)blockIdx.y;
    }
    const int blk = nblk - 1 - rank;  // the blocks with the longest lengths first
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const PairLanes ln(lane);
    const int G = hq / hkv;
    const int tok0 = blk * WAVES;
    const int tcount = min(WAVES, tokens - tok0);
    const int Lmax = start + tok0 + tcount;  // the block's longest length
    const int split_pages = S / PAGE;
    const int last_entry = (start + tokens + PAGE - 1) / PAGE - 1;
    // FUSED: every split of the block; else the splits of group blockIdx.x
    const int s_first = FUSED ? 0 : (int)blockIdx.x * GROUP;
    const int s_end = FUSED ? (Lmax + S - 1) / S
                            : min(((int)blockIdx.x + 1) * GROUP, (Lmax + S - 1) / S);
    if (s_first >= s_end)
        return;

    // The pages [0, np) of split s that the block needs, copied by LDS DMA: 64 lanes x
    // 16 bytes per instruction, lane l to image bytes 16 l .. of its piece; piece
    // i of the split goes to wave i % WAVES, which is always piece wave % QPP of a page.
    int k_off, v_off;  // this lane's source element in that piece of a page
    {
        const int pos = (wave % QPP) * 64 + lane;  // 16-byte position in the page image
        const int r = pos / CPR;
        k_off = r * D + 8 * ((pos % CPR) ^ kswz<D>(r));
        v_off = 8 * pos;
    }
    auto pages_of = [&](int s) { return (min(s * S + S, Lmax) - s * S + PAGE - 1) / PAGE; };
    // The block-table entries of split s, one per lane (lane < split_pages): read
    // with one vector load a phase ahead of the copies that use them, which take
    // each page id from its lane by v_readlane (no scalar load to wait for per page).
    auto entries = [&](int s) {
        return btrow[min(s * split_pages + min(lane, split_pages - 1), last_entry)];
    };
    auto dma = [&](uint16_t *img, const uint16_t *__restrict__ cache, int off, int s,
                   int ent) {
        const int n = pages_of(s) * QPP;
        for (int i = wave; i < n; i += WAVES) {
            const int slot = i / QPP;
            const int64_t phys = __builtin_amdgcn_readlane(ent, slot);
            const uint16_t *src = cache + (phys * hkv + g) * PG + off;
            uint16_t *dst = img + slot * PG + (wave % QPP) * 512;
#if defined(__HIP_DEVICE_COMPILE__)
            __builtin_amdgcn_global_load_lds(
                (const void __attribute__((address_space(1))) *)src,
                (void __attribute__((address_space(3))) *)dst, 16, 0, 0);
#else
            (void)src, (void)dst;
#endif
        }
    };
    int ent_cur = entries(s_first);
    dma(k_img, k_cache, k_off, s_first, ent_cur);

    // the block's query tiles: token t's rows r = query head g * G + r (zero past G)
    for (int i = threadIdx.x; i < WAVES * 16 * CPR; i += WAVES * 64) {
        const int t = i / (16 * CPR), r = (i / CPR) % 16, c = i % CPR;
        const uint4 v =
            (t < tcount && r < G)
                ? *reinterpret_cast<const uint4 *>(q + (int64_t)(tok0 + t) * q_row_stride +
                                                   (int64_t)(g * G + r) * D + 8 * c)
                : make_uint4(0, 0, 0, 0);
        *reinterpret_cast<uint4 *>(&q_img[t][r * D + 8 * (c ^ qswz<D>(r))]) = v;
    }

    const bool live = wave < tcount;
    const int Lt = start + tok0 + wave + 1;  // this wave's token's length (if live)
    const uint16_t *qrow = &q_img[wave][ln.lr() * D];
    const int qz = qswz<D>(ln.lr());
    auto qfrag = [&](int cc) {
        return as_bf16x8(
            *reinterpret_cast<const uint4 *>(qrow + 8 * ((ln.lg() * P::KCH + cc) ^ qz)));
    };
    const int kz = kswz<D>(ln.krow());  // the same for token rows krow and krow + 4
    const uint16_t *kbase = k_img + ln.kslot() * PG + ln.krow() * D;
    const uint16_t *vbase = v_img + ln.vslot() * PG + ln.lr() * PAGE + ln.vrun();

    // the token's fold of its current group of splits, and (FUSED) of its groups
    float Mg = -INFINITY, lgr = 0.f, Mt = -INFINITY, lt = 0.f;
    f32x4_t og[P::DB], ot[P::DB];
#pragma unroll
    for (int db = 0; db < P::DB; ++db)
        og[db] = ot[db] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    for (int s = s_first; s < s_end; ++s) {
        const int t0 = s * S;
        wait_dma_and_barrier();  // K pages of s in (and the query tiles); V buffer free
        dma(v_img, v_cache, v_off, s, ent_cur);
        // the next split's entries, for its K copies after the second barrier
        const int ent_next = s + 1 < s_end ? entries(s + 1) : 0;
        const bool act = live && t0 < Lt;  // wave-uniform
        const int t1 = min(t0 + S, Lt);
        const int vp = (t1 - t0 + PAGE - 1) / PAGE;  // the token's pages in the split
        const int npair = act ? (vp + 1) / 2 : 0;
        // every pair of the split live in every token (the common case): straight-line
        // code without masks or per-pair branches, so loads and arithmetic of
        // neighbouring pairs can overlap
        const bool whole = act && S == 2 * PAGE * WAVES && t0 + S <= Lt;
        float sv[WAVES][2][4], mp[WAVES];
        float M = -INFINITY;
        auto load_k = [&](int p, uint4 (&kf)[2][P::KCH]) {
#pragma unroll
            for (int b = 0; b < 2; ++b)
#pragma unroll
                for (int cc = 0; cc < P::KCH; ++cc)
                    kf[b][cc] = *reinterpret_cast<const uint4 *>(
                        kbase + 2 * p * PG + 4 * b * D + 8 * ((ln.lg() * P::KCH + cc) ^ kz));
        };
        if (whole) {
            // two pairs at a time: four independent MFMA chains in flight
#pragma unroll
            for (int p = 0; p < WAVES; p += 2) {
                uint4 kf[2][2][P::KCH];
                load_k(p, kf[0]);
                load_k(p + 1, kf[1]);
                float sv2[2][2][4], m2[2];
                full_pairs_scores<D, 2>(kf, qfrag, scale_log2, sv2, m2);
#pragma unroll
                for (int i = 0; i < 2; ++i) {
#pragma unroll
                    for (int b = 0; b < 2; ++b)
#pragma unroll
                        for (int j = 0; j < 4; ++j)
                            sv[p + i][b][j] = sv2[i][b][j];
                    mp[p + i] = m2[i];
                    M = fmaxf(M, m2[i]);
                }
            }
        } else if (act) {
#pragma unroll
            for (int p = 0; p < WAVES; ++p) {
                if (p < npair) {
                    uint4 kf[2][P::KCH];
                    load_k(p, kf);
                    mp[p] = pair_scores<D, true>(kf, run_keep(p, t0, t1, vp, ln),
                                                 pair_full(p, t0, t1), qfrag, scale_log2, sv[p]);
                    M = fmaxf(M, mp[p]);
                }
            }
        }
        wait_dma_and_barrier();  // V pages of s in; K buffer free
        if (s + 1 < s_end)
            dma(k_img, k_cache, k_off, s + 1, ent_next);
        ent_cur = ent_next;
        if (!act)
            continue;

        // the split's (l, acc): pair p's partial with weight 2^(m_p - M), in pair
        // order, as the decode combines its waves (wave p holding pair p)
        float l = 0.f;
        f32x4_t a[P::DB];
#pragma unroll
        for (int db = 0; db < P::DB; ++db)
            a[db] = f32x4_t{0.f, 0.f, 0.f, 0.f};
        auto pass2 = [&](auto all_c) {
            constexpr bool all = decltype(all_c)::value;
#pragma unroll
            for (int p = 0; p < WAVES; ++p) {
                if (all || p < npair) {
                    uint4 vf[P::DB];
#pragma unroll
                    for (int db = 0; db < P::DB; ++db)
                        vf[db] = *reinterpret_cast<const uint4 *>(vbase + 2 * p * PG +
                                                                  16 * db * PAGE);
                    if (!all && !pair_full(p, t0, t1))
                        mask_runs<D>(vf, run_keep(p, t0, t1, vp, ln), vf);
                    float m_run = -INFINITY, l_run = 0.f;
                    f32x4_t acc[P::DB];
                    pair_pv<D, true>(sv[p], mp[p], vf, m_run, l_run, acc);
                    const float cw = (m_run == -INFINITY) ? 0.f : exp2_hw(m_run - M);
                    l = fmaf(cw, l_run, l);
#pragma unroll
                    for (int db = 0; db < P::DB; ++db)
#pragma unroll
                        for (int j = 0; j < 4; ++j)
                            a[db][j] = fmaf(cw, acc[db][j], a[db][j]);
                }
            }
        };
        if (whole) {
            pass2(std::true_type{});
        } else {
            pass2(std::false_type{});
            if (npair < WAVES) {  // the decode's idle waves, each adding fma(0, +0, .)
                l = fmaf(0.f, 0.f, l);
#pragma unroll
                for (int db = 0; db < P::DB; ++db)
#pragma unroll
                    for (int j = 0; j < 4; ++j)
                        a[db][j] = fmaf(0.f, 0.f, a[db][j]);
            }
        }
        // the split into the token's group, as the decode group kernel folds it
        {
            const float Mn = fmaxf(Mg, M);
            const float al = exp2_hw(Mg - Mn), be = exp2_hw(M - Mn);
            lgr = fold_step(lgr, al, be, l);
#pragma unroll
            for (int db = 0; db < P::DB; ++db)
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    og[db][j] = fold_step(og[db][j], al, be, a[db][j]);
            Mg = Mn;
        }
        // the token's group ends here: at a group boundary or its last split
        if (s % GROUP == GROUP - 1 || t0 + S >= Lt) {
            if constexpr (FUSED) {  // the group into the token's total, as the merge does
                const float Mn = fmaxf(Mt, Mg);
                const float al = exp2_hw(Mt - Mn), be = exp2_hw(Mg - Mn);
                lt = fold_step(lt, al, be, lgr);
#pragma unroll
                for (int db = 0; db < P::DB; ++db)
#pragma unroll
                    for (int j = 0; j < 4; ++j)
                        ot[db][j] = fold_step(ot[db][j], al, be, og[db][j]);
                Mt = Mn;
            } else if (ln.lr() < G) {
                float *dst = ws + part_off(tok0 + wave, g, s / GROUP, ln.lr(), hkv, npmax, G,
                                           IST<D>);
#pragma unroll
                for (int db = 0; db < P::DB; ++db)
                    *reinterpret_cast<float4 *>(dst + 16 * db + 4 * ln.lg()) =
                        make_float4(og[db][0], og[db][1], og[db][2], og[db][3]);
                if (ln.lg() == 0)
                    *reinterpret_cast<float4 *>(dst + D) = make_float4(Mg, lgr, 0.f, 0.f);
            }
            Mg = -INFINITY;
            lgr = 0.f;
#pragma unroll
            for (int db = 0; db < P::DB; ++db)
                og[db] = f32x4_t{0.f, 0.f, 0.f, 0.f};
        }
    }

    if constexpr (FUSED) {
        if (live && ln.lr() < G) {
            uint16_t *dst = out + (int64_t)(tok0 + wave) * out_row_stride +
                            (int64_t)(g * G + ln.lr()) * D + 4 * ln.lg();
#pragma unroll
            for (int db = 0; db < P::DB; ++db)
                *reinterpret_cast<uint2 *>(dst + 16 * db) =
                    make_uint2(pack_bf16x2(ot[db][0] / lt, ot[db][1] / lt),
                               pack_bf16x2(ot[db][2] / lt, ot[db][3] / lt));
        }
    }
}

// One thread per 16-byte chunk of a (token, kv head) row.  K rows are stored
// token-major ([token][d]): the K chunk is copied whole.  V rows are stored
// head-dim-major ([d][token]): the V chunk's 8 values go to 8 rows of the page.
// Any head_dim (a multiple of 8) and page size.  32-bit index arithmetic: the host
// bounds tokens * hkv * (d / 8) below 2^31.
__global__ __launch_bounds__(256) void kv_append_kernel(
    const uint16_t *__restrict__ k_new, int64_t ks, const uint16_t *__restrict__ v_new, int64_t vs,
    const int32_t *__restrict__ slots, int tokens, uint16_t *__restrict__ k_cache,
    uint16_t *__restrict__ v_cache, int64_t num_pages, int hkv, int d, int page)
{
    const int cpr = d / 8;  // chunks per head row
    const int idx = (int)blockIdx.x * 256 + (int)threadIdx.x;
    if (idx >= tokens * hkv * cpr)
        return;
    const int t = idx / (hkv * cpr);
    const int h = (idx / cpr) % hkv;
    const int c = idx % cpr;
    const int64_t slot = slots[t];
    if (slot < 0 || slot >= num_pages * page)
        return;
    const int64_t pg = slot / page, off = slot % page;
    *reinterpret_cast<uint4 *>(k_cache + ((pg * hkv + h) * page + off) * d + 8 * c) =
        *reinterpret_cast<const uint4 *>(k_new + (int64_t)t * ks + h * d + 8 * c);
    const uint4 v = *reinterpret_cast<const uint4 *>(v_new + (int64_t)t * vs + h * d + 8 * c);
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
    uint16_t *vd = v_cache + ((pg * hkv + h) * d + 8 * c) * page + off;
#pragma unroll
    for (int e = 0; e < 8; ++e)
        vd[(int64_t)e * page] = (uint16_t)((e & 1) ? (w[e >> 1] >> 16) : (w[e >> 1] & 0xffffu));
}

// Page size 16 and head_dim up to 128: one workgroup of 16 * (d / 8) threads per
// (16 consecutive tokens, kv head), thread (t, c) holding chunk c of token t's row
// as in kv_append_kernel.  When the 16 tokens fill one page in order (a prompt
// chunk: slots page * 16 + 0 .. 15), their V chunks are transposed through LDS and
// each head-dim row of the page is written whole (32 bytes, two 16-byte stores)
// instead of as 16 separate 2-byte stores; otherwise (decode appends, ragged
// chunks) every thread stores its chunk's 8 values as kv_append_kernel does.
__global__ __launch_bounds__(256) void kv_append_page_kernel(
    const uint16_t *__restrict__ k_new, int64_t ks, const uint16_t *__restrict__ v_new, int64_t vs,
    const int32_t *__restrict__ slots, int tokens, uint16_t *__restrict__ k_cache,
    uint16_t *__restrict__ v_cache, int64_t num_pages, int hkv, int d)
{
    constexpr int T = 16;  // tokens per workgroup = page size
    __shared__ __attribute__((aligned(16))) uint16_t vt[T][128 + 8];
    __shared__ int broken;
    const int cpr = d / 8;
    const int t0 = (int)blockIdx.x * T, h = (int)blockIdx.y;
    const int t = (int)threadIdx.x / cpr, c = (int)threadIdx.x % cpr;
    const bool real = t0 + t < tokens;
    int64_t slot = real ? (int64_t)slots[t0 + t] : -1;
    if (slot >= num_pages * T)
        slot = -1;
    if (threadIdx.x == 0)
        broken = 0;
    __syncthreads();
    // the tile fills one page in order unless some token breaks the pattern
    const int64_t first = real ? (int64_t)slots[t0] : -1;
    if (c == 0 && (slot < 0 || first % T != 0 || slot != first + t || tokens - t0 < T))
        broken = 1;
    uint4 v = make_uint4(0, 0, 0, 0);
    const int64_t pg = slot / T, off = slot % T;
    if (slot >= 0) {
        *reinterpret_cast<uint4 *>(k_cache + ((pg * hkv + h) * T + off) * d + 8 * c) =
            *reinterpret_cast<const uint4 *>(k_new + (int64_t)(t0 + t) * ks + h * d + 8 * c);
        v = *reinterpret_cast<const uint4 *>(v_new + (int64_t)(t0 + t) * vs + h * d + 8 * c);
    }
    __syncthreads();  // broken settled
    if (!broken) {
        *reinterpret_cast<uint4 *>(&vt[t][8 * c]) = v;
        __syncthreads();
        uint16_t *vp = v_cache + (first / T * hkv + h) * (int64_t)d * T;
        for (int i = threadIdx.x; i < 2 * d; i += T * cpr) {  // row dd, tokens 8 * half ..
            const int dd = i >> 1, half = i & 1;
            uint32_t w[4];
#pragma unroll
            for (int j = 0; j < 4; ++j)
                w[j] = (uint32_t)vt[8 * half + 2 * j][dd] |
                       ((uint32_t)vt[8 * half + 2 * j + 1][dd] << 16);
            *reinterpret_cast<uint4 *>(vp + (int64_t)dd * T + 8 * half) =
                make_uint4(w[0], w[1], w[2], w[3]);
        }
    } else if (slot >= 0) {
        const uint32_t w[4] = {v.x, v.y, v.z, v.w};
        uint16_t *vd = v_cache + ((pg * hkv + h) * d + 8 * c) * T + off;
#pragma unroll
        for (int e = 0; e < 8; ++e)
            vd[e * T] = (uint16_t)((e & 1) ? (w[e >> 1] >> 16) : (w[e >> 1] & 0xffffu));
    }
}

// Floats of group (or split) partials in the decode workspace; the plan, when the
// split size has groups, follows them.
int64_t partial_floats(int64_t rows, int hq, int d, int max_kv_len, int split)
{
    const int64_t nsmax = ((int64_t)max_kv_len + split - 1) / split;
    const int64_t gs = splits_per_partial(split);
    return rows * hq * ((nsmax + gs - 1) / gs) * (int64_t)(d + 4);
}

// Compute units of the current device, looked up once per device.
int cu_count()
{
    constexpr int kDevMax = 64;
    static std::atomic<int> cache[kDevMax];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kDevMax)
        return 0;
    int n = cache[dev].load(std::memory_order_relaxed);
    if (n == 0) {
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
            return 0;
        cache[dev].store(n, std::memory_order_relaxed);
    }
    return n;
}

// Plan mode (whole rows, longest first) when the batch gives the compute units at
// least 1.5 (row, kv head) units each; below that a row's groups are spread over
// many workgroups instead.  Measured at the bench's lengths (U{1..32768}, 64q/4kv,
// d128, 256 CUs), plan against grid mode: batch 256 1469 vs 1745 us, 128 804 vs
// 898, 112 709 vs 788, 96 652 vs 691, 64 494 vs 481, 32 231 vs 223.  Only the
// schedule changes, never a bit of the output.
bool use_plan(int64_t rows, int hkv, int ncu)
{
    return ncu > 0 && ncu <= kPlanCuMax && 2 * rows * hkv >= 3 * (int64_t)ncu &&
           (rows + ncu / hkv + 1) * hkv < ((int64_t)1 << 22);  // the grid mode's x bound
}

template <int D>
hipError_t launch_attn_d(const AttnArgs &a, hipStream_t s)
{
    const int nsmax = (a.max_kv_len + a.split - 1) / a.split;
    const int gs = splits_per_partial(a.split);
    const int npmax = (nsmax + gs - 1) / gs;  // partials per (row, query head), at most
    const float scale_log2 = (float)((double)a.scale * 1.4426950408889634);
    const dim3 b1(WAVES * 64);
    const int32_t *row_chunks = nullptr;
    if (gs > 1) {
        const int ncu = cu_count();
        if (use_plan(a.rows, a.hkv, ncu)) {
            int32_t *plan = reinterpret_cast<int32_t *>(a.ws + partial_floats(a.rows, a.hq, a.d,
                                                                              a.max_kv_len, a.split));
            attn_plan_kernel<<<1, 1024, 0, s>>>(a.kv_lens, (int)a.rows, a.hkv, a.split,
                                                a.max_kv_len, ncu, plan);
            const int64_t items = a.rows + ncu / a.hkv + 1;
            attn_group_kernel<D, true><<<dim3((unsigned)(items * a.hkv)), b1, 0, s>>>(
                a.q, a.q_row_stride, a.k_cache, a.v_cache, a.block_table, a.bt_stride, a.kv_lens,
                a.hq, a.hkv, a.split, a.max_kv_len, npmax, (int)a.rows, plan, scale_log2, a.ws,
                a.out, a.out_row_stride);
            row_chunks = plan + kPlanHdr;
        } else {
            attn_group_kernel<D, false><<<dim3((unsigned)(npmax * a.hkv), 1, (unsigned)a.rows), b1, 0, s>>>(
                a.q, a.q_row_stride, a.k_cache, a.v_cache, a.block_table, a.bt_stride, a.kv_lens,
                a.hq, a.hkv, a.split, a.max_kv_len, npmax, (int)a.rows, nullptr, scale_log2, a.ws,
                a.out, a.out_row_stride);
        }
    } else
        attn_split_kernel<D><<<dim3((unsigned)(nsmax * a.hkv), 1, (unsigned)a.rows), b1, 0, s>>>(
            a.q, a.q_row_stride, a.k_cache, a.v_cache, a.block_table, a.bt_stride, a.kv_lens,
            a.hq, a.hkv, a.split, a.max_kv_len, nsmax, scale_log2, a.ws);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess)
        return e;
    const int64_t items = a.rows * a.hq;
    const dim3 g2((unsigned)((items + 3) / 4)), b2(256);
    attn_merge_kernel<D><<<g2, b2, 0, s>>>(a.ws, a.kv_lens, 0, a.rows, a.hq, a.hkv,
                                           a.split * gs, a.max_kv_len, npmax, row_chunks, a.out,
                                           a.out_row_stride);
    return hipGetLastError();
}

// The fused schedule needs enough token blocks to occupy the chip (one
// workgroup per compute unit); short chunks use the split schedule.
bool prefill_fused(int64_t tokens, int hkv, int d)
{
    (void)d;
    const int64_t blocks = (tokens + WAVES - 1) / WAVES;
    return blocks * hkv >= 256;
}

template <int D, bool FUSED>
hipError_t launch_prefill_sched(const PrefillArgs &a, hipStream_t s)
{
    const int nblk = (int)((a.tokens + WAVES - 1) / WAVES);
    const int nsmax = (int)((a.start + a.tokens + a.split - 1) / a.split);
    const int npmax = (nsmax + GROUP - 1) / GROUP;  // group partials per token, at most
    const float scale_log2 = (float)((double)a.scale * 1.4426950408889634);
    const dim3 blk(WAVES * 64);
    if constexpr (FUSED) {
        attn_prefill_kernel<D, true><<<dim3((unsigned)(nblk * a.hkv)), blk, 0, s>>>(
            a.q, a.q_row_stride, a.k_cache, a.v_cache, a.block_table_row, (int)a.start,
            (int)a.tokens, a.hq, a.hkv, a.split, scale_log2, a.out, a.out_row_stride, npmax,
            nullptr);
        return hipGetLastError();
    } else {
        attn_prefill_kernel<D, false>
            <<<dim3((unsigned)npmax, (unsigned)a.hkv, (unsigned)nblk), blk, 0, s>>>(
                a.q, a.q_row_stride, a.k_cache, a.v_cache, a.block_table_row, (int)a.start,
                (int)a.tokens, a.hq, a.hkv, a.split, scale_log2, a.out, a.out_row_stride,
                npmax, a.ws);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess)
            return e;
        const int64_t items = a.tokens * a.hq;
        attn_merge_kernel<D><<<dim3((unsigned)((items + 3) / 4)), dim3(256), 0, s>>>(
            a.ws, nullptr, (int)a.start, a.tokens, a.hq, a.hkv, a.split * GROUP,
            (int)(a.start + a.tokens), npmax, nullptr, a.out, a.out_row_stride);
        return hipGetLastError();
    }
}

template <int D>
hipError_t launch_prefill_d(const PrefillArgs &a, hipStream_t s)
{
    return prefill_fused(a.tokens, a.hkv, D) ? launch_prefill_sched<D, true>(a, s)
                                             : launch_prefill_sched<D, false>(a, s);
}

}  // namespace

size_t attn_workspace_bytes(int64_t rows, int hq, int d, int max_kv_len, int split)
{
    const int64_t plan = splits_per_partial(split) > 1 ? plan_words(rows) : 0;
    return (size_t)(partial_floats(rows, hq, d, max_kv_len, split) + plan) * sizeof(float);
}

hipError_t launch_decode_attn(const AttnArgs &a, hipStream_t s)
{
    return a.d == 128 ? launch_attn_d<128>(a, s) : launch_attn_d<64>(a, s);
}

size_t prefill_workspace_bytes(int64_t tokens, int hq, int hkv, int d, int64_t start, int split)
{
    if (prefill_fused(tokens, hkv, d))
        return 0;
    const int64_t nsmax = (start + tokens + split - 1) / split;
    return (size_t)(tokens * hq * ((nsmax + GROUP - 1) / GROUP)) * (size_t)(d + 4) * sizeof(float);
}

hipError_t launch_prefill_attn(const PrefillArgs &a, hipStream_t s)
{
    return a.d == 128 ? launch_prefill_d<128>(a, s) : launch_prefill_d<64>(a, s);
}

hipError_t launch_kv_append(const uint16_t *k_new, int64_t ks, const uint16_t *v_new, int64_t vs,
                            const int32_t *slots, int64_t tokens, uint16_t *k_cache,
                            uint16_t *v_cache, int64_t num_pages, int hkv, int d, int page,
                            hipStream_t s)
{
    if (page == 16 && d <= 128) {
        const dim3 grid((unsigned)((tokens + 15) / 16), (unsigned)hkv), block(16 * (d / 8));
        kv_append_page_kernel<<<grid, block, 0, s>>>(k_new, ks, v_new, vs, slots, (int)tokens,
                                                     k_cache, v_cache, num_pages, hkv, d);
        return hipGetLastError();
    }
    const int64_t n = tokens * hkv * (d / 8);
    const dim3 grid((unsigned)((n + 255) / 256)), block(256);
    kv_append_kernel<<<grid, block, 0, s>>>(k_new, ks, v_new, vs, slots, (int)tokens, k_cache,
                                            v_cache, num_pages, hkv, d, page);
    return hipGetLastError();
}

}  // namespace rbi
