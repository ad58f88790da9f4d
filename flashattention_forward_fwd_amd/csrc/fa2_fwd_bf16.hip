// fa2_fwd_bf16.hip -- FlashAttention-2 forward with 16-bit (bf16 or fp16) in/out,
// for gfx950: one kernel template serves the one-pass forward, the split-KV
// partials, the sliding window and dropout, at head dimensions 32 to 256.
//
// One work-group owns kBr = 128 query rows of one (batch, head) and streams the
// K/V tiles of that head through LDS (the Q-outer / KV-inner order and the
// sequence-length parallelism of "Flash Attention 全解析（上）" section 3.2.1).
// Each of its four wavefronts owns 32 of those rows and reads the same K/V tile
// (the "Sliced-Q" split of section 3.2.2: no reduction between wavefronts).
//
// Per K/V tile of kBc = 64 keys, one wavefront computes
//   S^T = K_j Q_i^T                      (bf16 MFMA 32x32x16, fp32 accumulate)
//   masked scores -> -inf                (only on tiles that cross the causal
//                                         diagonal or the end of the keys)
//   m'  = max(m, rowmax S * c)           (c = scale * log2 e, base-2 domain)
//   P~  = 2^(S c - m'),  alpha = 2^(m - m')
//   l   = alpha l + rowsum P~,  O~^T = alpha O~^T + V_j^T P~^T   (bf16 MFMA)
// and after the last tile O = O~ / l and LSE = (m + log2 l) ln 2 -- the online
// softmax update of "FlashAttention 怎么做? online softmax 怎么更新?" section
// "推导 / 关键公式", with the division deferred to the end as in
// "FlashAttention-2 算法架构升级" section 一.2.
//
// MI355X-specific choices:
//  * K and V tiles go from HBM straight into LDS with asynchronous 16-byte
//    buffer loads (LDS DMA, no register staging), double-buffered, one barrier
//    per tile; rows past Lk lie outside the buffer range and arrive as zeros.
//    Each 1 KiB transfer lands contiguously, so bank spreading is done by an XOR
//    swizzle of the 16-byte chunks within a row, chosen at load time.
//  * Software pipelining inside the wavefront: the exponentials of tile j run
//    on the VALU while the MFMA unit computes the scores of tile j+1, and the
//    max of tile j+1 is taken while the P~V product of tile j runs.  K is
//    loaded two tiles ahead, V one.
//  * Scores are computed transposed (keys down the MFMA rows, queries across the
//    lanes).  A lane then holds 16 keys of ONE query per 32x32 accumulator, so
//    the row max / row sum need one exchange between the two wavefront halves,
//    alpha is per lane, and the accumulator is already the B operand of the
//    P~V product.
//  * V stays row-major in LDS; the A operand of the P~V product (8 keys of one
//    d column per lane) is read with the gfx950 transposing LDS read
//    (ds_read_b64_tr_b16), two reads of 4 keys each.
//  * Q stays in registers for the whole K/V loop (read from HBM once).
#include "fa2_internal.h"

namespace fa2 {
namespace {

// The kernels run on bf16 (E = __bf16) or fp16 (E = _Float16) inputs: 8- and
// 4-element vectors of E, and the 32x32x16 matrix-core product for each.
template <typename E> struct V16 {
    typedef E x8 __attribute__((ext_vector_type(8)));
    typedef E x4 __attribute__((ext_vector_type(4)));
};
typedef V16<__bf16>::x8 bf16x8;
typedef V16<_Float16>::x8 f16x8;
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ f32x16 mfma_32x32x16(bf16x8 a, bf16x8 b, f32x16 c)
{
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x16 mfma_32x32x16(f16x8 a, f16x8 b, f32x16 c)
{
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
}

#define LDS_AS __attribute__((address_space(3)))

// d = 96: a row is 192 bytes in HBM but takes a d = 128 row (256 bytes) in LDS,
// so the 1 KiB transfers, the swizzles and the transposing reads of d = 128
// apply unchanged; the four chunks past column 95 are never loaded or read.
template <int D> struct Tile {
    static constexpr int kLdsD = D == 96 ? 128 : D;          // row length in LDS
    static constexpr int kRowBytes = 2 * kLdsD;              // one K or V row in LDS, 16-bit
    static constexpr int kGRowBytes = 2 * D;                 // one K or V row in HBM
    static constexpr int kChunks = kRowBytes / 16;           // 16-byte chunks per LDS row
    static constexpr int kGChunks = kGRowBytes / 16;         // ... that hold data
    static constexpr int kRowsPerXfer = 1024 / kRowBytes;    // rows per 1 KiB wave transfer
    static constexpr int kXfersPerWave = kBc * kRowBytes / 1024 / kWaves;
    static constexpr int kBytes = kBc * kRowBytes;           // one tile in LDS
    static constexpr int kGBytes = kBc * kGRowBytes;         // one tile in HBM
    // K swizzle repeats every kKPeriod transfers (see swz_k), V swizzle every
    // kVPeriod (d = 256: a transfer holds two rows, the V swizzle spans four).
    static constexpr int kKPeriod = kLdsD == 256 ? 8 : kLdsD == 128 ? 4 : kLdsD == 64 ? 2 : 1;
    static constexpr int kVPeriod = kLdsD == 256 ? 2 : 1;
    static constexpr int kElems = kBc * kLdsD;               // elements per LDS tile
    static_assert(kXfersPerWave * kWaves * 1024 == kBc * kRowBytes, "tile must split into 1 KiB transfers");
    static_assert(kXfersPerWave % kKPeriod == 0 && kXfersPerWave % kVPeriod == 0,
                  "a wave's transfers must start at a swizzle period");

    // K: chunk q of row r is stored at chunk q ^ swz_k(r).  The score MFMA reads
    // the same logical chunk from 32 consecutive rows; this spreads any 256
    // consecutive bytes of those reads over all 64 banks (d = 64: two rows, and
    // d = 32: four rows, share a 256-byte line; the row within the line already
    // separates them, the swizzle separates the lines; d = 256: each row spans
    // two lines, the swizzle moves the chunk within the row's first 16).
    static __device__ __forceinline__ int swz_k(int r)
    {
        return kLdsD >= 128 ? (r & 15) : kLdsD == 64 ? ((r >> 1) & 7) : ((r >> 2) & 3);
    }
    // V: the transposing read takes 64 consecutive bytes (4 chunks) from each of
    // 4 consecutive rows; moving each row's 4-chunk group to a different
    // 64-byte bank group keeps those 4 rows conflict-free (d = 32: the 4 rows
    // are one 256-byte line already).
    static __device__ __forceinline__ int swz_v(int r)
    {
        return kLdsD >= 128 ? 4 * (r & 3) : kLdsD == 64 ? 4 * ((r >> 1) & 1) : 0;
    }
};

// Buffer-resource word 3 for raw (unswizzled, unformatted) buffer access on gfx9.
constexpr int kRawBufferFlags = 0x00020000;

// Per-lane byte offsets of the tile loads.  Transfer x of wavefront w moves
// 1 KiB block b = w * kXfersPerWave + x of the LDS tile; lane l lands at byte
// 16 l of the block, i.e. row b * kRowsPerXfer + l / kChunks, physical chunk
// l % kChunks, and reads that row's logical chunk from HBM (offsets from the
// first row of its swizzle period).  The K swizzle depends on b % kKPeriod, the
// V swizzle on b % kVPeriod.  d = 96: a lane whose logical chunk lies past
// column 95 loads nothing (k_on / v_on false).
template <int D> struct LoadOffsets {
    int k[Tile<D>::kKPeriod];
    int v[Tile<D>::kVPeriod];
    bool k_on[Tile<D>::kKPeriod];
    bool v_on[Tile<D>::kVPeriod];
};

template <int D>
__device__ __forceinline__ LoadOffsets<D> load_offsets(int lane)
{
    using T = Tile<D>;
    LoadOffsets<D> o;
    const int phys = lane % T::kChunks;
#pragma unroll
    for (int b = 0; b < T::kKPeriod; ++b) {
        const int row = b * T::kRowsPerXfer + lane / T::kChunks;
        const int logical = phys ^ T::swz_k(row);
        o.k[b] = row * T::kGRowBytes + 16 * logical;
        o.k_on[b] = T::kGChunks == T::kChunks || logical < T::kGChunks;
    }
#pragma unroll
    for (int b = 0; b < T::kVPeriod; ++b) {
        const int row = b * T::kRowsPerXfer + lane / T::kChunks;
        const int logical = phys ^ T::swz_v(row);
        o.v[b] = row * T::kGRowBytes + 16 * logical;
        o.v_on[b] = T::kGChunks == T::kChunks || logical < T::kGChunks;
    }
    return o;
}

// Issue this wavefront's share of the asynchronous HBM -> LDS copy of tile
// `tile` of K (IS_V false) or V.  Rows past Lk lie outside the buffer range
// and arrive as zeros; their keys are masked to -inf.
template <int D, bool IS_V>
__device__ __forceinline__ void load_tile_async(__amdgpu_buffer_rsrc_t src, int tile, uint16_t *dst,
                                                int wave, const LoadOffsets<D> &off)
{
    using T = Tile<D>;
#pragma unroll
    for (int x = 0; x < T::kXfersPerWave; ++x) {
        const int b = wave * T::kXfersPerWave + x;
        const int voff = IS_V ? off.v[x % T::kVPeriod] : off.k[x % T::kKPeriod];
        const bool on = IS_V ? off.v_on[x % T::kVPeriod] : off.k_on[x % T::kKPeriod];
        const int row0 = (IS_V ? b - b % T::kVPeriod : b - b % T::kKPeriod) * T::kRowsPerXfer;
        const int soff = tile * T::kGBytes + row0 * T::kGRowBytes;
        if (on) __builtin_amdgcn_raw_ptr_buffer_load_lds(src, (LDS_AS void *)(dst + b * 512), 16, voff, soff, 0, 0);
    }
}

// Where a step issues the copies of the next tiles: at its start, or (d = 64)
// after its P~V products, from a closure the loop passes in.  Measured on MI355X,
// the d = 64 loop written that way compiles to 156 VGPRs instead of 210, so three
// work-groups share a CU (LDS allows it at d = 64), and runs 8-11 % faster; the
// same form costs up to 3 % at d = 32 and 3-20 % at d >= 96 (issued late), so
// every other head dimension keeps the copies at the start of the step.
template <int D> constexpr bool kLateTileLoads = D == 64;
struct NoTileLoads {
    __device__ void operator()() const {}
};

// Threshold (base-2 units) for moving the running max.  While a row's max has
// not grown by more than this, the old reference max is kept: P~ = 2^(S c - m)
// is then at most 2^2, l and O~ keep the same reference, and nothing is
// rescaled.  O = O~ / l and LSE = m + log2 l are unchanged by the choice of m,
// but the rounding is not: P~ enters the P~V product rounded to 16 bits while l
// sums it unrounded, so when one key dominates a row, O carries that key's
// rounding error (up to 2^-8 relative) unless its P~ is exactly 1, i.e. the
// reference is the row's true max.  A small threshold moves the reference to
// the true max more often; measured on MI355X, 2 instead of 8 halves the worst
// O error on large score ranges (Q x 4: 1.66e-2 -> 0.97e-2) for about 1 % of
// time on N(0, 1) inputs, where the max rarely grows that much after the first
// tile.
constexpr float kRescaleThreshold = 2.0f;

// S^T = K_j Q_i^T for one wavefront: two 32x32 tiles of (keys x queries).
template <int D, typename E>
__device__ __forceinline__ void scores(const LDS_AS char *kb, const typename V16<E>::x8 (&qf)[D / 16],
                                       f32x16 (&s)[2], int k_lane)
{
    using e8 = typename V16<E>::x8;
    using T = Tile<D>;
#pragma unroll
    for (int t = 0; t < 2; ++t) {
        s[t] = f32x16{};
#pragma unroll
        for (int c = 0; c < D / 16; ++c) {
            const int off = (32 * t * T::kRowBytes + k_lane) ^ (32 * c);
            const e8 a = *reinterpret_cast<const LDS_AS e8 *>(kb + off);
            s[t] = mfma_32x32x16(a, qf[c], s[t]);
        }
    }
}

// Keys past Lk, (causal) keys after the lane's query and (window) keys outside
// [qrow - wl, qrow + wr] get -inf.  Element (t, i) of this lane holds key
// k0 + 4 hh + off(t, i), off = 32 t + 8 (i / 4) + i % 4; without a window the
// visible keys are those up to one last key, so each element costs one compare
// of the constant off against a per-lane limit and one select.
template <bool CAUSAL, bool WINDOW>
__device__ __forceinline__ void mask_scores(f32x16 (&s)[2], int k0, int Lk, int qrow, int hh, int wl, int wr)
{
    if (!WINDOW) {
        const int last = CAUSAL ? min(qrow, Lk - 1) : Lk - 1;      // last visible key
        const int lim = last - k0 - 4 * hh;
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
            for (int i = 0; i < 16; ++i)
                s[t][i] = 32 * t + 8 * (i / 4) + (i % 4) > lim ? -INFINITY : s[t][i];
        return;
    }
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const int key = k0 + 32 * t + 8 * (i / 4) + 4 * hh + (i % 4);
            bool hidden = key >= Lk || (CAUSAL && key > qrow);
            hidden = hidden || (wl >= 0 && key < qrow - wl) || (wr >= 0 && key > qrow + wr);
            s[t][i] = hidden ? -INFINITY : s[t][i];
        }
}

// Row max (base-2 units) of a score tile: this lane's 32 keys, then the other half's.
__device__ __forceinline__ float row_max_scaled(const f32x16 (&s)[2], float c2)
{
    float mx = s[0][0];
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int i = 0; i < 16; ++i)
            mx = fmaxf(mx, s[t][i]);
    mx = halves_max(mx);
    return mx * c2;
}

// Moves the reference max when some row of the wavefront grew past the
// threshold, and rescales O~ and l by alpha = 2^(m - m') right there: the branch
// is the same on every lane and rarely taken, so the common step spends no
// exponential or select on it.
// EMPTY_ROWS: a row may have seen no visible key yet (m = -inf; only in a
// causal K/V range that starts after some of the wavefront's rows).  Such a
// row keeps m = -inf and alpha = 1 until its first visible key arrives.
template <int D, bool EMPTY_ROWS>
__device__ __forceinline__ void update_max(float &m, float m_tile, f32x16 (&acc_o)[D / 32], float &lpart)
{
    const float m_cand = fmaxf(m, m_tile);
    if (__builtin_amdgcn_ballot_w64(m_cand - m > kRescaleThreshold) == 0) return;
    float alpha = __builtin_amdgcn_exp2f(m - m_cand);
    if (EMPTY_ROWS && m_cand == -INFINITY) alpha = 1.0f;
    m = m_cand;
    lpart *= alpha;
#pragma unroll
    for (int t = 0; t < D / 32; ++t)
        acc_o[t] *= alpha;
}

// The max the probabilities are taken against: a row that has seen no visible
// key (m = -inf, all its scores -inf) uses 0, so its probabilities are 0.
template <bool EMPTY_ROWS>
__device__ __forceinline__ float reference_max(float m)
{
    return (EMPTY_ROWS && m == -INFINITY) ? 0.0f : m;
}

// Dropout keep bytes of one score tile for this lane (the lane's query qrow is
// q0 + lane % 32 with q0 a multiple of 32, so qrow % 4 == lane % 4).
template <bool DROPOUT>
__device__ __forceinline__ DropMask tile_mask(const DropoutParams &dp, int k0, int qrow, int lane, int bh)
{
    if (DROPOUT) return mask_query_lanes(dp, k0, qrow, lane, bh);
    return DropMask{};
}

// P~ = 2^(S c - m) as bf16 B operands (one per 16-key chunk: slots 0-3 are keys
// 16c + 4hh + 0..3, slots 4-7 keys 16c + 8 + 4hh + 0..3), and its row sum.
// DROPOUT: the row sum is taken before the mask; dropped entries become 0 in the
// operands (the 1 / keep-rate factor is applied to O at the end).
template <typename E, bool DROPOUT = false>
__device__ __forceinline__ float probabilities(const f32x16 (&s)[2], float c2, float m, typename V16<E>::x8 (&pf)[4],
                                               const DropMask &mk = DropMask{}, uint32_t thr = 256)
{
    float rs = 0.f;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
        const int t = c >> 1, i0 = 8 * (c & 1);
        f32x8 v8;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            v8[e] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[t][i0 + e], c2, -m));
            rs += v8[e];
            if (DROPOUT) v8[e] = keep(mk, t, i0 + e, thr) ? v8[e] : 0.0f;
        }
        pf[c] = __builtin_convertvector(v8, typename V16<E>::x8);
    }
    return rs;
}

// O~^T += V_j^T P~^T; the A operand of chunk c is two transposing reads
// (keys 16c + 4hh + 0..3 and 16c + 8 + 4hh + 0..3).
template <int D, typename E>
__device__ __forceinline__ void accumulate_pv(const LDS_AS char *vb, const typename V16<E>::x8 (&pf)[4],
                                              f32x16 (&acc_o)[D / 32], int v_lane)
{
    using e8 = typename V16<E>::x8;
    using T = Tile<D>;
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            const int off0 = (16 * c * T::kRowBytes + v_lane) ^ (64 * dt);
            const int off1 = off0 + 8 * T::kRowBytes;
            const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS_AS i16x4 *)(vb + off0));
            const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS_AS i16x4 *)(vb + off1));
            const e8 a = __builtin_bit_cast(e8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
            acc_o[dt] = mfma_32x32x16(a, pf[c], acc_o[dt]);
        }
}

// One step of the pipelined loop for tile j: probabilities of tile j (VALU)
// while the scores of tile j+1 run (MFMA), then O~ += P~_j V_j (MFMA) while the
// max of tile j+1 is taken (VALU).  Where kLateTileLoads<D>, the step issues the
// copies of the next tiles (late_loads) after its P~V products; otherwise the
// caller has issued them before the step.
template <int D, typename E, bool CAUSAL, bool EMPTY_ROWS, bool WINDOW, bool DROPOUT,
          typename Loads = NoTileLoads>
__device__ __forceinline__ void pipelined_step(Loads &&late_loads, const LDS_AS char *k_next, const LDS_AS char *v_cur,
                                               const typename V16<E>::x8 (&qf)[D / 16], f32x16 (&acc_o)[D / 32],
                                               f32x16 (&s_cur)[2], float &m, float &lpart,
                                               float c2, int j, int t0, int plain_lo, int n_plain, int Lk,
                                               int qrow, int hh, int k_lane, int v_lane, int wl, int wr,
                                               const DropoutParams &dp, int lane, int bh)
{
    typename V16<E>::x8 pf[4];
    const DropMask mk = tile_mask<DROPOUT>(dp, (t0 + j) * kBc, qrow, lane, bh);
    const float rs = probabilities<E, DROPOUT>(s_cur, c2, reference_max<EMPTY_ROWS>(m), pf, mk, dp.threshold);
    f32x16 s_next[2];
    scores<D, E>(k_next, qf, s_next, k_lane);
    accumulate_pv<D, E>(v_cur, pf, acc_o, v_lane);
    if constexpr (kLateTileLoads<D>) late_loads();
    float mt = row_max_scaled(s_next, c2);
    // The row sum and the next max are consumed after the branch below; this
    // use keeps their VALU work in this block, between the MFMAs, instead of
    // letting it sink past the branch where nothing overlaps it.
    asm volatile("" ::"v"(rs), "v"(mt));
    lpart += rs;
    // Tiles on the causal diagonal, a window edge or the key tail (few): mask,
    // take the max again.
    if (j + 1 >= n_plain || (WINDOW && j + 1 < plain_lo)) {
        mask_scores<CAUSAL, WINDOW>(s_next, (t0 + j + 1) * kBc, Lk, qrow, hh, wl, wr);
        mt = row_max_scaled(s_next, c2);
    }
    update_max<D, EMPTY_ROWS>(m, mt, acc_o, lpart);
    s_cur[0] = s_next[0];
    s_cur[1] = s_next[1];
}

// SPLIT: the work-group covers one of p.n_splits contiguous ranges of its
// query tile's K/V tiles and writes the fp32 partial O (normalised by its own
// row sum) and partial LSE of that range; rows that see no key of the range
// get LSE = -inf and no O.  Otherwise it covers all tiles and writes bf16 O.
// D = 256: the Q fragment (64 VGPRs) and the O accumulators (128) leave no room
// for two wavefronts per SIMD, so that instance runs one wavefront per SIMD with
// the accumulation registers in use (and one work-group per CU: 128 KiB of LDS).
// WINDOW (with CAUSAL and SPLIT false): key j is visible to query i iff
// (p.wl < 0 or j >= i - p.wl) and (p.wr < 0 or j <= i + p.wr); the work-group
// visits only the tiles that hold a key visible to one of its rows, and a row
// that sees no key gets O = 0 and LSE = -inf.
// DROPOUT (SPLIT and WINDOW false): each probability is kept iff its generator
// byte is below p.drop.threshold (the keep mask of tile_mask), and O is scaled by
// p.drop.keep_scale; m, l and the LSE are those without dropout.
template <int D, bool CAUSAL, bool SPLIT, bool WINDOW = false, typename E = __bf16, bool DROPOUT = false>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(D == 256 ? 1 : 2)))
void fa2_fwd_bf16_kernel(FwdParams p)
{
    using T = Tile<D>;
    using e8 = typename V16<E>::x8;
    using e4 = typename V16<E>::x4;
    static_assert(!WINDOW || (!CAUSAL && !SPLIT), "the window replaces the causal mask; no split");
    static_assert(!DROPOUT || (!SPLIT && !WINDOW), "dropout runs in the one-pass forward only");
    // Rows without a visible key in a visited tile range: a causal range that
    // starts after tile 0, or a window (rows at a window edge of the block).
    constexpr bool kEmptyRows = (SPLIT && CAUSAL) || WINDOW;
    constexpr int kDc = D / 16;          // 16-wide d chunks of the QK^T product
    constexpr int kDt = D / 32;          // 32-row d tiles of the output
    // Tile t of K lives in sK0 / sK1 by the parity of t, same for V.  Four
    // separate variables (not one array) let the compiler see that reading one
    // buffer does not depend on a transfer into another, so it does not wait
    // for the transfers in flight before every LDS read.
    __shared__ __attribute__((aligned(1024))) uint16_t sK0[T::kElems];
    __shared__ __attribute__((aligned(1024))) uint16_t sK1[T::kElems];
    __shared__ __attribute__((aligned(1024))) uint16_t sV0[T::kElems];
    __shared__ __attribute__((aligned(1024))) uint16_t sV1[T::kElems];

    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
    const int lane = tid % kWave;
    const int l32 = lane & 31;
    const int hh = lane >> 5;

    int bh, qt, split = 0;
    if (SPLIT) {
        split = blockIdx.x % p.n_splits;
        map_workgroup(blockIdx.x / p.n_splits, p.n_wg / p.n_splits, p.n_qtiles, bh, qt);
    } else {
        map_workgroup(blockIdx.x, p.n_wg, p.n_qtiles, bh, qt);
    }
    const int n_kv_all = kv_tiles_for(qt, p.Lq, p.Lk, CAUSAL);
    // This work-group's K/V tiles: [t0, t0 + n_kv).
    int t0 = SPLIT ? (int)((int64_t)split * n_kv_all / p.n_splits) : 0;
    int n_kv = SPLIT ? (int)((int64_t)(split + 1) * n_kv_all / p.n_splits) - t0 : n_kv_all;
    if (WINDOW) {
        // Keys visible to some row of the block: [key_lo, key_hi).
        const int q_first = qt * kBr;
        const int q_last = min(q_first + kBr - 1, p.Lq - 1);
        const int64_t key_lo = p.wl < 0 ? 0 : max((int64_t)0, (int64_t)q_first - p.wl);
        const int64_t key_hi = p.wr < 0 ? p.Lk : min((int64_t)p.Lk, (int64_t)q_last + p.wr + 1);
        t0 = 0;
        n_kv = 0;
        if (key_hi > key_lo) {
            t0 = (int)(key_lo / kBc);
            n_kv = (int)((key_hi + kBc - 1) / kBc) - t0;
        }
    }
    // Partial-result row of (split, bh, query 0 of this head).
    const size_t part_row0 = ((size_t)split * p.B * p.H + bh) * p.Lq;
    if (SPLIT && n_kv == 0) {                 // empty range: every row is empty
        const int r = qt * kBr + tid;
        if (tid < kBr && r < p.Lq) p.lse[part_row0 + r] = -INFINITY;
        return;
    }

    const uint16_t *Q = static_cast<const uint16_t *>(p.q) + (size_t)bh * p.Lq * D;
    const size_t kv_off = (size_t)bh * p.Lk * D;
    const __amdgpu_buffer_rsrc_t rK = __builtin_amdgcn_make_buffer_rsrc(
        (void *)(static_cast<const uint16_t *>(p.k) + kv_off), 0, p.Lk * T::kGRowBytes, kRawBufferFlags);
    const __amdgpu_buffer_rsrc_t rV = __builtin_amdgcn_make_buffer_rsrc(
        (void *)(static_cast<const uint16_t *>(p.v) + kv_off), 0, p.Lk * T::kGRowBytes, kRawBufferFlags);
    const LoadOffsets<D> loff = load_offsets<D>(lane);

    const int q0 = qt * kBr + wave * kRowsPerWave;    // first row of this wavefront
    const int qrow = q0 + l32;                        // this lane's query row
    const bool wave_active = q0 < p.Lq;               // wave-uniform

    // Tiles this wavefront computes, counted from t0: [0, n_plain) need no mask,
    // [n_plain, n_wave) cross the causal diagonal or the end of the keys; the
    // work-group's other tiles are masked for all of its rows (it only helps
    // load them).  Window: [plain_lo, n_plain) need no mask, the tiles before
    // plain_lo cross the left edge of some row's window.
    int n_wave = 0, n_plain = 0, plain_lo = 0;
    if (WINDOW) {
        if (wave_active) {
            const int wave_qlast = min(q0 + kRowsPerWave - 1, p.Lq - 1);
            int end = t0 + n_kv;
            if (p.wr >= 0) end = (int)min((int64_t)end, ((int64_t)wave_qlast + p.wr) / kBc + 1);
            n_wave = max(end - t0, 0);
            // A tile needs no mask when the window of every row of the wave holds it.
            const int64_t left = p.wl < 0 ? 0 : (int64_t)wave_qlast - p.wl;     // last row's left edge
            const int64_t first_plain = left <= 0 ? 0 : (left + kBc - 1) / kBc;
            int64_t end_plain = p.Lk / kBc;
            if (p.wr >= 0) end_plain = min(end_plain, ((int64_t)q0 + p.wr + 1) / kBc);
            plain_lo = (int)min(max(first_plain - t0, (int64_t)0), (int64_t)n_wave);
            n_plain = (int)min(max(end_plain - t0, (int64_t)0), (int64_t)n_wave);
        }
    } else if (wave_active) {
        const int wave_qlast = min(q0 + kRowsPerWave - 1, p.Lq - 1);
        const int end = CAUSAL ? min(t0 + n_kv, wave_qlast / kBc + 1) : t0 + n_kv;
        int plain = min(end, p.Lk / kBc);
        if (CAUSAL) plain = min(plain, (q0 + 1) / kBc);
        n_wave = max(end - t0, 0);
        n_plain = min(max(plain - t0, 0), n_wave);
    }

    // Local tile j (global tile t0 + j) of K lives in sK[j % 2], of V in
    // sV[j % 2].  Iteration j reads K_{j+1} (next scores) and V_j, and loads
    // K_{j+2} and V_{j+1}.
    load_tile_async<D, false>(rK, t0, sK0, wave, loff);
    load_tile_async<D, true>(rV, t0, sV0, wave, loff);
    if (n_kv > 1)
        load_tile_async<D, false>(rK, t0 + 1, sK1, wave, loff);

    // Q fragment: lane holds Q[qrow][16c + 8hh .. +7] for every chunk c.
    e8 qf[kDc];
#pragma unroll
    for (int c = 0; c < kDc; ++c) {
        u32x4 raw = {0u, 0u, 0u, 0u};
        if (qrow < p.Lq)
            raw = *reinterpret_cast<const u32x4 *>(Q + (size_t)qrow * D + 16 * c + 8 * hh);
        qf[c] = __builtin_bit_cast(e8, raw);
    }

    // Per-lane LDS byte offsets.
    // K (score A operand): row 32t + l32, logical chunk 2c + hh.  Because 2c and
    // hh occupy different bits, chunk (2c + hh) ^ s == 2c ^ (hh ^ s).
    const int k_lane = l32 * T::kRowBytes + 16 * (hh ^ T::swz_k(l32));
    // V (transposing read): lane = 16g + 4e + r supplies row 4(g/2) + e (plus the
    // chunk/read offset), columns 16(g%2) + 4r of d tile dt.
    const int vg = lane >> 4, ve = (lane >> 2) & 3, vr = lane & 3;
    const int v_row = 4 * (vg >> 1) + ve;
    const int v_lane = v_row * T::kRowBytes + 64 * (T::swz_v(v_row) >> 2) + 32 * (vg & 1) + 8 * vr;

    f32x16 acc_o[kDt];
#pragma unroll
    for (int t = 0; t < kDt; ++t)
        acc_o[t] = f32x16{};
    float m = -INFINITY;     // reference max (base-2 units), per query row
    float lpart = 0.f;       // running sum over this lane's half of the keys
    const float c2 = p.scale_log2;

    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();

    // Scores of the first tile.  Its max becomes the reference (O~ and l are 0).
    f32x16 s_cur[2];
    if (n_wave > 0) {
        scores<D, E>((const LDS_AS char *)sK0, qf, s_cur, k_lane);
        if (n_plain == 0 || (WINDOW && plain_lo > 0))
            mask_scores<CAUSAL, WINDOW>(s_cur, t0 * kBc, p.Lk, qrow, hh, p.wl, p.wr);
        m = row_max_scaled(s_cur, c2);
    }
    __syncthreads();                          // sK0 may now be refilled

    // Every wavefront passes the same n_kv barriers.  The pipelined loop is
    // unrolled over two tiles so each buffer is fixed at compile time.
    int j = 0;
    if constexpr (kLateTileLoads<D>) {
        while (j + 1 < n_wave) {
            // as below, with the copies of the next tiles issued inside the step
            auto loads_even = [&]() {
                if (j + 2 < n_kv) load_tile_async<D, false>(rK, t0 + j + 2, sK0, wave, loff);
                load_tile_async<D, true>(rV, t0 + j + 1, sV1, wave, loff);
            };
            pipelined_step<D, E, CAUSAL, kEmptyRows, WINDOW, DROPOUT>(loads_even,
                (const LDS_AS char *)sK1, (const LDS_AS char *)sV0, qf, acc_o, s_cur, m, lpart, c2, j, t0,
                plain_lo, n_plain, p.Lk, qrow, hh, k_lane, v_lane, p.wl, p.wr, p.drop, lane, bh);
            __builtin_amdgcn_s_waitcnt(0);
            __syncthreads();
            if (++j + 1 >= n_wave) break;
            auto loads_odd = [&]() {
                if (j + 2 < n_kv) load_tile_async<D, false>(rK, t0 + j + 2, sK1, wave, loff);
                load_tile_async<D, true>(rV, t0 + j + 1, sV0, wave, loff);
            };
            pipelined_step<D, E, CAUSAL, kEmptyRows, WINDOW, DROPOUT>(loads_odd,
                (const LDS_AS char *)sK0, (const LDS_AS char *)sV1, qf, acc_o, s_cur, m, lpart, c2, j, t0,
                plain_lo, n_plain, p.Lk, qrow, hh, k_lane, v_lane, p.wl, p.wr, p.drop, lane, bh);
            __builtin_amdgcn_s_waitcnt(0);
            __syncthreads();
            ++j;
        }
    } else {
    while (j + 1 < n_wave) {
        // even tile j: K_{j+1} in sK1, V_j in sV0; loads K_{j+2} -> sK0, V_{j+1} -> sV1
        if (j + 2 < n_kv) load_tile_async<D, false>(rK, t0 + j + 2, sK0, wave, loff);
        load_tile_async<D, true>(rV, t0 + j + 1, sV1, wave, loff);
        pipelined_step<D, E, CAUSAL, kEmptyRows, WINDOW, DROPOUT>(NoTileLoads{},
            (const LDS_AS char *)sK1, (const LDS_AS char *)sV0, qf, acc_o, s_cur, m, lpart, c2, j, t0,
            plain_lo, n_plain, p.Lk, qrow, hh, k_lane, v_lane, p.wl, p.wr, p.drop, lane, bh);
        __builtin_amdgcn_s_waitcnt(0);        // this wave's loads have landed
        __syncthreads();                      // ... everyone's, and the read buffers are free
        if (++j + 1 >= n_wave) break;
        // odd tile j: K_{j+1} in sK0, V_j in sV1; loads K_{j+2} -> sK1, V_{j+1} -> sV0
        if (j + 2 < n_kv) load_tile_async<D, false>(rK, t0 + j + 2, sK1, wave, loff);
        load_tile_async<D, true>(rV, t0 + j + 1, sV0, wave, loff);
        pipelined_step<D, E, CAUSAL, kEmptyRows, WINDOW, DROPOUT>(NoTileLoads{},
            (const LDS_AS char *)sK0, (const LDS_AS char *)sV1, qf, acc_o, s_cur, m, lpart, c2, j, t0,
            plain_lo, n_plain, p.Lk, qrow, hh, k_lane, v_lane, p.wl, p.wr, p.drop, lane, bh);
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
        ++j;
    }
    }
    if (j < n_wave) {                         // last computed tile: no next scores
        const bool odd = j & 1;
        if (j + 2 < n_kv) load_tile_async<D, false>(rK, t0 + j + 2, odd ? sK1 : sK0, wave, loff);
        if (j + 1 < n_kv) load_tile_async<D, true>(rV, t0 + j + 1, odd ? sV0 : sV1, wave, loff);
        e8 pf[4];
        const DropMask mk = tile_mask<DROPOUT>(p.drop, (t0 + j) * kBc, qrow, lane, bh);
        lpart += probabilities<E, DROPOUT>(s_cur, c2, reference_max<kEmptyRows>(m), pf, mk, p.drop.threshold);
        accumulate_pv<D, E>((const LDS_AS char *)(odd ? sV1 : sV0), pf, acc_o, v_lane);
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
        ++j;
    }
    for (; j < n_kv; ++j) {                   // this wave only helps load
        const bool odd = j & 1;
        if (j + 2 < n_kv) load_tile_async<D, false>(rK, t0 + j + 2, odd ? sK1 : sK0, wave, loff);
        if (j + 1 < n_kv) load_tile_async<D, true>(rV, t0 + j + 1, odd ? sV0 : sV1, wave, loff);
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
    }

    if (!wave_active) return;
    const float l = halves_sum(lpart);
    if (qrow >= p.Lq) return;
    if (SPLIT) {
        float lse = -INFINITY;
        if (l > 0.0f) {                       // the row saw a key of this range
            const float inv_l = 1.0f / l;
            float *Op = static_cast<float *>(p.o) + (part_row0 + qrow) * D;
#pragma unroll
            for (int dt = 0; dt < kDt; ++dt)
#pragma unroll
                for (int a = 0; a < 4; ++a) {
                    const f32x4 v4 = {acc_o[dt][4 * a + 0] * inv_l, acc_o[dt][4 * a + 1] * inv_l,
                                      acc_o[dt][4 * a + 2] * inv_l, acc_o[dt][4 * a + 3] * inv_l};
                    *reinterpret_cast<f32x4 *>(Op + 32 * dt + 8 * a + 4 * hh) = v4;
                }
            lse = (m + __builtin_amdgcn_logf(l)) * kLn2;
        }
        if (hh == 0) p.lse[part_row0 + qrow] = lse;
        return;
    }
    // A window can leave a row without a visible key: O = 0, LSE = -inf.
    const bool seen = !WINDOW || l > 0.0f;
    const float inv_l = seen ? (DROPOUT ? p.drop.keep_scale : 1.0f) / l : 0.0f;
    uint16_t *O = static_cast<uint16_t *>(p.o) + ((size_t)bh * p.Lq + qrow) * D;
#pragma unroll
    for (int dt = 0; dt < kDt; ++dt)
#pragma unroll
        for (int a = 0; a < 4; ++a) {
            const f32x4 v4 = {acc_o[dt][4 * a + 0] * inv_l, acc_o[dt][4 * a + 1] * inv_l,
                              acc_o[dt][4 * a + 2] * inv_l, acc_o[dt][4 * a + 3] * inv_l};
            const e4 b4 = __builtin_convertvector(v4, e4);
            *reinterpret_cast<e4 *>(O + 32 * dt + 8 * a + 4 * hh) = b4;
        }
    if (hh == 0)
        p.lse[(size_t)bh * p.Lq + qrow] = (m + __builtin_amdgcn_logf(l)) * kLn2;
}

template <typename E>
hipError_t launch(const FwdParams &p, int d, bool causal, FwdVariant v, hipStream_t stream)
{
    const dim3 grid(p.n_wg), block(kThreads);
    with_head_dim<true, true>(d, [&](auto dim) {
        constexpr int D = decltype(dim)::value;
        switch (v) {
        case FwdVariant::kPlain:
            if (causal) hipLaunchKernelGGL((fa2_fwd_bf16_kernel<D, true, false, false, E>), grid, block, 0, stream, p);
            else        hipLaunchKernelGGL((fa2_fwd_bf16_kernel<D, false, false, false, E>), grid, block, 0, stream, p);
            break;
        case FwdVariant::kSplit:
            if (causal) hipLaunchKernelGGL((fa2_fwd_bf16_kernel<D, true, true, false, E>), grid, block, 0, stream, p);
            else        hipLaunchKernelGGL((fa2_fwd_bf16_kernel<D, false, true, false, E>), grid, block, 0, stream, p);
            break;
        case FwdVariant::kWindow:
            hipLaunchKernelGGL((fa2_fwd_bf16_kernel<D, false, false, true, E>), grid, block, 0, stream, p);
            break;
        case FwdVariant::kDropout:
            if (causal)
                hipLaunchKernelGGL((fa2_fwd_bf16_kernel<D, true, false, false, E, true>), grid, block, 0, stream, p);
            else
                hipLaunchKernelGGL((fa2_fwd_bf16_kernel<D, false, false, false, E, true>), grid, block, 0, stream, p);
            break;
        }
    });
    return hipGetLastError();
}

}  // namespace

hipError_t launch_fwd16(const FwdParams &p, int d, bool causal, bool f16, FwdVariant v, hipStream_t stream)
{
    return f16 ? launch<_Float16>(p, d, causal, v, stream) : launch<__bf16>(p, d, causal, v, stream);
}

}  // namespace fa2
