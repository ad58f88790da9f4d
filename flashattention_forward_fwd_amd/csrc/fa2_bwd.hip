// fa2_bwd.hip -- FlashAttention-2 backward pass, bf16 or fp16 in/out, for gfx950.
//
// The backward needs the probabilities P of the forward but the forward keeps
// only O and one logsumexp per row, so every score block is rebuilt from Q, K
// and the saved logsumexp ("FlashAttention 怎么做? online softmax 怎么更新?",
// section "Recomputation").  With P = exp(scale * Q K^T - LSE) (masked keys 0)
// and dO the gradient of O, the gradients are the derivative of the forward
// definition:
//   D_i = sum_t dO_it O_it        (= sum_j P_ij dP_ij)
//   dV  = P^T dO                  dP = dO V^T
//   dS  = P * (dP - D)            dQ = scale dS K        dK = scale dS^T Q
//
// Three kernels, enqueued in order on one stream, no atomics (run-to-run
// bitwise identical results):
//  1. prep: per row, D_i and lse_i * log2(e) into the caller's workspace.
//  2. dK/dV: one work-group per block of 128 keys of one (batch, head); for
//     each group of 32 keys one wavefront (K in registers) computes P and
//     accumulates dV^T, another (V in registers) takes that P through LDS one
//     step later and accumulates dK^T, while 64-row tiles of Q and dO (and
//     their D and lse) stream through LDS.  Under the causal mask only the query tiles at
//     or below the block's first key are visited.  d = 256: 64 keys per
//     work-group, each accumulator split along d between two wavefronts
//     (fa2_bwd_dkdv256_kernel), so two wavefronts still share a SIMD.
//  3. dQ: one work-group per tile of 128 query rows, laid out like the forward
//     kernel: each wavefront keeps Q and dO of its 32 rows in registers and
//     accumulates dQ^T while 64-key tiles of K and V stream through LDS.  d =
//     256: a wavefront pair per 32 rows, one holding Q, one dO, each
//     accumulating half of dQ^T over 32-key tiles (fa2_bwd_dq256_kernel).
// dQ is computed by its own pass (S and dP rebuilt a second time) instead of
// being accumulated across key blocks with atomics, which would make the sum
// order, and so the rounding, depend on scheduling.
//
// With dropout (keep mask Z, keep scale ks = 256 / t, A = P * Z * ks the matrix
// the forward multiplied V by): dV = A^T dO, dP = (dO V^T) * Z * ks,
// D_i = sum_j A_ij (dO V^T)_ij = sum_t dO_it O_it as before, dS = P * (dP - D).
// The dV wavefront draws the mask, accumulates (P * Z)^T dO (ks is applied to dV
// at the end) and hands P to the dK wavefront with the sign bit set on dropped
// entries (P >= 0, so the sign carries the mask bit; a dropped 0 is -0), so the
// generator runs once per (row, key) in that kernel.  The prep kernel stores
// D / ks, so dS / ks = P * (dO V^T * Z - D / ks) needs no product with ks per
// entry; dK and dQ take the factor ks with the scale at the end.
//
// Every product runs on v_mfma_f32_32x32x16_bf16 with fp32 accumulation.  A
// 32x32 score accumulator puts one key (dK/dV kernel) or one query (dQ kernel)
// on each lane with 16 entries of the other index, in groups of four; that is
// the operand layout of the following product once the contraction index is
// permuted the same way on both operands, so P and dS feed the next MFMA
// straight from registers (rounded to bf16, nearest even).  Operands whose
// contraction index runs down the rows of a row-major LDS tile (dO^T, Q^T, K^T)
// come from the gfx950 transposing LDS read ds_read_b64_tr_b16.
#include "fa2_internal.h"

namespace fa2 {
namespace {

// bf16 (E = __bf16) or fp16 (E = _Float16) elements: 8- and 4-element vectors
// of E and the 32x32x16 matrix-core product for each.
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

#define LDS_AS __attribute__((address_space(3)))

__device__ __forceinline__ f32x16 mfma_32x32x16(bf16x8 a, bf16x8 b, f32x16 c)
{
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x16 mfma_32x32x16(f16x8 a, f16x8 b, f32x16 c)
{
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
}

constexpr int kRawBufferFlags = 0x00020000;   // raw buffer access, gfx9 resource word 3
constexpr float kLog2e = 1.44269504088896340736f;

constexpr int kKeysPerWave = 32;                  // dK/dV: keys owned by one wavefront

// A row-major bf16 tile [rows][D] in LDS, its 16-byte chunks XOR-swizzled by
// row.  The swizzle serves both read patterns the backward uses:
//  * ds_read_b128 of one logical chunk from 16 consecutive rows (the A operand
//    of a product contracting over d): the rows land in 16 different chunks;
//  * ds_read_b64_tr_b16 of 4 consecutive rows x 4 consecutive logical chunks
//    (the transposed A operand): the 4 rows land in 4 different aligned groups
//    of 4 chunks, so the 16 (row, chunk) pairs are 16 different chunks.
// For d = 64 two rows, for d = 32 four rows share one 256-byte line; the row
// within the line separates them; for d = 256 the swizzle moves a chunk within
// the first or second 256 bytes of its row.  d = 96: a 192-byte row takes a d = 128 row
// (256 bytes) in LDS, with the d = 128 swizzle; the chunks past column 95 are
// neither loaded nor read.
template <int D> struct BTile {
    static constexpr int kLdsD = D == 96 ? 128 : D;          // row length in LDS
    static constexpr int kRowBytes = 2 * kLdsD;              // LDS row
    static constexpr int kGRowBytes = 2 * D;                 // HBM row
    static constexpr int kChunks = kRowBytes / 16;
    static constexpr int kGChunks = kGRowBytes / 16;         // chunks that hold data
    static constexpr int kRowsPerXfer = 1024 / kRowBytes;   // rows per 1 KiB DMA transfer
    static __device__ __forceinline__ int swz(int r)
    {
        return kLdsD >= 128 ? (((r & 3) << 2) | ((r >> 2) & 3))
             : kLdsD == 64  ? ((((r >> 1) & 1) << 2) | ((r >> 2) & 3))
                            : ((r >> 2) & 3);
    }
    // Byte address in the tile of logical byte x of row r.
    static __device__ __forceinline__ int addr(int r, int x)
    {
        return r * kRowBytes + 16 * ((x >> 4) ^ swz(r)) + (x & 15);
    }
};

// Issue this wavefront's share of the asynchronous HBM -> LDS copy of rows
// [row0, row0 + ROWS) of a [*, D] bf16 tensor into an LDS tile (swizzled as
// BTile).  Rows past the end of the buffer range arrive as zeros.  Transfer b
// moves 1 KiB: lane l lands at byte 16 l, i.e. row b * rows_per_xfer + l / chunks
// and physical chunk l % chunks, and reads that row's logical chunk.
template <int D, int ROWS, int NWAVES = kWaves>
__device__ __forceinline__ void load_tile(__amdgpu_buffer_rsrc_t src, int row0, uint16_t *dst, int wave, int lane)
{
    using T = BTile<D>;
    constexpr int kXfers = ROWS * T::kRowBytes / 1024;
    static_assert(kXfers % NWAVES == 0 || NWAVES % kXfers == 0, "tile must split evenly over the wavefronts");
    constexpr int kPerWave = kXfers >= NWAVES ? kXfers / NWAVES : 1;
    if (kXfers < NWAVES && wave >= kXfers) return;    // small tile: the first waves copy it
#pragma unroll
    for (int x = 0; x < kPerWave; ++x) {
        const int b = wave * kPerWave + x;
        const int r = b * T::kRowsPerXfer + lane / T::kChunks;
        const int logical = (lane % T::kChunks) ^ T::swz(r);
        // The whole offset goes in the VGPR operand, which the range check covers.
        const int voff = (row0 + r) * T::kGRowBytes + 16 * logical;
        if (T::kGChunks == T::kChunks || logical < T::kGChunks)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(src, (LDS_AS void *)(dst + b * 512), 16, voff, 0, 0, 0);
    }
}

// A operand contracting over d: row `row` of a tile, logical d chunk 16c + 8hh.
template <int D, typename E>
__device__ __forceinline__ typename V16<E>::x8 read_rows_op(const LDS_AS char *tile, int row, int c, int hh)
{
    return *reinterpret_cast<const LDS_AS typename V16<E>::x8 *>(tile + BTile<D>::addr(row, 2 * (16 * c + 8 * hh)));
}

// Transposed A operand for a product contracting over the tile's rows: lane l
// receives column 32 dt + l % 32 at rows 16c + 4hh + 0..3 (slots 0-3) and
// 16c + 8 + 4hh + 0..3 (slots 4-7), hh = l / 32.  Lane 16g + 4e + r supplies the
// address of row 4(g/2) + e (+16c, +8 for the second read), columns
// 32 dt + 16(g%2) + 4r .. +3.
//
// The swizzle depends on the row's low four bits only, so for a d tile dt the
// reads of chunk c sit 16 c rows past those of chunk 0: ColsOffsets holds the
// per-lane byte offsets of chunk 0 (rows 4(g/2) + e and that + 8), computed once
// per wavefront, and read_cols_op adds the compile-time 16 c rows.
template <int D> struct ColsOffsets {
    int lo[D / 32], hi[D / 32];
};
template <int D>
__device__ __forceinline__ ColsOffsets<D> cols_offsets(int lane)
{
    const int g = lane >> 4, e = (lane >> 2) & 3, r = lane & 3;
    const int row = 4 * (g >> 1) + e;
    ColsOffsets<D> o;
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt) {
        const int x = 2 * (32 * dt + 16 * (g & 1) + 4 * r);
        o.lo[dt] = BTile<D>::addr(row, x);
        o.hi[dt] = BTile<D>::addr(row + 8, x);
    }
    return o;
}
template <int D, typename E>
__device__ __forceinline__ typename V16<E>::x8 read_cols_op(const LDS_AS char *tile, const ColsOffsets<D> &o, int dt,
                                                            int c)
{
    const LDS_AS char *t = tile + 16 * c * BTile<D>::kRowBytes;
    const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS_AS i16x4 *)(t + o.lo[dt]));
    const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS_AS i16x4 *)(t + o.hi[dt]));
    return __builtin_bit_cast(typename V16<E>::x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
}

// The same operand at a lane offset computed beforehand: row l32 (+ 32 rows for
// the second half) and logical chunk 16c + 8hh are BTile::addr(l32, 2 (16c + 8hh))
// + 32 h rows, since the swizzle depends on the row's low four bits only.
template <typename E>
__device__ __forceinline__ typename V16<E>::x8 read_rows_at(const LDS_AS char *tile, int off)
{
    return *reinterpret_cast<const LDS_AS typename V16<E>::x8 *>(tile + off);
}

// x unchanged, but opaque to the optimiser at this point of the program: per-lane
// LDS offsets re-issued inside a loop are added to the (constant) buffer address
// at each use, which folds into the instruction's offset field, instead of one
// register per (buffer, offset) pair being kept across the loop.
__device__ __forceinline__ int opaque(int x)
{
    asm volatile("" : "+v"(x));
    return x;
}

// 16 bytes of a 16-bit row from global memory (zero when `valid` is false).
template <typename E>
__device__ __forceinline__ typename V16<E>::x8 load_row_chunk(const uint16_t *p, bool valid)
{
    u32x4 raw = {0u, 0u, 0u, 0u};
    if (valid) raw = *reinterpret_cast<const u32x4 *>(p);
    return __builtin_bit_cast(typename V16<E>::x8, raw);
}

// Store one lane's share of a transposed accumulator (rows = d, columns =
// token) as bf16: the lane holds column l % 32 (token `row`), d positions
// 32 dt + 8a + 4hh + 0..3 in accumulator entries 4a .. 4a+3.
template <int D, typename E>
__device__ __forceinline__ void store_tokens(uint16_t *dst_row, const f32x16 (&acc)[D / 32], float mul, int hh)
{
    using e4 = typename V16<E>::x4;
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
        for (int a = 0; a < 4; ++a) {
            const f32x4 v4 = {acc[dt][4 * a + 0] * mul, acc[dt][4 * a + 1] * mul, acc[dt][4 * a + 2] * mul,
                              acc[dt][4 * a + 3] * mul};
            *reinterpret_cast<e4 *>(dst_row + 32 * dt + 8 * a + 4 * hh) = __builtin_convertvector(v4, e4);
        }
}

// Entry i of a 32x32 score accumulator lies at offset 8(i/4) + i%4 (0..27) from
// the lane's first index `base` (a key or a query row); entries outside [lo, hi]
// are set to `fill`.  The bounds are brought to entry offsets once per call,
// clamped to [-1, 64] (an empty range becomes [64, 64]), so each entry costs one
// unsigned compare and one select.
__device__ __forceinline__ void keep_range(f32x16 &x, int64_t base, int64_t lo, int64_t hi, float fill)
{
    const int64_t a64 = lo - base, b64 = hi - base;
    int a = (int)(a64 < -1 ? -1 : a64 > 64 ? 64 : a64);
    int b = (int)(b64 < -1 ? -1 : b64 > 64 ? 64 : b64);
    if (b < a) a = b = 64;
    const unsigned span = (unsigned)(b - a);
#pragma unroll
    for (int i = 0; i < 16; ++i)
        x[i] = (unsigned)(8 * (i / 4) + (i % 4) - a) > span ? fill : x[i];
}

// ---------------------------------------------------------------- 1. prep
// D_i = sum_t dO_it O_it (fp32) and lse2_i = lse_i * log2(e); D/8 threads per row
// (a power of two for the butterfly sum: d = 96 takes 16, the last 4 idle).
template <int D> constexpr int kPrepThreadsPerRow = D == 96 ? 16 : D / 8;

template <int D, typename E>
__global__ __launch_bounds__(256) void fa2_bwd_prep_kernel(const uint16_t *o, const uint16_t *dout, const float *lse,
                                                           float *lse2, float *delta, int64_t rows, float dmul)
{
    constexpr int kTpr = kPrepThreadsPerRow<D>;
    const int64_t gid = (int64_t)blockIdx.x * 256 + threadIdx.x;
    const int64_t row = gid / kTpr;
    const int part = (int)(gid % kTpr);
    float acc = 0.f;
    if (row < rows && part < D / 8) {
        const f32x8 a = __builtin_convertvector(*reinterpret_cast<const typename V16<E>::x8 *>(o + row * D + 8 * part), f32x8);
        const f32x8 b = __builtin_convertvector(*reinterpret_cast<const typename V16<E>::x8 *>(dout + row * D + 8 * part), f32x8);
#pragma unroll
        for (int i = 0; i < 8; ++i)
            acc = __builtin_fmaf(a[i], b[i], acc);
    }
#pragma unroll
    for (int off = kTpr / 2; off > 0; off >>= 1)
        acc += __shfl_xor(acc, off, kTpr);
    if (row < rows && part == 0) {
        delta[row] = acc * dmul;
        lse2[row] = lse[row] * kLog2e;
    }
}

// ---------------------------------------------------------------- 2. dK, dV
// Work-group id -> (batch*head, key block).  Under the causal mask the first
// key block sees the most query tiles, so blocks run from the first to the last
// across all heads (longest first); heads are the fast index.
//
// Eight wavefronts, two per SIMD.  For each group of 32 keys, wavefront g
// (0-3) computes S = Q K^T and P for query tile t, accumulates dV^T += dO^T P,
// and leaves P (bf16) in LDS; wavefront 4 + g takes that P one step later,
// computes dP = dO V^T and dS = P (dP - D) for tile t - 1 and accumulates
// dK^T += Q^T dS.  Each wavefront then holds one 32-key x d accumulator and one
// of K, V (about 160-190 registers, so two share a SIMD); holding both
// accumulators in one wavefront needs about 400 and leaves one wavefront per
// SIMD with nothing to hide its latencies.  The one-step lag keeps a single
// barrier per step: Q/dO tiles are triple-buffered (t + 1 loading, t read by
// the dV wavefronts, t - 1 by the dK wavefronts) and P double-buffered.
//
// d = 256: a wavefront's K (or V) of 32 keys and its accumulator would take 192
// registers; fa2_bwd_dkdv256_kernel below splits the accumulators along d instead.
template <int D> struct DkdvShape {
    static_assert(D <= 128, "d = 256 runs fa2_bwd_dkdv256_kernel");
    static constexpr int kWaves = 8;                           // wavefronts per work-group
    static constexpr int kGroups = kWaves / 2;                 // 32-key groups (one dV, one dK wave each)
    static constexpr int kKeyBlock = kGroups * kKeysPerWave;   // keys per work-group
    static constexpr int kRowTile = 64;                        // query rows per LDS tile
    static constexpr int kHalves = kRowTile / 32;              // 32-row score tiles per row tile
    static constexpr int kPChunks = kRowTile / 16;             // 16-row operand chunks per row tile
    static constexpr int kThreads = kWaves * kWave;
};

// Wavefronts per SIMD the register allocation is held to: at d = 32 (without
// dropout) the kernel fits 128 VGPRs (97-109), so two work-groups (58 KiB of LDS
// each) share a CU and four wavefronts a SIMD; measured on MI355X 16-20 % faster
// than two.  Every other instance keeps two (d = 32 with dropout would spill).
template <int D, bool DROPOUT> constexpr int kDkdvWavesPerEU = D == 32 && !DROPOUT ? 4 : 2;

template <int D, bool MASKED, typename E, bool DROPOUT>
__global__ __launch_bounds__(DkdvShape<D>::kThreads)
__attribute__((amdgpu_waves_per_eu(kDkdvWavesPerEU<D, DROPOUT>, kDkdvWavesPerEU<D, DROPOUT>)))
void fa2_bwd_dkdv_kernel(BwdParams p)
{
    using T = BTile<D>;
    using S = DkdvShape<D>;
    using e8 = typename V16<E>::x8;
    constexpr int kDc = D / 16;
    constexpr int kDt = D / 32;
    constexpr int kRowTile = S::kRowTile;
    constexpr int kKeyBlock = S::kKeyBlock;
    constexpr int kTileElems = kRowTile * T::kLdsD;
    __shared__ __attribute__((aligned(1024))) uint16_t sQ0[kTileElems];
    __shared__ __attribute__((aligned(1024))) uint16_t sQ1[kTileElems];
    __shared__ __attribute__((aligned(1024))) uint16_t sQ2[kTileElems];
    __shared__ __attribute__((aligned(1024))) uint16_t sO0[kTileElems];   // dO tiles
    __shared__ __attribute__((aligned(1024))) uint16_t sO1[kTileElems];
    __shared__ __attribute__((aligned(1024))) uint16_t sO2[kTileElems];
    // P of one tile: [key group][chunk c][lane] x 16 bytes, in the lane order of the B operand
    // (one array for both buffers: its accesses are known not to touch the tiles
    // that asynchronous copies are filling)
    __shared__ __attribute__((aligned(1024))) e8 sP[2][S::kGroups * S::kPChunks * kWave];
    // per buffer: lse2 of the tile's rows at 0, their D at 64 (a 32-row tile
    // leaves the upper halves unused)
    __shared__ __attribute__((aligned(256))) float sStat0[128];
    __shared__ __attribute__((aligned(256))) float sStat1[128];
    __shared__ __attribute__((aligned(256))) float sStat2[128];

    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
    const int lane = tid % kWave;
    const int l32 = lane & 31;
    const int hh = lane >> 5;
    const bool is_dk = wave >= S::kGroups;          // wave-uniform role
    const int grp = wave % S::kGroups;              // 32-key group

    const int n_bh = p.B * p.H;
    const int bh = blockIdx.x % n_bh;
    const int kb = blockIdx.x / n_bh;
    const int kw0 = kb * kKeyBlock + grp * kKeysPerWave;   // first key of this wavefront
    const int key = kw0 + l32;                              // this lane's key
    // Query tiles [t0, t_end) of the work-group: those holding a query that sees
    // one of its keys; this key group's own range is [wt0, wt_end).  MASKED: key
    // j is visible to query i iff (wl < 0 or j >= i - wl) and (wr < 0 or j <= i + wr),
    // i.e. i in [j - wr, j + wl].
    int t0 = 0, t_end = (p.Lq + kRowTile - 1) / kRowTile, wt0 = 0, wt_end = t_end;
    if (MASKED) {
        const int64_t k_first = (int64_t)kb * kKeyBlock;
        const int64_t k_last = min(k_first + kKeyBlock - 1, (int64_t)p.Lk - 1);
        const int64_t q_lo = p.wr < 0 ? 0 : max((int64_t)0, k_first - p.wr);
        const int64_t q_hi = p.wl < 0 ? p.Lq : min((int64_t)p.Lq, k_last + p.wl + 1);
        t0 = t_end = 0;
        if (q_hi > q_lo) {
            t0 = (int)(q_lo / kRowTile);
            t_end = (int)((q_hi + kRowTile - 1) / kRowTile);
        }
        const int64_t wq_lo = p.wr < 0 ? 0 : max((int64_t)0, (int64_t)kw0 - p.wr);
        const int64_t wq_hi = p.wl < 0 ? p.Lq : min((int64_t)p.Lq, (int64_t)kw0 + kKeysPerWave + p.wl);
        wt0 = max(t0, (int)(wq_lo / kRowTile));
        wt_end = min(t_end, (int)((wq_hi + kRowTile - 1) / kRowTile));
    }

    const size_t row_off = (size_t)bh * p.Lq;
    const __amdgpu_buffer_rsrc_t rQ = __builtin_amdgcn_make_buffer_rsrc(
        (void *)(static_cast<const uint16_t *>(p.q) + row_off * D), 0, p.Lq * T::kGRowBytes, kRawBufferFlags);
    const __amdgpu_buffer_rsrc_t rO = __builtin_amdgcn_make_buffer_rsrc(
        (void *)(static_cast<const uint16_t *>(p.dout) + row_off * D), 0, p.Lq * T::kGRowBytes, kRawBufferFlags);
    const __amdgpu_buffer_rsrc_t rL = __builtin_amdgcn_make_buffer_rsrc(
        (void *)(p.lse2 + row_off), 0, p.Lq * 4, kRawBufferFlags);
    const __amdgpu_buffer_rsrc_t rD = __builtin_amdgcn_make_buffer_rsrc(
        (void *)(p.delta + row_off), 0, p.Lq * 4, kRawBufferFlags);

    // Tile t lives in buffer set (t - t0) % 3: Q, dO, and lse2 (loaded by wave 0)
    // and D (wave 1) of its 64 rows.
    // The loops below run three steps per trip, so that every slot is fixed at
    // compile time.
    auto load = [&](int t, uint16_t *q, uint16_t *o, float *st) {
        load_tile<D, kRowTile, S::kWaves>(rQ, t * kRowTile, q, wave, lane);
        load_tile<D, kRowTile, S::kWaves>(rO, t * kRowTile, o, wave, lane);
        if (wave < 2)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(wave == 0 ? rL : rD, (LDS_AS void *)(st + 64 * wave),
                                                     4, 4 * (t * kRowTile + lane), 0, 0, 0);
    };
    if (t0 < t_end) load(t0, sQ0, sO0, sStat0);

    // K (dV wavefronts) or V (dK wavefronts) of this lane's key as B operands
    // (d chunk 16c + 8hh); zero past Lk.
    const uint16_t *Xr = static_cast<const uint16_t *>(is_dk ? p.v : p.k) + ((size_t)bh * p.Lk + key) * D;
    e8 xf[kDc];
#pragma unroll
    for (int c = 0; c < kDc; ++c)
        xf[c] = load_row_chunk<E>(Xr + 16 * c + 8 * hh, key < p.Lk);

    const ColsOffsets<D> coff = cols_offsets<D>(lane);
    // Lane offsets of the Q and dO rows operands (read_rows_at).
    int roff[kDc];
#pragma unroll
    for (int c = 0; c < kDc; ++c)
        roff[c] = BTile<D>::addr(l32, 2 * (16 * c + 8 * hh));
    f32x16 acc[kDt];                       // dV^T (wavefronts 0-3) or dK^T (4-7)
#pragma unroll
    for (int t = 0; t < kDt; ++t)
        acc[t] = f32x16{};
    const float c2 = p.scale_log2;

    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();

    // Step t: the dV wavefronts work on tile t, the dK wavefronts on tile t - 1.
    // Each role runs a loop of its own (the same trip count, so the same
    // barriers): in one shared loop the register allocator kept the accumulator
    // of the two roles in different registers and copied it on every step.
    if (!is_dk) {
        auto step = [&](int t, const uint16_t *q, const uint16_t *o, const float *sts, uint16_t *qn, uint16_t *on,
                        float *stn) {
            if (t + 1 < t_end) load(t + 1, qn, on, stn);
            if (t >= wt0 && t < wt_end) {
                const LDS_AS char *qb = (const LDS_AS char *)q;
                const LDS_AS char *ob = (const LDS_AS char *)o;
                const LDS_AS float *st = (const LDS_AS float *)sts;
                int ro[kDc];
#pragma unroll
                for (int c = 0; c < kDc; ++c)
                    ro[c] = opaque(roff[c]);
                ColsOffsets<D> co;
#pragma unroll
                for (int dt = 0; dt < kDt; ++dt) {
                    co.lo[dt] = opaque(coff.lo[dt]);
                    co.hi[dt] = opaque(coff.hi[dt]);
                }
                // S = Q K^T for the tile's rows (32-row halves h) x this group's 32
                // keys.  Entry i of half h is row 32h + 8(i/4) + 4hh + i%4.
                f32x16 s[S::kHalves];
#pragma unroll
                for (int h = 0; h < S::kHalves; ++h) {
                    s[h] = f32x16{};
#pragma unroll
                    for (int c = 0; c < kDc; ++c)
                        s[h] = mfma_32x32x16(read_rows_at<E>(qb + 32 * h * T::kRowBytes, ro[c]), xf[c], s[h]);
                }
                // Does every (row, key) pair of this tile and key group lie in the window?
                const bool need_mask =
                    MASKED && !((p.wl < 0 || (int64_t)kw0 >= (int64_t)t * kRowTile + kRowTile - 1 - p.wl) &&
                                (p.wr < 0 || (int64_t)kw0 + kKeysPerWave - 1 <= (int64_t)t * kRowTile + p.wr));
                // Chunk c (B operand of the products over the tile's rows) holds
                // rows 16c + 8(e/4) + 4hh + e%4, e = 0..7: entries 8(c%2) + e of half c/2.
                LDS_AS e8 *pdst = (LDS_AS e8 *)sP[t & 1] + grp * S::kPChunks * kWave;
                DropMask mk;
                if (DROPOUT)
#pragma unroll
                    for (int h = 0; h < S::kHalves; ++h)
                        mk.y[h] = mask_key_lanes_one(p.drop, t * kRowTile, h, key, lane, bh);
                // P = 2^(S c - lse2), in place.
#pragma unroll
                for (int c = 0; c < S::kPChunks; ++c) {
                    const int h = c >> 1, i0 = 8 * (c & 1);
                    const f32x4 l4a = *reinterpret_cast<const LDS_AS f32x4 *>(st + 16 * c + 4 * hh);
                    const f32x4 l4b = *reinterpret_cast<const LDS_AS f32x4 *>(st + 16 * c + 8 + 4 * hh);
#pragma unroll
                    for (int e = 0; e < 8; ++e)
                        s[h][i0 + e] = __builtin_amdgcn_exp2f(
                            __builtin_fmaf(s[h][i0 + e], c2, -(e < 4 ? l4a[e] : l4b[e - 4])));
                }
                // Pairs outside the window -> 0: one branch per tile, the same on
                // every lane (a test per entry would split the loop into blocks).
                if (need_mask) {
                    // rows that see this lane's key: [key - wr, key + wl]
                    const int64_t r_lo = p.wr >= 0 ? (int64_t)key - p.wr : INT64_MIN / 2;
                    const int64_t r_hi = p.wl >= 0 ? (int64_t)key + p.wl : INT64_MAX / 2;
#pragma unroll
                    for (int h = 0; h < S::kHalves; ++h)
                        keep_range(s[h], (int64_t)t * kRowTile + 32 * h + 4 * hh, r_lo, r_hi, 0.f);
                }
                e8 pf[S::kPChunks];
#pragma unroll
                for (int c = 0; c < S::kPChunks; ++c) {
                    const int h = c >> 1, i0 = 8 * (c & 1);
                    f32x8 v8;
#pragma unroll
                    for (int e = 0; e < 8; ++e) {
                        v8[e] = s[h][i0 + e];
                        if (DROPOUT && !keep(mk, h, i0 + e, p.drop.threshold)) v8[e] = -v8[e];
                    }
                    pf[c] = __builtin_convertvector(v8, e8);
                    pdst[c * kWave + lane] = pf[c];
                    if (DROPOUT) {
                        // dropped (negative) entries -> 0 for this wavefront's product
                        typedef short s8 __attribute__((ext_vector_type(8)));
                        const s8 bits = __builtin_bit_cast(s8, pf[c]);
                        pf[c] = __builtin_bit_cast(e8, __builtin_elementwise_max(bits, s8{}));
                    }
                }
                // dV^T += dO^T P (contraction over the tile's rows).
#pragma unroll
                for (int dt = 0; dt < kDt; ++dt)
#pragma unroll
                    for (int c = 0; c < S::kPChunks; ++c)
                        acc[dt] = mfma_32x32x16(read_cols_op<D, E>(ob, co, dt, c), pf[c], acc[dt]);
            }
            __builtin_amdgcn_s_waitcnt(0);    // this wave's loads of tile t+1 have landed
            __syncthreads();                  // ... everyone's; P of tile t is visible; old buffers free
        };
        // Tile t is in slot (t - t0) % 3.
        for (int t = t0; t <= t_end; t += 3) {
            step(t, sQ0, sO0, sStat0, sQ1, sO1, sStat1);
            if (t + 1 <= t_end) step(t + 1, sQ1, sO1, sStat1, sQ2, sO2, sStat2);
            if (t + 2 <= t_end) step(t + 2, sQ2, sO2, sStat2, sQ0, sO0, sStat0);
        }
    } else {
        // Step t works on tile tk = t - 1, in slot (tk - t0) % 3, and loads tile
        // t + 1 into slot (t + 1 - t0) % 3.
        auto step = [&](int t, const uint16_t *q, const uint16_t *o, const float *sts, uint16_t *qn, uint16_t *on,
                        float *stn) {
            if (t + 1 < t_end) load(t + 1, qn, on, stn);
            const int tk = t - 1;
            if (tk >= wt0 && tk < wt_end) {
                const LDS_AS char *qb = (const LDS_AS char *)q;
                const LDS_AS char *ob = (const LDS_AS char *)o;
                const LDS_AS float *st = (const LDS_AS float *)sts;
                int ro[kDc];
#pragma unroll
                for (int c = 0; c < kDc; ++c)
                    ro[c] = opaque(roff[c]);
                ColsOffsets<D> co;
#pragma unroll
                for (int dt = 0; dt < kDt; ++dt) {
                    co.lo[dt] = opaque(coff.lo[dt]);
                    co.hi[dt] = opaque(coff.hi[dt]);
                }
                // dP = dO V^T, same layout as S.
                f32x16 dp[S::kHalves];
#pragma unroll
                for (int h = 0; h < S::kHalves; ++h) {
                    dp[h] = f32x16{};
#pragma unroll
                    for (int c = 0; c < kDc; ++c)
                        dp[h] = mfma_32x32x16(read_rows_at<E>(ob + 32 * h * T::kRowBytes, ro[c]), xf[c], dp[h]);
                }
                const LDS_AS e8 *psrc = (const LDS_AS e8 *)sP[tk & 1] + grp * S::kPChunks * kWave;
                e8 dsf[S::kPChunks];
#pragma unroll
                for (int c = 0; c < S::kPChunks; ++c) {
                    const int h = c >> 1, i0 = 8 * (c & 1);
                    const e8 pc = psrc[c * kWave + lane];
                    const f32x4 d4a = *reinterpret_cast<const LDS_AS f32x4 *>(st + 64 + 16 * c + 4 * hh);
                    const f32x4 d4b = *reinterpret_cast<const LDS_AS f32x4 *>(st + 64 + 16 * c + 8 + 4 * hh);
                    f32x8 v8;
#pragma unroll
                    for (int e = 0; e < 8; ++e) {   // dS = P (dP - D)
                        const float dl = e < 4 ? d4a[e] : d4b[e - 4];
                        if (DROPOUT) {   // dS / ks, dl = D / ks
                            const float pr = (float)pc[e];
                            v8[e] = __builtin_fabsf(pr) * (__builtin_signbit(pr) ? -dl : dp[h][i0 + e] - dl);
                        } else {
                            v8[e] = (float)pc[e] * (dp[h][i0 + e] - dl);
                        }
                    }
                    dsf[c] = __builtin_convertvector(v8, e8);
                }
                // dK^T += Q^T dS (contraction over the tile's rows).
#pragma unroll
                for (int dt = 0; dt < kDt; ++dt)
#pragma unroll
                    for (int c = 0; c < S::kPChunks; ++c)
                        acc[dt] = mfma_32x32x16(read_cols_op<D, E>(qb, co, dt, c), dsf[c], acc[dt]);
            }
            __builtin_amdgcn_s_waitcnt(0);
            __syncthreads();
        };
        for (int t = t0; t <= t_end; t += 3) {
            step(t, sQ2, sO2, sStat2, sQ1, sO1, sStat1);
            if (t + 1 <= t_end) step(t + 1, sQ0, sO0, sStat0, sQ2, sO2, sStat2);
            if (t + 2 <= t_end) step(t + 2, sQ1, sO1, sStat1, sQ0, sO0, sStat0);
        }
    }

    if (key >= p.Lk) return;
    const size_t kv_row = (size_t)bh * p.Lk + key;
    if (is_dk)
        store_tokens<D, E>(static_cast<uint16_t *>(p.dk) + kv_row * D, acc,
                           DROPOUT ? p.scale * p.drop.keep_scale : p.scale, hh);
    else       store_tokens<D, E>(static_cast<uint16_t *>(p.dv) + kv_row * D, acc, DROPOUT ? p.drop.keep_scale : 1.0f, hh);
}

// d = 256 with two wavefronts per SIMD: the accumulators are split along d.
// For each group of 32 keys four wavefronts share the work of one step:
//  * SV (wavefront g):      K in registers; S = Q K^T and P for query tile t, P
//                           to LDS, dV^T[0:128) += dO^T P;
//  * VH (wavefront 4 + g):  P of tile t - 1 from LDS, dV^T[128:256) += dO^T P;
//  * PK (wavefront 2 + g):  V in registers; dP = dO V^T and dS = P (dP - D) for
//                           tile t - 1, dS to LDS, dK^T[0:128) += Q^T dS;
//  * KH (wavefront 6 + g):  dS of tile t - 2 from LDS, dK^T[128:256) += Q^T dS.
// Wavefronts w and w + 4 share a SIMD, so each SIMD carries one role that
// holds K or V (24 MFMAs a step) and one that does not (8 MFMAs).  The lags
// keep one barrier per step: Q tiles are held four deep (t + 1 loading, t, t - 1,
// t - 2), dO and the row statistics three deep, P and dS two deep.  The
// products, and the order of every accumulation, are those of the kernel above
// (32-row Q / dO tiles, 64 keys per work-group: the ten tiles take 130 KiB of LDS).
struct Dkdv256 {
    static constexpr int kWaves = 8;
    static constexpr int kGroups = 2;
    static constexpr int kKeyBlock = kGroups * kKeysPerWave;
    static constexpr int kRowTile = 32;
    static constexpr int kPChunks = 2;
    static constexpr int kThreads = kWaves * kWave;
};

// store_tokens for one half of d (four 32-wide d tiles); dst_row points at the half.
template <typename E>
__device__ __forceinline__ void store_tokens_half(uint16_t *dst_row, const f32x16 (&acc)[4], float mul, int hh)
{
    using e4 = typename V16<E>::x4;
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
#pragma unroll
        for (int a = 0; a < 4; ++a) {
            const f32x4 v4 = {acc[dt][4 * a + 0] * mul, acc[dt][4 * a + 1] * mul, acc[dt][4 * a + 2] * mul,
                              acc[dt][4 * a + 3] * mul};
            *reinterpret_cast<e4 *>(dst_row + 32 * dt + 8 * a + 4 * hh) = __builtin_convertvector(v4, e4);
        }
}

template <bool MASKED, typename E, bool DROPOUT>
__global__ __launch_bounds__(Dkdv256::kThreads) __attribute__((amdgpu_waves_per_eu(2, 2)))
void fa2_bwd_dkdv256_kernel(BwdParams p)
{
    constexpr int D = 256;
    using T = BTile<D>;
    using S = Dkdv256;
    using e8 = typename V16<E>::x8;
    constexpr int kDc = D / 16;
    constexpr int kRowTile = S::kRowTile;
    constexpr int kKeyBlock = S::kKeyBlock;
    constexpr int kTileElems = kRowTile * T::kLdsD;
    constexpr int kPElems = S::kGroups * S::kPChunks * kWave;
    __shared__ __attribute__((aligned(1024))) uint16_t sQ0[kTileElems];
    __shared__ __attribute__((aligned(1024))) uint16_t sQ1[kTileElems];
    __shared__ __attribute__((aligned(1024))) uint16_t sQ2[kTileElems];
    __shared__ __attribute__((aligned(1024))) uint16_t sQ3[kTileElems];
    __shared__ __attribute__((aligned(1024))) uint16_t sO0[kTileElems];
    __shared__ __attribute__((aligned(1024))) uint16_t sO1[kTileElems];
    __shared__ __attribute__((aligned(1024))) uint16_t sO2[kTileElems];
    __shared__ __attribute__((aligned(1024))) e8 sP0[kPElems];
    __shared__ __attribute__((aligned(1024))) e8 sP1[kPElems];
    __shared__ __attribute__((aligned(1024))) e8 sS0[kPElems];     // dS
    __shared__ __attribute__((aligned(1024))) e8 sS1[kPElems];
    __shared__ __attribute__((aligned(256))) float sStat0[128];
    __shared__ __attribute__((aligned(256))) float sStat1[128];
    __shared__ __attribute__((aligned(256))) float sStat2[128];

    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
    const int lane = tid % kWave;
    const int l32 = lane & 31;
    const int hh = lane >> 5;
    const int grp = wave & 1;                       // 32-key group
    const bool k_side = (wave & 2) != 0;            // PK / KH (dK) or SV / VH (dV)
    const bool heavy = wave < 4;                    // SV / PK: K or V in registers

    const int n_bh = p.B * p.H;
    const int bh = blockIdx.x % n_bh;
    const int kb = blockIdx.x / n_bh;
    const int kw0 = kb * kKeyBlock + grp * kKeysPerWave;
    const int key = kw0 + l32;
    int t0 = 0, t_end = (p.Lq + kRowTile - 1) / kRowTile, wt0 = 0, wt_end = t_end;
    if (MASKED) {
        const int64_t k_first = (int64_t)kb * kKeyBlock;
        const int64_t k_last = min(k_first + kKeyBlock - 1, (int64_t)p.Lk - 1);
        const int64_t q_lo = p.wr < 0 ? 0 : max((int64_t)0, k_first - p.wr);
        const int64_t q_hi = p.wl < 0 ? p.Lq : min((int64_t)p.Lq, k_last + p.wl + 1);
        t0 = t_end = 0;
        if (q_hi > q_lo) {
            t0 = (int)(q_lo / kRowTile);
            t_end = (int)((q_hi + kRowTile - 1) / kRowTile);
        }
        const int64_t wq_lo = p.wr < 0 ? 0 : max((int64_t)0, (int64_t)kw0 - p.wr);
        const int64_t wq_hi = p.wl < 0 ? p.Lq : min((int64_t)p.Lq, (int64_t)kw0 + kKeysPerWave + p.wl);
        wt0 = max(t0, (int)(wq_lo / kRowTile));
        wt_end = min(t_end, (int)((wq_hi + kRowTile - 1) / kRowTile));
    }

    const size_t row_off = (size_t)bh * p.Lq;
    const __amdgpu_buffer_rsrc_t rQ = __builtin_amdgcn_make_buffer_rsrc(
        (void *)(static_cast<const uint16_t *>(p.q) + row_off * D), 0, p.Lq * T::kGRowBytes, kRawBufferFlags);
    const __amdgpu_buffer_rsrc_t rO = __builtin_amdgcn_make_buffer_rsrc(
        (void *)(static_cast<const uint16_t *>(p.dout) + row_off * D), 0, p.Lq * T::kGRowBytes, kRawBufferFlags);
    const __amdgpu_buffer_rsrc_t rL = __builtin_amdgcn_make_buffer_rsrc(
        (void *)(p.lse2 + row_off), 0, p.Lq * 4, kRawBufferFlags);
    const __amdgpu_buffer_rsrc_t rD = __builtin_amdgcn_make_buffer_rsrc(
        (void *)(p.delta + row_off), 0, p.Lq * 4, kRawBufferFlags);

    // Tile t: Q in slot (t - t0) % 4, dO and the statistics (lse2 at 0, D at 64)
    // in slot (t - t0) % 3.
    auto qbuf = [&](int t) {
        const int s = (t - t0) & 3;
        return s == 0 ? sQ0 : s == 1 ? sQ1 : s == 2 ? sQ2 : sQ3;
    };
    auto obuf = [&](int t) {
        const int s = (t - t0) % 3;
        return s == 0 ? sO0 : s == 1 ? sO1 : sO2;
    };
    auto sbuf = [&](int t) {
        const int s = (t - t0) % 3;
        return s == 0 ? sStat0 : s == 1 ? sStat1 : sStat2;
    };
    auto load = [&](int t) {
        load_tile<D, kRowTile, S::kWaves>(rQ, t * kRowTile, qbuf(t), wave, lane);
        load_tile<D, kRowTile, S::kWaves>(rO, t * kRowTile, obuf(t), wave, lane);
        if (wave == 0)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rL, (LDS_AS void *)(sbuf(t)), 4, 4 * (t * kRowTile + lane), 0, 0, 0);
        if (wave == 1)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rD, (LDS_AS void *)(sbuf(t) + 64), 4, 4 * (t * kRowTile + lane),
                                                     0, 0, 0);
    };
    if (t0 < t_end) load(t0);

    // K (SV) or V (PK) of this lane's key as B operands; zero past Lk.
    e8 xf[kDc];
    if (heavy) {
        const uint16_t *Xr = static_cast<const uint16_t *>(k_side ? p.v : p.k) + ((size_t)bh * p.Lk + key) * D;
#pragma unroll
        for (int c = 0; c < kDc; ++c)
            xf[c] = load_row_chunk<E>(Xr + 16 * c + 8 * hh, key < p.Lk);
    }
    const ColsOffsets<D> coff = cols_offsets<D>(lane);
    const int dt0 = heavy ? 0 : 4;                  // this wavefront's half of d
    f32x16 acc[4];
#pragma unroll
    for (int t = 0; t < 4; ++t)
        acc[t] = f32x16{};
    const float c2 = p.scale_log2;

    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();

    const int last = t_end + 1;                     // KH finishes tile t_end - 1 at step t_end + 1
    if (heavy && !k_side) {                         // SV
        for (int t = t0; t <= last; ++t) {
            if (t + 1 < t_end) load(t + 1);
            if (t >= wt0 && t < wt_end) {
                const LDS_AS char *qb = (const LDS_AS char *)qbuf(t);
                const LDS_AS char *ob = (const LDS_AS char *)obuf(t);
                const LDS_AS float *st = (const LDS_AS float *)sbuf(t);
                f32x16 s = f32x16{};
#pragma unroll
                for (int c = 0; c < kDc; ++c)
                    s = mfma_32x32x16(read_rows_op<D, E>(qb, l32, c, hh), xf[c], s);
                const bool need_mask =
                    MASKED && !((p.wl < 0 || (int64_t)kw0 >= (int64_t)t * kRowTile + kRowTile - 1 - p.wl) &&
                                (p.wr < 0 || (int64_t)kw0 + kKeysPerWave - 1 <= (int64_t)t * kRowTile + p.wr));
                LDS_AS e8 *pdst = (LDS_AS e8 *)((t & 1) ? sP1 : sP0) + grp * S::kPChunks * kWave;
                DropMask mk;
                if (DROPOUT) mk.y[0] = mask_key_lanes_one(p.drop, t * kRowTile, 0, key, lane, bh);
#pragma unroll
                for (int c = 0; c < S::kPChunks; ++c) {
                    const int i0 = 8 * c;
                    const f32x4 l4a = *reinterpret_cast<const LDS_AS f32x4 *>(st + 16 * c + 4 * hh);
                    const f32x4 l4b = *reinterpret_cast<const LDS_AS f32x4 *>(st + 16 * c + 8 + 4 * hh);
#pragma unroll
                    for (int e = 0; e < 8; ++e)
                        s[i0 + e] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[i0 + e], c2, -(e < 4 ? l4a[e] : l4b[e - 4])));
                }
                if (need_mask) {
                    const int64_t r_lo = p.wr >= 0 ? (int64_t)key - p.wr : INT64_MIN / 2;
                    const int64_t r_hi = p.wl >= 0 ? (int64_t)key + p.wl : INT64_MAX / 2;
                    keep_range(s, (int64_t)t * kRowTile + 4 * hh, r_lo, r_hi, 0.f);
                }
                e8 pf[S::kPChunks];
#pragma unroll
                for (int c = 0; c < S::kPChunks; ++c) {
                    f32x8 v8;
#pragma unroll
                    for (int e = 0; e < 8; ++e) {
                        v8[e] = s[8 * c + e];
                        if (DROPOUT && !keep(mk, 0, 8 * c + e, p.drop.threshold)) v8[e] = -v8[e];
                    }
                    pf[c] = __builtin_convertvector(v8, e8);
                    pdst[c * kWave + lane] = pf[c];
                    if (DROPOUT) {
                        typedef short s8 __attribute__((ext_vector_type(8)));
                        const s8 bits = __builtin_bit_cast(s8, pf[c]);
                        pf[c] = __builtin_bit_cast(e8, __builtin_elementwise_max(bits, s8{}));
                    }
                }
#pragma unroll
                for (int dt = 0; dt < 4; ++dt)
#pragma unroll
                    for (int c = 0; c < S::kPChunks; ++c)
                        acc[dt] = mfma_32x32x16(read_cols_op<D, E>(ob, coff, dt, c), pf[c], acc[dt]);
            }
            __builtin_amdgcn_s_waitcnt(0);
            __syncthreads();
        }
    } else if (!k_side) {                           // VH
        for (int t = t0; t <= last; ++t) {
            if (t + 1 < t_end) load(t + 1);
            const int tv = t - 1;
            if (tv >= wt0 && tv < wt_end) {
                const LDS_AS char *ob = (const LDS_AS char *)obuf(tv);
                const LDS_AS e8 *psrc = (const LDS_AS e8 *)((tv & 1) ? sP1 : sP0) + grp * S::kPChunks * kWave;
                e8 pf[S::kPChunks];
#pragma unroll
                for (int c = 0; c < S::kPChunks; ++c) {
                    pf[c] = psrc[c * kWave + lane];
                    if (DROPOUT) {
                        typedef short s8 __attribute__((ext_vector_type(8)));
                        const s8 bits = __builtin_bit_cast(s8, pf[c]);
                        pf[c] = __builtin_bit_cast(e8, __builtin_elementwise_max(bits, s8{}));
                    }
                }
#pragma unroll
                for (int dt = 0; dt < 4; ++dt)
#pragma unroll
                    for (int c = 0; c < S::kPChunks; ++c)
                        acc[dt] = mfma_32x32x16(read_cols_op<D, E>(ob, coff, 4 + dt, c), pf[c], acc[dt]);
            }
            __builtin_amdgcn_s_waitcnt(0);
            __syncthreads();
        }
    } else if (heavy) {                             // PK
        for (int t = t0; t <= last; ++t) {
            if (t + 1 < t_end) load(t + 1);
            const int tk = t - 1;
            if (tk >= wt0 && tk < wt_end) {
                const LDS_AS char *qb = (const LDS_AS char *)qbuf(tk);
                const LDS_AS char *ob = (const LDS_AS char *)obuf(tk);
                const LDS_AS float *st = (const LDS_AS float *)sbuf(tk);
                f32x16 dp = f32x16{};
#pragma unroll
                for (int c = 0; c < kDc; ++c)
                    dp = mfma_32x32x16(read_rows_op<D, E>(ob, l32, c, hh), xf[c], dp);
                const LDS_AS e8 *psrc = (const LDS_AS e8 *)((tk & 1) ? sP1 : sP0) + grp * S::kPChunks * kWave;
                LDS_AS e8 *ddst = (LDS_AS e8 *)((tk & 1) ? sS1 : sS0) + grp * S::kPChunks * kWave;
                e8 dsf[S::kPChunks];
#pragma unroll
                for (int c = 0; c < S::kPChunks; ++c) {
                    const int i0 = 8 * c;
                    const e8 pc = psrc[c * kWave + lane];
                    const f32x4 d4a = *reinterpret_cast<const LDS_AS f32x4 *>(st + 64 + 16 * c + 4 * hh);
                    const f32x4 d4b = *reinterpret_cast<const LDS_AS f32x4 *>(st + 64 + 16 * c + 8 + 4 * hh);
                    f32x8 v8;
#pragma unroll
                    for (int e = 0; e < 8; ++e) {
                        const float dl = e < 4 ? d4a[e] : d4b[e - 4];
                        if (DROPOUT) {
                            const float pr = (float)pc[e];
                            v8[e] = __builtin_fabsf(pr) * (__builtin_signbit(pr) ? -dl : dp[i0 + e] - dl);
                        } else {
                            v8[e] = (float)pc[e] * (dp[i0 + e] - dl);
                        }
                    }
                    dsf[c] = __builtin_convertvector(v8, e8);
                    ddst[c * kWave + lane] = dsf[c];
                }
#pragma unroll
                for (int dt = 0; dt < 4; ++dt)
#pragma unroll
                    for (int c = 0; c < S::kPChunks; ++c)
                        acc[dt] = mfma_32x32x16(read_cols_op<D, E>(qb, coff, dt, c), dsf[c], acc[dt]);
            }
            __builtin_amdgcn_s_waitcnt(0);
            __syncthreads();
        }
    } else {                                        // KH
        for (int t = t0; t <= last; ++t) {
            if (t + 1 < t_end) load(t + 1);
            const int tq = t - 2;
            if (tq >= wt0 && tq < wt_end) {
                const LDS_AS char *qb = (const LDS_AS char *)qbuf(tq);
                const LDS_AS e8 *dsrc = (const LDS_AS e8 *)((tq & 1) ? sS1 : sS0) + grp * S::kPChunks * kWave;
                e8 dsf[S::kPChunks];
#pragma unroll
                for (int c = 0; c < S::kPChunks; ++c)
                    dsf[c] = dsrc[c * kWave + lane];
#pragma unroll
                for (int dt = 0; dt < 4; ++dt)
#pragma unroll
                    for (int c = 0; c < S::kPChunks; ++c)
                        acc[dt] = mfma_32x32x16(read_cols_op<D, E>(qb, coff, 4 + dt, c), dsf[c], acc[dt]);
            }
            __builtin_amdgcn_s_waitcnt(0);
            __syncthreads();
        }
    }

    if (key >= p.Lk) return;
    const size_t kv_row = (size_t)bh * p.Lk + key;
    uint16_t *dst = static_cast<uint16_t *>(k_side ? p.dk : p.dv) + kv_row * D + 32 * dt0;
    const float mul = k_side ? (DROPOUT ? p.scale * p.drop.keep_scale : p.scale) : (DROPOUT ? p.drop.keep_scale : 1.0f);
    store_tokens_half<E>(dst, acc, mul, hh);
}

// ---------------------------------------------------------------- 3. dQ
// Probabilities of one 32-key score tile (keys x this lane's query, first key
// k0; entry i is key k0 + 8(i/4) + 4hh + i%4) set to 0 where the key is past Lk
// or (MASKED) outside the window of query qrow.
template <bool MASKED>
__device__ __forceinline__ void mask_hidden(f32x16 &pt, int k0, int qrow, int hh, const BwdParams &p)
{
    // keys this lane's query sees: [qrow - wl, qrow + wr] within [0, Lk)
    int64_t lo = 0, hi = (int64_t)p.Lk - 1;
    if (MASKED && p.wl >= 0) lo = max(lo, (int64_t)qrow - p.wl);
    if (MASKED && p.wr >= 0) hi = min(hi, (int64_t)qrow + p.wr);
    keep_range(pt, (int64_t)k0 + 4 * hh, lo, hi, 0.f);
}

// d = 256: Q, dO and the dQ accumulator would take 256 registers;
// fa2_bwd_dq256_kernel below splits the work between wavefront pairs instead.
template <int D, bool MASKED, typename E, bool DROPOUT>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2)))
void fa2_bwd_dq_kernel(BwdParams p)
{
    static_assert(D <= 128, "d = 256 runs fa2_bwd_dq256_kernel");
    using T = BTile<D>;
    using e8 = typename V16<E>::x8;
    constexpr int kDc = D / 16;
    constexpr int kDt = D / 32;
    constexpr int kTileElems = kBc * T::kLdsD;
    __shared__ __attribute__((aligned(1024))) uint16_t sK0[kTileElems];
    __shared__ __attribute__((aligned(1024))) uint16_t sK1[kTileElems];
    __shared__ __attribute__((aligned(1024))) uint16_t sV0[kTileElems];
    __shared__ __attribute__((aligned(1024))) uint16_t sV1[kTileElems];

    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
    const int lane = tid % kWave;
    const int l32 = lane & 31;
    const int hh = lane >> 5;

    int bh, qt;
    map_workgroup(blockIdx.x, p.n_wg, p.n_blocks, bh, qt);
    // K/V tiles [t0, t0 + n_kv) hold a key some row of the block sees (MASKED:
    // the window of the forward's window kernel; causal is (-1, 0)).
    int t0 = 0, n_kv = (p.Lk + kBc - 1) / kBc;
    if (MASKED) {
        const int q_first = qt * kBr;
        const int q_last = min(q_first + kBr - 1, p.Lq - 1);
        const int64_t key_lo = p.wl < 0 ? 0 : max((int64_t)0, (int64_t)q_first - p.wl);
        const int64_t key_hi = p.wr < 0 ? p.Lk : min((int64_t)p.Lk, (int64_t)q_last + p.wr + 1);
        n_kv = 0;
        if (key_hi > key_lo) {
            t0 = (int)(key_lo / kBc);
            n_kv = (int)((key_hi + kBc - 1) / kBc) - t0;
        }
    }

    const size_t kv_off = (size_t)bh * p.Lk * D;
    const __amdgpu_buffer_rsrc_t rK = __builtin_amdgcn_make_buffer_rsrc(
        (void *)(static_cast<const uint16_t *>(p.k) + kv_off), 0, p.Lk * T::kGRowBytes, kRawBufferFlags);
    const __amdgpu_buffer_rsrc_t rV = __builtin_amdgcn_make_buffer_rsrc(
        (void *)(static_cast<const uint16_t *>(p.v) + kv_off), 0, p.Lk * T::kGRowBytes, kRawBufferFlags);

    const int q0 = qt * kBr + wave * kRowsPerWave;
    const int qrow = q0 + l32;
    const bool row_ok = qrow < p.Lq;
    const bool wave_active = q0 < p.Lq;

    // Tiles this wavefront computes, counted from t0: [0, n_wave); those in
    // [plain_lo, n_plain) are seen whole by every row of the wavefront, the others
    // cross a window edge or the end of the keys and are masked per element.
    int n_wave = 0, n_plain = 0, plain_lo = 0;
    if (wave_active) {
        const int wave_qlast = min(q0 + kRowsPerWave - 1, p.Lq - 1);
        int64_t end = t0 + n_kv, first_plain = 0, end_plain = p.Lk / kBc;
        if (MASKED) {
            if (p.wr >= 0) end = min(end, ((int64_t)wave_qlast + p.wr) / kBc + 1);
            const int64_t left = p.wl < 0 ? 0 : (int64_t)wave_qlast - p.wl;
            first_plain = left <= 0 ? 0 : (left + kBc - 1) / kBc;
            if (p.wr >= 0) end_plain = min(end_plain, ((int64_t)q0 + p.wr + 1) / kBc);
        }
        n_wave = (int)max(end - t0, (int64_t)0);
        plain_lo = (int)min(max(first_plain - t0, (int64_t)0), (int64_t)n_wave);
        n_plain = (int)min(max(end_plain - t0, (int64_t)0), (int64_t)n_wave);
    }

    load_tile<D, kBc>(rK, t0 * kBc, sK0, wave, lane);
    load_tile<D, kBc>(rV, t0 * kBc, sV0, wave, lane);

    const size_t qoff = ((size_t)bh * p.Lq + qrow);
    const uint16_t *Qr = static_cast<const uint16_t *>(p.q) + qoff * D;
    const uint16_t *Or = static_cast<const uint16_t *>(p.dout) + qoff * D;
    e8 qf[kDc], of[kDc];
#pragma unroll
    for (int c = 0; c < kDc; ++c) {
        qf[c] = load_row_chunk<E>(Qr + 16 * c + 8 * hh, row_ok);
        of[c] = load_row_chunk<E>(Or + 16 * c + 8 * hh, row_ok);
    }
    const float lse2 = row_ok ? p.lse2[qoff] : 0.f;
    const float dlt = row_ok ? p.delta[qoff] : 0.f;
    const ColsOffsets<D> coff = cols_offsets<D>(lane);
    // Lane offsets of the K and V rows operands (read_rows_at).
    int roff[kDc];
#pragma unroll
    for (int c = 0; c < kDc; ++c)
        roff[c] = BTile<D>::addr(l32, 2 * (16 * c + 8 * hh));

    f32x16 acc[kDt];
#pragma unroll
    for (int t = 0; t < kDt; ++t)
        acc[t] = f32x16{};
    const float c2 = p.scale_log2;

    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();

    // One step per K/V tile; the loop runs two steps per trip so that every
    // buffer is fixed at compile time.
    auto step = [&](int j, const uint16_t *sKc, const uint16_t *sVc, uint16_t *sKn, uint16_t *sVn) {
        if (j + 1 < n_kv) {
            load_tile<D, kBc>(rK, (t0 + j + 1) * kBc, sKn, wave, lane);
            load_tile<D, kBc>(rV, (t0 + j + 1) * kBc, sVn, wave, lane);
        }
        const LDS_AS char *kbuf = (const LDS_AS char *)sKc;
        const LDS_AS char *vbuf = (const LDS_AS char *)sVc;
        int ro[kDc];
#pragma unroll
        for (int c = 0; c < kDc; ++c)
            ro[c] = opaque(roff[c]);
        ColsOffsets<D> co;
#pragma unroll
        for (int dt = 0; dt < kDt; ++dt) {
            co.lo[dt] = opaque(coff.lo[dt]);
            co.hi[dt] = opaque(coff.hi[dt]);
        }
        auto rows_op = [&](const LDS_AS char *tile, int t, int c) {
            return read_rows_at<E>(tile + 32 * t * BTile<D>::kRowBytes, ro[c]);
        };
        if (j < n_wave) {
            // Entry i of score tile t is key 64(t0 + j) + 32t + 8(i/4) + 4hh + i%4.
            const bool need_mask = j < plain_lo || j >= n_plain;
            if constexpr (DROPOUT) {
                // S^T = K Q^T and dP^T = V dO^T for the 32 keys of half t (keys x
                // this wavefront's queries).
                auto products = [&](int t, f32x16 &s_t, f32x16 &dp_t) {
                    s_t = f32x16{};
                    dp_t = f32x16{};
#pragma unroll
                    for (int c = 0; c < kDc; ++c)
                        s_t = mfma_32x32x16(rows_op(kbuf, t, c), qf[c], s_t);
#pragma unroll
                    for (int c = 0; c < kDc; ++c)
                        dp_t = mfma_32x32x16(rows_op(vbuf, t, c), of[c], dp_t);
                };
                // dS / ks of half t (dlt = D / ks, keep bytes y of that half) as the B
                // operands of key chunks 2t, 2t + 1.
                auto dscores = [&](int t, f32x16 &s_t, const f32x16 &dp_t, const u32x4 &y, e8 *dsf) {
#pragma unroll
                    for (int i = 0; i < 16; ++i)
                        s_t[i] = __builtin_amdgcn_exp2f(__builtin_fmaf(s_t[i], c2, -lse2));
                    if (need_mask) mask_hidden<MASKED>(s_t, (t0 + j) * kBc + 32 * t, qrow, hh, p);
#pragma unroll
                    for (int h = 0; h < 2; ++h) {
                        f32x8 ds8;
#pragma unroll
                        for (int e = 0; e < 8; ++e) {
                            const int i = 8 * h + e;
                            const bool kept = ((y[i / 4] >> (8 * (i % 4))) & 0xFFu) < p.drop.threshold;
                            ds8[e] = s_t[i] * (kept ? dp_t[i] - dlt : -dlt);
                        }
                        dsf[h] = __builtin_convertvector(ds8, e8);
                    }
                };
                // One 32-key half at a time (products, keep bytes, dS, dQ update):
                // the generator's registers and one half's accumulators fit beside
                // Q, dO and dQ in the register budget of two wavefronts per SIMD.
#pragma unroll
                for (int t = 0; t < 2; ++t) {
                    const u32x4 y = mask_query_lanes_one(p.drop, (t0 + j) * kBc, t, qrow, lane, bh);
                    f32x16 s_t, dp_t;
                    products(t, s_t, dp_t);
                    e8 dsf[2];
                    dscores(t, s_t, dp_t, y, dsf);
                    // dQ^T += K^T dS^T over the half's keys.
#pragma unroll
                    for (int dt = 0; dt < kDt; ++dt)
#pragma unroll
                        for (int h = 0; h < 2; ++h)
                            acc[dt] = mfma_32x32x16(read_cols_op<D, E>(kbuf, co, dt, 2 * t + h), dsf[h], acc[dt]);
                }
            } else {
                // S^T = K Q^T and dP^T = V dO^T: (keys x this wavefront's queries).
                f32x16 s[2], dp[2];
#pragma unroll
                for (int t = 0; t < 2; ++t) {
                    s[t] = f32x16{};
                    dp[t] = f32x16{};
#pragma unroll
                    for (int c = 0; c < kDc; ++c)
                        s[t] = mfma_32x32x16(rows_op(kbuf, t, c), qf[c], s[t]);
#pragma unroll
                    for (int c = 0; c < kDc; ++c)
                        dp[t] = mfma_32x32x16(rows_op(vbuf, t, c), of[c], dp[t]);
                }
                // Pin the order of these 32 reads and products so that each read is
                // issued two products ahead (the compiler's own schedule read each
                // operand just before its product and waited out the full LDS latency).
                __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
#pragma unroll
                for (int i = 0; i < 4 * kDc - 2; ++i) {
                    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                    __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
                }
                __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
                // P = 2^(S c - lse2) in place; hidden pairs -> 0 under one branch per
                // tile (the same on every lane).
#pragma unroll
                for (int t = 0; t < 2; ++t)
#pragma unroll
                    for (int i = 0; i < 16; ++i)
                        s[t][i] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[t][i], c2, -lse2));
                if (need_mask)
#pragma unroll
                    for (int t = 0; t < 2; ++t)
                        mask_hidden<MASKED>(s[t], (t0 + j) * kBc + 32 * t, qrow, hh, p);
                e8 dsf[4];
#pragma unroll
                for (int c = 0; c < 4; ++c) {
                    const int t = c >> 1, i0 = 8 * (c & 1);
                    f32x8 ds8;
#pragma unroll
                    for (int e = 0; e < 8; ++e)
                        ds8[e] = s[t][i0 + e] * (dp[t][i0 + e] - dlt);
                    dsf[c] = __builtin_convertvector(ds8, e8);
                }
                // dQ^T += K^T dS^T (contraction over the tile's keys).
#pragma unroll
                for (int dt = 0; dt < kDt; ++dt)
#pragma unroll
                    for (int c = 0; c < 4; ++c)
                        acc[dt] = mfma_32x32x16(read_cols_op<D, E>(kbuf, co, dt, c), dsf[c], acc[dt]);
            }
        }
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
    };
    for (int j = 0; j < n_kv; j += 2) {
        step(j, sK0, sV0, sK1, sV1);
        if (j + 1 < n_kv) step(j + 1, sK1, sV1, sK0, sV0);
    }

    if (!row_ok) return;
    store_tokens<D, E>(static_cast<uint16_t *>(p.dq) + qoff * D, acc, DROPOUT ? p.scale * p.drop.keep_scale : p.scale,
                       hh);
}

// d = 256 dQ with two wavefronts per SIMD: for each group of 32 query rows a
// pair of wavefronts, on one SIMD, splits the work of a 32-key tile step:
//  * X (wavefront g):     Q in registers; S and P for key tile j (P to LDS in
//                         fp32, the dropout keep bit in its sign), dQ^T[0:128)
//                         += K^T dS^T for tile j - 2;
//  * Y (wavefront 4 + g): dO in registers; dP for tile j - 1, P from LDS,
//                         dS = P (dP - D) to LDS, dQ^T[128:256) += K^T dS^T.
// K tiles are held four deep (j + 1 loading, j, j - 1, j - 2), V three deep, P
// and dS two deep: one barrier per step, 160 KiB of LDS.  The products, the fp32
// P in dS and the order of every accumulation are those of fa2_bwd_dq_kernel, so
// dQ is bitwise the same.
struct Dq256 {
    static constexpr int kWaves = 8;
    static constexpr int kPairs = 4;
    static constexpr int kTileKeys = 32;
    static constexpr int kPChunks = 2;
    static constexpr int kThreads = kWaves * kWave;
};

template <bool MASKED, typename E, bool DROPOUT>
__global__ __launch_bounds__(Dq256::kThreads) __attribute__((amdgpu_waves_per_eu(2, 2)))
void fa2_bwd_dq256_kernel(BwdParams p)
{
    constexpr int D = 256;
    using T = BTile<D>;
    using S = Dq256;
    using e8 = typename V16<E>::x8;
    constexpr int kDc = D / 16;
    constexpr int kBk = S::kTileKeys;
    constexpr int kTileElems = kBk * T::kLdsD;
    constexpr int kPElems = S::kPairs * S::kPChunks * kWave;
    __shared__ __attribute__((aligned(1024))) uint16_t sK0[kTileElems];
    __shared__ __attribute__((aligned(1024))) uint16_t sK1[kTileElems];
    __shared__ __attribute__((aligned(1024))) uint16_t sK2[kTileElems];
    __shared__ __attribute__((aligned(1024))) uint16_t sK3[kTileElems];
    __shared__ __attribute__((aligned(1024))) uint16_t sV0[kTileElems];
    __shared__ __attribute__((aligned(1024))) uint16_t sV1[kTileElems];
    __shared__ __attribute__((aligned(1024))) uint16_t sV2[kTileElems];
    __shared__ __attribute__((aligned(1024))) f32x8 sP0[kPElems];   // P in fp32
    __shared__ __attribute__((aligned(1024))) f32x8 sP1[kPElems];
    __shared__ __attribute__((aligned(1024))) e8 sS0[kPElems];     // dS
    __shared__ __attribute__((aligned(1024))) e8 sS1[kPElems];

    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
    const int lane = tid % kWave;
    const int l32 = lane & 31;
    const int hh = lane >> 5;
    const int pair = wave & 3;
    const bool is_x = wave < 4;

    int bh, qt;
    map_workgroup(blockIdx.x, p.n_wg, p.n_blocks, bh, qt);
    // 32-key tiles [t0, t0 + n_kv) hold a key some row of the block sees.
    int t0 = 0, n_kv = (p.Lk + kBk - 1) / kBk;
    if (MASKED) {
        const int q_first = qt * kBr;
        const int q_last = min(q_first + kBr - 1, p.Lq - 1);
        const int64_t key_lo = p.wl < 0 ? 0 : max((int64_t)0, (int64_t)q_first - p.wl);
        const int64_t key_hi = p.wr < 0 ? p.Lk : min((int64_t)p.Lk, (int64_t)q_last + p.wr + 1);
        n_kv = 0;
        if (key_hi > key_lo) {
            t0 = (int)(key_lo / kBk);
            n_kv = (int)((key_hi + kBk - 1) / kBk) - t0;
        }
    }

    const size_t kv_off = (size_t)bh * p.Lk * D;
    const __amdgpu_buffer_rsrc_t rK = __builtin_amdgcn_make_buffer_rsrc(
        (void *)(static_cast<const uint16_t *>(p.k) + kv_off), 0, p.Lk * T::kGRowBytes, kRawBufferFlags);
    const __amdgpu_buffer_rsrc_t rV = __builtin_amdgcn_make_buffer_rsrc(
        (void *)(static_cast<const uint16_t *>(p.v) + kv_off), 0, p.Lk * T::kGRowBytes, kRawBufferFlags);

    const int q0 = qt * kBr + pair * kRowsPerWave;
    const int qrow = q0 + l32;
    const bool row_ok = qrow < p.Lq;
    const bool pair_active = q0 < p.Lq;

    // Tiles this pair computes, counted from t0: [0, n_wave); those in
    // [plain_lo, n_plain) are seen whole by every row of the pair.
    int n_wave = 0, n_plain = 0, plain_lo = 0;
    if (pair_active) {
        const int pair_qlast = min(q0 + kRowsPerWave - 1, p.Lq - 1);
        int64_t end = t0 + n_kv, first_plain = 0, end_plain = p.Lk / kBk;
        if (MASKED) {
            if (p.wr >= 0) end = min(end, ((int64_t)pair_qlast + p.wr) / kBk + 1);
            const int64_t left = p.wl < 0 ? 0 : (int64_t)pair_qlast - p.wl;
            first_plain = left <= 0 ? 0 : (left + kBk - 1) / kBk;
            if (p.wr >= 0) end_plain = min(end_plain, ((int64_t)q0 + p.wr + 1) / kBk);
        }
        n_wave = (int)max(end - t0, (int64_t)0);
        plain_lo = (int)min(max(first_plain - t0, (int64_t)0), (int64_t)n_wave);
        n_plain = (int)min(max(end_plain - t0, (int64_t)0), (int64_t)n_wave);
    }

    // Local tile j (global t0 + j): K in slot j % 4, V in slot j % 3.
    auto kbuf = [&](int j) {
        const int s = j & 3;
        return s == 0 ? sK0 : s == 1 ? sK1 : s == 2 ? sK2 : sK3;
    };
    auto vbuf = [&](int j) {
        const int s = j % 3;
        return s == 0 ? sV0 : s == 1 ? sV1 : sV2;
    };
    auto load = [&](int j) {
        load_tile<D, kBk, S::kWaves>(rK, (t0 + j) * kBk, kbuf(j), wave, lane);
        load_tile<D, kBk, S::kWaves>(rV, (t0 + j) * kBk, vbuf(j), wave, lane);
    };
    if (n_kv > 0) load(0);

    // Q (X) or dO (Y) of this lane's row as B operands; zero past Lq.
    const size_t qoff = (size_t)bh * p.Lq + qrow;
    const uint16_t *Rr = static_cast<const uint16_t *>(is_x ? p.q : p.dout) + qoff * D;
    e8 rf[kDc];
#pragma unroll
    for (int c = 0; c < kDc; ++c)
        rf[c] = load_row_chunk<E>(Rr + 16 * c + 8 * hh, row_ok);
    const float stat = row_ok ? (is_x ? p.lse2[qoff] : p.delta[qoff]) : 0.f;   // lse2 (X) or D (Y)
    const ColsOffsets<D> coff = cols_offsets<D>(lane);
    const int dt0 = is_x ? 0 : 4;
    f32x16 acc[4];
#pragma unroll
    for (int t = 0; t < 4; ++t)
        acc[t] = f32x16{};
    const float c2 = p.scale_log2;

    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();

    // dQ^T[half] += K^T dS^T over the tile's 32 keys (B operands dsf).
    auto dq_update = [&](const LDS_AS char *kb, const e8 (&dsf)[S::kPChunks]) {
#pragma unroll
        for (int dt = 0; dt < 4; ++dt)
#pragma unroll
            for (int c = 0; c < S::kPChunks; ++c)
                acc[dt] = mfma_32x32x16(read_cols_op<D, E>(kb, coff, dt0 + dt, c), dsf[c], acc[dt]);
    };
    const int last = n_kv + 1;                      // X finishes its dQ of tile n_kv - 1 at step n_kv + 1
    if (is_x) {
        for (int j = 0; j <= last; ++j) {
            if (j + 1 < n_kv) load(j + 1);
            if (j < n_wave) {
                // S^T = K Q^T (keys x this pair's queries), P = 2^(S c - lse2).
                const LDS_AS char *kb = (const LDS_AS char *)kbuf(j);
                f32x16 s = f32x16{};
#pragma unroll
                for (int c = 0; c < kDc; ++c)
                    s = mfma_32x32x16(read_rows_op<D, E>(kb, l32, c, hh), rf[c], s);
#pragma unroll
                for (int i = 0; i < 16; ++i)
                    s[i] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[i], c2, -stat));
                if (j < plain_lo || j >= n_plain) mask_hidden<MASKED>(s, (t0 + j) * kBk, qrow, hh, p);
                u32x4 y = {};
                if (DROPOUT) y = mask_query_lanes_one(p.drop, (t0 + j) * kBk, 0, qrow, lane, bh);
                LDS_AS f32x8 *pdst = (LDS_AS f32x8 *)((j & 1) ? sP1 : sP0) + pair * S::kPChunks * kWave;
#pragma unroll
                for (int c = 0; c < S::kPChunks; ++c) {
                    f32x8 v8;
#pragma unroll
                    for (int e = 0; e < 8; ++e) {
                        const int i = 8 * c + e;
                        v8[e] = s[i];
                        if (DROPOUT && ((y[i / 4] >> (8 * (i % 4))) & 0xFFu) >= p.drop.threshold) v8[e] = -v8[e];
                    }
                    pdst[c * kWave + lane] = v8;
                }
            }
            const int jq = j - 2;
            if (jq >= 0 && jq < n_wave) {
                const LDS_AS e8 *dsrc = (const LDS_AS e8 *)((jq & 1) ? sS1 : sS0) + pair * S::kPChunks * kWave;
                e8 dsf[S::kPChunks];
#pragma unroll
                for (int c = 0; c < S::kPChunks; ++c)
                    dsf[c] = dsrc[c * kWave + lane];
                dq_update((const LDS_AS char *)kbuf(jq), dsf);
            }
            __builtin_amdgcn_s_waitcnt(0);
            __syncthreads();
        }
    } else {
        for (int j = 0; j <= last; ++j) {
            if (j + 1 < n_kv) load(j + 1);
            const int jk = j - 1;
            if (jk >= 0 && jk < n_wave) {
                // dP^T = V dO^T, dS = P (dP - D) (dropout: dS / ks with D / ks).
                const LDS_AS char *vb = (const LDS_AS char *)vbuf(jk);
                f32x16 dp = f32x16{};
#pragma unroll
                for (int c = 0; c < kDc; ++c)
                    dp = mfma_32x32x16(read_rows_op<D, E>(vb, l32, c, hh), rf[c], dp);
                const LDS_AS f32x8 *psrc = (const LDS_AS f32x8 *)((jk & 1) ? sP1 : sP0) + pair * S::kPChunks * kWave;
                LDS_AS e8 *ddst = (LDS_AS e8 *)((jk & 1) ? sS1 : sS0) + pair * S::kPChunks * kWave;
                e8 dsf[S::kPChunks];
#pragma unroll
                for (int c = 0; c < S::kPChunks; ++c) {
                    const f32x8 pc = psrc[c * kWave + lane];
                    f32x8 v8;
#pragma unroll
                    for (int e = 0; e < 8; ++e) {
                        const float pr = pc[e];
                        if (DROPOUT)
                            v8[e] = __builtin_fabsf(pr) * (__builtin_signbit(pr) ? -stat : dp[8 * c + e] - stat);
                        else
                            v8[e] = pr * (dp[8 * c + e] - stat);
                    }
                    dsf[c] = __builtin_convertvector(v8, e8);
                    ddst[c * kWave + lane] = dsf[c];
                }
                dq_update((const LDS_AS char *)kbuf(jk), dsf);
            }
            __builtin_amdgcn_s_waitcnt(0);
            __syncthreads();
        }
    }

    if (!row_ok) return;
    store_tokens_half<E>(static_cast<uint16_t *>(p.dq) + qoff * D + 32 * dt0, acc,
                         DROPOUT ? p.scale * p.drop.keep_scale : p.scale, hh);
}

template <int D, typename E, bool DROPOUT = false>
hipError_t launch_bwd_d(const BwdParams &p, bool masked, int64_t rows, const void *o, const float *lse,
                        hipStream_t stream)
{
    const int64_t threads = rows * kPrepThreadsPerRow<D>;
    hipLaunchKernelGGL((fa2_bwd_prep_kernel<D, E>), dim3((unsigned)((threads + 255) / 256)), dim3(256), 0, stream,
                       static_cast<const uint16_t *>(o), static_cast<const uint16_t *>(p.dout), lse,
                       const_cast<float *>(p.lse2), const_cast<float *>(p.delta), rows,
                       DROPOUT ? 1.0f / p.drop.keep_scale : 1.0f);
    BwdParams pk = p;
    if constexpr (D == 256) {
        pk.n_blocks = (p.Lk + Dkdv256::kKeyBlock - 1) / Dkdv256::kKeyBlock;
        pk.n_wg = pk.n_blocks * p.B * p.H;
        if (masked)
            hipLaunchKernelGGL((fa2_bwd_dkdv256_kernel<true, E, DROPOUT>), dim3(pk.n_wg), dim3(Dkdv256::kThreads), 0,
                               stream, pk);
        else
            hipLaunchKernelGGL((fa2_bwd_dkdv256_kernel<false, E, DROPOUT>), dim3(pk.n_wg), dim3(Dkdv256::kThreads), 0,
                               stream, pk);
    } else {
        pk.n_blocks = (p.Lk + DkdvShape<D>::kKeyBlock - 1) / DkdvShape<D>::kKeyBlock;
        pk.n_wg = pk.n_blocks * p.B * p.H;
        if (masked)
            hipLaunchKernelGGL((fa2_bwd_dkdv_kernel<D, true, E, DROPOUT>), dim3(pk.n_wg), dim3(DkdvShape<D>::kThreads),
                               0, stream, pk);
        else
            hipLaunchKernelGGL((fa2_bwd_dkdv_kernel<D, false, E, DROPOUT>), dim3(pk.n_wg), dim3(DkdvShape<D>::kThreads),
                               0, stream, pk);
    }
    BwdParams pq = p;
    pq.n_blocks = (p.Lq + kBr - 1) / kBr;
    pq.n_wg = pq.n_blocks * p.B * p.H;
    if constexpr (D == 256) {
        if (masked) hipLaunchKernelGGL((fa2_bwd_dq256_kernel<true, E, DROPOUT>), dim3(pq.n_wg), dim3(Dq256::kThreads), 0, stream, pq);
        else        hipLaunchKernelGGL((fa2_bwd_dq256_kernel<false, E, DROPOUT>), dim3(pq.n_wg), dim3(Dq256::kThreads), 0, stream, pq);
    } else {
        if (masked) hipLaunchKernelGGL((fa2_bwd_dq_kernel<D, true, E, DROPOUT>), dim3(pq.n_wg), dim3(kThreads), 0, stream, pq);
        else        hipLaunchKernelGGL((fa2_bwd_dq_kernel<D, false, E, DROPOUT>), dim3(pq.n_wg), dim3(kThreads), 0, stream, pq);
    }
    return hipGetLastError();
}

}  // namespace

hipError_t launch_bwd16(const BwdParams &p, int d, bool f16, bool dropout, const void *o, const float *lse,
                        hipStream_t stream)
{
    const int64_t rows = (int64_t)p.B * p.H * p.Lq;
    const bool masked = p.wl >= 0 || p.wr >= 0;
    hipError_t err = hipSuccess;
    with_head_dim<true, true>(d, [&](auto dim) {
        constexpr int D = decltype(dim)::value;
        if (f16) err = dropout ? launch_bwd_d<D, _Float16, true>(p, masked, rows, o, lse, stream)
                               : launch_bwd_d<D, _Float16, false>(p, masked, rows, o, lse, stream);
        else     err = dropout ? launch_bwd_d<D, __bf16, true>(p, masked, rows, o, lse, stream)
                               : launch_bwd_d<D, __bf16, false>(p, masked, rows, o, lse, stream);
    });
    return err;
}

}  // namespace fa2
