// fa2_fwd_bf16.hip -- FlashAttention-2 forward, bf16 in/out, for gfx950.
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
// Layout choices (MI355X-specific):
//  * Scores are computed transposed (keys down the MFMA rows, queries across the
//    lanes).  A lane then holds 16 keys of ONE query per 32x32 accumulator, so
//    the row max / row sum need one exchange between the two wavefront halves,
//    alpha is per lane, and the accumulator is already the B operand of the
//    P~V product (up to a fixed permutation of keys that V^T in LDS absorbs).
//  * K is kept row-major in LDS (the A operand reads 8 consecutive d).
//    V is transposed into LDS with keys in that permuted order, so the A operand
//    of the P~V product is one 16-byte read.
//  * Q stays in registers for the whole K/V loop (read from HBM once).
#include "fa2_internal.h"

namespace fa2 {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// LDS row pitches (elements).  The extra 8 elements (16 bytes) shift successive
// rows across banks.
template <int D> struct Lds {
    static constexpr int kPitch = D + 8;         // K tile, row-major [key][d]
    static constexpr int vPitch = kBc + 8;       // V tile, transposed [d][key']
};

// Position of key `kk` (0..63 within a tile) in the transposed V tile.
// Accumulator entry i of the 32x32 score tile t, in lane half h, is key
// 32t + 8(i/4) + 4h + i%4.  The P~V MFMA over 16 keys (chunk c) takes 8 of
// these per lane: entries 8(c%2)..8(c%2)+7 of tile c/2.  Storing key kk at
// 16c + 8h + 4(a%2) + b  (a = (kk%32)/8, b = kk%4) makes those 8 keys one
// contiguous 16-byte run at column 16c + 8h.
__device__ __forceinline__ int vt_pos_of_group(int kg)   // kg = kk / 4
{
    const int t = kg >> 3, a = (kg >> 1) & 3, h = kg & 1;
    const int c = 2 * t + (a >> 1);
    return 16 * c + 8 * h + 4 * (a & 1);
}

template <int D>
__device__ __forceinline__ void stage_kv_tile(const uint16_t *__restrict__ K,
                                              const uint16_t *__restrict__ V,
                                              int k0, int Lk, int tid,
                                              uint16_t *sK, uint16_t *sVt)
{
    constexpr int KP = Lds<D>::kPitch, VP = Lds<D>::vPitch;
    constexpr int kChunksPerRow = D / 8;                     // 16-byte chunks
    // K: row-major copy, 16 bytes per access, consecutive threads along a row.
#pragma unroll
    for (int r = 0; r < kBc * kChunksPerRow / kThreads; ++r) {
        const int c = tid + kThreads * r;
        const int row = c / kChunksPerRow;
        const int col = (c % kChunksPerRow) * 8;
        u32x4 val = {0u, 0u, 0u, 0u};
        if (k0 + row < Lk)
            val = *reinterpret_cast<const u32x4 *>(K + (size_t)(k0 + row) * D + col);
        *reinterpret_cast<u32x4 *>(sK + row * KP + col) = val;
    }
    // V: each thread takes 4 consecutive keys x 8 consecutive d and writes the
    // 8 transposed runs of 4 keys (8 bytes each).
    constexpr int kGroups = (kBc / 4) * kChunksPerRow;
#pragma unroll
    for (int g0 = 0; g0 < kGroups; g0 += kThreads) {
        const int g = g0 + tid;
        if (kGroups % kThreads != 0 && g >= kGroups) break;
        const int dc = g % kChunksPerRow;
        const int kg = g / kChunksPerRow;
        u32x4 rows[4];
#pragma unroll
        for (int b = 0; b < 4; ++b) {
            const int key = k0 + 4 * kg + b;
            rows[b] = u32x4{0u, 0u, 0u, 0u};
            if (key < Lk)
                rows[b] = *reinterpret_cast<const u32x4 *>(V + (size_t)key * D + dc * 8);
        }
        const int pos = vt_pos_of_group(kg);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const uint32_t r0 = rows[0][e], r1 = rows[1][e], r2 = rows[2][e], r3 = rows[3][e];
            // element 2e of each row is the low half, element 2e+1 the high half
            const u32x2 lo = {__builtin_amdgcn_perm(r1, r0, 0x05040100u),
                              __builtin_amdgcn_perm(r3, r2, 0x05040100u)};
            const u32x2 hi = {__builtin_amdgcn_perm(r1, r0, 0x07060302u),
                              __builtin_amdgcn_perm(r3, r2, 0x07060302u)};
            *reinterpret_cast<u32x2 *>(sVt + (8 * dc + 2 * e) * VP + pos) = lo;
            *reinterpret_cast<u32x2 *>(sVt + (8 * dc + 2 * e + 1) * VP + pos) = hi;
        }
    }
}

template <int D, bool CAUSAL>
__global__ __launch_bounds__(kThreads)
void fa2_fwd_bf16_kernel(FwdParams p)
{
    constexpr int KP = Lds<D>::kPitch, VP = Lds<D>::vPitch;
    constexpr int kDc = D / 16;          // 16-wide d chunks of the QK^T product
    constexpr int kDt = D / 32;          // 32-row d tiles of the output
    __shared__ __attribute__((aligned(16))) uint16_t sK[kBc * KP];
    __shared__ __attribute__((aligned(16))) uint16_t sVt[D * VP];

    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
    const int lane = tid % kWave;
    const int l32 = lane & 31;
    const int hh = lane >> 5;

    int bh, qt;
    map_workgroup(blockIdx.x, p.n_wg, p.n_qtiles, bh, qt);

    const uint16_t *Q = static_cast<const uint16_t *>(p.q) + (size_t)bh * p.Lq * D;
    const uint16_t *K = static_cast<const uint16_t *>(p.k) + (size_t)bh * p.Lk * D;
    const uint16_t *V = static_cast<const uint16_t *>(p.v) + (size_t)bh * p.Lk * D;

    const int q0 = qt * kBr + wave * kRowsPerWave;    // first row of this wavefront
    const int qrow = q0 + l32;                        // this lane's query row
    const bool wave_active = q0 < p.Lq;               // wave-uniform
    const int wave_qlast = min(q0 + kRowsPerWave - 1, p.Lq - 1);

    // Q fragment: lane holds Q[qrow][16c + 8hh .. +7] for every chunk c.
    bf16x8 qf[kDc];
#pragma unroll
    for (int c = 0; c < kDc; ++c) {
        u32x4 raw = {0u, 0u, 0u, 0u};
        if (qrow < p.Lq)
            raw = *reinterpret_cast<const u32x4 *>(Q + (size_t)qrow * D + 16 * c + 8 * hh);
        qf[c] = __builtin_bit_cast(bf16x8, raw);
    }

    f32x16 acc_o[kDt];
#pragma unroll
    for (int t = 0; t < kDt; ++t)
        acc_o[t] = f32x16{};
    float m = -INFINITY;     // running max (base-2 units), per query row
    float lpart = 0.f;       // running sum over this lane's half of the keys

    const float c2 = p.scale_log2;
    const int n_kv = kv_tiles_for(qt, p.Lq, p.Lk, CAUSAL);

    for (int j = 0; j < n_kv; ++j) {
        const int k0 = j * kBc;
        __syncthreads();                       // everyone is done with the previous tile
        stage_kv_tile<D>(K, V, k0, p.Lk, tid, sK, sVt);
        __syncthreads();

        if (!wave_active) continue;
        if (CAUSAL && k0 > wave_qlast) continue;   // every key is masked for this wave

        // S^T (two 32x32 tiles of keys x queries)
        f32x16 s[2];
#pragma unroll
        for (int t = 0; t < 2; ++t) {
            s[t] = f32x16{};
#pragma unroll
            for (int c = 0; c < kDc; ++c) {
                const bf16x8 a = *reinterpret_cast<const bf16x8 *>(sK + (32 * t + l32) * KP + 16 * c + 8 * hh);
                s[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[c], s[t], 0, 0, 0);
            }
        }

        const bool need_mask = (k0 + kBc > p.Lk) || (CAUSAL && k0 + kBc - 1 > q0);
        if (need_mask) {
#pragma unroll
            for (int t = 0; t < 2; ++t)
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    const int key = k0 + 32 * t + 8 * (i / 4) + 4 * hh + (i % 4);
                    const bool hidden = key >= p.Lk || (CAUSAL && key > qrow);
                    s[t][i] = hidden ? -INFINITY : s[t][i];
                }
        }

        // running max over the row (this lane's 32 keys, then the other half's)
        float mx = s[0][0];
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
            for (int i = 0; i < 16; ++i)
                mx = fmaxf(mx, s[t][i]);
        mx = fmaxf(mx, swap_halves(mx));
        const float m_new = fmaxf(m, mx * c2);
        const float alpha = __builtin_amdgcn_exp2f(m - m_new);

        float rs = 0.f;
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const float e = __builtin_amdgcn_exp2f(__builtin_fmaf(s[t][i], c2, -m_new));
                s[t][i] = e;
                rs += e;
            }
        lpart = __builtin_fmaf(lpart, alpha, rs);
        m = m_new;

#pragma unroll
        for (int t = 0; t < kDt; ++t)
            acc_o[t] *= alpha;

        // P~^T as bf16 B operands, one per 16-key chunk
        bf16x8 pf[4];
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            const int t = c >> 1, i0 = 8 * (c & 1);
            const f32x8 v8 = {s[t][i0 + 0], s[t][i0 + 1], s[t][i0 + 2], s[t][i0 + 3],
                              s[t][i0 + 4], s[t][i0 + 5], s[t][i0 + 6], s[t][i0 + 7]};
            pf[c] = __builtin_convertvector(v8, bf16x8);
        }

        // O~^T += V^T P~^T
#pragma unroll
        for (int dt = 0; dt < kDt; ++dt)
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                const bf16x8 a = *reinterpret_cast<const bf16x8 *>(sVt + (32 * dt + l32) * VP + 16 * c + 8 * hh);
                acc_o[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pf[c], acc_o[dt], 0, 0, 0);
            }
    }

    if (!wave_active) return;
    const float l = lpart + swap_halves(lpart);
    if (qrow >= p.Lq) return;
    const float inv_l = 1.0f / l;
    uint16_t *O = static_cast<uint16_t *>(p.o) + ((size_t)bh * p.Lq + qrow) * D;
#pragma unroll
    for (int dt = 0; dt < kDt; ++dt)
#pragma unroll
        for (int a = 0; a < 4; ++a) {
            const f32x4 v4 = {acc_o[dt][4 * a + 0] * inv_l, acc_o[dt][4 * a + 1] * inv_l,
                              acc_o[dt][4 * a + 2] * inv_l, acc_o[dt][4 * a + 3] * inv_l};
            const bf16x4 b4 = __builtin_convertvector(v4, bf16x4);
            *reinterpret_cast<bf16x4 *>(O + 32 * dt + 8 * a + 4 * hh) = b4;
        }
    if (hh == 0)
        p.lse[(size_t)bh * p.Lq + qrow] = (m + __builtin_amdgcn_logf(l)) * kLn2;
}

}  // namespace

hipError_t launch_fwd_bf16(const FwdParams &p, int d, bool causal, hipStream_t stream)
{
    const dim3 grid(p.n_wg), block(kThreads);
    if (d == 64) {
        if (causal) hipLaunchKernelGGL((fa2_fwd_bf16_kernel<64, true>), grid, block, 0, stream, p);
        else        hipLaunchKernelGGL((fa2_fwd_bf16_kernel<64, false>), grid, block, 0, stream, p);
    } else {
        if (causal) hipLaunchKernelGGL((fa2_fwd_bf16_kernel<128, true>), grid, block, 0, stream, p);
        else        hipLaunchKernelGGL((fa2_fwd_bf16_kernel<128, false>), grid, block, 0, stream, p);
    }
    return hipGetLastError();
}

}  // namespace fa2
