// fa2_decode.hip -- split-KV partial results for a handful of query rows
// (decoding: one new token, or a few, against a long K/V history).
//
// With Lq <= kDecodeMaxRows the matrix cores have nothing to do: the MFMA kernel
// computes 32 rows per wavefront for the one that exists, and its LDS staging
// serves a reuse that is not there.  This kernel instead streams K and V from HBM
// straight into registers, as long coalesced rows, with many loads in flight per
// lane, and does the few multiply-adds per element on the vector ALU in fp32.
// It is the first stage of FlashDecoding ("Flash Attention 全解析（上）", section
// 4.3: the K/V sequence split across work-groups, each producing a partial result
// and its logsumexp); the merge kernel is the second.
//
// Work-group (bh, split s): keys [lo, hi) of the split.  A key row is D/8
// 16-byte chunks; kLanes (D/8 rounded up to a power of two) consecutive lanes
// hold one key, so one wavefront load covers 64 / kLanes consecutive keys of K
// (and of V) -- contiguous memory.  Each lane keeps, per query row r, the online
// softmax state of the keys its lane group saw: max m (base-2 units), sum l and
// the 8 output columns of its chunk.  Every step loads kUnroll key groups of K
// and V per wavefront before using any (2 kUnroll loads of 16 bytes in flight
// per lane), takes the dot products (partial sums reduced across the kLanes lanes
// of a key), moves the max once per step, and accumulates.  At the end the lane
// groups of a wavefront, then the four wavefronts, are merged with the same
// rescale-by-max rule, and lane group 0 of wavefront 0 writes O_s = O~ / l (fp32)
// and L_s; a row that sees no key of the range gets L_s = -inf and no O_s.
#include "fa2_internal.h"

namespace fa2 {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x8 __attribute__((ext_vector_type(8)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// 8 elements of E (bf16 or fp16) from their 16 raw bytes, widened to fp32.
template <typename E>
__device__ __forceinline__ f32x8 widen8(u32x4 raw)
{
    typedef E e8 __attribute__((ext_vector_type(8)));
    return __builtin_convertvector(__builtin_bit_cast(e8, raw), f32x8);
}

constexpr int kDecodeThreads = 256;

// kUnroll key groups per step: 8 for one row; 4 for more rows, whose per-row state
// and scores take the registers (so that two or more wavefronts share a SIMD).
template <int D, int R> struct DecodeShape {
    static constexpr int kChunks = D / 8;                               // 16-byte chunks per row
    static constexpr int kLanes = kChunks <= 4 ? 4 : kChunks <= 8 ? 8 : kChunks <= 16 ? 16 : 32;
    static constexpr int kKeysPerLoad = kWave / kLanes;                 // keys per wavefront load
    static constexpr int kUnroll = R == 1 ? 8 : 4;
    static constexpr int kKeysPerStep = kDecodeThreads / kLanes * kUnroll;
};

// Combine the state (m, l, acc) of another lane group into this one.
template <int R>
__device__ __forceinline__ void combine(float (&m)[R], float (&l)[R], f32x8 (&acc)[R], const float (&m2)[R],
                                        const float (&l2)[R], const f32x8 (&acc2)[R])
{
#pragma unroll
    for (int r = 0; r < R; ++r) {
        const float mn = fmaxf(m[r], m2[r]);
        // an empty side (m = -inf, l = 0) contributes nothing; keep 0 * inf out
        const float a = m[r] == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(m[r] - mn);
        const float b = m2[r] == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(m2[r] - mn);
        l[r] = l[r] * a + l2[r] * b;
        acc[r] = acc[r] * a + acc2[r] * b;
        m[r] = mn;
    }
}

template <int D, int R, typename E>
__global__ __launch_bounds__(kDecodeThreads) void fa2_decode_kernel(FwdParams p)
{
    using S = DecodeShape<D, R>;
    constexpr int kUnroll = S::kUnroll;
    const int tid = threadIdx.x;
    const int wave = tid / kWave;
    const int lane = tid % kWave;
    const int chunk = lane % S::kLanes;                  // this lane's 16-byte chunk of a row
    const bool has_chunk = chunk < S::kChunks;           // d = 96: lanes 12..15 of a group idle
    const int group = lane / S::kLanes;                  // key group within the wavefront load

    const int split = blockIdx.x % p.n_splits;
    const int bh = blockIdx.x / p.n_splits;
    // Keys of this split; under the causal mask no row sees a key >= Lq.
    const int kmax = p.wr == 0 ? min(p.Lk, p.Lq) : p.Lk;   // (wr = 0: causal)
    const int lo = (int)((int64_t)split * kmax / p.n_splits);
    const int hi = (int)((int64_t)(split + 1) * kmax / p.n_splits);

    // Q rows of this head, pre-scaled by scale * log2(e); zero for rows >= Lq.
    f32x8 qv[R];
#pragma unroll
    for (int r = 0; r < R; ++r) {
        u32x4 raw = {0u, 0u, 0u, 0u};
        if (r < p.Lq && has_chunk)
            raw = *reinterpret_cast<const u32x4 *>(static_cast<const uint16_t *>(p.q) +
                                                   ((size_t)bh * p.Lq + r) * D + 8 * chunk);
        qv[r] = widen8<E>(raw) * p.scale_log2;
    }

    float m[R], l[R];
    f32x8 acc[R];
#pragma unroll
    for (int r = 0; r < R; ++r) {
        m[r] = -INFINITY;
        l[r] = 0.0f;
        acc[r] = f32x8{};
    }

    const uint16_t *Kh = static_cast<const uint16_t *>(p.k) + (size_t)bh * p.Lk * D;
    const uint16_t *Vh = static_cast<const uint16_t *>(p.v) + (size_t)bh * p.Lk * D;
    const int first = lo + wave * S::kKeysPerLoad + group;   // this lane's first key
    constexpr int kStride = kDecodeThreads / S::kLanes;      // keys between a lane's successive loads

    for (int base = 0; lo + base < hi; base += S::kKeysPerStep) {
        u32x4 kr[kUnroll], vr[kUnroll];
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            const int key = first + base + u * kStride;
            kr[u] = u32x4{0u, 0u, 0u, 0u};
            vr[u] = u32x4{0u, 0u, 0u, 0u};
            if (key < hi && has_chunk) {
                kr[u] = *reinterpret_cast<const u32x4 *>(Kh + (size_t)key * D + 8 * chunk);
                vr[u] = *reinterpret_cast<const u32x4 *>(Vh + (size_t)key * D + 8 * chunk);
            }
        }
        float s[kUnroll][R];
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            const f32x8 kf = widen8<E>(kr[u]);
#pragma unroll
            for (int r = 0; r < R; ++r) {
                float d = 0.0f;
#pragma unroll
                for (int e = 0; e < 8; ++e)
                    d = __builtin_fmaf(qv[r][e], kf[e], d);
#pragma unroll
                for (int off = 1; off < S::kLanes; off <<= 1)
                    d += __shfl_xor(d, off, S::kLanes);
                const int key = first + base + u * kStride;
                const bool hidden = key >= hi || (p.wr == 0 && key > r);
                s[u][r] = hidden ? -INFINITY : d;
            }
        }
#pragma unroll
        for (int r = 0; r < R; ++r) {
            float mb = s[0][r];
#pragma unroll
            for (int u = 1; u < kUnroll; ++u)
                mb = fmaxf(mb, s[u][r]);
            const float mn = fmaxf(m[r], mb);
            if (mn == -INFINITY) continue;               // nothing visible yet
            const float alpha = __builtin_amdgcn_exp2f(m[r] - mn);   // 0 when m was -inf
            l[r] *= alpha;
            acc[r] *= alpha;
#pragma unroll
            for (int u = 0; u < kUnroll; ++u) {
                const float pu = __builtin_amdgcn_exp2f(s[u][r] - mn);
                l[r] += pu;
                acc[r] += pu * widen8<E>(vr[u]);
            }
            m[r] = mn;
        }
    }

    // Merge the lane groups of the wavefront (lanes with the same chunk).
#pragma unroll
    for (int off = S::kLanes; off < kWave; off <<= 1) {
        float m2[R], l2[R];
        f32x8 acc2[R];
#pragma unroll
        for (int r = 0; r < R; ++r) {
            m2[r] = __shfl_xor(m[r], off);
            l2[r] = __shfl_xor(l[r], off);
#pragma unroll
            for (int e = 0; e < 8; ++e)
                acc2[r][e] = __shfl_xor(acc[r][e], off);
        }
        combine<R>(m, l, acc, m2, l2, acc2);
    }
    // Merge the four wavefronts through LDS (lane group 0 of each).
    __shared__ float sM[kWaves][R][S::kLanes], sL[kWaves][R][S::kLanes];
    __shared__ f32x8 sAcc[kWaves][R][S::kLanes];
    if (lane < S::kLanes) {
#pragma unroll
        for (int r = 0; r < R; ++r) {
            sM[wave][r][lane] = m[r];
            sL[wave][r][lane] = l[r];
            sAcc[wave][r][lane] = acc[r];
        }
    }
    __syncthreads();
    if (wave != 0 || lane >= S::kLanes) return;
#pragma unroll
    for (int w = 1; w < kWaves; ++w) {
        float m2[R], l2[R];
        f32x8 acc2[R];
#pragma unroll
        for (int r = 0; r < R; ++r) {
            m2[r] = sM[w][r][lane];
            l2[r] = sL[w][r][lane];
            acc2[r] = sAcc[w][r][lane];
        }
        combine<R>(m, l, acc, m2, l2, acc2);
    }
    const size_t part_row0 = ((size_t)split * p.B * p.H + bh) * p.Lq;
#pragma unroll
    for (int r = 0; r < R; ++r) {
        if (r >= p.Lq) break;
        float lse = -INFINITY;
        if (l[r] > 0.0f) {
            if (has_chunk) {
                const f32x8 o = acc[r] * (1.0f / l[r]);
                float *Op = static_cast<float *>(p.o) + (part_row0 + r) * D + 8 * chunk;
                *reinterpret_cast<f32x4 *>(Op) = f32x4{o[0], o[1], o[2], o[3]};
                *reinterpret_cast<f32x4 *>(Op + 4) = f32x4{o[4], o[5], o[6], o[7]};
            }
            lse = (m[r] + __builtin_amdgcn_logf(l[r])) * kLn2;
        }
        if (lane == 0) p.lse[part_row0 + r] = lse;
    }
}

}  // namespace

namespace {
template <typename E>
void launch_decode_e(const FwdParams &p, int d, hipStream_t stream)
{
    const dim3 grid(p.n_wg), block(kDecodeThreads);
    with_head_dim<true, true>(d, [&](auto dim) {
        constexpr int D = decltype(dim)::value;
        switch (p.Lq) {
        case 1: hipLaunchKernelGGL((fa2_decode_kernel<D, 1, E>), grid, block, 0, stream, p); break;
        case 2: hipLaunchKernelGGL((fa2_decode_kernel<D, 2, E>), grid, block, 0, stream, p); break;
        case 3: hipLaunchKernelGGL((fa2_decode_kernel<D, 3, E>), grid, block, 0, stream, p); break;
        default: hipLaunchKernelGGL((fa2_decode_kernel<D, 4, E>), grid, block, 0, stream, p); break;
        }
    });
}
}  // namespace

hipError_t launch_decode(const FwdParams &p, int d, bool f16, hipStream_t stream)
{
    if (f16) launch_decode_e<_Float16>(p, d, stream);
    else     launch_decode_e<__bf16>(p, d, stream);
    return hipGetLastError();
}

}  // namespace fa2
