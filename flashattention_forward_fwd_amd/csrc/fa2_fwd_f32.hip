// fa2_fwd_f32.hip -- FlashAttention-2 forward with fp32 in/out, for gfx950.
//
// Same tiling and online-softmax update as the bf16 kernel (Q tile of 128 rows
// per work-group, 32 rows per wavefront, K/V tiles of 64 keys through LDS,
// transposed scores, deferred division), but every product runs on the fp32
// matrix-core instruction (32x32x2, fp32 in, fp32 accumulate) and the
// probabilities stay fp32: no step is taken in reduced precision.
//
// Operand placement for the 32x32x2 fp32 MFMA (one k pair per instruction, the
// lower lane half supplies k-slot 0 and the upper half k-slot 1):
//  * S^T = K Q^T: instruction `c` contracts d = c (lower half) and d = D/2 + c
//    (upper half), so each lane reads 4 consecutive d of its K row per 16 bytes.
//  * O~^T += V^T P~^T: instruction i of score tile t contracts the two keys the
//    lane halves hold in accumulator entry i (32t + 8(i/4) + 4h + i%4), so the
//    probabilities are used in place and V stays row-major in LDS.
#include "fa2_internal.h"

namespace fa2 {
namespace {

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

template <int D> struct LdsF {
    static constexpr int pitch = D + 4;    // floats per K or V row in LDS
};

template <int D, bool CAUSAL>
__global__ __launch_bounds__(kThreads)
void fa2_fwd_f32_kernel(FwdParams p)
{
    constexpr int P = LdsF<D>::pitch;
    constexpr int kHalf = D / 2;
    constexpr int kDt = D / 32;
    __shared__ __attribute__((aligned(16))) float sK[kBc * P];
    __shared__ __attribute__((aligned(16))) float sV[kBc * P];

    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
    const int lane = tid % kWave;
    const int l32 = lane & 31;
    const int hh = lane >> 5;

    int bh, qt;
    map_workgroup(blockIdx.x, p.n_wg, p.n_qtiles, bh, qt);

    const float *Q = static_cast<const float *>(p.q) + (size_t)bh * p.Lq * D;
    const float *K = static_cast<const float *>(p.k) + (size_t)bh * p.Lk * D;
    const float *V = static_cast<const float *>(p.v) + (size_t)bh * p.Lk * D;

    const int q0 = qt * kBr + wave * kRowsPerWave;
    const int qrow = q0 + l32;
    const bool wave_active = q0 < p.Lq;
    const int wave_qlast = min(q0 + kRowsPerWave - 1, p.Lq - 1);

    // Q fragment: lane holds Q[qrow][hh*D/2 .. hh*D/2 + D/2 - 1]
    f32x4 qf[kHalf / 4];
#pragma unroll
    for (int c = 0; c < kHalf / 4; ++c) {
        qf[c] = f32x4{0.f, 0.f, 0.f, 0.f};
        if (qrow < p.Lq)
            qf[c] = *reinterpret_cast<const f32x4 *>(Q + (size_t)qrow * D + hh * kHalf + 4 * c);
    }

    f32x16 acc_o[kDt];
#pragma unroll
    for (int t = 0; t < kDt; ++t)
        acc_o[t] = f32x16{};
    float m = -INFINITY;
    float lpart = 0.f;

    const float c2 = p.scale_log2;
    const int n_kv = kv_tiles_for(qt, p.Lq, p.Lk, CAUSAL);

    for (int j = 0; j < n_kv; ++j) {
        const int k0 = j * kBc;
        __syncthreads();
        constexpr int kChunks = D / 4;                       // 16-byte chunks per row
#pragma unroll
        for (int r = 0; r < kBc * kChunks / kThreads; ++r) {
            const int c = tid + kThreads * r;
            const int row = c / kChunks;
            const int col = (c % kChunks) * 4;
            f32x4 kv = {0.f, 0.f, 0.f, 0.f}, vv = {0.f, 0.f, 0.f, 0.f};
            if (k0 + row < p.Lk) {
                kv = *reinterpret_cast<const f32x4 *>(K + (size_t)(k0 + row) * D + col);
                vv = *reinterpret_cast<const f32x4 *>(V + (size_t)(k0 + row) * D + col);
            }
            *reinterpret_cast<f32x4 *>(sK + row * P + col) = kv;
            *reinterpret_cast<f32x4 *>(sV + row * P + col) = vv;
        }
        __syncthreads();

        if (!wave_active) continue;
        if (CAUSAL && k0 > wave_qlast) continue;

        f32x16 s[2];
#pragma unroll
        for (int t = 0; t < 2; ++t) {
            s[t] = f32x16{};
            const float *krow = sK + (32 * t + l32) * P + hh * kHalf;
#pragma unroll
            for (int c = 0; c < kHalf / 4; ++c) {
                const f32x4 a = *reinterpret_cast<const f32x4 *>(krow + 4 * c);
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    s[t] = __builtin_amdgcn_mfma_f32_32x32x2f32(a[e], qf[c][e], s[t], 0, 0, 0);
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

        float mx = s[0][0];
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
            for (int i = 0; i < 16; ++i)
                mx = fmaxf(mx, s[t][i]);
        mx = halves_max(mx);
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
        for (int dt = 0; dt < kDt; ++dt) {
            acc_o[dt] *= alpha;
#pragma unroll
            for (int t = 0; t < 2; ++t)
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    const int key = 32 * t + 8 * (i / 4) + 4 * hh + (i % 4);
                    const float a = sV[key * P + 32 * dt + l32];
                    acc_o[dt] = __builtin_amdgcn_mfma_f32_32x32x2f32(a, s[t][i], acc_o[dt], 0, 0, 0);
                }
        }
    }

    if (!wave_active) return;
    const float l = halves_sum(lpart);
    if (qrow >= p.Lq) return;
    float *O = static_cast<float *>(p.o) + ((size_t)bh * p.Lq + qrow) * D;
#pragma unroll
    for (int dt = 0; dt < kDt; ++dt)
#pragma unroll
        for (int a = 0; a < 4; ++a) {
            const f32x4 v4 = {acc_o[dt][4 * a + 0] / l, acc_o[dt][4 * a + 1] / l,
                              acc_o[dt][4 * a + 2] / l, acc_o[dt][4 * a + 3] / l};
            *reinterpret_cast<f32x4 *>(O + 32 * dt + 8 * a + 4 * hh) = v4;
        }
    if (hh == 0)
        p.lse[(size_t)bh * p.Lq + qrow] = (m + __builtin_amdgcn_logf(l)) * kLn2;
}

}  // namespace

hipError_t launch_fwd_f32(const FwdParams &p, int d, bool causal, hipStream_t stream)
{
    const dim3 grid(p.n_wg), block(kThreads);
    with_head_dim(d, [&](auto dim) {
        constexpr int D = decltype(dim)::value;
        if (causal) hipLaunchKernelGGL((fa2_fwd_f32_kernel<D, true>), grid, block, 0, stream, p);
        else        hipLaunchKernelGGL((fa2_fwd_f32_kernel<D, false>), grid, block, 0, stream, p);
    });
    return hipGetLastError();
}

}  // namespace fa2
