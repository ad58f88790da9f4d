// fa2_merge.hip -- combine partial attention results over disjoint key sets.
//
// Each part s holds, per query row, the output normalised by its own row sum,
// O_s, and its logsumexp L_s.  The result over the union of the key sets is
//     M = max_s L_s,   W = sum_s 2^((L_s - M) log2 e),
//     O = sum_s 2^((L_s - M) log2 e) O_s / W,   LSE = M + ln W,
// the two-part combine of "FlashAttention 怎么做? online softmax 怎么更新?"
// (follow-up "多卡(ring attention)怎么合并两段结果?") taken over n parts, which
// is also the reduce step of FlashDecoding ("Flash Attention 全解析（上）",
// section 4.3): rescale every part by the global max, sum, normalise.
//
// The kernel is bound by HBM bandwidth (it reads n_parts (d + 1) fp32 values
// and writes d 16-bit values (bf16 or fp16, round to nearest even) plus one fp32
// per row), so it is laid out for
// coalescing, not for the matrix cores: d/4 consecutive threads own one row,
// each reading 16 contiguous bytes of every part and writing 8 bytes of O.
#include "fa2_internal.h"

namespace fa2 {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kMergeThreads = 256;
constexpr float kLog2e = 1.44269504088896340736f;

template <int D, typename E>
__global__ __launch_bounds__(kMergeThreads)
void fa2_merge_kernel(const float *__restrict__ o_parts, const float *__restrict__ lse_parts,
                      int n_parts, int64_t rows, uint16_t *__restrict__ o, float *__restrict__ lse)
{
    typedef E e4 __attribute__((ext_vector_type(4)));
    constexpr int kThreadsPerRow = D / 4;
    const int64_t g = (int64_t)blockIdx.x * kMergeThreads + threadIdx.x;
    const int64_t row = g / kThreadsPerRow;
    const int c = (int)(g % kThreadsPerRow);        // this thread's 4 columns: 4c .. 4c + 3
    if (row >= rows) return;

    // Unrolled so the loads of several parts are in flight together (the part
    // loops are latency-bound when rows are few and parts many, as in decoding).
    float mx = -INFINITY;
#pragma unroll 8
    for (int s = 0; s < n_parts; ++s)
        mx = fmaxf(mx, lse_parts[(size_t)s * rows + row]);

    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    float wsum = 0.f;
    if (mx != -INFINITY) {
#pragma unroll 4
        for (int s = 0; s < n_parts; ++s) {
            const float ls = lse_parts[(size_t)s * rows + row];
            if (ls == -INFINITY) continue;          // empty part: its O_s was never written
            // (ls - mx) is exactly 0 for the largest part, so its weight is exactly 1.
            const float w = __builtin_amdgcn_exp2f((ls - mx) * kLog2e);
            const f32x4 os = *reinterpret_cast<const f32x4 *>(o_parts + ((size_t)s * rows + row) * D + 4 * c);
            wsum += w;
            acc += w * os;
        }
    }
    const float inv = wsum > 0.f ? 1.0f / wsum : 0.f;
    *reinterpret_cast<e4 *>(o + row * D + 4 * c) = __builtin_convertvector(acc * inv, e4);
    if (c == 0)
        lse[row] = wsum > 0.f ? mx + __builtin_amdgcn_logf(wsum) * kLn2 : -INFINITY;
}

}  // namespace

hipError_t launch_merge(const float *o_parts, const float *lse_parts, int n_parts, int64_t rows,
                        int d, bool f16, void *o, float *lse, hipStream_t stream)
{
    const int64_t threads = rows * (d / 4);
    const dim3 grid((unsigned)((threads + kMergeThreads - 1) / kMergeThreads)), block(kMergeThreads);
    uint16_t *ob = static_cast<uint16_t *>(o);
    with_head_dim<true, true>(d, [&](auto dim) {
        constexpr int D = decltype(dim)::value;
        if (f16)
            hipLaunchKernelGGL((fa2_merge_kernel<D, _Float16>), grid, block, 0, stream, o_parts, lse_parts, n_parts,
                               rows, ob, lse);
        else
            hipLaunchKernelGGL((fa2_merge_kernel<D, __bf16>), grid, block, 0, stream, o_parts, lse_parts, n_parts,
                               rows, ob, lse);
    });
    return hipGetLastError();
}

}  // namespace fa2
