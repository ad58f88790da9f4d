// fa2_internal.h -- launch parameters and device helpers shared by the HIP kernels
// of libfa2.so.  Not part of the C ABI (that is include/fa2.h).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "fa2_dropout.h"

namespace fa2 {

// Everything a forward kernel needs; passed by value as the kernel argument.
struct FwdParams {
    const void *q;
    const void *k;
    const void *v;
    void *o;
    float *lse;
    int B, H, Lq, Lk;
    float scale_log2;   // scale * log2(e): scores are handled in base 2 on the device
    int n_qtiles;       // ceil(Lq / rows per work-group)
    int n_splits;       // K/V ranges per query tile (1: plain forward)
    int n_wg;           // n_qtiles * B * H * n_splits
    int wl, wr;         // window kernels: key j visible to query i iff
                        // (wl < 0 or j >= i - wl) and (wr < 0 or j <= i + wr)
    DropoutParams drop; // dropout kernels: keep mask and scale
};

// Everything a backward kernel needs (q, k, v, dout bf16 inputs; dq, dk, dv bf16
// outputs; lse2 = lse * log2(e) and delta = rowsum(dO * O), fp32 per query row).
struct BwdParams {
    const void *q;
    const void *k;
    const void *v;
    const void *dout;
    void *dq;
    void *dk;
    void *dv;
    const float *lse2;
    const float *delta;
    int B, H, Lq, Lk;
    float scale;        // softmax scale; dQ and dK are multiplied by it
    float scale_log2;   // scale * log2(e)
    int n_blocks;       // per head: key blocks (dK/dV kernel) or query tiles (dQ kernel)
    int n_wg;           // n_blocks * B * H
    int wl, wr;         // key j visible to query i iff (wl < 0 or j >= i - wl) and
                        // (wr < 0 or j <= i + wr); causal is (-1, 0), full (-1, -1)
    DropoutParams drop; // dropout kernels: keep mask and scale
};

constexpr int kWave = 64;          // CDNA wavefront width
constexpr int kWaves = 4;          // wavefronts per work-group
constexpr int kThreads = kWave * kWaves;
constexpr int kRowsPerWave = 32;   // query rows owned by one wavefront (one 32-wide MFMA tile)
constexpr int kBr = kWaves * kRowsPerWave;   // query rows per work-group
constexpr int kBc = 64;            // keys per K/V tile
constexpr float kLn2 = 0.693147180559945309417f;

// Work-group id -> (batch*head, query tile).
//
// Query tiles run from the last to the first across all heads (heads are the
// fast index): under the causal mask the last query tile has the most key
// tiles, so the long work-groups start first and the short ones fill the tail
// (longest-processing-time-first).  The dispatcher hands consecutive
// work-group ids to the eight XCDs in turn, so with this order each XCD serves
// a fixed subset of heads, and its resident work-groups walk the K/V tiles of
// those heads at about the same pace.
__device__ __forceinline__ void map_workgroup(int w, int n_wg, int n_qtiles, int &bh, int &qt)
{
    const int n_bh = n_wg / n_qtiles;
    qt = n_qtiles - 1 - w / n_bh;
    bh = w % n_bh;
}

// Number of K/V tiles a query tile visits.  Causal: only tiles holding a key
// j <= the tile's last valid query row; tiles masked for every row are skipped.
__host__ __device__ __forceinline__ int kv_tiles_for(int qt, int Lq, int Lk, bool causal)
{
    int n = (Lk + kBc - 1) / kBc;
    if (causal) {
        int qlast = qt * kBr + kBr - 1;
        if (qlast > Lq - 1) qlast = Lq - 1;
        const int nc = qlast / kBc + 1;
        if (nc < n) n = nc;
    }
    return n;
}

// The two values of a lane pair (l, l + 32), one per wavefront half.  One
// v_permlane32_swap (a VALU op on gfx950) swaps the upper half of its first
// operand with the lower half of its second; given x twice, every lane ends up
// with {own x, partner's x} in some order.
struct HalfPair {
    float a, b;
};
__device__ __forceinline__ HalfPair half_pair(float x)
{
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return {__uint_as_float(r[0]), __uint_as_float(r[1])};
}
// max / sum of x over the lane pair (l, l + 32); the same value on both lanes.
__device__ __forceinline__ float halves_max(float x)
{
    const HalfPair p = half_pair(x);
    return fmaxf(p.a, p.b);
}
__device__ __forceinline__ float halves_sum(float x)
{
    const HalfPair p = half_pair(x);
    return p.a + p.b;
}

}  // namespace fa2

// Host-side launchers, defined next to their kernels.
namespace fa2 {
// Calls f(std::integral_constant<int, D>{}) for the head dimension d: 32, 64,
// 128, 96 where WITH_96 (the 16-bit forward and backward kernels and the
// merge) and 256 where WITH_256 (the 16-bit forward kernels and the merge); the
// entry points reject every other value before a launch.
template <bool WITH_96 = false, bool WITH_256 = false, typename F>
inline void with_head_dim(int d, F f)
{
    if (d == 32) f(std::integral_constant<int, 32>{});
    else if (d == 64) f(std::integral_constant<int, 64>{});
    else if (WITH_96 && d == 96) f(std::integral_constant<int, WITH_96 ? 96 : 128>{});
    else if (WITH_256 && d == 256) f(std::integral_constant<int, WITH_256 ? 256 : 128>{});
    else f(std::integral_constant<int, 128>{});
}
// The 16-bit forward kernels, bf16 or (f16) fp16 elements.  kSplit writes the
// split-KV partials (p.o, p.lse: the fp32 partial arrays indexed by (split,
// b*h, row)); kWindow takes its keys from p.wl, p.wr (causal unused); kDropout
// applies p.drop.
enum class FwdVariant { kPlain, kSplit, kWindow, kDropout };
hipError_t launch_fwd16(const FwdParams &p, int d, bool causal, bool f16, FwdVariant v, hipStream_t stream);
hipError_t launch_fwd_f32(const FwdParams &p, int d, bool causal, hipStream_t stream);
// Backward: D and lse2 into p.delta / p.lse2 from o and lse, then dK/dV, then dQ,
// for the keys p.wl / p.wr leave visible; dropout: the keep mask of p.drop.
hipError_t launch_bwd16(const BwdParams &p, int d, bool f16, bool dropout, const void *o, const float *lse,
                        hipStream_t stream);
// Merge of split partials into o (bf16, or fp16 where f16) and lse.
hipError_t launch_merge(const float *o_parts, const float *lse_parts, int n_parts, int64_t rows,
                        int d, bool f16, void *o, float *lse, hipStream_t stream);
// Split-KV partials for Lq <= kDecodeMaxRows, same outputs as the kSplit
// forward; p.n_wg = B * H * p.n_splits.
constexpr int kDecodeMaxRows = 4;
hipError_t launch_decode(const FwdParams &p, int d, bool f16, hipStream_t stream);
}  // namespace fa2
