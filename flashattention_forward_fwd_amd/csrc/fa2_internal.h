// fa2_internal.h -- launch parameters and device helpers shared by the HIP kernels
// of libfa2.so.  Not part of the C ABI (that is include/fa2.h).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

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
    int n_wg;           // n_qtiles * B * H
};

constexpr int kWave = 64;          // CDNA wavefront width
constexpr int kWaves = 4;          // wavefronts per work-group
constexpr int kThreads = kWave * kWaves;
constexpr int kRowsPerWave = 32;   // query rows owned by one wavefront (one 32-wide MFMA tile)
constexpr int kBr = kWaves * kRowsPerWave;   // query rows per work-group
constexpr int kBc = 64;            // keys per K/V tile
constexpr int kXcds = 8;           // accelerator complex dies on MI355X
constexpr float kLn2 = 0.693147180559945309417f;

// Work-group id -> (batch*head, query tile).
//
// The dispatcher hands consecutive work-group ids to the XCDs in turn, and each
// XCD has its own L2.  Remapping so that the ids an XCD receives are consecutive
// in the logical order keeps the query tiles of one (batch, head) -- which read
// the same K and V -- on one XCD.  Within a (batch, head) the tiles run from the
// last to the first: under the causal mask the last query tile has the most key
// tiles, so the long work-groups start first and the short ones fill the tail.
__device__ __forceinline__ void map_workgroup(int w, int n_wg, int n_qtiles, int &bh, int &qt)
{
    const int xcd = w % kXcds;
    const int slot = w / kXcds;
    const int per = n_wg / kXcds;
    const int rem = n_wg % kXcds;
    const int logical = xcd * per + (xcd < rem ? xcd : rem) + slot;
    bh = logical / n_qtiles;
    qt = n_qtiles - 1 - (logical - bh * n_qtiles);
}

// Number of K/V tiles a query tile visits.  Causal: only tiles holding a key
// j <= the tile's last valid query row; tiles masked for every row are skipped.
__device__ __forceinline__ int kv_tiles_for(int qt, int Lq, int Lk, bool causal)
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

// Exchange with the lane 32 positions away (the other half of the wavefront).
__device__ __forceinline__ float swap_halves(float x)
{
    return __shfl_xor(x, 32, kWave);
}

}  // namespace fa2

// Host-side launchers (one per element type), defined next to their kernels.
namespace fa2 {
hipError_t launch_fwd_bf16(const FwdParams &p, int d, bool causal, hipStream_t stream);
hipError_t launch_fwd_f32(const FwdParams &p, int d, bool causal, hipStream_t stream);
}  // namespace fa2
