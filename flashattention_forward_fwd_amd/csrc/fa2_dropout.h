// fa2_dropout.h -- the dropout keep mask on the device: Philox4x32-10 and the
// lane exchanges that hand every lane the bytes of its own (query, key) pairs.
// Part of libfa2.so's kernels; not part of the C ABI.
//
// Mask: byte (j mod 4) of word (i mod 4) of Philox4x32-10 (Salmon, Moraes, Dror,
// Shaw, "Parallel random numbers: as easy as 1, 2, 3", SC'11) at counter
// (j / 4, i / 4, b*H + h, offset) and key (seed low, seed high) is compared with
// the threshold t: the pair (query i, key j) keeps its probability iff byte < t.
// One generator call covers a block of 4 queries x 4 keys.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fa2 {

typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

// Dropout settings of one call.
struct DropoutParams {
    uint32_t seed_lo, seed_hi;   // Philox key
    uint32_t offset;             // fourth counter word
    uint32_t threshold;          // keep iff byte < threshold, 1..256
    float keep_scale;            // 256 / threshold
};

// Philox4x32-10: ten rounds of two 32x32->64-bit products (multipliers
// 0xD2511F53 and 0xCD9E8D57), the key bumped by the Weyl constants 0x9E3779B9 and
// 0xBB67AE85 between rounds.  The key is wave-uniform, so its schedule runs on
// the scalar unit.
__device__ __forceinline__ u32x4_t philox4x32_10(uint32_t c0, uint32_t c1, uint32_t c2, uint32_t c3,
                                                 uint32_t k0, uint32_t k1)
{
#pragma unroll
    for (int r = 0; r < 10; ++r) {
        const uint32_t hi0 = __umulhi(0xD2511F53u, c0), lo0 = 0xD2511F53u * c0;
        const uint32_t hi1 = __umulhi(0xCD9E8D57u, c2), lo1 = 0xCD9E8D57u * c2;
        c0 = hi1 ^ c1 ^ k0;
        c1 = lo1;
        c2 = hi0 ^ c3 ^ k1;
        c3 = lo0;
        k0 += 0x9E3779B9u;
        k1 += 0xBB67AE85u;
    }
    return u32x4_t{c0, c1, c2, c3};
}

// x[s] from a 4-element vector with a lane-dependent index s.
__device__ __forceinline__ uint32_t pick4(u32x4_t x, int s)
{
    const uint32_t a = (s & 1) ? x[1] : x[0];
    const uint32_t b = (s & 1) ? x[3] : x[2];
    return (s & 2) ? b : a;
}

// Transpose across each group of four consecutive lanes: lane s of the group
// holds x = X[s][0..3]; afterwards lane v holds y[u] = X[u][v].  Lane s offers
// X[s][s ^ k] to the lane s ^ k (DPP quad permutation "xor k").
__device__ __forceinline__ u32x4_t quad_transpose(u32x4_t x, int s)
{
    const uint32_t e0 = pick4(x, s);
    const uint32_t e1 = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)pick4(x, s ^ 1), 0xB1, 0xF, 0xF, false);
    const uint32_t e2 = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)pick4(x, s ^ 2), 0x4E, 0xF, 0xF, false);
    const uint32_t e3 = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)pick4(x, s ^ 3), 0x1B, 0xF, 0xF, false);
    // now e_k = X[s ^ k][s]; y[u] = e_{u ^ s}
    const u32x4_t e = {e0, e1, e2, e3};
    return u32x4_t{pick4(e, s), pick4(e, 1 ^ s), pick4(e, 2 ^ s), pick4(e, 3 ^ s)};
}

// Byte transpose within a lane: c[b] byte w = w_in[w] byte b.
__device__ __forceinline__ u32x4_t byte_transpose(u32x4_t w)
{
    u32x4_t c;
#pragma unroll
    for (int b = 0; b < 4; ++b)
        c[b] = ((w[0] >> (8 * b)) & 0xFFu) | (((w[1] >> (8 * b)) & 0xFFu) << 8) |
               (((w[2] >> (8 * b)) & 0xFFu) << 16) | (((w[3] >> (8 * b)) & 0xFFu) << 24);
    return c;
}

// Keep bytes of one 64 x 32 score block held as two 32x32 accumulators, for
// one lane.  Word g of y[t] covers entries 4g .. 4g + 3 of accumulator t (the
// four consecutive indices of the lane's column), one byte each, least
// significant first.
struct DropMask {
    u32x4_t y[2];
};

// Entry e (0..15) of accumulator t is kept iff its byte is below the threshold.
__device__ __forceinline__ bool keep(const DropMask &mk, int t, int e, uint32_t threshold)
{
    return ((mk.y[t][e / 4] >> (8 * (e % 4))) & 0xFFu) < threshold;
}

// One query per lane (the forward and dQ kernels): lane l holds query `qrow`
// (qrow % 4 == l % 4) and, in accumulator t, keys k0 + 32t + 8(e/4) + 4(l/32)
// + e%4.  The four keys of one row of four entries form one 4-key block, and the
// four lanes of a quad hold the four queries of one 4-query block, so each lane
// of the quad draws one block per accumulator (its own index s as the 4-key
// group) and the transpose hands every lane the word of its own query.
__device__ __forceinline__ DropMask mask_query_lanes(const DropoutParams &dp, int k0, int qrow, int lane, int bh)
{
    DropMask mk;
    const int s = lane & 3, hh = lane >> 5;
#pragma unroll
    for (int t = 0; t < 2; ++t) {
        const uint32_t kblock = (uint32_t)(k0 / 4 + 8 * t + 2 * s + hh);
        mk.y[t] = quad_transpose(philox4x32_10(kblock, (uint32_t)qrow / 4u, (uint32_t)bh, dp.offset,
                                               dp.seed_lo, dp.seed_hi), s);
    }
    return mk;
}

// One key per lane (the dK/dV kernel): lane l holds key `key` (key % 4 == l % 4)
// and, in accumulator t, query rows r0 + 32t + 8(e/4) + 4(l/32) + e%4.  Each
// lane of a quad draws the block of one 4-row group; its bytes are transposed
// within the lane (word w byte b -> word b byte w: the 4 rows of key b) and then
// across the quad, so every lane gets the rows of its own key.
__device__ __forceinline__ DropMask mask_key_lanes(const DropoutParams &dp, int r0, int key, int lane, int bh)
{
    DropMask mk;
    const int s = lane & 3, hh = lane >> 5;
#pragma unroll
    for (int t = 0; t < 2; ++t) {
        const uint32_t rblock = (uint32_t)(r0 / 4 + 8 * t + 2 * s + hh);
        mk.y[t] = quad_transpose(byte_transpose(philox4x32_10((uint32_t)key / 4u, rblock, (uint32_t)bh, dp.offset,
                                                              dp.seed_lo, dp.seed_hi)), s);
    }
    return mk;
}

}  // namespace fa2
