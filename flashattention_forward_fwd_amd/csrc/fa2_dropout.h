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
// the scalar unit.  Each product is one v_mad_u64_u32 (both halves at once), each
// three-way XOR one v_bitop3_b32 (truth table 0x96).
__device__ __forceinline__ u32x4_t philox4x32_10(uint32_t c0, uint32_t c1, uint32_t c2, uint32_t c3,
                                                 uint32_t k0, uint32_t k1)
{
#pragma unroll
    for (int r = 0; r < 10; ++r) {
        const uint64_t p0 = (uint64_t)0xD2511F53u * c0;
        const uint64_t p1 = (uint64_t)0xCD9E8D57u * c2;
        c0 = __builtin_amdgcn_bitop3_b32((uint32_t)(p1 >> 32), c1, k0, 0x96);
        c1 = (uint32_t)p1;
        c2 = __builtin_amdgcn_bitop3_b32((uint32_t)(p0 >> 32), c3, k1, 0x96);
        c3 = (uint32_t)p0;
        k0 += 0x9E3779B9u;
        k1 += 0xBB67AE85u;
    }
    return u32x4_t{c0, c1, c2, c3};
}

// x from lane (this lane XOR 1) / (this lane XOR 2) of the quad (DPP quad_perm
// [1,0,3,2] and [2,3,0,1]).
__device__ __forceinline__ uint32_t from_lane_xor1(uint32_t x)
{
    return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0xB1, 0xF, 0xF, false);
}
__device__ __forceinline__ uint32_t from_lane_xor2(uint32_t x)
{
    return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x4E, 0xF, 0xF, false);
}

// Transpose across each group of four consecutive lanes: lane s of the group
// holds x = X[s][0..3]; afterwards lane v holds y[u] = X[u][v].  Two butterfly
// stages: lanes s and s ^ 1 swap the words whose index differs from s in bit 0,
// then lanes s and s ^ 2 the words whose index differs from s in bit 1
// (afterwards word w of lane s holds X[s ^ e][w ^ e] with e = s ^ w, = X[w][s]).
__device__ __forceinline__ u32x4_t quad_transpose(u32x4_t x, int s)
{
    const bool b0 = s & 1, b1 = (s >> 1) & 1;
    {
        const uint32_t r01 = from_lane_xor1(b0 ? x[0] : x[1]);
        const uint32_t r23 = from_lane_xor1(b0 ? x[2] : x[3]);
        x[0] = b0 ? r01 : x[0];
        x[1] = b0 ? x[1] : r01;
        x[2] = b0 ? r23 : x[2];
        x[3] = b0 ? x[3] : r23;
    }
    {
        const uint32_t r02 = from_lane_xor2(b1 ? x[0] : x[2]);
        const uint32_t r13 = from_lane_xor2(b1 ? x[1] : x[3]);
        x[0] = b1 ? r02 : x[0];
        x[2] = b1 ? x[2] : r02;
        x[1] = b1 ? r13 : x[1];
        x[3] = b1 ? x[3] : r13;
    }
    return x;
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
__device__ __forceinline__ u32x4_t mask_query_lanes_one(const DropoutParams &dp, int k0, int t, int qrow, int lane,
                                                        int bh)
{
    const int s = lane & 3, hh = lane >> 5;
    const uint32_t kblock = (uint32_t)(k0 / 4 + 8 * t + 2 * s + hh);
    return quad_transpose(philox4x32_10(kblock, (uint32_t)qrow / 4u, (uint32_t)bh, dp.offset, dp.seed_lo, dp.seed_hi),
                          s);
}
__device__ __forceinline__ DropMask mask_query_lanes(const DropoutParams &dp, int k0, int qrow, int lane, int bh)
{
    DropMask mk;
#pragma unroll
    for (int t = 0; t < 2; ++t)
        mk.y[t] = mask_query_lanes_one(dp, k0, t, qrow, lane, bh);
    return mk;
}

// One key per lane (the dK/dV kernel): lane l holds key `key` (key % 4 == l % 4)
// and, in accumulator t, query rows r0 + 32t + 8(e/4) + 4(l/32) + e%4.  Each
// lane of a quad draws the block of one 4-row group; its bytes are transposed
// within the lane (word w byte b -> word b byte w: the 4 rows of key b) and then
// across the quad, so every lane gets the rows of its own key.
__device__ __forceinline__ u32x4_t mask_key_lanes_one(const DropoutParams &dp, int r0, int t, int key, int lane,
                                                      int bh)
{
    const int s = lane & 3, hh = lane >> 5;
    const uint32_t rblock = (uint32_t)(r0 / 4 + 8 * t + 2 * s + hh);
    return quad_transpose(byte_transpose(philox4x32_10((uint32_t)key / 4u, rblock, (uint32_t)bh, dp.offset,
                                                       dp.seed_lo, dp.seed_hi)), s);
}

}  // namespace fa2
