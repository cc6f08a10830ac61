// Key-row scoring shared by the score kernels on gfx950: each K row is read with 16-byte
// loads, LPR lanes per row (whole 128-byte lines per instruction), the lane's slices are dotted
// with the same slices of G query rows in fp32 (bf16 dot2 or fp32 FMA), and DPP exchanges sum
// the LPR partial products of a row (pages of "The Condensate Theorem", metaphor-xennon blog,
// section 2.1: the scores q_i . k_j of every causal key).
#pragma once

#include "device_utils.h"

namespace ca {

// Loads the K rows of one streaming round: row groups gi0 + 4*uu (RPG = 64/LPR rows each, LPR
// lanes per row) of the chunk [r0, rend). Rows past the chunk's end are clamped to its last row
// (loaded, never used), so every load is unconditional. Non-temporal loads.
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));

// 16-byte load of a key-row slice that is read once: non-temporal, so the stream does not
// evict what the kernels write meanwhile.
__device__ __forceinline__ uint4 load_row16_nt(const uint4 *p) {
    const u32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t *>(p));
    return make_uint4(v.x, v.y, v.z, v.w);
}

template <int LPR, int P, int U>
__device__ __forceinline__ void load_round(const uint4 *__restrict__ kbase, int r0, int rend, int gi0,
                                           int lane, uint4 (&dst)[U][P]) {
    constexpr int RQ = P * LPR;      // 16-byte words per row
    constexpr int RPG = 64 / LPR;    // rows per wavefront load
    const int sl = lane % LPR;
#pragma unroll
    for (int uu = 0; uu < U; ++uu) {
        int row = r0 + (gi0 + 4 * uu) * RPG + lane / LPR;
        row = row < rend ? row : rend - 1;
        const uint4 *src = kbase + (int64_t)row * RQ;
#pragma unroll
        for (int p = 0; p < P; ++p) dst[uu][p] = load_row16_nt(src + p * LPR + sl);
    }
}

// Sum of the G partial dot products over the LPR lanes of a row. Each exchange halves the
// queries a lane carries while it carries several, so the result has G lanes per row, one per
// query: query (lane % LPR) / (LPR / G) of the row.
template <int LPR, int G>
__device__ __forceinline__ float reduce_row(const float (&acc)[G], int lane) {
    if constexpr (LPR == 16) {
        const bool lo = (lane & 8) == 0;
        if constexpr (G == 4) {
            const float k0 = lo ? acc[0] : acc[2], s0 = lo ? acc[2] : acc[0];
            const float k1 = lo ? acc[1] : acc[3], s1 = lo ? acc[3] : acc[1];
            const float a0 = k0 + dpp_mirror16(s0);
            const float a1 = k1 + dpp_mirror16(s1);
            const bool b4 = (lane & 4) != 0;
            float x = (b4 ? a1 : a0) + dpp_half_mirror(b4 ? a0 : a1);
            x += dpp_xor2(x);
            return x + dpp_xor1(x);
        } else if constexpr (G == 2) {
            float x = (lo ? acc[0] : acc[1]) + dpp_mirror16(lo ? acc[1] : acc[0]);
            x += dpp_half_mirror(x);
            x += dpp_xor2(x);
            return x + dpp_xor1(x);
        } else {
            float x = acc[0] + dpp_mirror16(acc[0]);
            x += dpp_half_mirror(x);
            x += dpp_xor2(x);
            return x + dpp_xor1(x);
        }
    } else {
        const bool hi = (lane & 4) != 0;
        if constexpr (G == 4) {
            const float k0 = hi ? acc[2] : acc[0], s0 = hi ? acc[0] : acc[2];
            const float k1 = hi ? acc[3] : acc[1], s1 = hi ? acc[1] : acc[3];
            const float a0 = k0 + dpp_half_mirror(s0);
            const float a1 = k1 + dpp_half_mirror(s1);
            const bool hi1 = (lane & 2) != 0;
            const float b0 = (hi1 ? a1 : a0) + dpp_xor2(hi1 ? a0 : a1);
            return b0 + dpp_xor1(b0);
        } else if constexpr (G == 2) {
            float x = (hi ? acc[1] : acc[0]) + dpp_half_mirror(hi ? acc[0] : acc[1]);
            x += dpp_xor2(x);
            return x + dpp_xor1(x);
        } else {
            float x = acc[0] + dpp_half_mirror(acc[0]);
            x += dpp_xor2(x);
            return x + dpp_xor1(x);
        }
    }
}

// Order-preserving key of one K row for the G queries of a unit: the lane's P slices of the row
// dotted with the same slices of each query (fp32), summed over the row's LPR lanes, mapped by
// score_key. The lanes of query (lane % LPR) / (LPR / G) hold its key. Every kernel that scores
// rows uses this function, so a row's key has the same bits wherever it is computed.
template <typename T, int LPR, int P, int G>
__device__ __forceinline__ uint32_t row_key(const uint4 (&kr)[P], const uint4 (&qr)[G][P], int lane) {
    float acc[G];
#pragma unroll
    for (int t = 0; t < G; ++t) {
        float x = 0.f;
#pragma unroll
        for (int p = 0; p < P; ++p) x = dot16(kr[p], qr[t][p], x, T());
        acc[t] = x;
    }
    return score_key(reduce_row<LPR, G>(acc, lane));
}

}  // namespace ca
