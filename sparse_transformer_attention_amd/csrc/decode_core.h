// Shared pieces of the two decode kernels on gfx950 (pages of "The Condensate Theorem",
// metaphor-xennon blog: section 2.1 Definition 1, C_i = {0} u {i-W+1..i} u Top-k_i; section
// 2.2.3, the top-k part over R_i = {1..i-W}; section 2.3, the softmax restricted to C_i times V).
//
// Work unit: (batch, KV head, query group) with up to G query vectors reading one KV head.
//   decode_stream   per unit, wpb workgroups of two blocks of 256 key rows each (interleaved over
//                   the units: workgroup s serves unit s % units). Every K row is read once
//                   (16-byte non-temporal loads, LPR lanes per row) and dotted with the unit's G
//                   queries in fp32 (row_key); per block and query a 32-byte record: four of its
//                   rows (key, offset) and a key X that every other row of the block stays at or
//                   below (with the mass diagnostic also the block's largest score and its sum of
//                   exp2((s - m_b) * scale)). Its last workgroups make the softmax partials of the
//                   anchor and window rows, in chunks of kWinChunkRows per query vector.
//   decode_finish   one workgroup per query vector: the exact top-k' from the records, C_i to
//                   out_idx, and the restricted softmax times V.
#pragma once

#include "ca_internal.h"
#include "device_utils.h"
#include "score_core.h"

namespace ca {
namespace dec {

constexpr int kRows = 256;         // key rows per block
constexpr int kBW = 2;             // blocks per stream workgroup
constexpr int kNT = kBW * 256;     // threads per workgroup (both kernels)
constexpr int kWaves = kNT / 64;

struct DecodeArgs {
    int64_t n, nq;
    int Hq, Hkv, g, W, topk, cap;
    int64_t groups;     // units per (batch, KV head)
    int nblk;           // blocks of 256 rows per unit (rows 0 .. 256 nblk - 1)
    uint32_t nvec;      // query vectors per KV head (g * nq)
    int row_base;       // n - nq - W: last candidate row of vector idx is row_base + idx / g
    uint32_t units;     // work units
    float scale_log2e;
    int64_t rstride;    // scratch keys per query (256 nblk)
    uint4 *rec;         // [units][G][nblk][2] records: {k1, k2, k3, k4}, {offsets o1..o4 (8 bits
                        // each), X, m_b, l_b (float bits; mass diagnostic only)}
    uint32_t *scratch;  // [units][G][rstride] fallback keys
    int32_t *out_idx;   // [nqv][cap]
    float *out;         // [nqv][D] (null: select only)
    float *mass;        // [nqv][4] (null: no diagnostic)
    float *win;         // [nqv][nch][D + 2] anchor-and-window partials (decode_stream's last
                        // workgroups), or null (no output)
    int nch;            // chunks of kWinChunkRows rows per query vector (win only)
};

template <int N>
__device__ __forceinline__ uint32_t ror_u32(uint32_t x) { return dpp_u32<0x120 + N>(x, x); }

// ---- reductions over the 16 lanes of a DPP row (every lane gets the result) ----

__device__ __forceinline__ uint64_t row16_max_u64(uint64_t v) {
#define CA_ROW_MAX_STEP(N)                                                            \
    {                                                                                 \
        const uint32_t hi = ror_u32<N>((uint32_t)(v >> 32)), lo = ror_u32<N>((uint32_t)v); \
        const uint64_t o = ((uint64_t)hi << 32) | lo;                                 \
        v = o > v ? o : v;                                                            \
    }
    CA_ROW_MAX_STEP(8) CA_ROW_MAX_STEP(4) CA_ROW_MAX_STEP(2) CA_ROW_MAX_STEP(1)
#undef CA_ROW_MAX_STEP
    return v;
}
__device__ __forceinline__ uint32_t row16_max_u32(uint32_t v) {
    uint32_t o;
    o = ror_u32<8>(v); v = o > v ? o : v;
    o = ror_u32<4>(v); v = o > v ? o : v;
    o = ror_u32<2>(v); v = o > v ? o : v;
    o = ror_u32<1>(v); v = o > v ? o : v;
    return v;
}
__device__ __forceinline__ float row16_sum_f32(float x) {
    x += __uint_as_float(ror_u32<8>(__float_as_uint(x)));
    x += __uint_as_float(ror_u32<4>(__float_as_uint(x)));
    x += __uint_as_float(ror_u32<2>(__float_as_uint(x)));
    x += __uint_as_float(ror_u32<1>(__float_as_uint(x)));
    return x;
}

// Streaming layout of a key row (as in every score kernel: row_key gives the same bits).
template <typename T, int D>
struct StreamShape {
    static constexpr int EB = sizeof(T);
    static constexpr int RB = D * EB;                // bytes per key row
    static constexpr int LPR = RB >= 256 ? 16 : 8;   // lanes per row
    static constexpr int RPG = 64 / LPR;             // rows per wavefront load
    static constexpr int P = RB / (16 * LPR);        // 16-byte loads per lane per row
    static constexpr int NG = 64 / RPG;              // row groups of a wavefront's 64 rows
    static constexpr int U = 16 / P < NG ? 16 / P : NG;  // row groups per round
    static constexpr int TR = 4 * RPG;               // rows per staged tile
    static_assert(P >= 1 && NG % U == 0 && U % 4 == 0, "layout");
};

// Row offset (within its block) of staged position p of a block: a staged tile of TR rows holds
// row RPG * (p % 4) + p / 4 of the tile at position p.
template <int TR, int RPG>
__device__ __forceinline__ int staged_row(int p) {
    return TR * (p / TR) + RPG * (p % 4) + (p % TR) / 4;
}

// One query vector of a unit: where it sits and what its set looks like.
struct QInfo {
    bool valid;
    uint32_t qv;              // flat query vector (b*Hq + h)*nq + r
    int i, rl, kp, wlo, base, wcount, nbq;
};

template <int G>
__device__ __forceinline__ QInfo query_info(const DecodeArgs &a, uint32_t bk, uint32_t grp, int t) {
    QInfo qi;
    const uint32_t g = (uint32_t)a.g;
    const uint32_t b = bk / (uint32_t)a.Hkv, kvh = bk - b * (uint32_t)a.Hkv;
    const uint32_t idx = grp * G + (uint32_t)t;
    qi.valid = idx < a.nvec;
    const uint32_t idc = qi.valid ? idx : a.nvec - 1;
    const uint32_t qh = idc / g, hh = idc - qh * g;
    qi.qv = (b * (uint32_t)a.Hq + kvh * g + hh) * (uint32_t)a.nq + qh;
    qi.i = (int)(a.n - a.nq) + (int)qh;
    qi.rl = qi.i - a.W;
    const int n_r = qi.rl >= 1 ? qi.rl : 0;
    qi.kp = a.topk < n_r ? a.topk : n_r;
    qi.wlo = qi.i - a.W + 1 > 0 ? qi.i - a.W + 1 : 0;
    qi.base = qi.wlo > 0 ? 1 : 0;
    qi.wcount = qi.i - qi.wlo + 1;
    qi.nbq = qi.rl >= 1 ? (qi.rl >> 8) + 1 : 0;
    return qi;
}

// The unit's G query slices of this lane (zero past the last query vector), stream layout.
template <typename T, int D, int G>
__device__ __forceinline__ void load_query_slices(const T *__restrict__ q, const DecodeArgs &a, uint32_t bk,
                                                  uint32_t grp, int lane, uint4 (&qr)[G][StreamShape<T, D>::P]) {
    using S = StreamShape<T, D>;
    const uint32_t g = (uint32_t)a.g;
    const int sl = lane % S::LPR;
#pragma unroll
    for (int t = 0; t < G; ++t) {
        const uint32_t idx = grp * G + t;
        if (idx < a.nvec) {
            const uint32_t qh = idx / g, hh = idx - qh * g;
            const uint4 *src = reinterpret_cast<const uint4 *>(q + (((int64_t)bk * g + hh) * a.nq + qh) * D);
#pragma unroll
            for (int p = 0; p < S::P; ++p) qr[t][p] = src[p * S::LPR + sl];
        } else {
#pragma unroll
            for (int p = 0; p < S::P; ++p) qr[t][p] = make_uint4(0, 0, 0, 0);
        }
    }
}


inline DecodeArgs decode_args(const Plan &pl, void *ws, int32_t *out_idx, float *out, float *mass) {
    DecodeArgs a;
    a.n = pl.n; a.nq = pl.nq; a.Hq = pl.Hq; a.Hkv = pl.Hkv; a.g = pl.g; a.W = pl.W;
    a.topk = pl.topk; a.cap = pl.cap; a.groups = pl.groups; a.nblk = pl.nblk;
    a.nvec = (uint32_t)(pl.g * pl.nq);
    a.row_base = (int)(pl.n - pl.nq - pl.W);
    a.units = (uint32_t)pl.units;
    a.scale_log2e = (float)(1.4426950408889634 / __builtin_sqrt((double)pl.d));
    a.rstride = pl.rstride;
    char *w = static_cast<char *>(ws);
    a.rec = reinterpret_cast<uint4 *>(w + pl.summ_offset);
    a.scratch = reinterpret_cast<uint32_t *>(w + pl.scratch_offset);
    a.out_idx = out_idx;
    a.out = out;
    a.mass = mass;
    a.nch = pl.win_chunks;
    a.win = pl.win_chunks > 0 ? reinterpret_cast<float *>(w + pl.win_offset) : nullptr;
    return a;
}


}  // namespace dec
}  // namespace ca
