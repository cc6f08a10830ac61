// Stage 1 of condensate attention for decode-shaped problems on gfx950 (pages of "The
// Condensate Theorem", metaphor-xennon blog: section 2.1 Definition 1,
// C_i = {0} u {i-W+1..i} u Top-k_i; section 2.2.3, the top-k part ranks the positions
// R_i = {1..i-W} outside the anchor and the window).
//
// score_keys: one workgroup per (unit, block of 256 key rows), where a unit is (batch, KV head,
// query group) with up to G query vectors reading the same KV head. Each wavefront requests its
// 64 rows at once, then computes the fp32 scores of the G queries; the block's K rows are read
// once (the only large HBM traffic of the path). It writes one order-preserving 32-bit key per
// (row, query), the best key of every tile of rows, and the block's best key per query. Small workgroups in a one-shot grid let the
// hardware dispatcher balance the stream across the CUs; no LDS lists, no atomics.
//
// Key buffer: [units][G][rstride] words, query-major. Rows are grouped in tiles of 4*RPG rows
// (RPG = rows one wavefront load covers); after 4 loads a lane holds its query's keys of rows
// r, r+RPG, r+2RPG, r+3RPG and stores them as one 16-byte word, so position p of a tile holds
// row RPG*(p%4) + p/4 of the tile. Block b covers rows [256b, 256b+256); row 0 (the anchor) and
// rows that are no candidate of the query hold key 0.
//
// The finish kernel then takes, per query, the bound from the block maxima and reads only the
// tiles whose best key reaches it.
#include "ca_internal.h"
#include "score_core.h"

namespace ca {
namespace {

constexpr int kBlockRows = 256;   // rows per block of the bound (4 wavefronts of score_keys)
constexpr int kKeysBW = 2;        // blocks per score_keys workgroup
constexpr bool kKeysNT = true;    // non-temporal key-row loads

struct KeysArgs {
    int64_t n, nq;
    int Hq, Hkv, g, W;
    int64_t groups, units;
    int64_t rstride;  // key rows per unit in the key buffer
    int nblk;         // blocks per unit
    uint32_t nvec;    // query vectors per KV head (g * nq)
    int row_base;     // n - nq - W: the last candidate row of query vector idx is row_base + idx / g
    uint32_t *keys;   // [units][G][rstride], tiles as described above
    uint32_t *bmax;   // [units][nblk][G]
    uint32_t *tmax;   // [units][G][rstride / (4*RPG)]: best key of each tile
};

// 16-byte load of a key-row slice; NTL: non-temporal (streamed once, kept out of the caches so
// that the key buffer written meanwhile stays there).
template <bool NTL>
__device__ __forceinline__ uint4 load_row16(const uint4 *p) {
    if constexpr (NTL) return load_row16_nt(p);
    else return *p;
}

// BW blocks of 256 rows per workgroup (4 wavefronts each).
template <typename T, int D, int G, int BW, bool NTL>
__global__ __launch_bounds__(256 * BW) __attribute__((amdgpu_waves_per_eu(sizeof(T) == 2 ? 5 : 4))) void score_keys_kernel(
    const T *__restrict__ q, const T *__restrict__ k, KeysArgs a) {
    constexpr int EB = sizeof(T);
    constexpr int RB = D * EB;               // bytes per key row
    constexpr int LPR = RB >= 256 ? 16 : 8;  // lanes per row
    constexpr int RPG = 64 / LPR;            // rows per wavefront load
    constexpr int P = RB / (16 * LPR);       // 16-byte loads per lane per row
    constexpr int NG = 64 / RPG;             // row groups of a wavefront's 64 rows
    constexpr int U = 16 / P < NG ? 16 / P : NG;  // row groups per round (<= 16 loads per lane)
    static_assert(P >= 1 && NG % U == 0 && U % 4 == 0, "layout");
    __shared__ uint32_t red[4 * BW][G];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    // Workgroup (unit, BW blocks), units ordered (batch * Hkv + KV head, query group); 32-bit
    // math. Wavefronts 4b..4b+3 take block b of the workgroup.
    const uint32_t wpb = ((uint32_t)a.nblk + BW - 1) / BW;  // workgroups per unit
    const uint32_t wg = blockIdx.x, ng = (uint32_t)a.groups;
    const uint32_t uu32 = wg / wpb;
    const int bi = (int)(wg - uu32 * wpb) * BW + wave / 4;
    const uint32_t bk = uu32 / ng;
    const uint32_t grp = uu32 - bk * ng;
    const int64_t u = (int64_t)bk * a.groups + grp;
    const uint32_t g = (uint32_t)a.g;
    const int sl = lane % LPR;
    const bool writer = sl % (LPR / G) == 0;
    const int my_t = sl / (LPR / G);
    // Last candidate row of the unit: that of its last query vector (rows grow with idx).
    const uint32_t idx0 = grp * G;
    const uint32_t idx_last = (idx0 + G - 1 < a.nvec ? idx0 + G - 1 : a.nvec - 1);
    const int rl_max = a.row_base + (int)(idx_last / g);
    const int row0 = bi * kBlockRows;
    const bool live = bi < a.nblk && row0 <= rl_max;  // the block has candidate rows
    const int rows_end = (row0 + kBlockRows < rl_max + 1) ? row0 + kBlockRows : rl_max + 1;
    const int rlo = row0 > 1 ? row0 : 1;  // row 0 (the anchor) is no candidate

    const uint4 *kbase = reinterpret_cast<const uint4 *>(k + (int64_t)bk * a.n * D);
    uint32_t *kout = a.keys + ((size_t)u * G + my_t) * a.rstride;
    uint32_t *tout = a.tmax + ((size_t)u * G + my_t) * (a.rstride / (4 * RPG));
    const int wrow0 = row0 + (wave % 4) * 64;  // this wavefront's 64 rows
    uint32_t best = 0u;
    if (live && wrow0 < rows_end) {
        // The queries (vector idx of the KV head: head bk*g + idx % g, row idx / g) and the last
        // candidate row of this lane's query.
        uint4 qr[G][P];  // this lane's slices of the queries (zero past the last query vector)
        int my_rlast = 0;
#pragma unroll
        for (int t = 0; t < G; ++t) {
            const uint32_t idx = idx0 + t;
            if (idx < a.nvec) {
                const uint32_t qh = idx / g, hh = idx - qh * g;
                const uint4 *src = reinterpret_cast<const uint4 *>(q + (((int64_t)bk * g + hh) * a.nq + qh) * D);
#pragma unroll
                for (int p = 0; p < P; ++p) qr[t][p] = src[p * LPR + sl];
                if (my_t == t) my_rlast = a.row_base + (int)qh;
            } else {
#pragma unroll
                for (int p = 0; p < P; ++p) qr[t][p] = make_uint4(0, 0, 0, 0);
            }
        }
#pragma unroll
        for (int r = 0; r < NG / U; ++r) {
            // Row groups r*U .. r*U+U-1 of the wavefront's rows, RPG rows each, all in flight.
            uint4 kr[U][P];
#pragma unroll
            for (int uu = 0; uu < U; ++uu) {
                int row = wrow0 + (r * U + uu) * RPG + lane / LPR;
                row = row < rows_end ? row : rows_end - 1;
                const uint4 *src = kbase + (int64_t)row * (P * LPR);
#pragma unroll
                for (int p = 0; p < P; ++p) kr[uu][p] = load_row16<NTL>(src + p * LPR + sl);
            }
#pragma unroll
            for (int u4 = 0; u4 < U; u4 += 4) {
                uint32_t kv4[4];
#pragma unroll
                for (int gg = 0; gg < 4; ++gg) {
                    const int uu = u4 + gg;
                    float acc[G];
#pragma unroll
                    for (int t = 0; t < G; ++t) {
                        float x = 0.f;
#pragma unroll
                        for (int p = 0; p < P; ++p) x = dot16(kr[uu][p], qr[t][p], x, T());
                        acc[t] = x;
                    }
                    const uint32_t key = score_key(reduce_row<LPR, G>(acc, lane));
                    const int row = wrow0 + (r * U + uu) * RPG + lane / LPR;
                    kv4[gg] = (row >= rlo && row < rows_end && row <= my_rlast) ? key : 0u;
                    best = kv4[gg] > best ? kv4[gg] : best;
                }
                // Tile of 4*RPG rows starting at the first of these row groups, and its best key
                // (over the lanes of the query's rows: LPR apart).
                const int tile0 = wrow0 + (r * U + u4) * RPG;
                if (writer)
                    *reinterpret_cast<uint4 *>(kout + tile0 + 4 * (lane / LPR)) =
                        make_uint4(kv4[0], kv4[1], kv4[2], kv4[3]);
                uint32_t tm = kv4[0] > kv4[1] ? kv4[0] : kv4[1];
                tm = kv4[2] > tm ? kv4[2] : tm;
                tm = kv4[3] > tm ? kv4[3] : tm;
                tm = lane_max_stride<LPR>(tm);
                if (writer && lane < LPR) tout[tile0 / (4 * RPG)] = tm;
            }
        }
    }
    // Best key per query over each block: lanes of the same query are LPR apart, then the
    // block's 4 wavefronts (0 for a block without candidate rows).
    best = lane_max_stride<LPR>(best);
    if (lane < LPR && writer) red[wave][my_t] = best;
    __syncthreads();
    if (tid < BW * G) {
        const int b2 = tid / G, t = tid % G;
        const int bi2 = (int)(wg - uu32 * wpb) * BW + b2;
        if (bi2 < a.nblk) {
            uint32_t m = 0u;
#pragma unroll
            for (int w = 0; w < 4; ++w) m = red[4 * b2 + w][t] > m ? red[4 * b2 + w][t] : m;
            a.bmax[((size_t)u * a.nblk + bi2) * G + t] = m;
        }
    }
}

}  // namespace

size_t stream_keys_bytes(const Plan &pl) {
    return (size_t)pl.units * (size_t)pl.rstride * pl.G * sizeof(uint32_t);
}

hipError_t launch_score_keys(const Plan &pl, const void *q, const void *k, void *ws, hipStream_t s) {
    KeysArgs a;
    a.n = pl.n; a.nq = pl.nq; a.Hq = pl.Hq; a.Hkv = pl.Hkv; a.g = pl.g; a.W = pl.W;
    a.groups = pl.groups; a.units = pl.units; a.rstride = pl.rstride; a.nblk = pl.nblk;
    a.nvec = (uint32_t)(pl.g * pl.nq);
    a.row_base = (int)(pl.n - pl.nq - pl.W);
    a.keys = reinterpret_cast<uint32_t *>(static_cast<char *>(ws) + pl.keys_offset);
    a.bmax = reinterpret_cast<uint32_t *>(static_cast<char *>(ws) + pl.bmax_offset);
    a.tmax = reinterpret_cast<uint32_t *>(static_cast<char *>(ws) + pl.tmax_offset);
    dim3 grid((unsigned)(pl.units * ((pl.nblk + kKeysBW - 1) / kKeysBW))), block(256 * kKeysBW);
#define CA_LAUNCH_SK(T, D, G) \
    hipLaunchKernelGGL((score_keys_kernel<T, D, G, kKeysBW, kKeysNT>), grid, block, 0, s,       \
                       static_cast<const T *>(q), static_cast<const T *>(k), a)
#define CA_LAUNCH_SK_G(T, D)                          \
    do {                                              \
        if (pl.G == 4) CA_LAUNCH_SK(T, D, 4);         \
        else if (pl.G == 2) CA_LAUNCH_SK(T, D, 2);    \
        else CA_LAUNCH_SK(T, D, 1);                   \
    } while (0)
    if (pl.dtype == 1) {
        if (pl.d == 128) CA_LAUNCH_SK_G(__bf16, 128); else CA_LAUNCH_SK_G(__bf16, 64);
    } else {
        if (pl.d == 128) CA_LAUNCH_SK_G(float, 128); else CA_LAUNCH_SK_G(float, 64);
    }
#undef CA_LAUNCH_SK_G
#undef CA_LAUNCH_SK
    return hipGetLastError();
}

}  // namespace ca
