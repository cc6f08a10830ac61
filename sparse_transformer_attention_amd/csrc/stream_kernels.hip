// Stage 1 of condensate attention for decode-shaped problems on gfx950 (pages of "The
// Condensate Theorem", metaphor-xennon blog: section 2.1 Definition 1,
// C_i = {0} u {i-W+1..i} u Top-k_i; section 2.2.3, the top-k part ranks the positions
// R_i = {1..i-W} outside the anchor and the window).
//
// score_keys: one workgroup per (unit, BW blocks of 256 key rows), where a unit is (batch, KV
// head, query group) with up to G query vectors reading the same KV head. Each wavefront
// requests its 64 rows at once, then computes the fp32 scores of the G queries (row_key); the
// K rows are read once (the only large HBM traffic of the path). The order-preserving 32-bit
// keys (0 for rows that are no candidate of the query: the anchor, the window, past the query)
// are staged in LDS; the workgroup's epilogue then writes, per tile of TR = 4*RPG rows (RPG =
// rows one wavefront load covers) and query, only a summary: the two best keys with their row
// offsets in the tile (ties: the smaller offset first) and the upper half of the third best key;
// and per block and query the block's best key. Writing every key (16 MiB at 131K) cost the
// stream more than its share of bandwidth; the summaries are ~1/5 of that. Small workgroups in a one-shot grid let the
// hardware dispatcher balance the stream across the CUs.
//
// The finish kernel takes, per query, a bound from the block maxima; a tile gives each of its two
// best rows whose key reaches it as candidates, and a tile whose third key may reach it as well
// is scored again there (row_key, the same bits).
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
    int64_t rstride;  // rows per unit covered by the summaries (nblk * 256)
    int nblk;         // blocks per unit
    uint32_t nvec;    // query vectors per KV head (g * nq)
    int row_base;     // n - nq - W: the last candidate row of query vector idx is row_base + idx / g
    uint32_t *best1;  // [units][G][rstride / TR]: best key of each tile
    uint2 *rest;      // [units][G][rstride / TR]: second key; offsets of the best (bits 0-7) and
                      // the second (bits 8-15), upper 16 bits of the third key (bits 16-31)
    uint32_t *bmax;   // [units][nblk][G]
    // Mass diagnostic (null: off): per block and query the largest candidate score m and
    // sum of exp2((s - m) * scale_log2e) over the block's candidate rows, [units][nblk][G][2].
    float2 *zsum;
    float scale_log2e;
};

// 16-byte load of a key-row slice; NTL: non-temporal (streamed once, kept out of the caches).
template <bool NTL>
__device__ __forceinline__ uint4 load_row16(const uint4 *p) {
    if constexpr (NTL) return load_row16_nt(p);
    else return *p;
}

// BW blocks of 256 rows per workgroup (4 wavefronts each).
template <typename T, int D, int G, int BW, bool NTL, bool MASS>
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
    constexpr int TR = 4 * RPG;               // rows per tile
    constexpr int WROWS = BW * kBlockRows;    // rows per workgroup
    __shared__ uint32_t red[4 * BW][G];
    __shared__ uint32_t kst[G][WROWS];        // keys of the workgroup's rows, per query

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    // Workgroup (unit, BW blocks), units ordered (batch * Hkv + KV head, query group); 32-bit
    // math. Wavefronts 4b..4b+3 take block b of the workgroup.
    const uint32_t wpb = ((uint32_t)a.nblk + BW - 1) / BW;  // workgroups per unit
    const uint32_t wg = blockIdx.x, ng = (uint32_t)a.groups;
    const uint32_t uu32 = wg / wpb;
    const int wg_row0 = (int)(wg - uu32 * wpb) * WROWS;
    const int bi = wg_row0 / kBlockRows + wave / 4;
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
                    const uint32_t key = row_key<T, LPR, P, G>(kr[uu], qr, lane);
                    const int row = wrow0 + (r * U + uu) * RPG + lane / LPR;
                    kv4[gg] = (row >= rlo && row < rows_end && row <= my_rlast) ? key : 0u;
                    best = kv4[gg] > best ? kv4[gg] : best;
                }
                // Keys of rows tile0 + RPG*gg + lane/LPR, staged as one 16-byte word: position p
                // of a staged tile holds row RPG*(p%4) + p/4 of the tile.
                const int tile0 = wrow0 + (r * U + u4) * RPG;
                if (writer)
                    *reinterpret_cast<uint4 *>(&kst[my_t][tile0 - wg_row0 + 4 * (lane / LPR)]) =
                        make_uint4(kv4[0], kv4[1], kv4[2], kv4[3]);
            }
        }
    } else {
        // Rows without candidates: key 0.
        for (int i = lane; i < G * 16; i += 64)
            *reinterpret_cast<uint4 *>(&kst[i / 16][wrow0 - wg_row0 + 4 * (i % 16)]) = make_uint4(0, 0, 0, 0);
    }
    // Best key per query over each block: lanes of the same query are LPR apart, then the
    // block's 4 wavefronts (0 for a block without candidate rows).
    best = lane_max_stride<LPR>(best);
    if (lane < LPR && writer) red[wave][my_t] = best;
    __syncthreads();
    const int nbw = (int)(a.nblk - wg_row0 / kBlockRows) < BW ? a.nblk - wg_row0 / kBlockRows : BW;
    if (tid < BW * G) {
        const int b2 = tid / G, t = tid % G;
        if (b2 < nbw) {
            uint32_t m = 0u;
#pragma unroll
            for (int w = 0; w < 4; ++w) m = red[4 * b2 + w][t] > m ? red[4 * b2 + w][t] : m;
            a.bmax[((size_t)u * a.nblk + wg_row0 / kBlockRows + b2) * G + t] = m;
        }
    }
    // Tile summaries, one thread per (query, tile) of the workgroup's blocks: the two best
    // (key, offset) in the ranking order (larger key, then smaller offset) and the third key.
    // With the mass diagnostic also the tile's sum of exp2((s - m) * scale) relative to its
    // block's best score m.
    const int nt = nbw * kBlockRows / TR;
    __shared__ float tsum[MASS ? G : 1][MASS ? BW * kBlockRows / TR : 1];
    constexpr bool mass = MASS;
    for (int x = tid; x < G * nt; x += 256 * BW) {
        const int t = x / nt, j = x - t * nt;
        float mb = 0.f, zs = 0.f;
        if constexpr (mass) {
            const int b2 = j * TR / kBlockRows;
            uint32_t mk = 0u;
#pragma unroll
            for (int w = 0; w < 4; ++w) mk = red[4 * b2 + w][t] > mk ? red[4 * b2 + w][t] : mk;
            mb = mk ? key_score(mk) : 0.f;
        }
        uint32_t k1 = 0u, o1 = 0u, k2 = 0u, o2 = 0u, k3 = 0u;
#pragma unroll
        for (int w4 = 0; w4 < TR / 4; ++w4) {
            const uint4 v = *reinterpret_cast<const uint4 *>(&kst[t][j * TR + 4 * w4]);
            const uint32_t kv[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
            for (int c = 0; c < 4; ++c) {  // staged position 4*w4 + c holds row offset RPG*c + w4
                const uint32_t key = kv[c], off = (uint32_t)(RPG * c + w4);
                if constexpr (mass) {
                    if (key) zs += exp2f((key_score(key) - mb) * a.scale_log2e);
                }
                const bool b1 = key > k1 || (key == k1 && off < o1);
                const bool b2 = key > k2 || (key == k2 && off < o2);
                k3 = b2 ? k2 : (key > k3 ? key : k3);
                k2 = b1 ? k1 : (b2 ? key : k2);
                o2 = b1 ? o1 : (b2 ? off : o2);
                k1 = b1 ? key : k1;
                o1 = b1 ? off : o1;
            }
        }
        const size_t o = ((size_t)u * G + t) * (size_t)(a.rstride / TR) + wg_row0 / TR + j;
        a.best1[o] = k1;
        a.rest[o] = make_uint2(k2, o1 | (o2 << 8) | (k3 & 0xFFFF0000u));
        if constexpr (mass) tsum[t][j] = zs;
    }
    if constexpr (mass) {
        // Per block and query: its tiles' sums in tile order.
        __syncthreads();
        constexpr int TPB = kBlockRows / TR;  // tiles per block
        if (tid < BW * G) {
            const int b2 = tid / G, t = tid % G;
            if (b2 < nbw) {
                uint32_t mk = 0u;
#pragma unroll
                for (int w = 0; w < 4; ++w) mk = red[4 * b2 + w][t] > mk ? red[4 * b2 + w][t] : mk;
                float l = 0.f;
#pragma unroll
                for (int jj = 0; jj < TPB; ++jj) l += tsum[t][b2 * TPB + jj];
                a.zsum[((size_t)u * a.nblk + wg_row0 / kBlockRows + b2) * G + t] =
                    make_float2(mk ? key_score(mk) : -INFINITY, mk ? l : 0.f);
            }
        }
    }
}

}  // namespace

hipError_t launch_score_keys(const Plan &pl, const void *q, const void *k, void *ws, hipStream_t s,
                             bool mass) {
    KeysArgs a;
    a.n = pl.n; a.nq = pl.nq; a.Hq = pl.Hq; a.Hkv = pl.Hkv; a.g = pl.g; a.W = pl.W;
    a.groups = pl.groups; a.units = pl.units; a.rstride = pl.rstride; a.nblk = pl.nblk;
    a.nvec = (uint32_t)(pl.g * pl.nq);
    a.row_base = (int)(pl.n - pl.nq - pl.W);
    char *w = static_cast<char *>(ws);
    a.best1 = reinterpret_cast<uint32_t *>(w + pl.best1_offset);
    a.rest = reinterpret_cast<uint2 *>(w + pl.rest_offset);
    a.bmax = reinterpret_cast<uint32_t *>(w + pl.bmax_offset);
    a.zsum = mass ? reinterpret_cast<float2 *>(w + pl.zsum_offset) : nullptr;
    a.scale_log2e = (float)(1.4426950408889634 / __builtin_sqrt((double)pl.d));
    dim3 grid((unsigned)(pl.units * ((pl.nblk + kKeysBW - 1) / kKeysBW))), block(256 * kKeysBW);
#define CA_LAUNCH_SK(T, D, G)                                                                      \
    do {                                                                                           \
        if (mass)                                                                                  \
            hipLaunchKernelGGL((score_keys_kernel<T, D, G, kKeysBW, kKeysNT, true>), grid, block, 0, s, \
                               static_cast<const T *>(q), static_cast<const T *>(k), a);            \
        else                                                                                       \
            hipLaunchKernelGGL((score_keys_kernel<T, D, G, kKeysBW, kKeysNT, false>), grid, block, 0, s, \
                               static_cast<const T *>(q), static_cast<const T *>(k), a);            \
    } while (0)
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
