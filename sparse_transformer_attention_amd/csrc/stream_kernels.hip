// Stage 1 of condensate attention for decode-shaped problems on gfx950, in two kernels (pages of
// "The Condensate Theorem", metaphor-xennon blog: section 2.1 Definition 1,
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
// filter: one workgroup per (unit, split of 1024 rows). The blocks are disjoint, so any value
// that at least k' of a query's block maxima reach (k' = min(k, |R_i|)) is reached by k'
// distinct candidates: a lower bound of the query's k-th key. The bound used is the lower edge
// of the radix bin that holds the k'-th largest maximum, a tight one. The workgroup keeps the
// keys of its split that reach the bound (the exact top-k of them when there are more than k)
// and writes them, as 64-bit ranking keys, with their count, to its segment of the query. The
// finish kernel merges the segments.
#include "ca_internal.h"
#include "score_core.h"
#include "select_core.h"

namespace ca {
namespace {

constexpr int kBlockRows = 256;   // rows per score_keys workgroup (block of the bound)
constexpr int kSplitRows = 1024;  // rows per filter workgroup
constexpr int kMaxBound = 512;    // block maxima used by the bound (merged in groups beyond)

struct KeysArgs {
    int64_t n, nq;
    int Hq, Hkv, g, W;
    int64_t groups, units;
    int64_t rstride;  // key rows per unit in the key buffer
    int nblk;         // blocks per unit
    uint32_t *keys;   // [units][G][rstride], tiles as described above
    uint32_t *bmax;   // [units][nblk][G]
    uint32_t *tmax;   // [units][G][rstride / (4*RPG)]: best key of each tile
};

template <typename T, int D, int G>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(sizeof(T) == 2 ? 5 : 4))) void score_keys_kernel(
    const T *__restrict__ q, const T *__restrict__ k, KeysArgs a) {
    constexpr int EB = sizeof(T);
    constexpr int RB = D * EB;               // bytes per key row
    constexpr int LPR = RB >= 256 ? 16 : 8;  // lanes per row
    constexpr int RPG = 64 / LPR;            // rows per wavefront load
    constexpr int P = RB / (16 * LPR);       // 16-byte loads per lane per row
    constexpr int NG = 64 / RPG;             // row groups of a wavefront's 64 rows
    constexpr int U = 16 / P < NG ? 16 / P : NG;  // row groups per round (<= 16 loads per lane)
    static_assert(P >= 1 && NG % U == 0 && U % 4 == 0, "layout");
    __shared__ uint32_t red[4][G];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int64_t u = blockIdx.x / a.nblk;
    const int bi = (int)(blockIdx.x - u * a.nblk);
    const int bk = (int)(u / a.groups);  // b * Hkv + kvh
    const int64_t grp = u - (int64_t)bk * a.groups;
    const int kvh = bk % a.Hkv;
    const int b = bk / a.Hkv;
    const int64_t nvec = (int64_t)a.g * a.nq;
    const int sl = lane % LPR;
    const bool writer = sl % (LPR / G) == 0;
    const int my_t = sl / (LPR / G);

    int64_t rlast[G];
    int64_t rl_max = 0;
#pragma unroll
    for (int t = 0; t < G; ++t) {
        const int64_t idx = grp * G + t;
        rlast[t] = idx < nvec ? (a.n - a.nq + idx / a.g) - a.W : 0;
        rl_max = rlast[t] > rl_max ? rlast[t] : rl_max;
    }
    uint32_t *bout = a.bmax + ((size_t)u * a.nblk + bi) * G;
    const int row0 = bi * kBlockRows;
    if (row0 > rl_max) {  // no candidate row of the unit in this block
        if (tid < G) bout[tid] = 0u;
        return;
    }
    const int rows_end = (int)((row0 + kBlockRows < rl_max + 1) ? row0 + kBlockRows : rl_max + 1);
    const int rlo = row0 > 1 ? row0 : 1;  // row 0 (the anchor) is no candidate
    int my_rlast = (int)rlast[0];
#pragma unroll
    for (int t = 1; t < G; ++t) my_rlast = (my_t == t) ? (int)rlast[t] : my_rlast;

    const uint4 *kbase = reinterpret_cast<const uint4 *>(k + (int64_t)bk * a.n * D);
    uint32_t *kout = a.keys + ((size_t)u * G + my_t) * a.rstride;
    uint32_t *tout = a.tmax + ((size_t)u * G + my_t) * (a.rstride / (4 * RPG));
    const int wrow0 = row0 + wave * 64;  // this wavefront's 64 rows
    uint32_t best = 0u;
    if (wrow0 < rows_end) {
        uint4 qr[G][P];  // this lane's slices of the queries (zero past the last query vector)
#pragma unroll
        for (int t = 0; t < G; ++t) {
            const int64_t idx = grp * G + t;
            if (idx < nvec) {
                const int h = kvh * a.g + (int)(idx % a.g);
                const uint4 *src = reinterpret_cast<const uint4 *>(q + (((int64_t)b * a.Hq + h) * a.nq + idx / a.g) * D);
#pragma unroll
                for (int p = 0; p < P; ++p) qr[t][p] = src[p * LPR + sl];
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
                for (int p = 0; p < P; ++p) kr[uu][p] = src[p * LPR + sl];
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
    // Best key per query over the block: lanes of the same query are LPR apart, then the waves.
    best = lane_max_stride<LPR>(best);
    if (lane < LPR && writer) red[wave][my_t] = best;
    __syncthreads();
    if (tid < G) {
        uint32_t m = 0u;
#pragma unroll
        for (int w = 0; w < 4; ++w) m = red[w][tid] > m ? red[w][tid] : m;
        bout[tid] = m;
    }
}

struct FilterArgs {
    int64_t n, nq;
    int Hq, Hkv, g, W, topk;
    int64_t groups, units;
    int64_t rstride;
    int nblk, nsplit;
    int rpg;               // rows per load of score_keys (tile = 4*rpg rows)
    const uint32_t *keys;  // [units][G][rstride]
    const uint32_t *bmax;  // [units][nblk][G]
    const uint32_t *tmax;  // [units][G][rstride / (4*rpg)]
    uint32_t *cnt;         // [nqv][nsplit]
    uint64_t *lists;       // [nqv][nsplit][topk]
};

template <int G>
__global__ __launch_bounds__(256) void filter_kernel(FilterArgs a) {
    // LDS: candidate lists [G][kSplitRows] (u64), radix histograms [4][320], counts and bounds.
    __shared__ uint64_t lst[G][kSplitRows];
    __shared__ uint32_t hist_all[4][320];
    __shared__ uint32_t lcnt[G], thr_s[G];
    constexpr int E = kMaxBound / 64;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int64_t u = blockIdx.x / a.nsplit;
    const int sp = (int)(blockIdx.x - u * a.nsplit);
    const int bk = (int)(u / a.groups);
    const int64_t grp = u - (int64_t)bk * a.groups;
    const int kvh = bk % a.Hkv;
    const int b = bk / a.Hkv;
    const int64_t nvec = (int64_t)a.g * a.nq;
    uint32_t *hist = hist_all[wave];

    int rlast[G];
    int64_t rl_max = 0;
#pragma unroll
    for (int t = 0; t < G; ++t) {
        const int64_t idx = grp * G + t;
        const int64_t rl = idx < nvec ? (a.n - a.nq + idx / a.g) - a.W : 0;
        rlast[t] = (int)rl;
        rl_max = rl > rl_max ? rl : rl_max;
    }
    // The split's tile maxima, requested first so that they arrive while the bounds are
    // computed: entry i of the loop below is query i / tps, tile i % tps of the split.
    const int row0 = sp * kSplitRows;
    const int rows_end = (int)((row0 + kSplitRows < rl_max + 1) ? row0 + kSplitRows : rl_max + 1);
    const int trows = 4 * a.rpg;              // rows per tile
    const int tps = kSplitRows / trows;       // tiles per split
    const int64_t ntq = a.rstride / trows;    // tiles per (unit, query)
    constexpr int TPT = (G * kSplitRows / 16 + 255) / 256;  // entries per thread (at most)
    uint32_t tmv[TPT];
#pragma unroll
    for (int e = 0; e < TPT; ++e) {
        const int i = tid + 256 * e;
        const int t = i / tps, tile0 = row0 + (i % tps) * trows;
        // A tile that starts below rows_end was written by score_keys.
        tmv[e] = (t < G && tile0 < rows_end)
                     ? a.tmax[((size_t)u * G + t) * ntq + tile0 / trows] : 0u;
    }

    // Wavefront t: the bound of query t, near the k'-th largest block maximum.
    const int64_t w_idx = grp * G + wave;
    const bool w_query = wave < G && w_idx < nvec;
    const int64_t w_rlast = w_query ? (a.n - a.nq + w_idx / a.g) - a.W : 0;
    const int kq = (int)(a.topk < w_rlast ? a.topk : w_rlast);
    if (wave < G) {
        uint32_t thr = 0u;
        if (w_query && kq > 0) {
            // Block maxima, merged into at most kMaxBound groups of consecutive blocks (the
            // maximum of a group is still one distinct candidate).
            const int per = (a.nblk + kMaxBound - 1) / kMaxBound;
            const int ngr = (a.nblk + per - 1) / per;
            const uint32_t *bm = a.bmax + (size_t)u * a.nblk * G + wave;
            uint32_t m[E];
#pragma unroll
            for (int e = 0; e < E; ++e) m[e] = 0u;
            for (int j = 0; j < per; ++j) {  // E independent loads per pass
#pragma unroll
                for (int e = 0; e < E; ++e) {
                    const int gi = lane + 64 * e, blk = gi * per + j;
                    if (gi < ngr && blk < a.nblk) {
                        const uint32_t x = bm[(size_t)blk * G];
                        m[e] = x > m[e] ? x : m[e];
                    }
                }
            }
            thr = wave_bound_u32(m, kq, hist);
        }
        // (0 keys are rows that are no candidate of the query.)
        if (lane == 0) { thr_s[wave] = thr > 1u ? thr : 1u; lcnt[wave] = 0u; }
    }
    __syncthreads();

    // Keys of the split that reach their query's bound: only tiles whose best key does are read
    // (position p of a tile holds row rpg*(p%4) + p/4 of the tile).
#pragma unroll
    for (int e = 0; e < TPT; ++e) {
        const int i = tid + 256 * e;
        const int t = i / tps;
        if (t < G && tmv[e] >= thr_s[t]) {
            const uint32_t th = thr_s[t];
            const int tile0 = row0 + (i % tps) * trows;
            const uint4 *src = reinterpret_cast<const uint4 *>(a.keys + ((size_t)u * G + t) * a.rstride + tile0);
            for (int w4 = 0; w4 < trows / 4; ++w4) {
                const uint4 v = src[w4];
                const uint32_t kv[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
                for (int c = 0; c < 4; ++c) {
                    const int row = tile0 + a.rpg * c + w4;  // position 4*w4 + c
                    if (kv[c] >= th && row >= 1 && row < rows_end && row <= rlast[t]) {
                        const uint32_t at = atomicAdd(&lcnt[t], 1u);
                        lst[t][at] = make_rank_key(kv[c], (uint32_t)row);
                    }
                }
            }
        }
    }
    __syncthreads();

    // Wavefront t: at most k of query t's keys (the exact top-k when there are more) to the
    // split's segment.
    if (w_query) {
        const int64_t qv = ((int64_t)b * a.Hq + kvh * a.g + (int)(w_idx % a.g)) * a.nq + w_idx / a.g;
        const int c = (int)lcnt[wave];
        uint64_t *dst = a.lists + ((size_t)qv * a.nsplit + sp) * a.topk;
        int outc;
        if (c > a.topk) {
            constexpr int RE = kSplitRows / 64;
            uint64_t kk[RE];
#pragma unroll
            for (int e = 0; e < RE; ++e) {
                const int f = lane + 64 * e;
                kk[e] = f < c ? lst[wave][f] : 0ull;
            }
            (void)wave_keep_top_u64(kk, a.topk, hist, lst[wave]);
            outc = a.topk;
        } else {
            outc = c;
        }
        wave_sync();
        for (int f = lane; f < outc; f += 64) dst[f] = lst[wave][f];
        if (lane == 0) a.cnt[(size_t)qv * a.nsplit + sp] = (uint32_t)outc;
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
    a.keys = reinterpret_cast<uint32_t *>(static_cast<char *>(ws) + pl.keys_offset);
    a.bmax = reinterpret_cast<uint32_t *>(static_cast<char *>(ws) + pl.bmax_offset);
    a.tmax = reinterpret_cast<uint32_t *>(static_cast<char *>(ws) + pl.tmax_offset);
    dim3 grid((unsigned)(pl.units * pl.nblk)), block(256);
#define CA_LAUNCH_SK(T, D, G) \
    hipLaunchKernelGGL((score_keys_kernel<T, D, G>), grid, block, 0, s, static_cast<const T *>(q), \
                       static_cast<const T *>(k), a)
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

hipError_t launch_filter(const Plan &pl, void *ws, hipStream_t s) {
    FilterArgs a;
    a.n = pl.n; a.nq = pl.nq; a.Hq = pl.Hq; a.Hkv = pl.Hkv; a.g = pl.g; a.W = pl.W; a.topk = pl.topk;
    a.groups = pl.groups; a.units = pl.units; a.rstride = pl.rstride; a.nblk = pl.nblk;
    a.nsplit = pl.wpu;
    a.rpg = pl.tile_rows / 4;
    a.keys = reinterpret_cast<const uint32_t *>(static_cast<char *>(ws) + pl.keys_offset);
    a.bmax = reinterpret_cast<const uint32_t *>(static_cast<char *>(ws) + pl.bmax_offset);
    a.tmax = reinterpret_cast<const uint32_t *>(static_cast<char *>(ws) + pl.tmax_offset);
    a.cnt = reinterpret_cast<uint32_t *>(ws) + 2 * pl.nqv * pl.wpu;
    a.lists = reinterpret_cast<uint64_t *>(static_cast<char *>(ws) + pl.lists_offset);
    dim3 grid((unsigned)(pl.units * pl.wpu)), block(256);
    if (pl.G == 4) hipLaunchKernelGGL(filter_kernel<4>, grid, block, 0, s, a);
    else if (pl.G == 2) hipLaunchKernelGGL(filter_kernel<2>, grid, block, 0, s, a);
    else hipLaunchKernelGGL(filter_kernel<1>, grid, block, 0, s, a);
    return hipGetLastError();
}

}  // namespace ca
