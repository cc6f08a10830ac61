// Stage 1 of condensate attention for decode-shaped problems on gfx950, in two kernels (pages of
// "The Condensate Theorem", metaphor-xennon blog: section 2.1 Definition 1,
// C_i = {0} u {i-W+1..i} u Top-k_i; section 2.2.3, the top-k part ranks the positions
// R_i = {1..i-W} outside the anchor and the window).
//
// score_keys: one workgroup per (unit, block of 256 key rows), where a unit is (batch, KV head,
// query group) with up to G query vectors reading the same KV head. It streams the block's K
// rows once (the only large HBM traffic of the path), computes the fp32 scores of its G
// queries, and writes one order-preserving 32-bit key per (row, query) plus the block's best key
// per query. No LDS lists, no barriers in the stream, no atomics: the grid is one-shot and the
// hardware dispatcher balances it.
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
    uint32_t *keys;   // [units][rstride][G]
    uint32_t *bmax;   // [units][nblk][G]
};

template <typename T, int D, int G>
__global__ __launch_bounds__(256) void score_keys_kernel(const T *__restrict__ q, const T *__restrict__ k,
                                                         KeysArgs a) {
    constexpr int EB = sizeof(T);
    constexpr int RB = D * EB;               // bytes per key row
    constexpr int LPR = RB >= 256 ? 16 : 8;  // lanes per row
    constexpr int RPG = 64 / LPR;            // rows per wavefront load
    constexpr int P = RB / (16 * LPR);       // 16-byte loads per lane per row
    constexpr int NG = 64 / RPG;             // row groups per wavefront (64 rows)
    constexpr int U = 8 / P < NG ? 8 / P : NG;  // row groups per round (<= 8 loads per lane)
    static_assert(P >= 1 && NG % U == 0, "layout");
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
    const int row0 = 1 + bi * kBlockRows;
    if (row0 > rl_max) {  // no candidate row of the unit in this block
        if (tid < G) bout[tid] = 0u;
        return;
    }
    const int rows_end = (int)((row0 + kBlockRows < rl_max + 1) ? row0 + kBlockRows : rl_max + 1);
    int my_rlast = (int)rlast[0];
#pragma unroll
    for (int t = 1; t < G; ++t) my_rlast = (my_t == t) ? (int)rlast[t] : my_rlast;

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

    const uint4 *kbase = reinterpret_cast<const uint4 *>(k + (int64_t)bk * a.n * D);
    uint32_t *kout = a.keys + (size_t)u * a.rstride * G;
    const int wrow0 = row0 + wave * 64;  // this wavefront's 64 rows
    uint32_t best = 0u;
    if (wrow0 < rows_end) {
#pragma unroll
        for (int r = 0; r < NG / U; ++r) {
            uint4 kr[U][P];
            // Row groups r*U*... of the wavefront's rows, RPG rows per load.
#pragma unroll
            for (int uu = 0; uu < U; ++uu) {
                int row = wrow0 + (r * U + uu) * RPG + lane / LPR;
                row = row < rows_end ? row : rows_end - 1;
                const uint4 *src = kbase + (int64_t)row * (P * LPR);
#pragma unroll
                for (int p = 0; p < P; ++p) kr[uu][p] = src[p * LPR + sl];
            }
#pragma unroll
            for (int uu = 0; uu < U; ++uu) {
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
                if (writer && row < rows_end) {
                    const uint32_t kv = row <= my_rlast ? key : 0u;
                    kout[(size_t)row * G + my_t] = kv;
                    best = kv > best ? kv : best;
                }
            }
        }
    }
    // Best key per query over the block: lanes of the same query are LPR apart.
#pragma unroll
    for (int off = LPR; off < 64; off <<= 1) {
        const uint32_t o = (uint32_t)__shfl_xor((int)best, off);
        best = o > best ? o : best;
    }
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
    const uint32_t *keys;  // [units][rstride][G]
    const uint32_t *bmax;  // [units][nblk][G]
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
    constexpr int RPT = kSplitRows / 256;  // rows per thread
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
    // The split's keys, requested first so that they arrive while the bounds are computed.
    const int row0 = 1 + sp * kSplitRows;
    const int rows_end = (int)((row0 + kSplitRows < rl_max + 1) ? row0 + kSplitRows : rl_max + 1);
    const uint32_t *kin = a.keys + (size_t)u * a.rstride * G;
    uint32_t kv[RPT][G];
#pragma unroll
    for (int j = 0; j < RPT; ++j) {
        const int row = row0 + tid + 256 * j;
        if (row < rows_end) {
            if constexpr (G == 4) {
                const uint4 v = *reinterpret_cast<const uint4 *>(kin + (size_t)row * 4);
                kv[j][0] = v.x; kv[j][1] = v.y; kv[j][2] = v.z; kv[j][3] = v.w;
            } else if constexpr (G == 2) {
                const uint2 v = *reinterpret_cast<const uint2 *>(kin + (size_t)row * 2);
                kv[j][0] = v.x; kv[j][1] = v.y;
            } else {
                kv[j][0] = kin[row];
            }
        } else {
#pragma unroll
            for (int t = 0; t < G; ++t) kv[j][t] = 0u;
        }
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

    // Keys of the split that reach their query's bound.
    uint32_t thr[G];
#pragma unroll
    for (int t = 0; t < G; ++t) thr[t] = thr_s[t];
#pragma unroll
    for (int j = 0; j < RPT; ++j) {
        const int row = row0 + tid + 256 * j;
#pragma unroll
        for (int t = 0; t < G; ++t) {
            const bool pass = row < rows_end && row <= rlast[t] && kv[j][t] >= thr[t];
            const uint64_t m = __ballot(pass);
            if (m != 0ull) {
                uint32_t base = 0u;
                if (lane == 0) base = atomicAdd(&lcnt[t], (uint32_t)__popcll(m));
                base = __builtin_amdgcn_readlane(base, 0);
                if (pass) lst[t][base + lanes_below(m)] = make_rank_key(kv[j][t], (uint32_t)row);
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
    a.keys = reinterpret_cast<const uint32_t *>(static_cast<char *>(ws) + pl.keys_offset);
    a.bmax = reinterpret_cast<const uint32_t *>(static_cast<char *>(ws) + pl.bmax_offset);
    a.cnt = reinterpret_cast<uint32_t *>(ws) + 2 * pl.nqv * pl.wpu;
    a.lists = reinterpret_cast<uint64_t *>(static_cast<char *>(ws) + pl.lists_offset);
    dim3 grid((unsigned)(pl.units * pl.wpu)), block(256);
    if (pl.G == 4) hipLaunchKernelGGL(filter_kernel<4>, grid, block, 0, s, a);
    else if (pl.G == 2) hipLaunchKernelGGL(filter_kernel<2>, grid, block, 0, s, a);
    else hipLaunchKernelGGL(filter_kernel<1>, grid, block, 0, s, a);
    return hipGetLastError();
}

}  // namespace ca
