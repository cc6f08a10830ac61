// Condensate attention for decode-shaped problems on gfx950 (pages of "The Condensate Theorem",
// metaphor-xennon blog: section 2.1 Definition 1, C_i = {0} u {i-W+1..i} u Top-k_i; section
// 2.2.3, the top-k part over R_i = {1..i-W}; section 2.3, the softmax restricted to C_i times V).
//
// Work unit: (batch, KV head, query group) with up to G query vectors reading one KV head. Two
// kernels:
//   decode_stream   per unit, wpb workgroups of two blocks of 256 key rows each (interleaved over
//                   the units: workgroup s serves unit s % units). Every K row is read once
//                   (16-byte non-temporal loads, LPR lanes per row) and dotted with the unit's G
//                   queries in fp32 (row_key); the order-preserving 32-bit keys (0 for rows
//                   outside R_i of a query) are staged in LDS. Per block and query, 16 lanes
//                   reduce the block's keys to a 32-byte record: four of its rows (key, offset)
//                   and a key X that every other row of the block stays at or below (with the
//                   mass diagnostic also the block's largest score m_b and its sum of
//                   exp2((s - m_b) * scale)).
//   decode_finish   one workgroup per query vector. All of its wavefronts compute the anchor-and-
//                   window softmax partials while the records load (one per thread). A bound T0
//                   comes from the blocks' best keys: the k'-th largest of them (k' blocks, so k'
//                   distinct rows, reach it: no row below it can be in the top k'). The record
//                   rows whose ranking key (score_key << 32) | ~position reaches the bound are
//                   gathered and cut to their exact top k' (one wavefront). A block whose X
//                   reaches the k'-th key has rows beyond its record that may rank: those are
//                   scored again (row_key, the same bits) and the cut repeated. C_i goes to
//                   out_idx, and the top-k rows' partials (weights exp2((s - m) * scale), s read
//                   back from the keys) merge with the window's into the output. Too many
//                   candidates or such blocks (dense clusters of high scores, exact ties) switch
//                   the query to an exact fallback: all its candidate rows scored into scratch
//                   keys and a workgroup radix select over them.
#include <type_traits>

#include "attend_core.h"
#include "ca_internal.h"
#include "device_utils.h"
#include "merge_core.h"
#include "score_core.h"
#include "select_core.h"

namespace ca {
namespace {

constexpr int kRows = 256;         // key rows per block
constexpr int kBW = 2;             // blocks per stream workgroup
constexpr int kNT = kBW * 256;     // threads per workgroup (both kernels)
constexpr int kWaves = kNT / 64;
constexpr int kCand = 1024;        // candidate keys per query held in LDS
constexpr int kDef = 64;           // blocks whose X reaches the threshold, held in LDS
constexpr int kResc = 8;           // such blocks scored again on the common path
constexpr int kSelMax = 256;       // largest k' of the common path (larger: the fallback)

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

// ---- decode_stream: keys of two blocks into LDS, then the block records ---------------------
template <typename T, int D, int G, bool MASS>
__global__ __launch_bounds__(kNT) __attribute__((amdgpu_waves_per_eu(sizeof(T) == 2 ? 5 : 4))) void decode_stream_kernel(
    const T *__restrict__ q, const T *__restrict__ k, DecodeArgs a) {
    __shared__ uint32_t kst[G][kBW * kRows];  // keys of the workgroup's rows, per query
    // Workgroup s: unit s % units, its part s / units.
    const uint32_t part = blockIdx.x / a.units;
    const uint32_t uu = blockIdx.x - part * a.units;
    using S = StreamShape<T, D>;
    constexpr int LPR = S::LPR, RPG = S::RPG, P = S::P, NG = S::NG, U = S::U, TR = S::TR;
    constexpr int WROWS = kBW * kRows;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const uint32_t ng = (uint32_t)a.groups;
    const int wg_row0 = (int)part * WROWS;
    const int bi = wg_row0 / kRows + wave / 4;
    const uint32_t bk = uu / ng, grp = uu - bk * ng;
    const uint32_t g = (uint32_t)a.g;
    const int sl = lane % LPR;
    const bool writer = sl % (LPR / G) == 0;
    const int my_t = sl / (LPR / G);
    const uint32_t idx0 = grp * G;
    const uint32_t idx_last = (idx0 + G - 1 < a.nvec ? idx0 + G - 1 : a.nvec - 1);
    const int rl_max = a.row_base + (int)(idx_last / g);
    const int row0 = bi * kRows;
    const bool live = bi < a.nblk && row0 <= rl_max;
    const int rows_end = (row0 + kRows < rl_max + 1) ? row0 + kRows : rl_max + 1;
    const int rlo = row0 > 1 ? row0 : 1;  // row 0 (the anchor) is no candidate
    const uint4 *kbase = reinterpret_cast<const uint4 *>(k + (int64_t)bk * a.n * D);
    const int wrow0 = row0 + (wave % 4) * 64;
    if (live && wrow0 < rows_end) {
        uint4 qr[G][P];
        load_query_slices<T, D, G>(q, a, bk, grp, lane, qr);
        int my_rlast = 0;
        {
            const uint32_t idx = idx0 + my_t;
            if (idx < a.nvec) my_rlast = a.row_base + (int)(idx / g);
        }
#pragma unroll
        for (int r = 0; r < NG / U; ++r) {
            uint4 kr[U][P];
#pragma unroll
            for (int uq = 0; uq < U; ++uq) {
                int row = wrow0 + (r * U + uq) * RPG + lane / LPR;
                row = row < rows_end ? row : rows_end - 1;
                const uint4 *src = kbase + (int64_t)row * (P * LPR);
#pragma unroll
                for (int p = 0; p < P; ++p) kr[uq][p] = load_row16_nt(src + p * LPR + sl);
            }
#pragma unroll
            for (int u4 = 0; u4 < U; u4 += 4) {
                uint32_t kv4[4];
#pragma unroll
                for (int gg = 0; gg < 4; ++gg) {
                    const int uq = u4 + gg;
                    const uint32_t key = row_key<T, LPR, P, G>(kr[uq], qr, lane);
                    const int row = wrow0 + (r * U + uq) * RPG + lane / LPR;
                    kv4[gg] = (row >= rlo && row < rows_end && row <= my_rlast) ? key : 0u;
                }
                // Keys of rows tile0 + RPG*gg + lane/LPR as one 16-byte word.
                const int tile0 = wrow0 + (r * U + u4) * RPG;
                if (writer)
                    *reinterpret_cast<uint4 *>(&kst[my_t][tile0 - wg_row0 + 4 * (lane / LPR)]) =
                        make_uint4(kv4[0], kv4[1], kv4[2], kv4[3]);
            }
        }
    } else {
        for (int x = lane; x < G * 16; x += 64)
            *reinterpret_cast<uint4 *>(&kst[x / 16][wrow0 - wg_row0 + 4 * (x % 16)]) = make_uint4(0, 0, 0, 0);
    }
    __syncthreads();
    // Records: 16 lanes per (block, query); lane j takes staged positions 16j .. 16j + 15. The
    // wavefronts without a record to write are done.
    const int nbw = a.nblk - wg_row0 / kRows < kBW ? a.nblk - wg_row0 / kRows : kBW;
    if (wave * 4 >= nbw * G) return;
    const int pr = tid >> 4, j = tid & 15;
    if (pr >= nbw * G) return;
    const int b2 = pr / G, t = pr % G;
    if (idx0 + t >= a.nvec) return;  // no query vector: no record
    const uint32_t *src = &kst[t][b2 * kRows + 16 * j];
    uint32_t kk[16];
#pragma unroll
    for (int w4 = 0; w4 < 4; ++w4) {
        const uint4 x = reinterpret_cast<const uint4 *>(src)[w4];
        kk[4 * w4] = x.x; kk[4 * w4 + 1] = x.y; kk[4 * w4 + 2] = x.z; kk[4 * w4 + 3] = x.w;
    }
    // This lane's two best rows as (key << 8 | 255 - offset) (ties: smaller offset first) and
    // the largest key of its other rows.
    uint64_t v1 = 0ull, v2 = 0ull;
    uint32_t k3 = 0u;
#pragma unroll
    for (int c = 0; c < 16; ++c) {
        const int off = staged_row<TR, RPG>(16 * j + c);
        const uint64_t x = ((uint64_t)kk[c] << 8) | (uint32_t)(255 - off);
        const bool b1 = x > v1, b2w = x > v2;
        const uint32_t drop = (uint32_t)((b1 ? v2 : (b2w ? v2 : x)) >> 8);
        k3 = drop > k3 ? drop : k3;
        v2 = b1 ? v1 : (b2w ? x : v2);
        v1 = b1 ? x : v1;
    }
    // Four rows of the block: the largest head of the 16 lanes, four times; X: the largest key
    // left (heads and the lanes' other rows).
    uint64_t e[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        const uint64_t m = row16_max_u64(v1);
        e[r] = m;
        const bool mine = v1 == m;
        v1 = mine ? v2 : v1;
        v2 = mine ? 0ull : v2;
    }
    const uint32_t xr = row16_max_u32((uint32_t)(v1 >> 8));
    const uint32_t x3 = row16_max_u32(k3);
    const uint32_t X = xr > x3 ? xr : x3;
    const uint32_t k1 = (uint32_t)(e[0] >> 8);
    float zl = 0.f, zm = -INFINITY;
    if constexpr (MASS) {
        zm = k1 ? key_score(k1) : -INFINITY;
        float zsum = 0.f;
#pragma unroll
        for (int c = 0; c < 16; ++c)
            if (kk[c]) zsum += exp2f((key_score(kk[c]) - zm) * a.scale_log2e);
        zl = row16_sum_f32(zsum);
    }
    const int blk = wg_row0 / kRows + b2;
    uint4 *rec = a.rec + (((size_t)uu * G + t) * (size_t)a.nblk + blk) * 2;
    if (j == 0) {
        rec[0] = make_uint4(k1, (uint32_t)(e[1] >> 8), (uint32_t)(e[2] >> 8), (uint32_t)(e[3] >> 8));
    } else if (j == 1) {
        uint32_t offs = 0u;
#pragma unroll
        for (int r = 0; r < 4; ++r) offs |= (255u - (uint32_t)(e[r] & 255u)) << (8 * r);
        rec[1] = make_uint4(offs, X, __float_as_uint(zm), __float_as_uint(zl));
    }
}

// Keeps the top kp of the n distinct non-zero ranking keys list[0..n) (n <= 64 E) in
// list[0..kp) and returns a value that exactly those reach. One wavefront.
template <int E>
__device__ __forceinline__ uint64_t keep_top(uint64_t *list, int n, int kp) {
    const int lane = threadIdx.x & 63;
    uint64_t kr[E];
#pragma unroll
    for (int e = 0; e < E; ++e) {
        const int c = lane + 64 * e;
        kr[e] = c < n ? list[c] : 0ull;
    }
    wave_sync();  // every key is in registers before the list is rewritten
    const uint64_t t = wave_kth_u64(kr, kp);
    int base = 0;
#pragma unroll
    for (int e = 0; e < E; ++e) {
        const bool ok = kr[e] != 0ull && kr[e] >= t;
        const uint64_t bal = __ballot(ok);
        if (ok) list[base + lanes_below(bal)] = kr[e];
        base += __popcll(bal);
    }
    wave_sync();
    return t;
}


// ---- decode_finish ---------------------------------------------------------------------------
template <int D>
struct FinShared {
    uint64_t cand[kCand];  // candidate ranking keys; after each cut the top k'
    union {
        uint32_t bmax[kNT];  // best keys of the round's blocks (threshold of the single wavefront)
        struct {
            int32_t js[2 * 512];    // fallback: selected positions
            SelectShared<kNT> ssh;  // fallback: radix select
        } fb;
    } x;
    uint64_t def[kDef];   // blocks whose X reached the threshold: X << 32 | block
    uint32_t doff[kDef];  // and their records' row offsets
    SoftmaxPartials<D, 2 * kWaves> part;  // [0, kWaves) anchor and window, then the top-k rows
    int wc[kWaves], wd[kWaves];           // per-wavefront counts of an append
    uint32_t tw[kWaves];                  // per-wavefront bounds
    uint32_t tb;                          // the single wavefront's bound
    float zm[kWaves], zl[kWaves];         // mass diagnostic: candidates' mass per wavefront
    uint64_t thr;
    int n, ndef, flag;
};

// Appends, in a fixed order (wavefront, then e, then lane), the keys key[e] with ok[e] of every
// wavefront after list[0..sh.n), and the blocks with okd (entry dk, offsets doff) after
// def[0..sh.ndef). Called by all threads; two workgroup barriers. Entries past the capacities
// are dropped (the counts still grow, so the caller sees the overflow).
template <int D, int E>
__device__ __forceinline__ void append_all(FinShared<D> &sh, const bool (&ok)[E], const uint64_t (&key)[E],
                                           bool okd, uint64_t dk, uint32_t doff) {
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    uint64_t bal[E];
    int tot = 0;
#pragma unroll
    for (int e = 0; e < E; ++e) {
        bal[e] = __ballot(ok[e]);
        tot += __popcll(bal[e]);
    }
    const uint64_t bd = __ballot(okd);
    if (lane == 0) {
        sh.wc[wave] = tot;
        sh.wd[wave] = __popcll(bd);
    }
    lds_barrier();
    int base = sh.n, dbase = sh.ndef, n_all = sh.n, d_all = sh.ndef;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
        const int c = sh.wc[w], d = sh.wd[w];
        base += w < wave ? c : 0;
        dbase += w < wave ? d : 0;
        n_all += c;
        d_all += d;
    }
#pragma unroll
    for (int e = 0; e < E; ++e) {
        const int pos = base + lanes_below(bal[e]);
        if (ok[e] && pos < kCand) sh.cand[pos] = key[e];
        base += __popcll(bal[e]);
    }
    {
        const int pos = dbase + lanes_below(bd);
        if (okd && pos < kDef) {
            sh.def[pos] = dk;
            sh.doff[pos] = doff;
        }
    }
    lds_barrier();
    if (threadIdx.x == 0) {
        sh.n = n_all;
        sh.ndef = d_all;
    }
}

// Keeps the top kp of the n distinct non-zero ranking keys list[0..n) (n <= 64 E, n > kp) in
// list[0..kp), in their list order, and returns the kp-th key. The search runs on the 32-bit
// score keys first; only equal score keys at the kp-th place need the 64-bit keys. One
// wavefront.
template <int E>
__device__ __forceinline__ uint64_t keep_top_fast(uint64_t *list, int n, int kp) {
    const int lane = threadIdx.x & 63;
    uint64_t kr[E];
    uint32_t sk[E];
#pragma unroll
    for (int e = 0; e < E; ++e) {
        const int c = lane + 64 * e;
        kr[e] = c < n ? list[c] : 0ull;
        sk[e] = (uint32_t)(kr[e] >> 32);
    }
    const uint32_t t32 = wave_loose_kth_u32(sk, kp, 0);
    int cnt = 0;
#pragma unroll
    for (int e = 0; e < E; ++e) cnt += __popcll(__ballot(sk[e] != 0u && sk[e] >= t32));
    if (cnt != kp) return keep_top<E>(list, n, kp);
    wave_sync();  // every key is in registers before the list is rewritten
    int base = 0;
    uint64_t kmin = ~0ull;
#pragma unroll
    for (int e = 0; e < E; ++e) {
        const bool ok = sk[e] != 0u && sk[e] >= t32;
        const uint64_t bal = __ballot(ok);
        if (ok) {
            list[base + lanes_below(bal)] = kr[e];
            kmin = kr[e] < kmin ? kr[e] : kmin;
        }
        base += __popcll(bal);
    }
    wave_sync();
    return wave_min_u64_dpp(kmin);
}

// Exact top kp of sh.cand[0..n) into sh.cand[0..kp); the threshold becomes the kp-th key (one
// wavefront; n <= kCand).
template <int D>
__device__ __forceinline__ void cut_exact(FinShared<D> &sh, int kp) {
    const int n = sh.n;
    if (n <= kp) return;
    uint64_t t;
    if (n <= 128) t = keep_top_fast<2>(sh.cand, n, kp);
    else if (n <= 256) t = keep_top_fast<4>(sh.cand, n, kp);
    else if (n <= 512) t = keep_top_fast<8>(sh.cand, n, kp);
    else t = keep_top<16>(sh.cand, n, kp);
    if ((threadIdx.x & 63) == 0) {
        sh.thr = t;
        sh.n = kp;
    }
}

// Deferred blocks whose X fell below the threshold's score key leave the list, in order (one
// wavefront).
template <int D>
__device__ __forceinline__ void filter_deferred(FinShared<D> &sh) {
    const int lane = threadIdx.x & 63;
    const int nd = sh.ndef;
    if (nd == 0 || nd > kDef) return;
    const uint32_t thi = (uint32_t)(sh.thr >> 32);
    const uint64_t d = lane < nd ? sh.def[lane] : 0ull;
    const uint32_t o = lane < nd ? sh.doff[lane] : 0u;
    wave_sync();
    const bool keep = d != 0ull && (uint32_t)(d >> 32) >= thi;
    const uint64_t bal = __ballot(keep);
    if (keep) {
        sh.def[lanes_below(bal)] = d;
        sh.doff[lanes_below(bal)] = o;
    }
    if (lane == 0) sh.ndef = __popcll(bal);
    wave_sync();
}

template <typename T, int D, int G, bool ATTEND, bool MASS>
__global__ __launch_bounds__(kNT) void decode_finish_kernel(const T *__restrict__ q, const T *__restrict__ k,
                                                            const T *__restrict__ v, DecodeArgs a) {
    static_assert(kDef <= 64 && kCand <= 64 * 16, "one wavefront holds the lists");
    using AS = AttendShape<D, T>;
    using S = StreamShape<T, D>;
    constexpr int UW = 9;  // window rows per lane requested before the selection (9 * 32 >= 257)
    __shared__ FinShared<D> sh;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const uint32_t uu = blockIdx.x / G;
    const int t = (int)(blockIdx.x - uu * G);
    const uint32_t ng = (uint32_t)a.groups;
    const uint32_t bk = uu / ng, grp = uu - bk * ng;
    const QInfo qi = query_info<G>(a, bk, grp, t);
    if (!qi.valid) return;
    const int kp = qi.kp;
    const size_t kv0 = (size_t)bk * (size_t)a.n * D;
    const T *kb = k + kv0, *vb = v + kv0;
    int32_t *row = a.out_idx + (size_t)qi.qv * a.cap;
    const uint4 *R = a.rec + ((size_t)uu * G + t) * (size_t)a.nblk * 2;
    // Requests first: the first round's records, then the first rows of the anchor and window.
    uint4 ra = make_uint4(0, 0, 0, 0), rb = make_uint4(0, 0, 0, 0);
    if (tid < qi.nbq && kp > 0) {
        ra = R[2 * tid];
        rb = R[2 * tid + 1];
    }
    const uint4 qs = reinterpret_cast<const uint4 *>(q + (size_t)qi.qv * D)[lane % AS::LPR];
    const int wn = qi.base + qi.wcount;  // anchor and window rows
    auto row_at = [&](int c) -> size_t { return c < qi.base ? 0 : (size_t)(qi.wlo - qi.base + c); };
    const int wstep = kWaves * AS::RPW;
    RowSlices<D, T, UW> rs;
    if constexpr (ATTEND) load_rows<D, T, UW>(rs, kb, vb, row_at, wn, wave * AS::RPW, wstep);
    if (tid == 0) {
        sh.n = 0;
        sh.ndef = 0;
        sh.flag = kp > kSelMax ? 1 : 0;
        sh.thr = 1ull << 32;  // any candidate key (>= 1) reaches it
    }
    // Anchor, window and padding entries of C_i (ascending: anchor, top-k', window, -1).
    for (int e = tid; e < a.cap; e += kNT) {
        if (e >= qi.base && e < qi.base + kp) continue;
        row[e] = e < qi.base ? 0 : (e < qi.base + kp + qi.wcount ? qi.wlo + (e - qi.base - kp) : -1);
    }
    // Rounds of kNT blocks (one record per thread).
    float zm = -INFINITY, zl = 0.f;
    for (int r0 = 0; r0 < qi.nbq && kp > 0; r0 += kNT) {
        const int blk = r0 + tid;
        const bool has = blk < qi.nbq;
        if (r0 > 0) {
            ra = has ? R[2 * (size_t)blk] : make_uint4(0, 0, 0, 0);
            rb = has ? R[2 * (size_t)blk + 1] : make_uint4(0, 0, 0, 0);
        }
        if constexpr (MASS) {
            const float bm = __uint_as_float(rb.z), bl = __uint_as_float(rb.w);
            if (has && bm != -INFINITY) {
                const float mn = fmaxf(zm, bm);
                zl = (zm == -INFINITY ? 0.f : zl * exp2f((zm - mn) * a.scale_log2e)) + bl * exp2f((bm - mn) * a.scale_log2e);
                zm = mn;
            }
        }
        // A bound from the round's best keys: with q = ceil(kp / 8), each wavefront's q-th
        // largest; their minimum is reached by q blocks of each wavefront, kp distinct rows in
        // all. A wavefront with fewer than q blocks leaves it to one wavefront searching all of
        // the round's best keys for their kp-th largest.
        {
            const int qk = (kp + kWaves - 1) / kWaves;
            const uint32_t b1[1] = {ra.x};
            const int nz = __popcll(__ballot(ra.x != 0u));
            const uint32_t tw = nz >= qk ? wave_loose_kth_u32(b1, qk, 0) : 0u;
            if (lane == 0) sh.tw[wave] = tw;
            sh.x.bmax[tid] = ra.x;
        }
        lds_barrier();
        {
            uint32_t t0 = 0xFFFFFFFFu;
#pragma unroll
            for (int w = 0; w < kWaves; ++w) t0 = sh.tw[w] < t0 ? sh.tw[w] : t0;
            if (t0 == 0u) {
                // (Uniform: every thread reads the same bounds.)
                if (wave == 0) {
                    uint32_t bm[kNT / 64];
                    int nzt = 0;
#pragma unroll
                    for (int e = 0; e < kNT / 64; ++e) {
                        bm[e] = sh.x.bmax[lane + 64 * e];
                        nzt += __popcll(__ballot(bm[e] != 0u));
                    }
                    const uint32_t tb = nzt >= kp ? wave_loose_kth_u32(bm, kp, 32) : 0u;
                    if (lane == 0) sh.tb = tb;
                }
                lds_barrier();
                t0 = sh.tb;
            }
            const uint64_t b0 = (uint64_t)t0 << 32;
            const uint64_t thr = b0 > sh.thr ? b0 : sh.thr;
            const uint32_t ks[4] = {ra.x, ra.y, ra.z, ra.w};
            const uint32_t offs = rb.x, X = rb.y;
            bool ok[4];
            uint64_t kk[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                kk[e] = make_rank_key(ks[e], (uint32_t)blk * kRows + ((offs >> (8 * e)) & 255u));
                ok[e] = has && ks[e] != 0u && kk[e] >= thr;
            }
            // X reaches the threshold's score key: rows beyond the record may rank.
            const bool okd = has && X != 0u && X >= (uint32_t)(thr >> 32);
            append_all<D, 4>(sh, ok, kk, okd, ((uint64_t)X << 32) | (uint32_t)blk, offs);
            if (tid == 0) sh.thr = thr;
        }
        __syncthreads();
        if (wave == 0) {
            if (sh.n > kCand || sh.ndef > kDef) {
                if (lane == 0) sh.flag = 1;
            } else if (!sh.flag) {
                cut_exact<D>(sh, kp);
                wave_sync();
                filter_deferred<D>(sh);
            }
        }
        __syncthreads();
        if (sh.flag) break;
    }
    // Blocks whose rows beyond their record may still rank: scored again, all wavefronts on one
    // block at a time (32 rows each), then the cut again.
    if (kp > 0 && !sh.flag && sh.ndef > 0) {
        if (sh.ndef > kResc) {
            __syncthreads();
            if (tid == 0) sh.flag = 1;
            __syncthreads();
        } else {
            constexpr int LPR = S::LPR, RPG = S::RPG, P = S::P;
            constexpr int RW = kRows / kWaves;  // rows per wavefront
            constexpr int NL = RW / RPG;        // row groups per wavefront
            uint4 qr[G][P];
            load_query_slices<T, D, G>(q, a, bk, grp, lane, qr);
            const uint4 *kbase = reinterpret_cast<const uint4 *>(kb);
            const int sl = lane % LPR;
            const bool mine = sl % (LPR / G) == 0 && sl / (LPR / G) == t;
            const uint64_t thr = sh.thr;
            const int nd = sh.ndef;
            for (int x = 0; x < nd; ++x) {
                const int blk = (int)(uint32_t)sh.def[x];
                const uint32_t offs = sh.doff[x];
                uint4 kr[NL][P];
#pragma unroll
                for (int u = 0; u < NL; ++u) {
                    int r = blk * kRows + wave * RW + u * RPG + lane / LPR;
                    r = r <= qi.rl ? r : qi.rl;
                    const uint4 *src = kbase + (int64_t)r * (P * LPR);
#pragma unroll
                    for (int p = 0; p < P; ++p) kr[u][p] = src[p * LPR + sl];
                }
                bool ok[NL];
                uint64_t kk[NL];
#pragma unroll
                for (int u = 0; u < NL; ++u) {
                    const uint32_t key = row_key<T, LPR, P, G>(kr[u], qr, lane);
                    const int off = wave * RW + u * RPG + lane / LPR;
                    const int r = blk * kRows + off;
                    const bool in_rec = ((offs & 255u) == (uint32_t)off) || (((offs >> 8) & 255u) == (uint32_t)off) ||
                                        (((offs >> 16) & 255u) == (uint32_t)off) || ((offs >> 24) == (uint32_t)off);
                    kk[u] = make_rank_key(key, (uint32_t)r);
                    ok[u] = mine && !in_rec && r >= 1 && r <= qi.rl && key != 0u && kk[u] >= thr;
                }
                append_all<D, NL>(sh, ok, kk, false, 0ull, 0u);
                __syncthreads();
            }
            if (wave == 0) {
                if (sh.n > kCand) {
                    if (lane == 0) sh.flag = 1;
                } else {
                    cut_exact<D>(sh, kp);
                }
            }
            __syncthreads();
        }
    }
    // Exact fallback: every candidate row of the query scored into its scratch keys, then the
    // workgroup radix select over the ranking keys that reach the threshold.
    if (kp > 0 && sh.flag) {
        constexpr int LPR = S::LPR, RPG = S::RPG, P = S::P;
        const uint64_t thr = sh.thr;
        uint32_t *sc = a.scratch + ((size_t)uu * G + t) * (size_t)a.rstride;
        uint4 qr[G][P];
        load_query_slices<T, D, G>(q, a, bk, grp, lane, qr);
        const uint4 *kbase = reinterpret_cast<const uint4 *>(kb);
        const int sl = lane % LPR;
        const bool mine = sl % (LPR / G) == 0 && sl / (LPR / G) == t;
        const int rows = qi.nbq * kRows;
        for (int r0 = wave * RPG; r0 < rows; r0 += kWaves * RPG) {
            const int r = r0 + lane / LPR;
            const int lr = r <= qi.rl ? r : qi.rl;
            const uint4 *src = kbase + (int64_t)lr * (P * LPR);
            uint4 kr[P];
#pragma unroll
            for (int p = 0; p < P; ++p) kr[p] = src[p * LPR + sl];
            const uint32_t key = row_key<T, LPR, P, G>(kr, qr, lane);
            if (mine) sc[r] = (r >= 1 && r <= qi.rl) ? key : 0u;
        }
        __threadfence_block();
        __syncthreads();
        auto key_at = [&](int64_t f64) -> uint64_t {
            const int f = (int)f64;
            const uint32_t kv = sc[f];
            const uint64_t rk = make_rank_key(kv, (uint32_t)f);
            return kv != 0u && rk >= thr ? rk : 0ull;
        };
        select_exact<kNT>(kGather + 1, (int64_t)rows, key_at, kp, sh.x.fb.js, nullptr, nullptr, sh.x.fb.ssh);
        // The top-k' as ranking keys (js holds their positions, ascending).
        for (int c = tid; c < kp; c += kNT) {
            const int32_t pos = sh.x.fb.js[c];
            sh.cand[c] = make_rank_key(sc[pos], (uint32_t)pos);
        }
        __syncthreads();
    }
    // The top-k' rows are sh.cand[0..kp), in an order fixed by the inputs. Their V rows are
    // requested first (partial of wavefront `wave`: rows c = wave*RPW + slot + u*kWaves*RPW);
    // while they load, the top-k' places in out_idx (the number of selected positions below)
    // and the anchor-and-window partial.
    constexpr int UT = 4;
    const int cs = lane % AS::LPR, slot = lane / AS::LPR;
    const int step = kWaves * AS::RPW;
    const uint32_t last_row = (uint32_t)(a.n - 1);
    uint4 vv[UT];
    uint32_t sk[UT];
    auto request = [&](int c0) {
#pragma unroll
        for (int u = 0; u < UT; ++u) {
            int c = c0 + u * step + slot;
            c = c < kp ? c : (kp > 0 ? kp - 1 : 0);
            const uint64_t key = sh.cand[c];
            uint32_t pos = (uint32_t)rank_key_pos(key);
            pos = pos < last_row ? pos : last_row;
            sk[u] = (uint32_t)(key >> 32);
            vv[u] = reinterpret_cast<const uint4 *>(vb + (size_t)pos * D)[cs];
        }
    };
    if (ATTEND && kp > 0) request(wave * AS::RPW);
    if (kp <= 64) {
        if (wave == kWaves - 1) {
            // One candidate per lane; every position broadcast in turn.
            const uint32_t pos = lane < kp ? (uint32_t)rank_key_pos(sh.cand[lane]) : 0xFFFFFFFFu;
            int rank = 0;
            for (int j = 0; j < kp; ++j) rank += __builtin_amdgcn_readlane(pos, j) < pos;
            if (lane < kp) row[qi.base + rank] = (int32_t)pos;
        }
    } else {
        const int kp8 = (kp + 7) & ~7;
        for (int cb = 64 * (kWaves - 1 - wave); cb < kp; cb += 64 * kWaves) {
            const int c = cb + lane;
            const uint32_t pos = c < kp ? (uint32_t)rank_key_pos(sh.cand[c]) : 0u;
            int rank = 0;
            for (int f0 = 0; f0 < kp8; f0 += 8) {
                // (Whole groups of 8 read: kp8 <= kSelMax <= kCand.)
                const uint4 *src = reinterpret_cast<const uint4 *>(sh.cand + f0);
                uint4 y[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) y[e] = src[e];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    rank += (f0 + 2 * e < kp) && ~y[e].x < pos;
                    rank += (f0 + 2 * e + 1 < kp) && ~y[e].z < pos;
                }
            }
            if (c < kp) row[qi.base + rank] = (int32_t)pos;
        }
    }
    if constexpr (ATTEND) {
        // Anchor and window: the requested rows, then any beyond them (long windows).
        {
            SlotState<D, T> st;
            auto use = [&](int c) { return c < wn; };
            accumulate_rows<D, T, UW>(st, rs, qs, use, wave * AS::RPW, wstep, a.scale_log2e);
            for (int c0 = wave * AS::RPW + UW * wstep; c0 < wn; c0 += UW * wstep) {
                load_rows<D, T, UW>(rs, kb, vb, row_at, wn, c0, wstep);
                accumulate_rows<D, T, UW>(st, rs, qs, use, c0, wstep, a.scale_log2e);
            }
            store_wave_partial<D, T>(st, a.scale_log2e, sh.part, wave);
        }
        // Top-k rows: weights exp2((s - m) * scale), m the largest selected score.
        float acc[AS::EPL];
#pragma unroll
        for (int e = 0; e < AS::EPL; ++e) acc[e] = 0.f;
        float l = 0.f;
        uint32_t kmax = 0u;
        for (int c = lane; c < kp; c += 64) {
            const uint32_t x = (uint32_t)(sh.cand[c] >> 32);
            kmax = x > kmax ? x : kmax;
        }
        const float m = kp > 0 ? key_score(wave_max_u32_dpp(kmax)) : -INFINITY;
        for (int c0 = wave * AS::RPW; c0 < kp; c0 += UT * step) {
            if (c0 != wave * AS::RPW) request(c0);
#pragma unroll
            for (int u = 0; u < UT; ++u) {
                if (c0 + u * step + slot < kp) {
                    const float w = exp2f((key_score(sk[u]) - m) * a.scale_log2e);
                    l += w;
                    accumulate16(acc, vv[u], w, T());
                }
            }
        }
        if constexpr (AS::LPR <= 8) {
            l = lane_pair_sum<8>(l);
#pragma unroll
            for (int e = 0; e < AS::EPL; ++e) acc[e] = lane_pair_sum<8>(acc[e]);
        }
        if constexpr (AS::LPR <= 16) {
            l = lane_pair_sum<16>(l);
#pragma unroll
            for (int e = 0; e < AS::EPL; ++e) acc[e] = lane_pair_sum<16>(acc[e]);
        }
        l = lane_pair_sum<32>(l);
#pragma unroll
        for (int e = 0; e < AS::EPL; ++e) acc[e] = lane_pair_sum<32>(acc[e]);
        const int slot_out = kWaves + wave;
        if (lane < AS::LPR) {
#pragma unroll
            for (int e = 0; e < AS::EPL; ++e) sh.part.acc[slot_out][cs * AS::EPL + e] = acc[e];
        }
        if (lane == 0) {
            sh.part.m[slot_out] = m;
            sh.part.l[slot_out] = l;
        }
        if constexpr (MASS) {
            const float mr = wave_max_f32_dpp(zm);
            const float lr = wave_sum_f32_dpp(zm == -INFINITY ? 0.f : zl * exp2f((zm - mr) * a.scale_log2e));
            if (lane == 0) {
                sh.zm[wave] = mr;
                sh.zl[wave] = lr;
            }
        }
        lds_barrier();
        float *o = a.out + (size_t)qi.qv * D;
        merge_partials<kNT, D, 2 * kWaves>(sh.part, 0, 2 * kWaves, a.scale_log2e, o);
        if constexpr (MASS) {
            // Mass diagnostic (section 3.2.2, the full-softmax mass outside C_i; sections
            // 2.2.1-2.2.3, the parts of C_i): the candidates' part from the blocks' sums, the
            // window part (with row 0) and the top-k part from the partials, row 0 from its score;
            // all relative to one maximum.
            if (wave == 0) {
                auto fold = [&](int p0, float *mo, float *lo) {
                    float mx = -INFINITY;
                    for (int p = p0; p < p0 + kWaves; ++p) mx = fmaxf(mx, sh.part.m[p]);
                    float sm = 0.f;
                    for (int p = p0; p < p0 + kWaves; ++p)
                        sm += sh.part.m[p] == -INFINITY ? 0.f : sh.part.l[p] * exp2f((sh.part.m[p] - mx) * a.scale_log2e);
                    *mo = mx;
                    *lo = sm;
                };
                float mw, lw, mt, lt;
                fold(0, &mw, &lw);
                fold(kWaves, &mt, &lt);
                float mr = -INFINITY;
                for (int p = 0; p < kWaves; ++p) mr = fmaxf(mr, sh.zm[p]);
                float lr = 0.f;
                for (int p = 0; p < kWaves; ++p)
                    lr += sh.zm[p] == -INFINITY ? 0.f : sh.zl[p] * exp2f((sh.zm[p] - mr) * a.scale_log2e);
                const uint4 k0 = reinterpret_cast<const uint4 *>(kb)[lane % AS::LPR];
                const float s0 = row_sum<AS::LPR>(dot16(k0, qs, 0.f, T()));
                const float mgm = fmaxf(mr, mw);
                auto rel = [&](float mx, float sm) { return mx == -INFINITY ? 0.f : sm * exp2f((mx - mgm) * a.scale_log2e); };
                const float zr = rel(mr, lr), zw = rel(mw, lw), zt = rel(mt, lt);
                const float z0 = exp2f((s0 - mgm) * a.scale_log2e);
                const float zf = zr + zw;
                if (lane == 0) {
                    float *mo = a.mass + (size_t)qi.qv * 4;
                    mo[0] = fmaxf(zr - zt, 0.f) / zf;
                    mo[1] = z0 / zf;
                    mo[2] = fmaxf(zw - z0, 0.f) / zf;
                    mo[3] = zt / zf;
                }
            }
        }
    }
}

}  // namespace

hipError_t launch_decode(const Plan &pl, const void *q, const void *k, const void *v, void *ws,
                         int32_t *out_idx, float *out, float *mass, hipStream_t s) {
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
    const bool attend = out != nullptr;
    const uint32_t wpb = (uint32_t)((pl.nblk + kBW - 1) / kBW);
    const dim3 sgrid((unsigned)((uint64_t)pl.units * wpb)), fgrid((unsigned)((uint64_t)pl.units * pl.G)), block(kNT);
    hipError_t e = hipSuccess;
#define CA_DEC(T, D, G)                                                                               \
    do {                                                                                              \
        const T *qt = static_cast<const T *>(q), *kt = static_cast<const T *>(k), *vt = static_cast<const T *>(v); \
        if (mass) hipLaunchKernelGGL((decode_stream_kernel<T, D, G, true>), sgrid, block, 0, s, qt, kt, a); \
        else hipLaunchKernelGGL((decode_stream_kernel<T, D, G, false>), sgrid, block, 0, s, qt, kt, a); \
        e = hipGetLastError();                                                                        \
        if (e != hipSuccess) return e;                                                                \
        if (mass) hipLaunchKernelGGL((decode_finish_kernel<T, D, G, true, true>), fgrid, block, 0, s, qt, kt, vt, a); \
        else if (attend) hipLaunchKernelGGL((decode_finish_kernel<T, D, G, true, false>), fgrid, block, 0, s, qt, kt, vt, a); \
        else hipLaunchKernelGGL((decode_finish_kernel<T, D, G, false, false>), fgrid, block, 0, s, qt, kt, vt, a); \
    } while (0)
#define CA_DEC_G(T, D)                                  \
    do {                                                \
        if (pl.G == 4) CA_DEC(T, D, 4);                 \
        else if (pl.G == 2) CA_DEC(T, D, 2);            \
        else CA_DEC(T, D, 1);                           \
    } while (0)
    if (pl.dtype == 1) {
        if (pl.d == 128) CA_DEC_G(__bf16, 128); else CA_DEC_G(__bf16, 64);
    } else {
        if (pl.d == 128) CA_DEC_G(float, 128); else CA_DEC_G(float, 64);
    }
#undef CA_DEC_G
#undef CA_DEC
    (void)e;
    return hipGetLastError();
}

}  // namespace ca
