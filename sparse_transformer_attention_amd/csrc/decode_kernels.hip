// Condensate attention for decode-shaped problems on gfx950, in one kernel (pages of "The
// Condensate Theorem", metaphor-xennon blog: section 2.1 Definition 1,
// C_i = {0} u {i-W+1..i} u Top-k_i; section 2.2.3, the top-k part over R_i = {1..i-W};
// section 2.3, the softmax restricted to C_i times V).
//
// Work unit: (batch, KV head, query group) with up to G query vectors reading one KV head. The
// grid holds one finisher workgroup per unit (first in the grid, so they start at once) and then,
// per unit, wpb stream workgroups of two blocks of 256 key rows each:
//   stream    every K row is read once (16-byte non-temporal loads, LPR lanes per row) and
//             dotted with the unit's G queries in fp32 (row_key); the order-preserving 32-bit
//             keys (0 for rows outside R_i of a query) are staged in LDS;
//   record    per block and query, 16 lanes reduce the block's keys to a record: four of its
//             rows (key, offset) and a key X that every other row of the block stays at or
//             below (with the mass diagnostic also the block's sum of exp2((s - m_b) * scale)
//             relative to its largest score m_b). The record's words are stored with
//             agent-scope relaxed stores (coherent across the XCDs' L2 caches, no cache
//             maintenance); once they have completed, a last word carries the call's tag.
//   finisher  computes the anchor-and-window softmax partials of the unit's query vectors, then
//             takes the records as they land (one wavefront per query vector, 64 blocks at a
//             time, polling their tags): it admits the record rows whose ranking key
//             (score_key << 32) | ~position reaches the query's running threshold and, whenever
//             its list holds more than k' keys, cuts it to its exact top k' (wave_keep_top_u64),
//             the k'-th kept key becoming the threshold (k' distinct rows reach it, so no row
//             below it can be in the top k'). A block whose X reaches the threshold when the
//             last record is in has rows beyond its record that may rank: those are scored again
//             (row_key, the same bits). What remains is the exact top-k' (ties toward the smaller
//             position): C_i goes to out_idx, and the restricted softmax is the window partial
//             merged with the top-k rows' V times exp2((s - m) * scale), s read back from the
//             keys. Too many such blocks (dense clusters of high scores, exact ties) switch a
//             query to an exact fallback: all its candidate rows scored into scratch keys and a
//             workgroup radix select over them.
// Tags: each unit has a 64-bit epoch word in the workspace header. Every workgroup of the unit
// reads it when it starts and tags its records with epoch + 1; the finisher advances the word to
// that tag once every record of the unit carries it (so every workgroup has read the word
// before it changes). Records left by earlier calls carry older tags, so the workspace needs no
// clearing and a replayed launch (graph) starts a fresh epoch by itself.
// Stream workgroups never wait for another workgroup; the finisher waits only for records of
// workgroups dispatched after it, which never wait, with a bounded poll.
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
constexpr int kNT = kBW * 256;     // threads per workgroup
constexpr int kWaves = kNT / 64;
constexpr int kCand = 512;         // running candidate keys per query held in LDS
constexpr int kDef = 128;          // blocks per query whose X reached the threshold, held in LDS
constexpr int kResc = 8;           // blocks per query scored again on the common path
constexpr int kSelMax = 256;       // largest k' of the common path (larger: the fallback)
constexpr int kRecWords = 4;       // 64-bit words per record
constexpr uint64_t kPollTicks = 200000000ull;  // finisher poll limit: 2 s of s_memrealtime

struct DecodeArgs {
    int64_t n, nq;
    int Hq, Hkv, g, W, topk, cap;
    int64_t groups;     // units per (batch, KV head)
    int nblk;           // blocks of 256 rows per unit (rows 0 .. 256 nblk - 1)
    uint32_t nvec;      // query vectors per KV head (g * nq)
    int row_base;       // n - nq - W: last candidate row of vector idx is row_base + idx / g
    uint32_t wpb;       // stream workgroups per unit
    uint32_t units;     // finisher workgroups at the start of the grid
    float scale_log2e;
    int64_t rstride;    // scratch keys per query (256 nblk)
    uint64_t *epoch;    // [units] epoch words (workspace header)
    uint64_t *rec;      // [units][G][nblk][4] records: (k1 | k2 << 32), (k3 | k4 << 32),
                        // (offsets o1..o4, 8 bits each | X << 32), tag
    float2 *zs;         // [units][G][nblk] mass diagnostic: (m_b, l_b), stored before the tag
    uint32_t *scratch;  // [units][G][rstride] fallback keys
    int32_t *out_idx;   // [nqv][cap]
    float *out;         // [nqv][D] (null: select only)
    float *mass;        // [nqv][4] (null: no diagnostic)
};

// ---- agent-scope relaxed accesses: coherent across the XCDs without cache maintenance ----
__device__ __forceinline__ void st_agent(uint64_t *p, uint64_t x) {
    __hip_atomic_store(p, x, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint64_t ld_agent(const uint64_t *p) {
    return __hip_atomic_load(const_cast<uint64_t *>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// The tag of a call whose unit epoch word reads e (never 0).
__device__ __forceinline__ uint64_t tag_after(uint64_t e) { return e + 1 == 0 ? 1 : e + 1; }

// ---- reductions over the 16 lanes of a DPP row (every lane gets the result) ----
template <int N>
__device__ __forceinline__ uint32_t ror_u32(uint32_t x) { return dpp_u32<0x120 + N>(x, x); }

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

// Window partial of one query vector: largest score, weight sum, anchor score, weighted V rows.
template <int D>
struct WinPartial {
    float m, l, s0, pad;
    float acc[D];
};

template <int D, int G>
struct DecShared {
    union {
        uint32_t kst[G][kBW * kRows];     // stream: keys of the workgroup's rows, per query
        struct {
            uint64_t cand[G][kCand];      // running candidates (ranking keys); then the top k'
            union {
                struct {
                    uint64_t def[G][kDef];     // blocks whose X reached the threshold: X << 32 | blk
                    int32_t spos[G][kSelMax];  // selected positions, ascending
                    uint32_t skey[G][kSelMax]; // and their score keys
                } q;
                struct {
                    int32_t js[2 * 512];       // fallback: selected positions
                    SelectShared<kNT> ssh;     // fallback: radix select
                } fb;
            } x;
            SoftmaxPartials<D, kWaves> part;  // window partials, then top-k partials
        } fin;
    } u;
    WinPartial<D> win[G];
    uint64_t thr[G];
    int ndef[G], flag[G], ncand[G];
    int timeout;
};

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

// ---- stream workgroup: keys of two blocks into LDS, then the block records ------------------
template <typename T, int D, int G, bool MASS>
__device__ __forceinline__ void stream_phase(const T *__restrict__ q, const T *__restrict__ k,
                                             const DecodeArgs &a, uint32_t uu, uint32_t part,
                                             DecShared<D, G> &sh) {
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
                    *reinterpret_cast<uint4 *>(&sh.u.kst[my_t][tile0 - wg_row0 + 4 * (lane / LPR)]) =
                        make_uint4(kv4[0], kv4[1], kv4[2], kv4[3]);
            }
        }
    } else {
        for (int x = lane; x < G * 16; x += 64)
            *reinterpret_cast<uint4 *>(&sh.u.kst[x / 16][wrow0 - wg_row0 + 4 * (x % 16)]) = make_uint4(0, 0, 0, 0);
    }
    __syncthreads();
    // Records: 16 lanes per (block, query); lane j takes staged positions 16j .. 16j + 15. The
    // wavefronts without a record to write are done.
    const int nbw = a.nblk - wg_row0 / kRows < kBW ? a.nblk - wg_row0 / kRows : kBW;
    if (wave * 4 >= nbw * G) return;
    const int pr = tid >> 4, j = tid & 15;
    if (pr >= nbw * G) return;
    // The call's tag (read before this workgroup's records exist, so before the finisher can
    // advance the epoch word).
    const uint64_t tag = tag_after(ld_agent(a.epoch + uu));
    const int b2 = pr / G, t = pr % G;
    const uint32_t *src = &sh.u.kst[t][b2 * kRows + 16 * j];
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
    const size_t rq = ((size_t)uu * G + t) * (size_t)a.nblk + blk;
    uint64_t *rec = a.rec + rq * kRecWords;
    if (j == 0) {
        uint32_t offs = 0u;
#pragma unroll
        for (int r = 0; r < 4; ++r) offs |= (255u - (uint32_t)(e[r] & 255u)) << (8 * r);
        st_agent(rec, (uint64_t)k1 | ((e[1] >> 8) << 32));
        st_agent(rec + 1, (e[2] >> 8) | ((e[3] >> 8) << 32));
        st_agent(rec + 2, (uint64_t)offs | ((uint64_t)X << 32));
        if constexpr (MASS)
            st_agent(reinterpret_cast<uint64_t *>(a.zs + rq),
                     (uint64_t)__float_as_uint(zm) | ((uint64_t)__float_as_uint(zl) << 32));
    }
    // The record's words have completed before its tag is stored.
    __builtin_amdgcn_s_waitcnt(0);
    if (j == 0) st_agent(rec + 3, tag);
}

// ---- finisher, window partials (all threads): the anchor and the window of each query -------
template <typename T, int D, int G, bool MASS>
__device__ __forceinline__ void window_partials(const T *__restrict__ q, const T *__restrict__ k,
                                                const T *__restrict__ v, const DecodeArgs &a, uint32_t uu,
                                                DecShared<D, G> &sh) {
    using AS = AttendShape<D, T>;
    constexpr int NW = kWaves / G;  // wavefronts per query vector
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const uint32_t ng = (uint32_t)a.groups;
    const uint32_t bk = uu / ng, grp = uu - bk * ng;
    const int t = wave / NW, wv = wave % NW;
    const QInfo qi = query_info<G>(a, bk, grp, t);
    const size_t kv0 = (size_t)bk * (size_t)a.n * D;
    const T *kb = k + kv0, *vb = v + kv0;
    const uint4 qs = reinterpret_cast<const uint4 *>(q + (size_t)qi.qv * D)[lane % AS::LPR];
    auto row_at = [&](int c) -> size_t { return c < qi.base ? 0 : (size_t)(qi.wlo - qi.base + c); };
    wave_partial<D, T, 5>(qs, kb, vb, row_at, qi.base + qi.wcount, wv, NW, a.scale_log2e, sh.u.fin.part, wave);
    float s0 = 0.f;
    if constexpr (MASS) {
        const uint4 k0 = reinterpret_cast<const uint4 *>(kb)[lane % AS::LPR];
        s0 = row_sum<AS::LPR>(dot16(k0, qs, 0.f, T()));
    }
    __syncthreads();
    if (wv == 0) {
        float mx = -INFINITY;
#pragma unroll
        for (int p = 0; p < NW; ++p) mx = fmaxf(mx, sh.u.fin.part.m[t * NW + p]);
        float f[NW], l = 0.f;
#pragma unroll
        for (int p = 0; p < NW; ++p) {
            const float mp = sh.u.fin.part.m[t * NW + p];
            f[p] = mp == -INFINITY ? 0.f : exp2f((mp - mx) * a.scale_log2e);
            l += f[p] * sh.u.fin.part.l[t * NW + p];
        }
        for (int col = lane; col < D; col += 64) {
            float acc = 0.f;
#pragma unroll
            for (int p = 0; p < NW; ++p) acc = fmaf(f[p], sh.u.fin.part.acc[t * NW + p][col], acc);
            sh.win[t].acc[col] = acc;
        }
        if (lane == 0) {
            sh.win[t].m = mx;
            sh.win[t].l = l;
            sh.win[t].s0 = s0;
        }
    }
    __syncthreads();
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

// ---- finisher, records of query t as they land (one wavefront) ------------------------------
// Keeps in LDS the running candidates (ranking keys that reach the threshold) and the blocks whose
// X reaches it; cuts the list to its exact top k' whenever it holds more. Mass diagnostic: the
// blocks' (m_b, l_b) merged per lane into (*zm, *zl).
template <typename T, int D, int G, bool MASS>
__device__ __forceinline__ void take_records(const DecodeArgs &a, uint32_t uu, int t, uint64_t tag,
                                             uint64_t t_start, DecShared<D, G> &sh, float *zm, float *zl) {
    const int lane = threadIdx.x & 63;
    const uint32_t ng = (uint32_t)a.groups;
    const uint32_t bk = uu / ng, grp = uu - bk * ng;
    const QInfo qi = query_info<G>(a, bk, grp, t);
    const size_t rq0 = ((size_t)uu * G + t) * (size_t)a.nblk;
    const uint64_t *R = a.rec + rq0 * kRecWords;
    const float2 *Z = a.zs + rq0;
    uint64_t *cand = sh.u.fin.cand[t];
    uint64_t *def = sh.u.fin.x.q.def[t];
    const int kp = qi.kp;
    // Any candidate key (>= 1) reaches the starting threshold.
    uint64_t thr = 1ull << 32;
    int n = 0, ndef = 0;
    bool timed_out = false;
    float ml = -INFINITY, ll = 0.f;
    auto append = [&](bool ok, uint64_t key) {
        const uint64_t bal = __ballot(ok);
        const int pos = n + lanes_below(bal);
        if (ok && pos < kCand) cand[pos] = key;
        n += __popcll(bal);
    };
    auto defer = [&](bool ok, uint64_t entry) {
        const uint64_t bal = __ballot(ok);
        const int pos = ndef + lanes_below(bal);
        if (ok && pos < kDef) def[pos] = entry;
        ndef += __popcll(bal);
    };
    // Exact top-kp of the list; the threshold becomes its kp-th key; blocks whose X fell below
    // the threshold's score key leave the deferred list.
    auto cut = [&]() {
        if (n > kp && n <= kCand) {
            thr = n <= 128 ? keep_top<2>(cand, n, kp) : keep_top<8>(cand, n, kp);
            n = kp;
        }
        if (ndef > 0 && ndef <= kDef) {
            const uint32_t thi = (uint32_t)(thr >> 32);
            uint64_t d[2];
#pragma unroll
            for (int e = 0; e < 2; ++e) {
                const int c = lane + 64 * e;
                d[e] = c < ndef ? def[c] : 0ull;
            }
            wave_sync();
            ndef = 0;
#pragma unroll
            for (int e = 0; e < 2; ++e) defer(d[e] != 0ull && (uint32_t)(d[e] >> 32) >= thi, d[e]);
            wave_sync();
        }
    };
    for (int b0 = 0; b0 < a.nblk; b0 += 64) {
        const int blk = b0 + lane;
        bool pend = blk < a.nblk;
        for (;;) {
            const uint64_t *rb = R + (size_t)(pend ? blk : 0) * kRecWords;
            const uint64_t tg = pend ? ld_agent(rb + 3) : 0ull;
            const bool ready = pend && tg == tag;
            uint64_t r0 = 0ull, r1 = 0ull, r2 = 0ull, zz = 0ull;
            if (ready) {
                // (Issued after the tag compared equal: the record's words completed before it.)
                asm volatile("" ::: "memory");
                r0 = ld_agent(rb);
                r1 = ld_agent(rb + 1);
                r2 = ld_agent(rb + 2);
                if constexpr (MASS) zz = ld_agent(reinterpret_cast<const uint64_t *>(Z + blk));
            }
            const bool have = ready && blk < qi.nbq && kp > 0;
            const uint32_t X = (uint32_t)(r2 >> 32), offs = (uint32_t)r2;
            const uint32_t ks[4] = {(uint32_t)r0, (uint32_t)(r0 >> 32), (uint32_t)r1, (uint32_t)(r1 >> 32)};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const uint64_t key = make_rank_key(ks[e], (uint32_t)blk * kRows + ((offs >> (8 * e)) & 255u));
                append(have && ks[e] != 0u && key >= thr, key);
            }
            // X >= the threshold's score key: rows beyond the record may rank.
            defer(have && X != 0u && X >= (uint32_t)(thr >> 32), ((uint64_t)X << 32) | (uint32_t)blk);
            if constexpr (MASS) {
                if (ready && blk < qi.nbq) {
                    const float bm = __uint_as_float((uint32_t)zz), bl = __uint_as_float((uint32_t)(zz >> 32));
                    if (bm != -INFINITY) {
                        const float mn = fmaxf(ml, bm);
                        ll = (ml == -INFINITY ? 0.f : ll * exp2f((ml - mn) * a.scale_log2e)) +
                             bl * exp2f((bm - mn) * a.scale_log2e);
                        ml = mn;
                    }
                }
            }
            pend = pend && !ready;
            if (__ballot(pend) == 0ull) break;
            if (__builtin_amdgcn_s_memrealtime() - t_start > kPollTicks) {
                timed_out = true;
                break;
            }
            __builtin_amdgcn_s_sleep(2);
        }
        if (timed_out) break;
        wave_sync();
        // Cut early (the threshold then rises above most blocks' X) and whenever another batch
        // of 64 records might not fit.
        if (n > 2 * kp || n > kCand - 256 || ndef > 32) cut();
    }
    wave_sync();
    cut();
    if (lane == 0) {
        sh.thr[t] = thr;
        sh.ndef[t] = ndef;
        sh.ncand[t] = n;
        sh.flag[t] = timed_out ? 2 : (ndef > kResc || n > kCand || kp > kSelMax) ? 1 : 0;
        if (timed_out) sh.timeout = 1;
    }
    *zm = ml;
    *zl = ll;
}

// ---- finisher: blocks whose rows beyond their record may rank, scored again (one wavefront) --
template <typename T, int D, int G>
__device__ __forceinline__ void rescore_deferred(const T *__restrict__ q, const T *__restrict__ k,
                                                 const DecodeArgs &a, uint32_t uu, int t,
                                                 DecShared<D, G> &sh) {
    using S = StreamShape<T, D>;
    constexpr int LPR = S::LPR, RPG = S::RPG, P = S::P;
    const int lane = threadIdx.x & 63;
    const uint32_t ng = (uint32_t)a.groups;
    const uint32_t bk = uu / ng, grp = uu - bk * ng;
    const QInfo qi = query_info<G>(a, bk, grp, t);
    const int ndef = sh.ndef[t];
    if (!qi.valid || qi.kp == 0 || ndef == 0 || sh.flag[t]) return;
    const uint64_t thr = sh.thr[t];
    uint64_t *cand = sh.u.fin.cand[t];
    int n = sh.ncand[t];
    const size_t rq0 = ((size_t)uu * G + t) * (size_t)a.nblk;
    uint4 qr[G][P];
    load_query_slices<T, D, G>(q, a, bk, grp, lane, qr);
    const uint4 *kbase = reinterpret_cast<const uint4 *>(k + (int64_t)bk * a.n * D);
    const int sl = lane % LPR;
    const bool mine = sl % (LPR / G) == 0 && sl / (LPR / G) == t;
    for (int x = 0; x < ndef; ++x) {
        const int blk = (int)(uint32_t)sh.u.fin.x.q.def[t][x];
        // The record's rows are in the list already (when they reach the threshold).
        const uint32_t offs = (uint32_t)ld_agent(a.rec + (rq0 + blk) * kRecWords + 2);
        for (int r0 = 0; r0 < kRows; r0 += 4 * RPG) {
            uint4 kr[4][P];
#pragma unroll
            for (int uq = 0; uq < 4; ++uq) {
                int row = blk * kRows + r0 + uq * RPG + lane / LPR;
                row = row <= qi.rl ? row : qi.rl;
                const uint4 *src = kbase + (int64_t)row * (P * LPR);
#pragma unroll
                for (int p = 0; p < P; ++p) kr[uq][p] = src[p * LPR + sl];
            }
#pragma unroll
            for (int uq = 0; uq < 4; ++uq) {
                const uint32_t key = row_key<T, LPR, P, G>(kr[uq], qr, lane);
                const int off = r0 + uq * RPG + lane / LPR;
                const int row = blk * kRows + off;
                const bool in_rec = ((offs & 255u) == (uint32_t)off) || (((offs >> 8) & 255u) == (uint32_t)off) ||
                                    (((offs >> 16) & 255u) == (uint32_t)off) || ((offs >> 24) == (uint32_t)off);
                const uint64_t rk = make_rank_key(key, (uint32_t)row);
                const bool ok = mine && !in_rec && row >= 1 && row <= qi.rl && key != 0u && rk >= thr;
                const uint64_t bal = __ballot(ok);
                const int pos = n + lanes_below(bal);
                if (ok && pos < kCand) cand[pos] = rk;
                n += __popcll(bal);
            }
        }
    }
    wave_sync();
    if (n > kCand) {
        if (lane == 0) sh.flag[t] = 1;
        return;
    }
    if (n > qi.kp) {
        (void)(n <= 128 ? keep_top<2>(cand, n, qi.kp) : keep_top<8>(cand, n, qi.kp));
        n = qi.kp;
    }
    if (lane == 0) sh.ncand[t] = n;
}

// ---- finisher, exact fallback for query t (all threads) -------------------------------------
// Every candidate row of the query scored into its scratch keys, then the workgroup radix select
// over the ranking keys that reach the threshold. Leaves the top-k' in cand[t][0..k').
template <typename T, int D, int G>
__device__ __forceinline__ void final_fallback(const T *__restrict__ q, const T *__restrict__ k,
                                               const DecodeArgs &a, uint32_t uu, int t,
                                               DecShared<D, G> &sh) {
    using S = StreamShape<T, D>;
    constexpr int LPR = S::LPR, RPG = S::RPG, P = S::P;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const uint32_t ng = (uint32_t)a.groups;
    const uint32_t bk = uu / ng, grp = uu - bk * ng;
    const QInfo qi = query_info<G>(a, bk, grp, t);
    const uint64_t thr = sh.thr[t];
    uint32_t *sc = a.scratch + ((size_t)uu * G + t) * (size_t)a.rstride;
    uint4 qr[G][P];
    load_query_slices<T, D, G>(q, a, bk, grp, lane, qr);
    const uint4 *kbase = reinterpret_cast<const uint4 *>(k + (int64_t)bk * a.n * D);
    const int sl = lane % LPR;
    const bool mine = sl % (LPR / G) == 0 && sl / (LPR / G) == t;
    const int rows = qi.nbq * kRows;
    for (int r0 = wave * RPG; r0 < rows; r0 += kWaves * RPG) {
        const int row = r0 + lane / LPR;
        const int lrow = row <= qi.rl ? row : qi.rl;
        const uint4 *src = kbase + (int64_t)lrow * (P * LPR);
        uint4 kr[P];
#pragma unroll
        for (int p = 0; p < P; ++p) kr[p] = src[p * LPR + sl];
        const uint32_t key = row_key<T, LPR, P, G>(kr, qr, lane);
        if (mine) sc[row] = (row >= 1 && row <= qi.rl) ? key : 0u;
    }
    __threadfence_block();
    __syncthreads();
    auto key_at = [&](int64_t f64) -> uint64_t {
        const int f = (int)f64;
        const uint32_t kv = sc[f];
        const uint64_t rk = make_rank_key(kv, (uint32_t)f);
        return kv != 0u && rk >= thr ? rk : 0ull;
    };
    select_exact<kNT>(kGather + 1, (int64_t)rows, key_at, qi.kp, sh.u.fin.x.fb.js, nullptr, nullptr, sh.u.fin.x.fb.ssh);
    // The top-k' as ranking keys (js holds their positions, ascending).
    for (int c = tid; c < qi.kp; c += kNT) {
        const int32_t pos = sh.u.fin.x.fb.js[c];
        sh.u.fin.cand[t][c] = make_rank_key(sc[pos], (uint32_t)pos);
    }
    if (tid == 0) sh.ncand[t] = qi.kp;
    __syncthreads();
}

// ---- finisher: the top-k' of query t in ascending position order, and out_idx (one wavefront)
template <int D, int G>
__device__ __forceinline__ void write_set(const DecodeArgs &a, const QInfo &qi, int t, DecShared<D, G> &sh) {
    const int lane = threadIdx.x & 63;
    const int kp = sh.timeout ? 0 : qi.kp;
    const uint64_t *cand = sh.u.fin.cand[t];
    // Each selected position's rank among the selected ones (8 keys per LDS round).
    const int kp8 = (kp + 7) & ~7;
    for (int c0 = 0; c0 < kp; c0 += 64) {
        const int c = c0 + lane;
        const uint64_t key = c < kp ? cand[c] : 0ull;
        const uint32_t pos = (uint32_t)rank_key_pos(key);
        int rank = 0;
        for (int f0 = 0; f0 < kp8; f0 += 8) {
            uint64_t y[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) y[e] = f0 + e < kp ? cand[f0 + e] : 0ull;
#pragma unroll
            for (int e = 0; e < 8; ++e) rank += (f0 + e < kp) && (uint32_t)rank_key_pos(y[e]) < pos;
        }
        if (c < kp) {
            sh.u.fin.x.q.spos[t][rank] = (int32_t)pos;
            sh.u.fin.x.q.skey[t][rank] = (uint32_t)(key >> 32);
        }
    }
    wave_sync();
    int32_t *row = a.out_idx + (size_t)qi.qv * a.cap;
    for (int c = lane; c < a.cap; c += 64) {
        int32_t val = -1;
        if (c < qi.base) val = 0;
        else if (c < qi.base + kp) val = sh.u.fin.x.q.spos[t][c - qi.base];
        else if (c < qi.base + kp + qi.wcount) val = qi.wlo + (c - qi.base - kp);
        row[c] = val;
    }
}

// ---- finisher: partial over the top-k rows of query t, wavefront part p of np ---------------
template <typename T, int D, int G>
__device__ __forceinline__ void topk_partial(const T *__restrict__ v, const DecodeArgs &a, uint32_t bk,
                                             const QInfo &qi, int t, int p, int np, DecShared<D, G> &sh,
                                             int slot_out) {
    using AS = AttendShape<D, T>;
    const int lane = threadIdx.x & 63;
    const int kp = (qi.valid && !sh.timeout) ? qi.kp : 0;
    const T *vb = v + (size_t)bk * (size_t)a.n * D;
    const uint32_t last_row = (uint32_t)(a.n - 1);
    const int cs = lane % AS::LPR, slot = lane / AS::LPR;
    float acc[AS::EPL];
#pragma unroll
    for (int e = 0; e < AS::EPL; ++e) acc[e] = 0.f;
    float l = 0.f;
    // The largest selected score: every weight is exp2((s - m) * scale) <= 1.
    uint32_t kmax = 0u;
    for (int c = lane; c < kp; c += 64) kmax = sh.u.fin.x.q.skey[t][c] > kmax ? sh.u.fin.x.q.skey[t][c] : kmax;
    const float m = kp > 0 ? key_score(wave_max_u32_dpp(kmax)) : -INFINITY;
    constexpr int UT = 8;  // rows per lane in flight
    const int step = np * AS::RPW;
    for (int c0 = p * AS::RPW; c0 < kp; c0 += UT * step) {
        uint4 vv[UT];
        float s[UT];
#pragma unroll
        for (int uq = 0; uq < UT; ++uq) {
            int c = c0 + uq * step + slot;
            c = c < kp ? c : kp - 1;
            uint32_t pos = (uint32_t)sh.u.fin.x.q.spos[t][c];
            pos = pos < last_row ? pos : last_row;
            vv[uq] = reinterpret_cast<const uint4 *>(vb + (size_t)pos * D)[cs];
            s[uq] = key_score(sh.u.fin.x.q.skey[t][c]);
        }
#pragma unroll
        for (int uq = 0; uq < UT; ++uq) {
            if (c0 + uq * step + slot < kp) {
                const float w = exp2f((s[uq] - m) * a.scale_log2e);
                l += w;
                accumulate16(acc, vv[uq], w, T());
            }
        }
    }
    // Sum over the row slots (lanes LPR apart).
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
    if (lane < AS::LPR) {
#pragma unroll
        for (int e = 0; e < AS::EPL; ++e) sh.u.fin.part.acc[slot_out][cs * AS::EPL + e] = acc[e];
    }
    if (lane == 0) {
        sh.u.fin.part.m[slot_out] = m;
        sh.u.fin.part.l[slot_out] = l;
    }
}

// ---- finisher workgroup ---------------------------------------------------------------------
template <typename T, int D, int G, bool ATTEND, bool MASS>
__device__ __forceinline__ void finisher(const T *__restrict__ q, const T *__restrict__ k,
                                         const T *__restrict__ v, const DecodeArgs &a, uint32_t uu,
                                         DecShared<D, G> &sh) {
    constexpr int NP = kWaves / G;  // wavefronts per query vector in the attend part
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const uint64_t t_start = __builtin_amdgcn_s_memrealtime();
    const uint64_t tag = tag_after(ld_agent(a.epoch + uu));
    const uint32_t ng = (uint32_t)a.groups;
    const uint32_t bk = uu / ng, grp = uu - bk * ng;
    if (tid == 0) sh.timeout = 0;
    if constexpr (ATTEND) window_partials<T, D, G, MASS>(q, k, v, a, uu, sh);
    else __syncthreads();
    // Records as they land; query 0 (always a valid vector) waits for every one of the unit's.
    float zm = -INFINITY, zl = 0.f;
    if (wave < G) {
        const QInfo qi = query_info<G>(a, bk, grp, wave);
        if (qi.valid) {
            take_records<T, D, G, MASS>(a, uu, wave, tag, t_start, sh, &zm, &zl);
            rescore_deferred<T, D, G>(q, k, a, uu, wave, sh);
        } else if (lane == 0) {
            sh.flag[wave] = 0;
            sh.ncand[wave] = 0;
        }
    }
    __syncthreads();
    for (int t = 0; t < G; ++t) {
        const QInfo qi = query_info<G>(a, bk, grp, t);
        if (qi.valid && qi.kp > 0 && sh.flag[t] && !sh.timeout) final_fallback<T, D, G>(q, k, a, uu, t, sh);
    }
    if (wave < G) {
        const QInfo qi = query_info<G>(a, bk, grp, wave);
        if (qi.valid) write_set<D, G>(a, qi, wave, sh);
    }
    if constexpr (ATTEND) {
        // (LDS-only barriers: the index rows' stores need not complete first.)
        lds_barrier();
        {
            const int t = wave % G, p = wave / G;
            const QInfo qi = query_info<G>(a, bk, grp, t);
            topk_partial<T, D, G>(v, a, bk, qi, t, p, NP, sh, wave);
        }
        lds_barrier();
        if (wave < G) {
            const int t = wave;
            const QInfo qi = query_info<G>(a, bk, grp, t);
            if (qi.valid) {
                using AS = AttendShape<D, T>;
                // Window partial and the NP top-k partials (slots t, t + G, ...), in that order.
                float mt = -INFINITY;
#pragma unroll
                for (int p = 0; p < NP; ++p) mt = fmaxf(mt, sh.u.fin.part.m[t + G * p]);
                const float mw = sh.win[t].m;
                const float mg = fmaxf(mw, mt);
                const float fw = mw == -INFINITY ? 0.f : exp2f((mw - mg) * a.scale_log2e);
                float f[NP], L = fw * sh.win[t].l, lt = 0.f;
#pragma unroll
                for (int p = 0; p < NP; ++p) {
                    const float mp = sh.u.fin.part.m[t + G * p];
                    f[p] = mp == -INFINITY ? 0.f : exp2f((mp - mg) * a.scale_log2e);
                    L += f[p] * sh.u.fin.part.l[t + G * p];
                    lt += mp == -INFINITY ? 0.f : exp2f((mp - mt) * a.scale_log2e) * sh.u.fin.part.l[t + G * p];
                }
                const float inv = 1.f / L;
                float *o = a.out + (size_t)qi.qv * D;
                for (int col = lane; col < D; col += 64) {
                    float x = fw * sh.win[t].acc[col];
#pragma unroll
                    for (int p = 0; p < NP; ++p) x = fmaf(f[p], sh.u.fin.part.acc[t + G * p][col], x);
                    o[col] = sh.timeout ? __builtin_nanf("") : x * inv;
                }
                (void)AS::LPR;
                if constexpr (MASS) {
                    // Mass diagnostic (section 3.2.2, the full-softmax mass outside C_i; sections
                    // 2.2.1-2.2.3, the parts of C_i): the candidates' part from the blocks' sums,
                    // the window part (with row 0) and the top-k part from the partials, row 0
                    // from its score; all relative to one maximum.
                    const float mr = wave_max_f32_dpp(zm);
                    const float lr = wave_sum_f32_dpp(zm == -INFINITY ? 0.f : zl * exp2f((zm - mr) * a.scale_log2e));
                    const float lw = sh.win[t].l, s0 = sh.win[t].s0;
                    const float mgm = fmaxf(mr, mw);
                    auto rel = [&](float mx, float sm) {
                        return mx == -INFINITY ? 0.f : sm * exp2f((mx - mgm) * a.scale_log2e);
                    };
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
    // Every record of the unit carries the tag (query 0 waited for each): every workgroup has read
    // the epoch word; the next call's tag follows this one.
    if (tid == 0 && !sh.timeout) st_agent(a.epoch + uu, tag);
}

template <typename T, int D, int G, bool ATTEND, bool MASS>
__global__ __launch_bounds__(kNT) __attribute__((amdgpu_waves_per_eu(sizeof(T) == 2 ? 5 : 4))) void decode_kernel(
    const T *__restrict__ q, const T *__restrict__ k, const T *__restrict__ v, DecodeArgs a) {
    __shared__ DecShared<D, G> sh;
    if (blockIdx.x < a.units) {
        finisher<T, D, G, ATTEND, MASS>(q, k, v, a, blockIdx.x, sh);
    } else {
        const uint32_t s = blockIdx.x - a.units;
        const uint32_t uu = s / a.wpb;
        stream_phase<T, D, G, MASS>(q, k, a, uu, s - uu * a.wpb, sh);
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
    a.wpb = (uint32_t)((pl.nblk + kBW - 1) / kBW);
    a.units = (uint32_t)pl.units;
    a.scale_log2e = (float)(1.4426950408889634 / __builtin_sqrt((double)pl.d));
    a.rstride = pl.rstride;
    char *w = static_cast<char *>(ws);
    a.epoch = reinterpret_cast<uint64_t *>(w);
    a.rec = reinterpret_cast<uint64_t *>(w + pl.summ_offset);
    a.zs = reinterpret_cast<float2 *>(w + pl.zsum_offset);
    a.scratch = reinterpret_cast<uint32_t *>(w + pl.scratch_offset);
    a.out_idx = out_idx;
    a.out = out;
    a.mass = mass;
    const bool attend = out != nullptr;
    const dim3 grid((unsigned)((uint64_t)pl.units * (a.wpb + 1))), block(kNT);
#define CA_DEC(T, D, G)                                                                               \
    do {                                                                                              \
        const T *qt = static_cast<const T *>(q), *kt = static_cast<const T *>(k), *vt = static_cast<const T *>(v); \
        if (mass) hipLaunchKernelGGL((decode_kernel<T, D, G, true, true>), grid, block, 0, s, qt, kt, vt, a); \
        else if (attend) hipLaunchKernelGGL((decode_kernel<T, D, G, true, false>), grid, block, 0, s, qt, kt, vt, a); \
        else hipLaunchKernelGGL((decode_kernel<T, D, G, false, false>), grid, block, 0, s, qt, kt, vt, a); \
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
    return hipGetLastError();
}

}  // namespace ca
