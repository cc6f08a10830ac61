// The end of the condensate-attention path on gfx950, one workgroup per query vector:
//   merge    exact top-k' of the query's candidates (ranking keys (score_key << 32) | ~position;
//            k' = min(k, |R_i|)): from the segments score_topk left, or from the key buffer of
//            score_keys, reading only the tiles whose best key reaches the query's bound;
//   assemble C_i = {0} u top-k' u {i-W+1..i} in ascending order, written to out_idx (pages of
//            "The Condensate Theorem", metaphor-xennon blog, section 2.1 Definition 1);
//   attend   (optional) the restricted softmax times V on that set, straight from LDS.
// Plus the standalone attend kernel for caller-supplied sets (flash_attention_on_subset of the
// section 5.2.2 sketch).
#include <type_traits>

#include "attend_core.h"
#include "ca_internal.h"
#include "device_utils.h"
#include "merge_core.h"
#include "score_core.h"
#include "select_core.h"

namespace ca {
namespace {

struct FinishArgs {
    int64_t n, nq;
    int Hq, Hkv, g, W, topk, cap, wpu, seg;
    float scale_log2e;
    const uint32_t *cnt;    // [nqv][wpu] keys in each segment
    const uint64_t *lists;  // [nqv][wpu][seg] segments of candidate ranking keys
    // Tile-summary path (score_keys): units of G query vectors, blocks and tiles of key rows.
    int G, nblk, tile_shift;  // rows per tile: 1 << tile_shift
    int64_t groups, rstride;
    uint32_t nvec;            // query vectors per KV head (g * nq)
    const uint32_t *best1;    // [units][G][rstride / tile_rows]
    const uint2 *rest;        // second key; offsets of the best two (bits 0-15), third key's upper half
    const uint32_t *bmax;     // [units][nblk][G]
    uint32_t *scratch;        // [nqv][rstride]
    const float *win;         // [nqv][D + 2] anchor-and-window partials (MFMA path), or null
    // Mass diagnostic (tile-summary path; null: off): per-block sums of score_keys and the
    // output [nqv][4] = excluded mass, anchor, window without position 0, top-k.
    const float2 *zsum;
    float *mass;
};

// Exact top-kp of n distinct non-zero ranking keys in gathered[0..n) (kp <= n <= kRankSelectMax, n <= NT,
// so the tail of gathered[] holds a copy clear of them) by rank counting: a key is selected when
// fewer than kp keys beat it; the selected positions are then placed by their rank among the
// selected ones (ascending) in js[0..kp). S lanes per candidate (S*n <= NT, S <= 16): lane s
// compares against keys s, s+S, ..., and the S counts are summed. All threads; ends with an
// LDS barrier.
constexpr int kRankSelectMax = 256;
static_assert(2 * kRankSelectMax <= kGather && 2 * 128 <= kGatherFor<128>, "rank select room");
template <int NT>
__device__ __forceinline__ void select_by_rank(int n, int kp, uint64_t *gathered, int32_t *js) {
    const int tid = threadIdx.x;
    int lg = 4;
    while (lg > 0 && (n << lg) > NT) --lg;
    const int S = 1 << lg, c = tid >> lg, sl = tid & (S - 1);
    const bool mine = c < n;
    const uint64_t x = gathered[mine ? c : 0];
    int above = 0;
    if (mine) {
#pragma unroll 4
        for (int f = sl; f < n; f += S) above += gathered[f] > x;
    }
    for (int off = 1; off < S; off <<= 1) above += __shfl_xor(above, off);
    const bool chosen = mine && above < kp;
    // Selected keys (0 = not) in the tail of gathered[], clear of [0, n).
    if (mine && sl == 0) gathered[kGatherFor<NT> - 1 - c] = chosen ? x : 0ull;
    lds_barrier();
    const int32_t pos = rank_key_pos(x);
    int rank = 0;
    if (chosen) {
#pragma unroll 4
        for (int f = sl; f < n; f += S) {
            const uint64_t y = gathered[kGatherFor<NT> - 1 - f];
            rank += y != 0ull && rank_key_pos(y) < pos;
        }
    }
    for (int off = 1; off < S; off <<= 1) rank += __shfl_xor(rank, off);
    if (chosen && sl == 0) js[rank] = pos;
    lds_barrier();
}

// Candidates from the segments of score_topk or of the MFMA passes (the first cnt[w] keys of
// each segment w of lists[w][0..seg)), gathered into LDS by wavefront 0 while the other wavefronts run
// overlap(); then the exact top-kp.
template <int NT, typename Overlap>
__device__ __forceinline__ void select_segments(const uint32_t *__restrict__ cnt,
                                                const uint64_t *__restrict__ lists, int wpu,
                                                int topk, int kp, int32_t *js, uint64_t *sel,
                                                uint64_t *gathered, SelectShared<NT> &sh,
                                                Overlap overlap) {
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    if (wave == 0) {
        // Every slot of every segment, four per lane in flight with their segments' lengths,
        // kept when inside its segment's length (compacted by ballot).
        constexpr int GU = 4;
        const int slots = wpu * topk;
        int base = 0;
        for (int f0 = 0; f0 < slots; f0 += 64 * GU) {
            uint64_t x[GU];
            uint32_t c[GU];
#pragma unroll
            for (int u = 0; u < GU; ++u) {
                const int f = f0 + u * 64 + lane, fc = f < slots ? f : slots - 1;
                x[u] = lists[fc];
                c[u] = cnt[fc / topk];
            }
#pragma unroll
            for (int u = 0; u < GU; ++u) {
                const int f = f0 + u * 64 + lane;
                const bool ok = f < slots && (uint32_t)(f % topk) < c[u];
                const uint64_t bal = __ballot(ok);
                const int pos = base + lanes_below(bal);
                if (ok && pos < kGatherFor<NT>) gathered[pos] = x[u];
                base += __popcll(bal);
            }
        }
        if (lane == 0) sh.sel_count = base;
    } else {
        overlap();
    }
    __syncthreads();
    const int n = sh.sel_count;
    __syncthreads();
    if (n >= kp && n <= kRankSelectMax && n <= NT) {
        select_by_rank<NT>(n, kp, gathered, js);
        return;
    }
    auto key_at = [&](int64_t f) -> uint64_t {
        const int w = (int)(f / topk);
        const int e = (int)(f - (int64_t)w * topk);
        return e < (int)cnt[w] ? lists[f] : 0ull;
    };
    select_exact<NT>(n, (int64_t)wpu * topk, key_at, kp, js, sel, gathered, sh);
}

// Candidates from the tile summaries of score_keys. The query's bound thr is the lower edge of
// the 10-bit radix bin that holds the k'-th largest of its block maxima (or of its tile maxima when
// there are fewer than 2k' blocks): k' distinct rows reach it, so it is a lower bound of the
// query's k-th key. Every key that reaches thr lies in a tile whose best key reaches it; such a
// tile contributes its one or two best rows that reach thr, and, when its third key may reach
// thr too, all its rows, scored again by rescore (the same bits as score_keys). The candidates go to gathered[] as ranking keys;
// then the exact top-kp. best1/rest point at the query's tiles, bm at its first block
// maximum (stride G); its candidate rows are 1..rl. tiles is LDS for kTileCap tile indices,
// ovf for kOvfCap. When the candidates do not fit (ties at the bound), every passing tile is
// scored into scratch (the query's rows) and selected from there. The other wavefronts run
// overlap() while wavefront 0 takes the bound.
//
// rescore(ntl, tile_at, emit): scores every row of the tiles tile_at(0..ntl) (-1: none) for
// this query, calling emit(key, row) for each of its candidate rows. All threads.
constexpr int kTileCap = 1024;
constexpr int kOvfCap = 64;

template <int NT, typename Overlap, typename Rescore>
__device__ __forceinline__ void select_tiles(const uint32_t *__restrict__ best1,
                                             const uint2 *__restrict__ rest,
                                             const uint32_t *__restrict__ bm, int G, int nblk,
                                             int tile_shift, int rl, int kp, int32_t *js,
                                             uint64_t *sel, uint64_t *gathered, int32_t *tiles,
                                             int32_t *ovf, uint32_t *scratch,
                                             SelectShared<NT> &sh, Overlap overlap,
                                             Rescore rescore) {
    static_assert(NT >= 256, "tile path: 256- or 1024-thread workgroups");
    constexpr int E = 8;   // block maxima per lane: at most 512 (merged in groups beyond)
    constexpr int TU = 8;  // tile maxima in flight per thread
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    // 32-bit indices: a query's key rows are fewer than 2^31.
    const int tile_rows = 1 << tile_shift;
    const int ntiles = (rl + tile_rows) >> tile_shift;  // tiles covering rows 0..rl
    // First tile maxima requested before the bound is known.
    uint32_t tm[TU];
#pragma unroll
    for (int e = 0; e < TU; ++e) {
        const int j = tid + NT * e;
        tm[e] = best1[j < ntiles ? j : 0];
    }
    if (wave == 0) {
        // Maxima of disjoint groups of rows: the blocks (256 rows), or the tiles when there are
        // fewer than 2k' blocks; merged into at most 64*E groups of consecutive ones.
        const bool by_tile = nblk < 2 * kp;
        const uint32_t *src = by_tile ? best1 : bm;
        const int stride = by_tile ? 1 : G;
        const int count = by_tile ? ntiles : nblk;
        const int per = (count + 64 * E - 1) / (64 * E);
        const int ngr = per == 1 ? count : (int)(((uint32_t)count + per - 1) / (uint32_t)per);
        uint32_t m[E];
#pragma unroll
        for (int e = 0; e < E; ++e) m[e] = 0u;
        for (int jj = 0; jj < per; ++jj) {  // E independent loads per pass, all issued first
            uint32_t x[E];
#pragma unroll
            for (int e = 0; e < E; ++e) {
                const int gi = lane + 64 * e, grp = gi * per + jj;
                x[e] = src[(gi < ngr && grp < count ? grp : 0) * stride];
            }
#pragma unroll
            for (int e = 0; e < E; ++e) {
                const int gi = lane + 64 * e, grp = gi * per + jj;
                if (gi < ngr && grp < count) m[e] = x[e] > m[e] ? x[e] : m[e];
            }
        }
        const uint32_t thr = wave_bound_u32(m, kp);
        if (lane == 0) { sh.pick[0] = thr > 1u ? thr : 1u; sh.pick[1] = 0u; sh.pick[2] = 0u; sh.sel_count = 0; }
    } else {
        overlap();
    }
    __syncthreads();
    const uint32_t thr = sh.pick[0];
    // Tiles whose best key reaches the bound, compacted into tiles[] (in any order: the
    // selection does not depend on it). jb is uniform.
    for (int jb = 0;; jb += NT * TU) {
        const int j0 = jb + tid;
#pragma unroll
        for (int e = 0; e < TU; ++e) {
            if (tm[e] >= thr && j0 + NT * e < ntiles) {
                const uint32_t at = atomicAdd(&sh.pick[1], 1u);
                if (at < (uint32_t)kTileCap) tiles[at] = j0 + NT * e;
            }
        }
        if (jb + NT * TU >= ntiles) break;
#pragma unroll
        for (int e = 0; e < TU; ++e) {
            const int j = j0 + NT * (TU + e);
            tm[e] = best1[j < ntiles ? j : 0];
        }
    }
    __syncthreads();
    const int nt = (int)sh.pick[1];
    bool fallback = nt > kTileCap;
    if (!fallback) {
        // Each passing tile gives its best rows that reach the bound, or, when its third key may
        // reach it as well (its upper half is kept: compared as the largest key with that
        // half), goes to the list of tiles scored again.
        for (int x = tid; x < nt; x += NT) {
            const int tile = tiles[x];
            const uint32_t k1 = best1[tile];
            const uint2 rs = rest[tile];
            // Both loads complete here (kept from being moved into the branches one by one).
            asm volatile("" ::"v"(k1), "v"(rs.x), "v"(rs.y));
            const uint32_t k2 = rs.x, o = rs.y, k3max = (rs.y & 0xFFFF0000u) | 0xFFFFu;
            if ((rs.y & 0xFFFF0000u) != 0u && k3max >= thr) {
                const uint32_t at = atomicAdd(&sh.pick[2], 1u);
                if (at < (uint32_t)kOvfCap) ovf[at] = tile;
            } else {
                // (Increments of 1 only: the compiler turns those into one atomic per wavefront.)
                const uint32_t row0 = (uint32_t)(tile << tile_shift);
                const int p1 = atomicAdd(&sh.sel_count, 1);
                if (p1 < kGather) gathered[p1] = make_rank_key(k1, row0 + (o & 0xFFu));
                if (k2 >= thr) {
                    const int p2 = atomicAdd(&sh.sel_count, 1);
                    if (p2 < kGather) gathered[p2] = make_rank_key(k2, row0 + ((o >> 8) & 0xFFu));
                }
            }
        }
        __syncthreads();
        const int no = (int)sh.pick[2];
        if (no > kOvfCap) {
            fallback = true;
        } else if (no > 0) {
            rescore(no, [&](int i) { return ovf[i]; }, [&](uint32_t key, int row) {
                if (key >= thr) {
                    const int pos = atomicAdd(&sh.sel_count, 1);
                    if (pos < kGather) gathered[pos] = make_rank_key(key, (uint32_t)row);
                }
            });
            __syncthreads();
        }
    }
    int n = fallback ? kGather + 1 : sh.sel_count;
    if (n > kGather) {
        // Too many candidates for LDS (exact ties at the bound): the keys of every passing tile
        // into scratch, then the selection over them.
        rescore(ntiles, [&](int i) { return best1[i] >= thr ? i : -1; },
                [&](uint32_t key, int row) { scratch[row] = key; });
        __threadfence_block();
        n = kGather + 1;
    }
    __syncthreads();
    if (n <= kRankSelectMax && n <= NT && n >= kp) {
        select_by_rank<NT>(n, kp, gathered, js);
        return;
    }
    // Keys from scratch for rows of passing tiles (others hold none that reach the bound).
    auto key_at = [&](int64_t f64) -> uint64_t {
        const int f = (int)f64;
        if (f < 1 || f > rl || best1[f >> tile_shift] < thr) return 0ull;
        const uint32_t kv = scratch[f];
        return kv >= thr ? make_rank_key(kv, (uint32_t)f) : 0ull;
    };
    select_exact<NT>(n, (int64_t)ntiles << tile_shift, key_at, kp, js, sel, gathered, sh);
}

// Scores every row of the tiles tile_at(0..ntl) (-1: none) for the query vector in slot t of
// unit (b, kvh, group gq) with row_key over the unit's G query vectors, as score_keys does (the
// same bits), and calls emit(key, row) for each row in [1, rl] (key 0 never reaches a bound). RPG
// rows per wavefront load, LPR lanes per row; one pass per NW*RPG rows. All threads.
template <typename T, int D, int NT, typename TileAt, typename Emit>
__device__ __forceinline__ void rescore_tiles(const T *__restrict__ q, const T *__restrict__ kb,
                                              const FinishArgs &a, uint32_t b, uint32_t kvh, uint32_t gq,
                                              int t, int rl, int ntl, TileAt tile_at, Emit emit) {
    constexpr int RB = D * (int)sizeof(T);
    constexpr int LPR = RB >= 256 ? 16 : 8, RPG = 64 / LPR, P = RB / (16 * LPR);
    constexpr int NW = NT / 64;
    const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int sl = lane % LPR;
    const uint32_t g = (uint32_t)a.g, bk = b * (uint32_t)a.Hkv + kvh;
    const int G = a.G;
    auto body = [&](auto gc) {
        constexpr int GC = decltype(gc)::value;
        uint4 qr[GC][P];
#pragma unroll
        for (int tt = 0; tt < GC; ++tt) {
            const uint32_t idx = gq * GC + tt;
            if (idx < a.nvec) {
                const uint32_t qh = idx / g, hh = idx - qh * g;
                const uint4 *src = reinterpret_cast<const uint4 *>(q + (((size_t)bk * g + hh) * a.nq + qh) * D);
#pragma unroll
                for (int p = 0; p < P; ++p) qr[tt][p] = src[p * LPR + sl];
            } else {
#pragma unroll
                for (int p = 0; p < P; ++p) qr[tt][p] = make_uint4(0, 0, 0, 0);
            }
        }
        const bool mine = sl / (LPR / GC) == t && sl % (LPR / GC) == 0;
        const int total = ntl << a.tile_shift;
        for (int r0 = wave * RPG; r0 < total; r0 += NW * RPG) {
            const int rr = r0 + lane / LPR;
            const int tile = rr < total ? tile_at(rr >> a.tile_shift) : -1;
            const int row = tile >= 0 ? (tile << a.tile_shift) + (rr & ((1 << a.tile_shift) - 1)) : 0;
            const int lrow = row < a.n ? row : (int)a.n - 1;
            const uint4 *src = reinterpret_cast<const uint4 *>(kb + (size_t)lrow * D);
            uint4 kr[P];
#pragma unroll
            for (int p = 0; p < P; ++p) kr[p] = src[p * LPR + sl];
            const uint32_t key = row_key<T, LPR, P, GC>(kr, qr, lane);
            if (mine && tile >= 0 && row >= 1 && row <= rl) emit(key, row);
        }
    };
    if (G == 4) body(std::integral_constant<int, 4>());
    else if (G == 2) body(std::integral_constant<int, 2>());
    else body(std::integral_constant<int, 1>());
}

// Rows per lane in flight in the attend phase (rows past the set's end are loaded as clamped
// duplicates, so these match the common sizes: 15 wavefronts x 4 rows x 5 cover the anchor and
// a window of up to 299 rows of 256 bytes in one round, 4 x 4 x 4 a top-64 part).
constexpr int kWindowU = 5;
constexpr int kTopU = 4;  // rows per lane in flight in the top-k part

template <typename T, int D, int NT, bool ATTEND, bool TILES>
__global__ __launch_bounds__(NT) void finish_kernel(const T *__restrict__ q, const T *__restrict__ k,
                                                    const T *__restrict__ v,
                                                    int32_t *__restrict__ out_idx,
                                                    float *__restrict__ out, FinishArgs a) {
    constexpr int NW = NT / 64;
    extern __shared__ int32_t fsm[];  // js[2*cap] positions, then sel[topk] keys
    __shared__ SelectShared<NT> ssh;
    __shared__ uint64_t gathered[kGatherFor<NT>];
    __shared__ int32_t tile_idx[TILES ? kTileCap : 1];
    __shared__ int32_t ovf_idx[TILES ? kOvfCap : 1];
    // Softmax partials: [0, NW) the anchor and window rows (wavefronts 1..NW-1 when wavefront 0
    // takes the bound), [NW, 2NW) the top-k rows.
    __shared__ SoftmaxPartials<D, ATTEND ? 2 * NW : 1> part;
    int32_t *js = fsm;
    uint64_t *sel = reinterpret_cast<uint64_t *>(fsm + 2 * a.cap);

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    // Query vector qv = (b*Hq + h)*nq + r (32-bit math: the plan keeps qv below 2^24).
    const int64_t qv = blockIdx.x;
    const uint32_t nq32 = (uint32_t)a.nq, hq32 = (uint32_t)a.Hq, g32 = (uint32_t)a.g;
    const uint32_t bh = (uint32_t)qv / nq32;
    const int64_t r = (uint32_t)qv - bh * nq32;
    const uint32_t b = bh / hq32, h = bh - b * hq32;
    const uint32_t kvh = h / g32;
    const int64_t i = a.n - a.nq + r;
    const int64_t wlo = (i - a.W + 1 > 0) ? i - a.W + 1 : 0;
    const int64_t rl = i - a.W;
    const int64_t n_r = rl >= 1 ? rl : 0;
    const int kp = (int)(a.topk < n_r ? a.topk : n_r);
    // Wavefronts of the top-k part: in 1024-thread workgroups as many as one round of kTopU
    // rows per lane needs (fewer partials to merge); in narrower ones every wavefront.
    constexpr int kTopRowsPerWave = AttendShape<D, T>::RPW * kTopU;
    const int top_waves = NT >= 1024 ? ((kp + kTopRowsPerWave - 1) / kTopRowsPerWave < NW
                                            ? (kp + kTopRowsPerWave - 1) / kTopRowsPerWave : NW)
                                     : NW;
    // js layout: [0 if the anchor is separate][top-k' ascending][window ascending]
    const int base = wlo > 0 ? 1 : 0;
    const int wcount = (int)(i - wlo + 1);
    // Tile-summary path: unit and slot of this query vector (vector index r*g + (h - kvh*g) of
    // its KV head).
    const uint32_t idx = (uint32_t)r * g32 + (h - kvh * g32);
    const uint32_t gq = TILES ? idx / (uint32_t)a.G : 0u;
    const int64_t u = ((int64_t)b * a.Hkv + kvh) * a.groups + gq;
    const int t = (int)(idx - gq * (uint32_t)(TILES ? a.G : 0));

    // Attend over the anchor and the window: the rows are known from the start, so they are
    // processed by the wavefronts that do not take the bound (all of them when there is no
    // top-k part).
    const size_t kv0 = ((size_t)b * a.Hkv + kvh) * (size_t)a.n * D;
    const T *kb = k + kv0, *vb = v + kv0;
    uint4 qs = make_uint4(0, 0, 0, 0);
    if constexpr (ATTEND) qs = reinterpret_cast<const uint4 *>(q + qv * D)[lane % AttendShape<D, T>::LPR];
    // MFMA path: mfma_window computed the anchor-and-window partial already; it goes to slot
    // NW - 1, next to the top-k rows' partials NW..2NW-1.
    const bool pre_win = a.win != nullptr;
    if constexpr (ATTEND) {
        // (Threads of the wavefronts after the first, which gathers the candidates; all of a
        // one-wavefront workgroup.)
        constexpr int E0 = NT > 64 ? 64 : 0;
        for (int e = tid - E0; pre_win && e >= 0 && e < D + 2; e += NT - E0) {
            const float x = a.win[(size_t)qv * (D + 2) + e];
            if (e == 0) part.m[NW - 1] = x;
            else if (e == 1) part.l[NW - 1] = x;
            else part.acc[NW - 1][e - 2] = x;
        }
    }
    auto window_part = [&](int wv, int nw) {
        if constexpr (ATTEND) {
            if (pre_win) return;
            auto row_at = [&](int c) -> size_t { return c < base ? 0 : (size_t)(wlo - base + c); };
            wave_partial<D, T, kWindowU>(qs, kb, vb, row_at, base + wcount, wv, nw, a.scale_log2e,
                                         part, wave);
        }
    };
    if (kp > 0) {
        auto overlap = [&]() { window_part(wave - 1, NW - 1); };
        if constexpr (TILES) {
            const size_t qt = ((size_t)u * a.G + t) * (size_t)(a.rstride >> a.tile_shift);
            select_tiles<NT>(a.best1 + qt, a.rest + qt,
                             a.bmax + (size_t)u * a.nblk * a.G + t, a.G, a.nblk, a.tile_shift,
                             (int)rl, kp, js + base, sel, gathered, tile_idx, ovf_idx,
                             a.scratch + qv * a.rstride, ssh, overlap,
                             [&](int ntl, auto tile_at, auto emit) {
                                 rescore_tiles<T, D, NT>(q, kb, a, b, kvh, gq, t, (int)rl, ntl, tile_at, emit);
                             });
        } else {
            select_segments<NT>(a.cnt + qv * a.wpu, a.lists + qv * a.wpu * a.seg, a.wpu, a.seg,
                                kp, js + base, sel, gathered, ssh, overlap);
        }
    } else {
        window_part(wave, NW);
    }
    const int count = base + kp + wcount;
    if (tid == 0 && base) js[0] = 0;
    for (int t = tid; t < wcount; t += NT) js[base + kp + t] = (int32_t)(wlo + t);
    lds_barrier();
    int32_t *row = out_idx + qv * a.cap;
    for (int t = tid; t < a.cap; t += NT) row[t] = t < count ? js[t] : -1;
    if constexpr (ATTEND) {
        if (kp > 0) {
            const int32_t *top = js + base;
            auto row_at = [&](int c) -> size_t { return (size_t)(uint32_t)top[c]; };
            if (wave < top_waves)
                wave_partial<D, T, kTopU>(qs, kb, vb, row_at, kp, wave, top_waves, a.scale_log2e, part, NW + wave);
        }
        // (The index row's stores need not complete before the merge: LDS only.)
        lds_barrier();
        // Window partials: NW-1 (from mfma_window), 1..NW-1 (wavefront 0 took the bound) or
        // 0..NW-1; top-k partials NW..2NW-1.
        const int p0 = pre_win ? NW - 1 : (kp > 0 ? 1 : 0);
        if constexpr (TILES) {
            if (a.mass && tid < 64) {
                // Mass diagnostic (pages of "The Condensate Theorem", metaphor-xennon blog:
                // section 3.2.2, the full-softmax mass outside C_i; sections 2.2.1-2.2.3, the
                // parts of C_i). Sum over the candidate rows R_i from score_keys' per-block
                // sums; the window part (with row 0) and the top-k part from the partials above;
                // row 0's own weight from its score. All relative to one maximum M.
                const float2 *zs = a.zsum + (size_t)u * a.nblk * a.G + t;
                float ml = -INFINITY, ll = 0.f;  // this lane's blocks lane, lane + 64, ...
                for (int blk = lane; blk < a.nblk; blk += 64) {
                    const float2 z = zs[(size_t)blk * a.G];
                    if (z.x != -INFINITY) {
                        const float mn = fmaxf(ml, z.x);
                        ll = (ml == -INFINITY ? 0.f : ll * exp2f((ml - mn) * a.scale_log2e)) +
                             z.y * exp2f((z.x - mn) * a.scale_log2e);
                        ml = mn;
                    }
                }
                const float mr = wave_max_f32_dpp(ml);
                const float lr = wave_sum_f32_dpp(ml == -INFINITY ? 0.f : ll * exp2f((ml - mr) * a.scale_log2e));
                auto range = [&](int q0, int q1, float &mx, float &sm) {
                    const int pc = lane < 2 * NW ? lane : 2 * NW - 1;
                    const float pm = lane >= q0 && lane < q1 ? part.m[pc] : -INFINITY;
                    const float pl = lane >= q0 && lane < q1 ? part.l[pc] : 0.f;
                    mx = wave_max_f32_dpp(pm);
                    sm = wave_sum_f32_dpp(pm == -INFINITY ? 0.f : pl * exp2f((pm - mx) * a.scale_log2e));
                };
                float mw, lw, mt = -INFINITY, lt = 0.f;
                range(p0, NW, mw, lw);
                if (kp > 0) range(NW, NW + top_waves, mt, lt);
                using S = AttendShape<D, T>;
                const uint4 k0 = reinterpret_cast<const uint4 *>(kb)[lane % S::LPR];
                const float s0 = row_sum<S::LPR>(dot16(k0, qs, 0.f, T()));
                const float mg = fmaxf(mr, mw);
                auto rel = [&](float mx, float sm) {
                    return mx == -INFINITY ? 0.f : sm * exp2f((mx - mg) * a.scale_log2e);
                };
                const float zr = rel(mr, lr), zw = rel(mw, lw), zt = rel(mt, lt);
                const float z0 = exp2f((s0 - mg) * a.scale_log2e);
                const float zf = zr + zw;
                if (lane == 0) {
                    float *mo = a.mass + qv * 4;
                    mo[0] = fmaxf(zr - zt, 0.f) / zf;
                    mo[1] = z0 / zf;
                    mo[2] = fmaxf(zw - z0, 0.f) / zf;
                    mo[3] = zt / zf;
                }
            }
        }
        merge_partials<NT, D>(part, p0, kp > 0 ? NW + top_waves : NW, a.scale_log2e, out + qv * D);
    }
}

// Caller-supplied sets: ordered compaction of the valid entries of the index row, then attend.
template <typename T, int D, int NT>
__global__ __launch_bounds__(NT) void attend_kernel(const T *__restrict__ q, const T *__restrict__ k,
                                                    const T *__restrict__ v,
                                                    const int32_t *__restrict__ idx,
                                                    float *__restrict__ out, FinishArgs a) {
    constexpr int NW = NT / 64;
    extern __shared__ int32_t js[];  // js[cap]
    __shared__ int wave_cnt[NW];
    __shared__ SoftmaxPartials<D, NW> part;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int64_t qv = blockIdx.x;  // (b*Hq + h)*nq + r, below 2^24
    const uint32_t nq32 = (uint32_t)a.nq, hq32 = (uint32_t)a.Hq;
    const uint32_t bh = (uint32_t)qv / nq32;
    const int64_t r = (uint32_t)qv - bh * nq32;
    const uint32_t b = bh / hq32, h = bh - b * hq32;
    const int64_t i = a.n - a.nq + r;
    const int32_t *row = idx + qv * a.cap;

    int count = 0;
    for (int c0 = 0; c0 < a.cap; c0 += NT) {
        const int c = c0 + tid;
        const int32_t j = c < a.cap ? row[c] : -1;
        const bool ok = j >= 0 && j <= i;
        const uint64_t m = __ballot(ok);
        if (lane == 0) wave_cnt[wave] = __popcll(m);
        __syncthreads();
        int off = count, tot = 0;
        for (int w2 = 0; w2 < NT / 64; ++w2) {
            off += w2 < wave ? wave_cnt[w2] : 0;
            tot += wave_cnt[w2];
        }
        if (ok) js[off + lanes_below(m)] = j;
        count += tot;
        __syncthreads();
    }
    float *o = out + qv * D;
    if (count == 0) {
        for (int t = tid; t < D; t += NT) o[t] = 0.f;
        return;
    }
    // Every listed position lies in [0, i], so it addresses a row of the KV head.
    const size_t kv0 = ((size_t)b * a.Hkv + h / (uint32_t)a.g) * (size_t)a.n * D;
    const uint4 qs = reinterpret_cast<const uint4 *>(q + qv * D)[lane % AttendShape<D, T>::LPR];
    auto row_at = [&](int c) -> size_t { return (size_t)(uint32_t)js[c]; };
    wave_partial<D, T, 2>(qs, k + kv0, v + kv0, row_at, count, wave, NW, a.scale_log2e, part, wave);
    __syncthreads();
    merge_partials<NT, D>(part, 0, NW, a.scale_log2e, o);
}

FinishArgs finish_args(const Plan &pl, const void *ws) {
    FinishArgs a;
    a.n = pl.n; a.nq = pl.nq; a.Hq = pl.Hq; a.Hkv = pl.Hkv; a.g = pl.g;
    a.W = pl.W; a.topk = pl.topk; a.cap = pl.cap; a.wpu = pl.wpu; a.seg = pl.seg;
    a.scale_log2e = (float)(1.4426950408889634 / __builtin_sqrt((double)pl.d));
    a.cnt = ws ? reinterpret_cast<const uint32_t *>(static_cast<const char *>(ws) + pl.slots_offset) + 2 * pl.nqv * pl.wpu
               : nullptr;
    a.lists = ws ? reinterpret_cast<const uint64_t *>(static_cast<const char *>(ws) + pl.lists_offset) : nullptr;
    a.G = pl.G; a.nblk = pl.nblk; a.tile_shift = pl.tile_rows == 32 ? 5 : 4; a.groups = pl.groups; a.rstride = pl.rstride;
    const char *wb = static_cast<const char *>(ws);
    const bool sm = ws && pl.stream;
    a.best1 = sm ? reinterpret_cast<const uint32_t *>(wb + pl.best1_offset) : nullptr;
    a.rest = sm ? reinterpret_cast<const uint2 *>(wb + pl.rest_offset) : nullptr;
    a.bmax = sm ? reinterpret_cast<const uint32_t *>(wb + pl.bmax_offset) : nullptr;
    a.scratch = sm ? reinterpret_cast<uint32_t *>(const_cast<char *>(wb) + pl.scratch_offset) : nullptr;
    a.nvec = (uint32_t)(pl.g * pl.nq);
    a.win = ws && pl.mfma ? reinterpret_cast<const float *>(wb + pl.win_offset) : nullptr;
    a.zsum = sm ? reinterpret_cast<const float2 *>(wb + pl.zsum_offset) : nullptr;
    a.mass = nullptr;
    return a;
}

// Few query vectors: 1024 threads each (latency); many: 256, or on the MFMA path, whose
// candidate lists hold at most 256 keys and whose window partials are computed already, 128
// (64 when topk <= 32): more query vectors in flight per CU.
constexpr int64_t kWideBelow = 4096;

template <typename T, int D, bool ATTEND>
hipError_t launch_finish_t(const Plan &pl, const void *ws, const void *q, const void *k,
                           const void *v, int32_t *out_idx, float *out, hipStream_t s, float *mass) {
    FinishArgs a = finish_args(pl, ws);
    a.mass = mass;
    const size_t shmem = (size_t)pl.cap * (2 * sizeof(int32_t)) + (size_t)pl.topk * sizeof(uint64_t);
    const bool tiles = pl.stream && ws != nullptr;
    const dim3 grid((unsigned)pl.nqv);
    const T *qt = static_cast<const T *>(q), *kt = static_cast<const T *>(k), *vt = static_cast<const T *>(v);
    const size_t fixed1024 = kGather * sizeof(uint64_t) + sizeof(SelectShared<1024>) +
                             (kTileCap + kOvfCap) * sizeof(int32_t) + sizeof(SoftmaxPartials<D, 32>);
    const bool wide = pl.nqv < kWideBelow && shmem + fixed1024 <= 64 * 1024;
#define CA_LAUNCH_FIN(NT, TILES)                                                                  \
    hipLaunchKernelGGL((finish_kernel<T, D, NT, ATTEND, TILES>), grid, dim3(NT), shmem, s, qt, kt, vt, \
                       out_idx, out, a)
    if (wide) {
        if (tiles) CA_LAUNCH_FIN(1024, true); else CA_LAUNCH_FIN(1024, false);
    } else if (tiles) {
        CA_LAUNCH_FIN(256, true);
    } else if (pl.mfma && pl.wpu * pl.seg <= kRankSelectMax && pl.topk <= 32) {
        CA_LAUNCH_FIN(64, false);
    } else if (pl.mfma && pl.wpu * pl.seg <= kRankSelectMax) {
        CA_LAUNCH_FIN(128, false);
    } else {
        CA_LAUNCH_FIN(256, false);
    }
#undef CA_LAUNCH_FIN
    return hipGetLastError();
}

template <typename T, int D>
hipError_t launch_attend_t(const Plan &pl, const void *q, const void *k, const void *v,
                           const int32_t *idx, float *out, hipStream_t s) {
    const FinishArgs a = finish_args(pl, nullptr);
    const size_t shmem = (size_t)pl.cap * sizeof(int32_t);
    const dim3 grid((unsigned)pl.nqv);
    const T *qt = static_cast<const T *>(q), *kt = static_cast<const T *>(k), *vt = static_cast<const T *>(v);
    const bool wide = pl.nqv < kWideBelow && shmem + sizeof(SoftmaxPartials<D, 16>) <= 64 * 1024;
    if (wide)
        hipLaunchKernelGGL((attend_kernel<T, D, 1024>), grid, dim3(1024), shmem, s, qt, kt, vt, idx, out, a);
    else
        hipLaunchKernelGGL((attend_kernel<T, D, 256>), grid, dim3(256), shmem, s, qt, kt, vt, idx, out, a);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_finish(const Plan &pl, const void *ws, const void *q, const void *k,
                         const void *v, int32_t *out_idx, float *out, hipStream_t s, float *mass) {
    const bool attend = out != nullptr;
#define CA_FIN(T, D) (attend ? launch_finish_t<T, D, true>(pl, ws, q, k, v, out_idx, out, s, mass) \
                             : launch_finish_t<T, D, false>(pl, ws, q, k, v, out_idx, out, s, nullptr))
    if (pl.dtype == 1) return pl.d == 128 ? CA_FIN(__bf16, 128) : CA_FIN(__bf16, 64);
    return pl.d == 128 ? CA_FIN(float, 128) : CA_FIN(float, 64);
#undef CA_FIN
}

hipError_t launch_gather_softmax_av(const Plan &pl, const void *q, const void *k, const void *v,
                                    const int32_t *idx, float *out, hipStream_t s) {
    if (pl.dtype == 1)
        return pl.d == 128 ? launch_attend_t<__bf16, 128>(pl, q, k, v, idx, out, s)
                           : launch_attend_t<__bf16, 64>(pl, q, k, v, idx, out, s);
    return pl.d == 128 ? launch_attend_t<float, 128>(pl, q, k, v, idx, out, s)
                       : launch_attend_t<float, 64>(pl, q, k, v, idx, out, s);
}

}  // namespace ca
