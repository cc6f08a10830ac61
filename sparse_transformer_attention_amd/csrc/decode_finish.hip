// decode_finish: the end of the decode path on gfx950, one workgroup per query vector (pages of
// "The Condensate Theorem", metaphor-xennon blog: section 2.1 Definition 1, C_i = {0} u
// {i-W+1..i} u Top-k_i; section 2.2.3, the top-k part over R_i = {1..i-W}, ties to the smaller
// position; section 2.3, the softmax restricted to C_i times V; section 3.2.2, the mass outside
// C_i).
//
// The records of decode_stream and the anchor-and-window chunk partials (made by decode_stream's
// window workgroups) are requested first. A bound T0 comes from the blocks' best keys (k' blocks,
// so k' distinct rows, reach it: no row below it can be in the top k'). The record rows whose
// ranking key (score_key << 32) | ~position reaches the bound are gathered in a fixed order; their
// V rows are requested at once, and the list is cut to its exact top k' by counting each key's
// rank on all wavefronts. A block whose X reaches the k'-th key has rows beyond its record that
// may rank: those are scored again (row_key, the same bits) and the cut repeated (their V rows
// are then requested after it). The top k''s places in out_idx are counted while the V rows
// load; the anchor-and-window partial and the top-k partials (weights exp2((s - m) * scale), s
// read back from the keys) merge into the output. Too many candidates or such blocks (dense
// clusters of high scores, exact ties) switch the query to an exact fallback: all its candidate
// rows scored into scratch keys and a workgroup radix select.
#include "attend_core.h"
#include "decode_core.h"
#include "merge_core.h"
#include "select_core.h"

namespace ca {
namespace dec {
namespace {

constexpr int kCand = 1024;        // candidate keys per query held in LDS
constexpr int kDef = 64;           // blocks whose X reaches the threshold, held in LDS
constexpr int kResc = 8;           // such blocks scored again on the common path
constexpr int kSelMax = 256;       // largest k' of the common path (larger: the fallback)
constexpr int kRankMax = 256;      // candidate lists cut by rank counting (longer: one wavefront)
static_assert(kSelMax <= kRankMax && 2 * kRankMax <= kCand, "rank_cut's output room");

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
    alignas(16) uint64_t cand[kCand];  // candidate ranking keys; after each cut the top k'
    union {
        uint32_t bmax[kNT];  // best keys of the round's blocks (threshold of the single wavefront)
        struct {
            int32_t js[2 * 512];    // fallback: selected positions
            SelectShared<kNT> ssh;  // fallback: radix select
        } fb;
    } x;
    uint64_t def[kDef];   // blocks whose X reached the threshold: X << 32 | block
    uint32_t doff[kDef];  // and their records' row offsets
    SoftmaxPartials<D, 2 * kWaves> part;  // [0, kWaves-1) anchor and window, then the top-k rows
    int wc[kWaves], wd[kWaves];           // per-wavefront counts of an append
    int anyd[kWaves];                     // per-wavefront: some block to list after the cut
    uint32_t tw[kWaves];                  // per-wavefront bounds
    uint32_t tb;                          // the single wavefront's bound
    float zm[kWaves], zl[kWaves];         // mass diagnostic: candidates' mass per wavefront
    uint64_t thr;
    int n, ndef, flag;
};

// Appends, in a fixed order (wavefront, then e, then lane), the keys key[e] with ok[e] of every
// wavefront after list[0..sh.n), and the blocks with okd (entry dk, offsets doff) after
// def[0..sh.ndef). Called by all threads; two workgroup barriers, after which the entries are
// visible; returns the new list length (sh.n and sh.ndef are written after the second barrier).
// Entries past the capacities are dropped (the counts still grow, so the caller sees the
// overflow).
template <int D, int E>
__device__ __forceinline__ int append_all(FinShared<D> &sh, const bool (&ok)[E], const uint64_t (&key)[E],
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
    return n_all;
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

// Exact top kp of the n distinct ranking keys sh.cand[0..n) (kp < n <= kRankMax), all threads:
// each key's rank (the number of keys above it) is counted by a group of 8 lanes (two keys per
// group, from the same reads); the keys of
// rank < kp go to sh.cand[0..kp) in descending order, and the threshold becomes the kp-th key.
// On the way, sh.anyd[wave] says whether some thread's block key X (0: none) reaches the new
// threshold's score key. Two barriers, on LDS traffic only (vector loads stay in flight).
template <int D>
__device__ __forceinline__ void rank_cut(FinShared<D> &sh, int n, int kp, uint32_t X) {
    const int tid = threadIdx.x;
    uint64_t *const top = sh.cand + (kCand - kRankMax);  // (past every read: n <= kRankMax)
    for (int c0 = 0; c0 < n; c0 += kNT / 4) {
        const int c = c0 + (tid >> 3), c1 = c + kNT / 8;
        const uint64_t key = c < n ? sh.cand[c] : ~0ull, key1 = c1 < n ? sh.cand[c1] : ~0ull;
        const uint2 r = group8_count(sh.cand, n, [&](uint64_t y, int s) { return y > (s ? key1 : key); });
        if ((tid & 7) == 0 && c < n && r.x < (uint32_t)kp) top[r.x] = key;
        if ((tid & 7) == 1 && c1 < n && r.y < (uint32_t)kp) top[r.y] = key1;
    }
    lds_barrier();
    const bool okd = X != 0u && X >= (uint32_t)(top[kp - 1] >> 32);
    const bool wany = __ballot(okd) != 0ull;
    if ((tid & 63) == 0) sh.anyd[tid >> 6] = wany ? 1 : 0;
    for (int c = tid; c < kp; c += kNT) sh.cand[c] = top[c];
    if (tid == 0) {
        sh.thr = top[kp - 1];
        sh.n = kp;
    }
    lds_barrier();
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
    __shared__ FinShared<D> sh;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    // Workgroup b serves query t = b / units of unit b % units: with the stream's interleaved
    // order (workgroups are dealt to the 8 XCDs in turn) it runs on the XCD whose L2 took the
    // unit's records when units is a multiple of 8.
    const int t = (int)(blockIdx.x / a.units);
    const uint32_t uu = blockIdx.x - (uint32_t)t * a.units;
    const uint32_t ng = (uint32_t)a.groups;
    const uint32_t bk = uu / ng, grp = uu - bk * ng;
    const QInfo qi = query_info<G>(a, bk, grp, t);
    if (!qi.valid) return;
    const int kp = qi.kp;
    const size_t kv0 = (size_t)bk * (size_t)a.n * D;
    const T *kb = k + kv0, *vb = v + kv0;
    int32_t *row = a.out_idx + (size_t)qi.qv * a.cap;
    const uint4 *R = a.rec + ((size_t)uu * G + t) * (size_t)a.nblk * 2;
    // Requests first: the first round's records, then the first anchor-and-window chunk partial
    // of each of wavefronts 1..kWaves-1 (made by decode_stream's window workgroups).
    uint4 ra = make_uint4(0, 0, 0, 0), rb = make_uint4(0, 0, 0, 0);
    if (tid < qi.nbq && kp > 0) {
        ra = R[2 * tid];
        rb = R[2 * tid + 1];
    }
    constexpr int NWW = kWaves - 1;
    constexpr int EW = D / 64;  // window partial elements per lane
    const int wv = wave - 1;
    float wm = -INFINITY, wl = 0.f, wacc[EW];
#pragma unroll
    for (int e = 0; e < EW; ++e) wacc[e] = 0.f;
    if (ATTEND && wave > 0 && wv < a.nch) {
        const float *src = a.win + ((size_t)qi.qv * a.nch + wv) * (D + 2);
        wm = src[0];
        wl = src[1];
#pragma unroll
        for (int e = 0; e < EW; ++e) wacc[e] = src[2 + lane + 64 * e];
    }
    // Mass diagnostic: the query slice and row 0's key, for row 0's score at the end (the last
    // wavefront, which the output merge leaves free).
    uint4 qs = make_uint4(0, 0, 0, 0), k0 = make_uint4(0, 0, 0, 0);
    if constexpr (MASS) {
        if (wave == kWaves - 1) {
            qs = reinterpret_cast<const uint4 *>(q + (size_t)qi.qv * D)[lane % AS::LPR];
            k0 = reinterpret_cast<const uint4 *>(kb)[lane % AS::LPR];
        }
    }
    // Wavefront w >= 1 merges chunks w - 1, w - 1 + NWW, ... into partial w - 1 (the first one
    // from the registers requested above).
    auto window_merge = [&]() {
        if constexpr (ATTEND) {
            if (wave > 0) {
                float m = wm, l = wl, acc[EW];
#pragma unroll
                for (int e = 0; e < EW; ++e) acc[e] = wacc[e];
                for (int c = wv + NWW; c < a.nch; c += NWW) {
                    const float *src = a.win + ((size_t)qi.qv * a.nch + c) * (D + 2);
                    const float pm = src[0], pl = src[1];
                    if (pm == -INFINITY) continue;  // (uniform: an empty chunk)
                    const float mn = fmaxf(m, pm);
                    const float f0 = m == -INFINITY ? 0.f : exp2f((m - mn) * a.scale_log2e);
                    const float f1 = exp2f((pm - mn) * a.scale_log2e);
                    l = l * f0 + pl * f1;
#pragma unroll
                    for (int e = 0; e < EW; ++e) acc[e] = acc[e] * f0 + src[2 + lane + 64 * e] * f1;
                    m = mn;
                }
#pragma unroll
                for (int e = 0; e < EW; ++e) sh.part.acc[wv][lane + 64 * e] = acc[e];
                if (lane == 0) {
                    sh.part.m[wv] = m;
                    sh.part.l[wv] = l;
                }
            }
        }
    };
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
    // V rows of the top k': lane slot `slot` of wavefront `wave` takes the rows
    // c = wave * RPW + slot + u * step of a list. With one round of records and at most UT * step
    // candidates, the candidates' V rows are requested before the cut (pv, with their keys pk)
    // and the cut's threshold then picks the members among them.
    constexpr int UT = 4;
    const int cs = lane % AS::LPR, slot = lane / AS::LPR;
    const int step = kWaves * AS::RPW;
    const uint32_t last_row = (uint32_t)(a.n - 1);
    uint4 pv[UT];
    uint64_t pk[UT];
    bool pre = false, resc = false;
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
        int n;  // candidates after the append (uniform)
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
            const uint32_t offs = rb.x;
            bool ok[4];
            uint64_t kk[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                kk[e] = make_rank_key(ks[e], (uint32_t)blk * kRows + ((offs >> (8 * e)) & 255u));
                ok[e] = has && ks[e] != 0u && kk[e] >= thr;
            }
            n = append_all<D, 4>(sh, ok, kk, false, 0ull, 0u);
            if (tid == 0) sh.thr = thr;
        }
        if (ATTEND && r0 == 0 && qi.nbq <= kNT && n <= UT * step) {
            pre = true;
#pragma unroll
            for (int u = 0; u < UT; ++u) {
                const int c = wave * AS::RPW + slot + u * step;
                pk[u] = c < n ? sh.cand[c] : 0ull;
                uint32_t pos = c < n ? (uint32_t)rank_key_pos(pk[u]) : 0u;
                pos = pos < last_row ? pos : last_row;
                pv[u] = reinterpret_cast<const uint4 *>(vb + (size_t)pos * D)[cs];
            }
        }
        // The cut. Rank counting (all wavefronts) also votes on the blocks to list below, so
        // that its last barrier serves for both; deferred blocks of earlier rounds are filtered
        // by wavefront 0 after it (and a barrier follows when there were any).
        bool voted = false;
        const uint32_t X = has ? rb.y : 0u;
        if (n > kCand) {
            if (tid == 0) sh.flag = 1;
        } else if (!sh.flag) {
            if (n > kp && n <= kRankMax) {
                const bool had_def = sh.ndef > 0;  // (uniform)
                rank_cut<D>(sh, n, kp, X);
                voted = true;
                if (had_def) {
                    if (wave == 0) filter_deferred<D>(sh);
                    lds_barrier();
                }
            } else if (wave == 0) {
                cut_exact<D>(sh, kp);
                wave_sync();
                filter_deferred<D>(sh);
            }
        }
        if (!voted) {
            lds_barrier();
            if (sh.flag) break;
        }
        {
            // Blocks whose X reaches the round's final threshold's score key: rows beyond the
            // record may rank. Usually there is none, and one barrier (or the cut's) says so.
            const bool okd = X != 0u && X >= (uint32_t)(sh.thr >> 32);
            if (!voted) {
                const bool wany = __ballot(okd) != 0ull;
                if (lane == 0) sh.anyd[wave] = wany ? 1 : 0;
                lds_barrier();
            }
            int any = 0;
#pragma unroll
            for (int w = 0; w < kWaves; ++w) any |= sh.anyd[w];
            if (any) {
                const bool no[1] = {false};
                const uint64_t nk[1] = {0ull};
                (void)append_all<D, 1>(sh, no, nk, okd, ((uint64_t)X << 32) | (uint32_t)blk, rb.x);
                __syncthreads();
                if (sh.ndef > kDef) {
                    __syncthreads();
                    if (tid == 0) sh.flag = 1;
                    __syncthreads();
                }
            }
        }
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
            resc = true;
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
    // The top-k' rows are sh.cand[0..kp), in an order fixed by the inputs. Unless they were
    // requested before the cut, their V rows are requested now; while they load, the top-k'
    // places in out_idx and the anchor-and-window partial.
    const bool use_pre = pre && !sh.flag && !resc;  // (uniform)
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
    if (ATTEND && kp > 0 && !use_pre) request(wave * AS::RPW);
    // Places of the top-k' in out_idx (positions ascending), on wavefronts w0 .. w0 + nw - 1: a
    // group of 8 lanes per two members counts the smaller positions. With the output, wavefronts 2..
    // do it while 0 and 1 write the merged output (the last one is kept for the mass diagnostic).
    auto place_top = [&](int w0, int nw) {
        if (wave < w0 || wave >= w0 + nw) return;
        const int rel = tid - 64 * w0;
        for (int c0 = 0; c0 < kp; c0 += nw * 16) {
            const int c = c0 + (rel >> 3), c1 = c + nw * 8;
            const uint32_t pos = c < kp ? (uint32_t)rank_key_pos(sh.cand[c]) : 0u;
            const uint32_t pos1 = c1 < kp ? (uint32_t)rank_key_pos(sh.cand[c1]) : 0u;
            // (The position is the complement of a key's low word.)
            const uint2 r = group8_count(sh.cand, kp, [&](uint64_t y, int s) { return ~(uint32_t)y < (s ? pos1 : pos); });
            if ((tid & 7) == 0 && c < kp) row[qi.base + r.x] = (int32_t)pos;
            if ((tid & 7) == 1 && c1 < kp) row[qi.base + r.y] = (int32_t)pos1;
        }
    };
    static_assert(D <= 128, "the merged output is written by wavefronts 0 and 1");
    if constexpr (!ATTEND) place_top(0, kWaves);
    if constexpr (ATTEND) {
        window_merge();
        // Top-k rows: weights exp2((s - m) * scale), m the largest selected score (the hardware
        // exponential: a weight below 2^-126 of the largest counts as 0, which no fp32 sum sees).
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
        if (use_pre) {
            // The candidates requested before the cut: the members are those reaching the
            // final threshold (the k'-th key, or the admission bound when all were kept).
            const uint64_t thr = sh.thr;
#pragma unroll
            for (int u = 0; u < UT; ++u) {
                if (pk[u] != 0ull && pk[u] >= thr) {
                    const float w = __builtin_amdgcn_exp2f((key_score((uint32_t)(pk[u] >> 32)) - m) * a.scale_log2e);
                    l += w;
                    accumulate16(acc, pv[u], w, T());
                }
            }
        } else {
            for (int c0 = wave * AS::RPW; c0 < kp; c0 += UT * step) {
                if (c0 != wave * AS::RPW) request(c0);
#pragma unroll
                for (int u = 0; u < UT; ++u) {
                    if (c0 + u * step + slot < kp) {
                        const float w = __builtin_amdgcn_exp2f((key_score(sk[u]) - m) * a.scale_log2e);
                        l += w;
                        accumulate16(acc, vv[u], w, T());
                    }
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
        const int slot_out = NWW + wave;
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
        merge_partials<kNT, D, 2 * kWaves>(sh.part, 0, NWW + kWaves, a.scale_log2e, o);
        place_top(2, MASS ? kWaves - 3 : kWaves - 2);
        if constexpr (MASS) {
            // Mass diagnostic (section 3.2.2, the full-softmax mass outside C_i; sections
            // 2.2.1-2.2.3, the parts of C_i): the candidates' part from the blocks' sums, the
            // window part (with row 0) and the top-k part from the partials, row 0 from its score;
            // all relative to one maximum. On the last wavefront, while the others write the
            // output.
            if (wave == kWaves - 1) {
                auto fold = [&](const float *pm, const float *pl, int np, float &mx, float &sm) {
                    const float m = lane < np ? pm[lane] : -INFINITY;
                    const float l = lane < np ? pl[lane] : 0.f;
                    mx = wave_max_f32_dpp(m);
                    sm = wave_sum_f32_dpp(m == -INFINITY ? 0.f : l * exp2f((m - mx) * a.scale_log2e));
                };
                float mw, lw, mt, lt, mr, lr;
                fold(sh.part.m, sh.part.l, NWW, mw, lw);
                fold(sh.part.m + NWW, sh.part.l + NWW, kWaves, mt, lt);
                fold(sh.zm, sh.zl, kWaves, mr, lr);
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
}  // namespace dec

hipError_t launch_decode_finish(const Plan &pl, const void *q, const void *k, const void *v, void *ws,
                                int32_t *out_idx, float *out, float *mass, hipStream_t s) {
    using namespace dec;
    const DecodeArgs a = decode_args(pl, ws, out_idx, out, mass);
    const dim3 grid((unsigned)((uint64_t)pl.units * pl.G)), block(kNT);
#define CA_DF(T, D, G)                                                                                \
    do {                                                                                              \
        const T *qt = static_cast<const T *>(q), *kt = static_cast<const T *>(k), *vt = static_cast<const T *>(v); \
        if (mass) hipLaunchKernelGGL((decode_finish_kernel<T, D, G, true, true>), grid, block, 0, s, qt, kt, vt, a); \
        else if (out) hipLaunchKernelGGL((decode_finish_kernel<T, D, G, true, false>), grid, block, 0, s, qt, kt, vt, a); \
        else hipLaunchKernelGGL((decode_finish_kernel<T, D, G, false, false>), grid, block, 0, s, qt, kt, vt, a); \
    } while (0)
#define CA_DF_G(T, D)                                   \
    do {                                                \
        if (pl.G == 4) CA_DF(T, D, 4);                  \
        else if (pl.G == 2) CA_DF(T, D, 2);             \
        else CA_DF(T, D, 1);                            \
    } while (0)
    if (pl.dtype == 1) {
        if (pl.d == 128) CA_DF_G(__bf16, 128); else CA_DF_G(__bf16, 64);
    } else {
        if (pl.d == 128) CA_DF_G(float, 128); else CA_DF_G(float, 64);
    }
#undef CA_DF_G
#undef CA_DF
    return hipGetLastError();
}


}  // namespace ca
