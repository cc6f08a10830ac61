// The end of the condensate-attention path on gfx950, one workgroup per query vector:
//   merge    exact top-k' of the query's candidates (ranking keys (score_key << 32) | ~position;
//            k' = min(k, |R_i|)) from the segments that score_topk or the MFMA passes left;
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
    const float *win;       // [nqv][D + 2] anchor-and-window partials (MFMA path), or null
    int64_t nqv;            // query vectors (the grid covers at least this many workgroups)
    // Mass diagnostic (MFMA path; null: off): per query the bound pass's (reference score m,
    // sum over R_i of exp2((s - m) * scale_log2e)), and the output [nqv][4] = excluded mass,
    // anchor, window without position 0, top-k.
    const float2 *zmass;
    int zw;  // zmass entries per query: 1 (MFMA path) or wpu (chunked path)
    float *mass;
};

// Workgroup grid of one workgroup per query vector: x up to 2^16, y the rest (a launch's
// workgroups times its width stay below 2^32 per dimension).
inline dim3 qv_grid(int64_t nqv) {
    const int64_t gx = nqv < 65536 ? nqv : 65536;
    return dim3((unsigned)gx, (unsigned)((nqv + gx - 1) / gx));
}

// Query vector of this workgroup (qv_grid layout); below nqv < 2^31 (the plan's limit).
__device__ __forceinline__ int64_t block_qv() {
    return (int64_t)blockIdx.y * gridDim.x + blockIdx.x;
}

// Exact top-kp of n distinct non-zero ranking keys in gathered[0..n) (kp <= n <= kRankSelectMax,
// n <= NT; gathered[n .. 64 ceil(n / 64)) holds 0 keys): the keys that reach the kp-th largest
// score key when exactly kp do, else by rank counting: each key's rank, the number of keys above
// it, is counted by a group of 8 lanes (four keys per group, group8_count4) and the keys of rank
// < kp are kept. They go to the tail of gathered[] (64 ceil(kp / 64) entries clear of every read
// of the first count, 0 past kp), and the same count on their positions places them ascending in
// js[0..kp) (their score keys in jk[0..kp)). All threads; two or three LDS barriers, the last at
// the end.
constexpr int kRankSelectMax = 256;
static_assert(kRankSelectMax <= kGather - kRankSelectMax && 128 <= kGatherFor<128> - 128, "rank select room");
template <int NT>
__device__ __forceinline__ void select_by_rank(int n, int kp, uint64_t *gathered, int32_t *js,
                                               uint32_t *jk = nullptr) {
    const int tid = threadIdx.x, part = tid & 7, lane = tid & 63;
    const int kp64 = 64 * ((kp + 63) / 64);
    uint64_t *const top = gathered + kGatherFor<NT> - kp64;
    for (int t = kp + tid; t < kp64; t += NT) top[t] = 0ull;
    // First, on wavefront 0: the kp-th largest 32-bit score key by a bitwise search (no pairwise
    // compares). When exactly kp keys reach it they are the top kp, in list order; otherwise
    // (equal score keys at the kp-th place) the rank count below decides on the 64-bit keys.
    __shared__ int found;
    if (tid < 64) {
        constexpr int E = NT / 64;  // (n <= NT)
        uint64_t kk[E];
        uint32_t sk[E];
#pragma unroll
        for (int e = 0; e < E; ++e) {
            const int c = lane + 64 * e;
            kk[e] = c < n ? gathered[c] : 0ull;
            sk[e] = (uint32_t)(kk[e] >> 32);
        }
        const uint32_t t32 = wave_loose_kth_u32(sk, kp, 0);
        int cnt = 0;
#pragma unroll
        for (int e = 0; e < E; ++e) cnt += __popcll(__ballot(sk[e] != 0u && sk[e] >= t32));
        if (cnt == kp) {
            int base = 0;
#pragma unroll
            for (int e = 0; e < E; ++e) {
                const bool ok = sk[e] != 0u && sk[e] >= t32;
                const uint64_t bal = __ballot(ok);
                if (ok) top[base + lanes_below(bal)] = kk[e];
                base += __popcll(bal);
            }
        }
        if (lane == 0) found = cnt == kp ? 1 : 0;
    }
    lds_barrier();
    for (int c0 = 0; !found && c0 < n; c0 += NT / 2) {
        uint64_t x[4];
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            const int c = c0 + (tid >> 3) + s * (NT / 8);
            x[s] = c < n ? gathered[c] : ~0ull;
        }
        const uint4 r = group8_count4(gathered, n, [&](uint64_t y, int s) { return y > x[s]; });
        const uint32_t rs[4] = {r.x, r.y, r.z, r.w};
        if (part < 4) {
            const int c = c0 + (tid >> 3) + part * (NT / 8);
            if (c < n && rs[part] < (uint32_t)kp) top[rs[part]] = x[part];
        }
    }
    if (!found) lds_barrier();
    for (int c0 = 0; c0 < kp; c0 += NT / 2) {
        uint64_t x[4];
        uint32_t p[4];
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            const int c = c0 + (tid >> 3) + s * (NT / 8);
            x[s] = c < kp ? top[c] : 0ull;
            p[s] = (uint32_t)rank_key_pos(x[s]);
        }
        // (A position is the complement of its key's low word.)
        const uint4 r = group8_count4(top, kp, [&](uint64_t y, int s) { return ~(uint32_t)y < p[s]; });
        const uint32_t rs[4] = {r.x, r.y, r.z, r.w};
        if (part < 4) {
            const int c = c0 + (tid >> 3) + part * (NT / 8);
            if (c < kp) {
                js[rs[part]] = (int32_t)p[part];
                if (jk) jk[rs[part]] = (uint32_t)(x[part] >> 32);  // its score key, in the same place
            }
        }
    }
    lds_barrier();
}

// Candidates from the segments of score_topk or of the MFMA passes (the first cnt[w] keys of
// each segment w of lists[w][0..seg)), gathered into LDS by wavefront 0 while the other wavefronts run
// overlap(); then the exact top-kp: positions to js[0..kp), ascending, and their score keys to
// jk[0..kp) (room for 2*kp).
template <int NT, typename Overlap>
__device__ __forceinline__ void select_segments(const uint32_t *__restrict__ cnt,
                                                const uint64_t *__restrict__ lists, int wpu,
                                                int topk, int kp, int32_t *js, uint64_t *sel,
                                                uint64_t *gathered, SelectShared<NT> &sh,
                                                Overlap overlap, uint32_t *jk) {
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    if (wave == 0) {
        // Every slot of every segment, four per lane in flight with their segments' lengths,
        // kept when inside its segment's length (compacted by ballot).
        // (Segments of a power-of-two length, as on the MFMA path, take shifts and masks
        // instead of integer divisions.)
        constexpr int GU = 4;
        const int slots = wpu * topk;
        const bool p2 = (topk & (topk - 1)) == 0;
        const int lg = p2 ? __builtin_ctz((unsigned)topk) : 0;
        int base = 0;
        for (int f0 = 0; f0 < slots; f0 += 64 * GU) {
            uint64_t x[GU];
            uint32_t c[GU];
#pragma unroll
            for (int u = 0; u < GU; ++u) {
                const int f = f0 + u * 64 + lane, fc = f < slots ? f : slots - 1;
                x[u] = lists[fc];
                c[u] = cnt[p2 ? fc >> lg : fc / topk];
            }
#pragma unroll
            for (int u = 0; u < GU; ++u) {
                const int f = f0 + u * 64 + lane;
                const int e = p2 ? (f & (topk - 1)) : f % topk;
                const bool ok = f < slots && (uint32_t)e < c[u];
                const uint64_t bal = __ballot(ok);
                const int pos = base + lanes_below(bal);
                if (ok && pos < kGatherFor<NT>) gathered[pos] = x[u];
                base += __popcll(bal);
            }
        }
        // 0 keys up to the next multiple of 64 (the rank count reads whole groups of 64).
        if (base + lane < kGatherFor<NT> && lane < 64 * ((base + 63) / 64) - base) gathered[base + lane] = 0ull;
        if (lane == 0) sh.sel_count = base;
    } else {
        overlap();
    }
    __syncthreads();
    const int n = sh.sel_count;
    __syncthreads();
    if (n >= kp && n <= kRankSelectMax && n <= NT) {
        select_by_rank<NT>(n, kp, gathered, js, jk);
        return;
    }
    auto key_at = [&](int64_t f) -> uint64_t {
        const int w = (int)(f / topk);
        const int e = (int)(f - (int64_t)w * topk);
        return e < (int)cnt[w] ? lists[f] : 0ull;
    };
    select_exact<NT>(n, (int64_t)wpu * topk, key_at, kp, js, sel, gathered, sh, jk);
}

// Rows per lane in flight in the attend phase (rows past the set's end are loaded as clamped
// duplicates, so these match the common sizes: 15 wavefronts x 4 rows x 5 cover the anchor and
// a window of up to 299 rows of 256 bytes in one round, 4 x 4 x 4 a top-64 part).
constexpr int kWindowU = 5;
constexpr int kTopU = 4;  // rows per lane in flight in the top-k part

template <typename T, int D, int NT, bool ATTEND>
__global__ __launch_bounds__(NT) void finish_kernel(const T *__restrict__ q, const T *__restrict__ k,
                                                    const T *__restrict__ v,
                                                    int32_t *__restrict__ out_idx,
                                                    float *__restrict__ out, FinishArgs a) {
    constexpr int NW = NT / 64;
    extern __shared__ int32_t fsm[];  // js[2*cap] positions, then sel[topk] keys
    __shared__ SelectShared<NT> ssh;
    __shared__ alignas(16) uint64_t gathered[kGatherFor<NT>];  // (16-byte reads in select_by_rank)
    // Softmax partials: [0, NW) the anchor and window rows (wavefronts 1..NW-1 when wavefront 0
    // takes the bound), [NW, 2NW) the top-k rows.
    __shared__ SoftmaxPartials<D, ATTEND ? 2 * NW : 1> part;
    int32_t *js = fsm;
    uint64_t *sel = reinterpret_cast<uint64_t *>(fsm + 2 * a.cap);
    uint32_t *jk = reinterpret_cast<uint32_t *>(sel + a.topk);  // score keys of the top-k' (2 topk)

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    // Query vector qv = (b*Hq + h)*nq + r (32-bit math: the plan keeps qv below 2^31).
    const int64_t qv = block_qv();
    if (qv >= a.nqv) return;
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
        select_segments<NT>(a.cnt + qv * a.wpu, a.lists + qv * a.wpu * a.seg, a.wpu, a.seg,
                            kp, js + base, sel, gathered, ssh, overlap, jk);
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
            // The selected rows' scores are those their candidate keys were ranked by (the
            // same fp32 products), so only their V rows are read.
            auto score_at = [&](int c) { return key_score(jk[c]); };
            if (wave < top_waves)
                wave_partial_scored<D, T, kTopU>(vb, row_at, score_at, kp, wave, top_waves, a.scale_log2e, part, NW + wave);
        }
        // (The index row's stores need not complete before the merge: LDS only.)
        lds_barrier();
        // Window partials: NW-1 (from mfma_window), 1..NW-1 (wavefront 0 took the bound) or
        // 0..NW-1; top-k partials NW..2NW-1.
        const int p0 = pre_win ? NW - 1 : (kp > 0 ? 1 : 0);
        if (a.mass && tid < 64) {
            // Mass diagnostic (pages of "The Condensate Theorem", metaphor-xennon blog: section
            // 3.2.2, the full-softmax mass outside C_i; sections 2.2.1-2.2.3, the parts of C_i):
            // the sum over the candidate rows R_i from the bound pass, the window part (with
            // row 0) and the top-k part from the partials above, row 0's own weight from its
            // score; all relative to one maximum.
            // (Rows of a query without candidates may enter its wavefront's sum in the bound
            // pass; R_i is empty for it, so the sum is not read.) The chunked path leaves one
            // sum per workgroup of the query's unit.
            float mr = -INFINITY, lr = 0.f;
            for (int w0 = 0; kp > 0 && w0 < a.zw; w0 += 64) {
                const float2 z = w0 + lane < a.zw ? a.zmass[qv * a.zw + w0 + lane] : make_float2(-INFINITY, 0.f);
                const float mx = wave_max_f32_dpp(z.x);
                const float sm = wave_sum_f32_dpp(z.x == -INFINITY ? 0.f : z.y * exp2f((z.x - mx) * a.scale_log2e));
                const float mn = fmaxf(mr, mx);
                lr = (mr == -INFINITY ? 0.f : lr * exp2f((mr - mn) * a.scale_log2e)) +
                     (mx == -INFINITY ? 0.f : sm * exp2f((mx - mn) * a.scale_log2e));
                mr = mn;
            }
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
    const int64_t qv = block_qv();  // (b*Hq + h)*nq + r, below 2^31
    if (qv >= a.nqv) return;
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
    const char *wb = static_cast<const char *>(ws);
    a.win = ws && pl.mfma ? reinterpret_cast<const float *>(wb + pl.win_offset) : nullptr;
    a.zmass = ws && !pl.stream ? reinterpret_cast<const float2 *>(wb + pl.zmass_offset) : nullptr;
    a.zw = pl.mfma ? 1 : pl.wpu;
    a.mass = nullptr;
    a.nqv = pl.nqv;
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
    const size_t shmem = (size_t)pl.cap * (2 * sizeof(int32_t)) + (size_t)pl.topk * (sizeof(uint64_t) + 2 * sizeof(uint32_t));
    const dim3 grid = qv_grid(pl.nqv);
    const T *qt = static_cast<const T *>(q), *kt = static_cast<const T *>(k), *vt = static_cast<const T *>(v);
    const size_t fixed1024 = kGather * sizeof(uint64_t) + sizeof(SelectShared<1024>) + sizeof(SoftmaxPartials<D, 32>);
    const bool wide = pl.nqv < kWideBelow && shmem + fixed1024 <= 64 * 1024;
#define CA_LAUNCH_FIN(NT)                                                                          \
    hipLaunchKernelGGL((finish_kernel<T, D, NT, ATTEND>), grid, dim3(NT), shmem, s, qt, kt, vt, out_idx, out, a)
    if (wide) {
        CA_LAUNCH_FIN(1024);
    } else if (pl.mfma && pl.wpu * pl.seg <= kRankSelectMax && pl.topk <= 32) {
        CA_LAUNCH_FIN(64);
    } else if (pl.mfma && pl.wpu * pl.seg <= kRankSelectMax) {
        CA_LAUNCH_FIN(128);
    } else {
        CA_LAUNCH_FIN(256);
    }
#undef CA_LAUNCH_FIN
    return hipGetLastError();
}

template <typename T, int D>
hipError_t launch_attend_t(const Plan &pl, const void *q, const void *k, const void *v,
                           const int32_t *idx, float *out, hipStream_t s) {
    const FinishArgs a = finish_args(pl, nullptr);
    const size_t shmem = (size_t)pl.cap * sizeof(int32_t);
    const dim3 grid = qv_grid(pl.nqv);
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
