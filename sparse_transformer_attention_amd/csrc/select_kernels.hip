// Stage 1 of condensate attention on gfx950: score every causal key and keep, per query, the
// candidates that can still be in its top-k (pages of "The Condensate Theorem", metaphor-xennon
// blog: section 2.1 Definition 1, C_i = {0} u {i-W+1..i} u Top-k_i; section 2.2.3, the top-k
// part ranks the positions R_i = {1..i-W} outside the anchor and the window).
//
// score_topk: a unit of work is (batch, KV head, query group): up to G query vectors that read
// the same KV head (the query heads of a GQA group and/or consecutive query rows). The key rows
// of the unit's candidate range {1..max_i (i-W)} are cut into chunks of `chunk` rows; the wpu
// workgroups serving a unit take every wpu-th chunk.
// For each chunk the workgroup streams the K rows once (16-byte loads, 8 lanes per row, whole
// 128-byte lines per instruction) and computes fp32 dot products for its G queries (bf16 dot2 or
// fp32 FMA, DPP lane reductions). A score that reaches its query's admission threshold is added
// to the query's running list in LDS at once (one LDS counter per query, one atomic per
// wavefront and query). At the end of a chunk, wavefront t looks after query t's list: a list
// that might not take another chunk is cut back to its exact top-k (radix select), and the
// threshold is raised to the largest of the list's own k-th key and the bounds the unit's other
// workgroups have published. Every one of those is a lower bound of the query's final k-th key,
// so no member of the final top-k is ever dropped: each workgroup publishes the k-th key of its
// list and its best key, and the k'-th largest of the best keys (distinct keys, one per
// workgroup) is a tight bound. At the end each workgroup writes the keys of its list that reach
// the best bound it can see (at most k), and their count, to its own segment. No two
// workgroups write the same word, so nothing waits on a contended atomic.
#include "ca_internal.h"
#include "score_core.h"
#include "select_core.h"

namespace ca {
namespace {

struct TopkArgs {
    int64_t n, nq;
    int Hq, Hkv, g, W, topk, chunk, rcap;
    int64_t groups, units, nwg;
    int wpu;
    uint32_t *tau;    // [nqv][wpu] published k-th keys (high words), cleared first
    uint32_t *top;    // [nqv][wpu] published best keys (high words), cleared first
    uint32_t *cnt;    // [nqv][wpu] keys each workgroup leaves for the query
    uint64_t *lists;  // [nqv][wpu][topk] those keys
    // Mass diagnostic (null: off): [nqv][wpu] per workgroup and query, a reference score m and
    // the sum of exp2((s - m) * scale_log2e) over the workgroup's rows of R_i.
    float2 *zpart;
    float scale_log2e;
};

constexpr int kSlotsRead = 128;  // published slots a workgroup reads (the first ones)

__global__ __launch_bounds__(256) void clear_words_kernel(uint32_t *__restrict__ w, int64_t n) {
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256)
        w[i] = 0u;
}

__device__ __forceinline__ uint32_t load_slot(const uint32_t *p) {
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

template <int G, int NS>
__device__ __forceinline__ void emit_keys(const uint32_t (&keyv)[NS], const int (&rowv)[NS], bool direct,
                                          uint32_t my_thr, bool writer, int my_t, int my_rlast, int row0,
                                          int rows_end, const uint64_t (&qmask)[G], uint64_t my_mask,
                                          uint32_t *rcnt, uint64_t *run, int rcap, int lane) {
    uint64_t *dst = run + (size_t)my_t * rcap;
    if (direct) {
#pragma unroll
        for (int e = 0; e < NS; ++e)
            if (writer && rowv[e] < rows_end)
                dst[rowv[e] - row0] = rowv[e] <= my_rlast ? make_rank_key(keyv[e], (uint32_t)rowv[e]) : 0ull;
        return;
    }
    uint64_t bal[NS];
    uint64_t any = 0ull;
#pragma unroll
    for (int e = 0; e < NS; ++e) {
        bal[e] = __ballot(writer && rowv[e] < rows_end && rowv[e] <= my_rlast && keyv[e] >= my_thr);
        any |= bal[e];
    }
    if (any == 0ull) return;
    uint32_t off = 0u;
#pragma unroll
    for (int t = 0; t < G; ++t) {
        uint32_t cnt_t = 0u;
#pragma unroll
        for (int e = 0; e < NS; ++e) cnt_t += (uint32_t)__popcll(bal[e] & qmask[t]);
        if (cnt_t != 0u) {
            uint32_t b0 = 0u;
            if (lane == 0) b0 = atomicAdd(&rcnt[t], cnt_t);
            b0 = __builtin_amdgcn_readlane(b0, 0);
            off = (my_t == t) ? b0 : off;
        }
    }
#pragma unroll
    for (int e = 0; e < NS; ++e) {
        const uint64_t m = bal[e] & my_mask;
        if ((m >> lane) & 1ull) dst[off + lanes_below(m)] = make_rank_key(keyv[e], (uint32_t)rowv[e]);
        off += (uint32_t)__popcll(m);
    }
}

template <typename T, int D, int G, int RE, bool MASS = false>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(RE <= 12 ? 4 : 2))) void score_topk_kernel(const T *__restrict__ q,
                                                         const T *__restrict__ k, TopkArgs a) {
    // LDS: run [G][rcap] (u64), hist [4][320], query rows [G][D] (T), list lengths [G],
    // admission thresholds [G].
    extern __shared__ __align__(16) uint32_t smem[];
    constexpr int EB = sizeof(T);
    constexpr int RB = D * EB;               // bytes per key row
    constexpr int LPR = RB >= 256 ? 16 : 8;  // lanes per row
    constexpr int RPG = 64 / LPR;            // rows per wavefront load
    constexpr int P = RB / (16 * LPR);       // 16-byte loads per lane per row
    constexpr int U = 8 / P;                 // row groups per wavefront round (8 loads per lane)
    // RE: run keys per lane during a cut (rcap <= 64 * RE)
    static_assert(G == 1 || G == 2 || G == 4, "G");
    static_assert(P >= 1 && P * U == 8, "rows of at least 128 bytes");

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int CH = a.chunk;
    const int cut_at = a.rcap - CH;  // a longer list might not take another chunk
    uint64_t *run = reinterpret_cast<uint64_t *>(smem);
    uint32_t *hist = smem + 2 * G * a.rcap + wave * 320;
    uint4 *qs = reinterpret_cast<uint4 *>(smem + 2 * G * a.rcap + 4 * 320);
    uint32_t *rcnt = smem + 2 * G * a.rcap + 4 * 320 + G * RB / 4;
    uint32_t *thr_s = rcnt + G;
    const int64_t nvec = (int64_t)a.g * a.nq;  // query vectors per KV head
    const int sl = lane % LPR;
    // After the row reduction lane sl of a row holds the score of query sl / (LPR / G); the
    // first lane of each such run writes it.
    const bool writer = sl % (LPR / G) == 0;
    const int my_t = sl / (LPR / G);
    uint64_t qmask[G];  // writer lanes of each query
#pragma unroll
    for (int t = 0; t < G; ++t) qmask[t] = __ballot(writer && my_t == t);
    uint64_t my_mask = qmask[0];  // writer lanes of this lane's query
#pragma unroll
    for (int t = 1; t < G; ++t) my_mask = (my_t == t) ? qmask[t] : my_mask;

    const bool shared_unit = a.wpu > 1;
    const int member = shared_unit ? (int)(blockIdx.x % a.wpu) : 0;
    const int nread = a.wpu < kSlotsRead ? a.wpu : kSlotsRead;
    for (int64_t u = shared_unit ? blockIdx.x / a.wpu : blockIdx.x; u < a.units;
         u += shared_unit ? a.units : a.nwg) {
        const int bk = (int)(u / a.groups);  // b * Hkv + kvh
        const int64_t grp = u - (int64_t)bk * a.groups;
        const int kvh = bk % a.Hkv;
        const int b = bk / a.Hkv;
        int64_t rlast[G];
        int64_t rl_max = 0;
#pragma unroll
        for (int t = 0; t < G; ++t) {
            const int64_t idx = grp * G + t;
            rlast[t] = idx < nvec ? (a.n - a.nq + idx / a.g) - a.W : 0;
            rl_max = rlast[t] > rl_max ? rlast[t] : rl_max;
        }
        if (rl_max < 1) continue;  // no query of the unit has candidates
        // The unit's query rows, staged in LDS (zero rows past the last query vector).
        if (tid < G * (RB / 16)) {
            const int t = tid / (RB / 16), w16 = tid % (RB / 16);
            const int64_t idx = grp * G + t;
            uint4 v = make_uint4(0, 0, 0, 0);
            if (idx < nvec) {
                const int h = kvh * a.g + (int)(idx % a.g);
                v = reinterpret_cast<const uint4 *>(q + (((int64_t)b * a.Hq + h) * a.nq + idx / a.g) * D)[w16];
            }
            qs[t * (RB / 16) + w16] = v;
        }
        if (tid < G) { rcnt[tid] = 0u; thr_s[tid] = 0u; }
        __syncthreads();
        int my_rlast = (int)rlast[0];
#pragma unroll
        for (int t = 1; t < G; ++t) my_rlast = (my_t == t) ? (int)rlast[t] : my_rlast;
        // Wavefront t owns query t of the unit: its running list and thresholds.
        const int64_t w_idx = grp * G + wave;
        const bool w_query = wave < G && w_idx < nvec;
        const int64_t w_rlast = w_query ? (a.n - a.nq + w_idx / a.g) - a.W : 0;
        const int64_t w_qv =
            w_query ? (((int64_t)b * a.Hq + kvh * a.g + (int)(w_idx % a.g)) * a.nq + w_idx / a.g) : 0;
        const int kq = (int)(a.topk < w_rlast ? a.topk : w_rlast);  // size of the query's top-k
        uint64_t *w_run = run + (size_t)(wave < G ? wave : 0) * a.rcap;
        uint32_t *w_tau = a.tau + w_qv * a.wpu;
        uint32_t *w_top = a.top + w_qv * a.wpu;
        // Published best keys are distinct candidates: once at least kq workgroups have
        // published one, the smallest of them is a lower bound of the k-th key.
        const bool use_min_bound = shared_unit && kq >= 1 && kq <= nread;
        int rc_seen = 0;        // list entries already scanned for the best key
        uint32_t tau_loc = 0u;  // high word of the list's k-th key once it has been cut back
        uint32_t tau_pub = 0u;  // k-th key published
        uint32_t best_loc = 0u; // best key seen
        uint32_t top_pub = 0u;  // best key published
        // Mass diagnostic: this lane's running sum for its query (writer lanes only), against a
        // reference that moves only when a score passes it by more than 64 / scale (each term
        // below 2^64).
        float zm = -INFINITY, zmc = 0.f, zl = 0.f;

        const uint4 *kbase = reinterpret_cast<const uint4 *>(k + (int64_t)bk * a.n * D);
        int64_t c = member;
        while (1 + c * CH <= rl_max) {
            const int row0 = (int)(1 + c * CH);
            const int rows_end = (int)((row0 + CH < rl_max + 1) ? row0 + CH : rl_max + 1);
            // Published bounds: requested now, reduced after the chunk's stream.
            uint32_t sl0 = 0u, sl1 = 0u, sb0 = 0u, sb1 = 0u;
            if (w_query && shared_unit) {
                if (lane < nread) sl0 = load_slot(w_tau + lane);
                if (lane + 64 < nread) sl1 = load_slot(w_tau + lane + 64);
                if (use_min_bound && lane < nread) sb0 = load_slot(w_top + lane);
                if (use_min_bound && lane + 64 < nread) sb1 = load_slot(w_top + lane + 64);
            }
            const uint32_t my_thr = thr_s[my_t];
            const bool direct = c == member;
            uint4 qr[G][P];  // this lane's slices of the queries
#pragma unroll
            for (int t = 0; t < G; ++t)
#pragma unroll
                for (int p = 0; p < P; ++p) qr[t][p] = qs[t * (RB / 16) + p * LPR + sl];
            const int ngroups = (rows_end - row0 + RPG - 1) / RPG;  // RPG rows per wavefront load
            for (int gi0 = wave; gi0 < ngroups; gi0 += 4 * U) {
                uint4 kr[U][P];
                load_round<LPR, P, U>(kbase, row0, rows_end, gi0, lane, kr);
                uint32_t keyv[U];
                int rowv[U];
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
                    const float sc = reduce_row<LPR, G>(acc, lane);
                    keyv[uu] = score_key(sc);
                    rowv[uu] = row0 + (gi0 + 4 * uu) * RPG + lane / LPR;
                    if (MASS && writer && rowv[uu] < rows_end && rowv[uu] <= my_rlast) {
                        if (sc > zm + 64.f / a.scale_log2e) {
                            zl = zm == -INFINITY ? 0.f : zl * __builtin_amdgcn_exp2f((zm - sc) * a.scale_log2e);
                            zm = sc;
                            zmc = sc * a.scale_log2e;
                        }
                        zl += __builtin_amdgcn_exp2f(__builtin_fmaf(sc, a.scale_log2e, -zmc));
                    }
                }
                emit_keys<G, U>(keyv, rowv, direct, my_thr, writer, my_t, my_rlast, row0, rows_end,
                                qmask, my_mask, rcnt, run, a.rcap, lane);
            }
            __syncthreads();

            // End of chunk: query `wave`'s list.
            if (w_query) {
                uint32_t thr = wave_max_u32_dpp(sl0 > sl1 ? sl0 : sl1);
                if (use_min_bound) {
                    int np;
                    (void)wave_excl_scan((sb0 != 0u) + (sb1 != 0u), &np);
                    if (np >= kq) {
                        const uint32_t m0 = sb0 ? sb0 : 0xFFFFFFFFu, m1 = sb1 ? sb1 : 0xFFFFFFFFu;
                        const uint32_t mb = wave_min_u32_dpp(m0 < m1 ? m0 : m1);
                        thr = thr > mb ? thr : mb;
                    }
                }
                int rc = direct ? rows_end - row0 : (int)rcnt[wave];
                if (rc > rc_seen) {
                    uint32_t bmax = 0u;
                    for (int f = rc_seen + lane; f < rc; f += 64) {
                        const uint32_t hi = (uint32_t)(w_run[f] >> 32);
                        bmax = hi > bmax ? hi : bmax;
                    }
                    bmax = wave_max_u32_dpp(bmax);
                    best_loc = bmax > best_loc ? bmax : best_loc;
                    if (rc > cut_at) {  // thin the list to about its top-k
                        uint64_t kk[RE];
#pragma unroll
                        for (int e = 0; e < RE; ++e) {
                            const int f = lane + 64 * e;
                            kk[e] = f < rc ? w_run[f] : 0ull;
                        }
                        uint32_t tk;
                        rc = wave_thin_u64(kk, a.topk, cut_at, hist, w_run, &tk);
                        tau_loc = tk > tau_loc ? tk : tau_loc;
                    }
                    if (lane == 0) rcnt[wave] = (uint32_t)rc;
                    rc_seen = rc;
                    if (shared_unit && lane == 0) {
                        if (tau_loc > tau_pub)
                            __hip_atomic_store(w_tau + member, tau_loc, __ATOMIC_RELAXED,
                                               __HIP_MEMORY_SCOPE_AGENT);
                        if (best_loc > top_pub)
                            __hip_atomic_store(w_top + member, best_loc, __ATOMIC_RELAXED,
                                               __HIP_MEMORY_SCOPE_AGENT);
                    }
                    tau_pub = tau_loc > tau_pub ? tau_loc : tau_pub;
                    top_pub = best_loc > top_pub ? best_loc : top_pub;
                }
                thr = thr > tau_loc ? thr : tau_loc;
                if (lane == 0) thr_s[wave] = thr;
            }
            __syncthreads();  // lengths and thresholds are read by every wavefront
            c += a.wpu;
        }

        if constexpr (MASS) {
            // Mass diagnostic: per query, the workgroup's lanes merged (each wavefront, then the
            // four through LDS), written by the query's wavefront.
            __shared__ float2 zred[4][G];
#pragma unroll
            for (int t = 0; t < G; ++t) {
                const float mt = wave_max_f32_dpp(my_t == t ? zm : -INFINITY);
                const float lt = wave_sum_f32_dpp(my_t == t && zm != -INFINITY
                                                      ? zl * __builtin_amdgcn_exp2f((zm - mt) * a.scale_log2e) : 0.f);
                if (lane == 0) zred[wave][t] = make_float2(mt, lt);
            }
            __syncthreads();
            if (w_query && lane == 0) {
                float mx = -INFINITY;
                for (int w = 0; w < 4; ++w) mx = fmaxf(mx, zred[w][wave].x);
                float sm = 0.f;
                for (int w = 0; w < 4; ++w)
                    sm += zred[w][wave].x == -INFINITY ? 0.f
                                                        : zred[w][wave].y * exp2f((zred[w][wave].x - mx) * a.scale_log2e);
                a.zpart[w_qv * a.wpu + member] = make_float2(mx, sm);
            }
        }
        // Leave the keys that reach the best visible bound (at most k of them), and their
        // count, in this workgroup's segment of the query.
        if (w_query) {
            int rc = (int)rcnt[wave];
            uint32_t thr = tau_loc;
            if (shared_unit) {
                uint32_t t0 = 0u, t1 = 0u;
                uint64_t m2[2] = {0ull, 0ull};
                if (lane < nread) {
                    t0 = load_slot(w_tau + lane);
                    const uint32_t bb = load_slot(w_top + lane);
                    m2[0] = bb ? make_rank_key(bb, (uint32_t)lane) : 0ull;
                }
                if (lane + 64 < nread) {
                    t1 = load_slot(w_tau + lane + 64);
                    const uint32_t bb = load_slot(w_top + lane + 64);
                    m2[1] = bb ? make_rank_key(bb, (uint32_t)(lane + 64)) : 0ull;
                }
                const uint32_t tg = wave_max_u32_dpp(t0 > t1 ? t0 : t1);
                thr = thr > tg ? thr : tg;
                // k-th largest of the published best keys (one per workgroup, so distinct).
                int have = (m2[0] != 0ull) + (m2[1] != 0ull);
                int nz;
                (void)wave_excl_scan(have, &nz);
                if (kq > 0 && nz >= kq) {
                    const uint32_t tb = wave_keep_top_u64(m2, kq, hist, nullptr);
                    thr = thr > tb ? thr : tb;
                }
            }
            // (0 entries are rows that are no candidate of the query: their high word is 0.)
            thr = thr > 1u ? thr : 1u;
            int cnt = 0;
            for (int f = lane; f < rc; f += 64) cnt += (uint32_t)(w_run[f] >> 32) >= thr;
            int tot;
            (void)wave_excl_scan(cnt, &tot);
            if (tot > a.topk) {  // more than k keys reach the bound: keep the exact top-k
                uint64_t kk[RE];
#pragma unroll
                for (int e = 0; e < RE; ++e) {
                    const int f = lane + 64 * e;
                    kk[e] = f < rc ? w_run[f] : 0ull;
                }
                const uint32_t tk = wave_keep_top_u64(kk, a.topk, hist, w_run);
                rc = a.topk;
                thr = thr > tk ? thr : tk;
                cnt = 0;
                for (int f = lane; f < rc; f += 64) cnt += (uint32_t)(w_run[f] >> 32) >= thr;
            }
            int pos = wave_excl_scan(cnt, &tot);
            uint64_t *dst = a.lists + (w_qv * a.wpu + member) * a.topk;
            for (int f = lane; f < rc; f += 64) {
                const uint64_t key = w_run[f];
                if ((uint32_t)(key >> 32) >= thr) {
                    if (pos < a.topk) dst[pos] = key;
                    ++pos;
                }
            }
            if (lane == 0) a.cnt[w_qv * a.wpu + member] = (uint32_t)(tot < a.topk ? tot : a.topk);
        }
        __syncthreads();  // LDS is reused by the next unit
    }
}

}  // namespace

size_t topk_lds_bytes(const Plan &pl) {
    return (size_t)pl.G * pl.rcap * sizeof(uint64_t) + 4 * 320 * sizeof(uint32_t) +
           (size_t)pl.G * pl.d * (pl.dtype == 1 ? 2 : 4) + 2 * (size_t)pl.G * sizeof(uint32_t);
}

hipError_t launch_score_select(const Plan &pl, const void *q, const void *k, void *ws,
                               hipStream_t s, bool mass) {
    uint32_t *tau = reinterpret_cast<uint32_t *>(static_cast<char *>(ws) + pl.slots_offset);
    const int64_t nslots = pl.nqv * pl.wpu;
    const int64_t cblocks = (2 * nslots + 255) / 256;
    hipLaunchKernelGGL(clear_words_kernel, dim3((unsigned)(cblocks < 1024 ? cblocks : 1024)), dim3(256),
                       0, s, tau, 2 * nslots);
    TopkArgs a;
    a.n = pl.n; a.nq = pl.nq; a.Hq = pl.Hq; a.Hkv = pl.Hkv; a.g = pl.g; a.W = pl.W;
    a.topk = pl.topk; a.chunk = pl.chunk; a.rcap = pl.rcap; a.groups = pl.groups;
    a.units = pl.units; a.nwg = pl.nwg; a.wpu = pl.wpu;
    a.tau = tau;
    a.top = tau + nslots;
    a.cnt = tau + 2 * nslots;
    a.lists = reinterpret_cast<uint64_t *>(static_cast<char *>(ws) + pl.lists_offset);
    a.zpart = mass ? reinterpret_cast<float2 *>(static_cast<char *>(ws) + pl.zmass_offset) : nullptr;
    a.scale_log2e = (float)(1.4426950408889634 / __builtin_sqrt((double)pl.d));
    const size_t shmem = topk_lds_bytes(pl);
    dim3 grid((unsigned)pl.nwg), block(256);
#define CA_LAUNCH_TK(T, D, G)                                                                     \
    do {                                                                                          \
        if (mass) /* (one run size for the mass variant: 24 keys per lane hold every run) */      \
            hipLaunchKernelGGL((score_topk_kernel<T, D, G, 24, true>), grid, block, shmem, s,    \
                               static_cast<const T *>(q), static_cast<const T *>(k), a);         \
        else if (pl.rcap == 512)                                                                  \
            hipLaunchKernelGGL((score_topk_kernel<T, D, G, 8>), grid, block, shmem, s,           \
                               static_cast<const T *>(q), static_cast<const T *>(k), a);         \
        else if (pl.rcap == 768)                                                                  \
            hipLaunchKernelGGL((score_topk_kernel<T, D, G, 12>), grid, block, shmem, s,          \
                               static_cast<const T *>(q), static_cast<const T *>(k), a);         \
        else                                                                                      \
            hipLaunchKernelGGL((score_topk_kernel<T, D, G, 24>), grid, block, shmem, s,          \
                               static_cast<const T *>(q), static_cast<const T *>(k), a);         \
    } while (0)
#define CA_LAUNCH_TK_G(T, D)                         \
    do {                                             \
        if (pl.G == 4) CA_LAUNCH_TK(T, D, 4);        \
        else if (pl.G == 2) CA_LAUNCH_TK(T, D, 2);   \
        else CA_LAUNCH_TK(T, D, 1);                  \
    } while (0)
    if (pl.dtype == 1) {
        if (pl.d == 128) CA_LAUNCH_TK_G(__bf16, 128); else CA_LAUNCH_TK_G(__bf16, 64);
    } else {
        if (pl.d == 128) CA_LAUNCH_TK_G(float, 128); else CA_LAUNCH_TK_G(float, 64);
    }
#undef CA_LAUNCH_TK_G
#undef CA_LAUNCH_TK
    return hipGetLastError();
}

}  // namespace ca
