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
// 128-byte lines per instruction), computes fp32 dot products for its G queries (bf16 dot2 or
// fp32 FMA, DPP lane reductions), and keeps the score keys in LDS. Then wavefront t updates
// query t's running list: keys below the admission threshold are dropped, the rest are added,
// and a list longer than k is cut back to its exact top-k (radix select). The threshold is the
// largest of the list's own k-th key and the k-th keys the unit's other workgroups have
// published in their slots; every one of them is a lower bound of the query's final k-th key,
// so no member of the final top-k is ever dropped. Each workgroup also publishes its best key;
// the k'-th largest of those (distinct keys, one per workgroup) is a lower bound too, and a much
// tighter one. At the end each workgroup writes the keys of its list that reach the best bound
// it can see, and their count, to its own segment. No two workgroups write the same word, so
// nothing waits on a contended atomic.
#include "ca_internal.h"
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
};

constexpr int kSlotsRead = 128;  // published slots a workgroup reads (the first ones)

__global__ __launch_bounds__(256) void clear_words_kernel(uint32_t *__restrict__ w, int64_t n) {
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256)
        w[i] = 0u;
}

__device__ __forceinline__ uint32_t load_slot(const uint32_t *p) {
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Loads the K rows of one streaming round: row groups gi0 + 4*uu (8 rows each) of the chunk
// [r0, rend). Rows past the chunk's end are clamped to its last row (loaded, never used), so
// every load is unconditional.
template <int P, int U>
__device__ __forceinline__ void load_round(const uint4 *__restrict__ kbase, int r0, int rend, int gi0,
                                           int lane, uint4 (&dst)[U][P]) {
    constexpr int RQ = P * 8;  // 16-byte words per row
    const int s = lane & 7;
#pragma unroll
    for (int uu = 0; uu < U; ++uu) {
        int row = r0 + (gi0 + 4 * uu) * 8 + (lane >> 3);
        row = row < rend ? row : rend - 1;
        const uint4 *src = kbase + (int64_t)row * RQ;
#pragma unroll
        for (int p = 0; p < P; ++p) dst[uu][p] = src[p * 8 + s];
    }
}

template <typename T, int D, int G, int RE>
__global__ __launch_bounds__(256) void score_topk_kernel(const T *__restrict__ q,
                                                         const T *__restrict__ k, TopkArgs a) {
    // LDS: keys32 [G][chunk], run [G][rcap] (u64), hist [4][320], query rows [G][D] (T)
    extern __shared__ __align__(16) uint32_t smem[];
    constexpr int EB = sizeof(T);
    constexpr int RB = D * EB;          // bytes per key row
    constexpr int P = RB / 128;         // 16-byte loads per lane per row (8 lanes per row)
    constexpr int U = 8 / P;            // row groups (8 rows each) per wavefront round
    // RE: run keys per lane during a cut (rcap == 64 * RE)
    static_assert(G == 1 || G == 2 || G == 4, "G");
    static_assert(P >= 1, "rows of at least 128 bytes");

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int CH = a.chunk;
    const int cut_at = a.rcap - CH;  // a longer list could not take another chunk
    uint32_t *keys32 = smem;
    uint64_t *run = reinterpret_cast<uint64_t *>(smem + G * CH);
    uint32_t *hist = smem + G * CH + 2 * G * a.rcap + wave * 320;
    uint4 *qs = reinterpret_cast<uint4 *>(smem + G * CH + 2 * G * a.rcap + 4 * 320);  // [G][RB/16]
    const int64_t nvec = (int64_t)a.g * a.nq;  // query vectors per KV head
    const int s = lane & 7;
    // After the 8-lane reduction the even lanes own one query's score each: query
    // 2*bit2 + bit1 of the lane (G == 4); lanes 0 and 4 of 8 own queries 0 and 1 (G == 2);
    // lane 0 of 8 owns query 0 (G == 1).
    const int my_t = (G == 4) ? (((lane >> 2) & 1) * 2 + ((lane >> 1) & 1)) : (G == 2) ? ((lane >> 2) & 1) : 0;
    const bool writer = (G == 4) ? ((lane & 1) == 0) : (G == 2) ? ((lane & 3) == 0) : ((lane & 7) == 0);

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
        __syncthreads();
        int64_t my_rlast = rlast[0];
#pragma unroll
        for (int t = 1; t < G; ++t) my_rlast = (my_t == t) ? rlast[t] : my_rlast;
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
        // The first kq workgroups' best keys are kq distinct candidates: their minimum is a
        // lower bound of the k-th key once all of them have published.
        const bool use_min_bound = shared_unit && kq >= 1 && kq <= 64 && kq <= nread;
        int rc = 0;             // keys in the running list
        uint32_t tau_loc = 0u;  // high word of its k-th key once it has been cut back
        uint32_t tau_pub = 0u;  // k-th key published
        uint32_t best_loc = 0u; // best key seen
        uint32_t top_pub = 0u;  // best key published

        const uint4 *kbase = reinterpret_cast<const uint4 *>(k + (int64_t)bk * a.n * D);
        int64_t c = member;
        while (1 + c * CH <= rl_max) {
            const int64_t row0 = 1 + c * CH;
            const int64_t rows_end = (row0 + CH < rl_max + 1) ? row0 + CH : rl_max + 1;
            const int nrows = (int)(rows_end - row0);
            const int64_t cn = c + a.wpu;
            // Published bounds: requested now, reduced after the chunk's stream.
            uint32_t sl0 = 0u, sl1 = 0u, sb = 0xFFFFFFFFu;
            if (w_query && shared_unit) {
                if (lane < nread) sl0 = load_slot(w_tau + lane);
                if (lane + 64 < nread) sl1 = load_slot(w_tau + lane + 64);
                if (use_min_bound && lane < kq) sb = load_slot(w_top + lane);
            }

            uint4 qr[G][P];  // this lane's slices of the queries
#pragma unroll
            for (int t = 0; t < G; ++t)
#pragma unroll
                for (int p = 0; p < P; ++p) qr[t][p] = qs[t * (RB / 16) + p * 8 + s];
            const int ngroups = (nrows + 7) >> 3;  // 8 rows per wavefront step
            for (int gi0 = wave; gi0 < ngroups; gi0 += 4 * U) {
                uint4 kr[U][P];
                load_round<P, U>(kbase, (int)row0, (int)rows_end, gi0, lane, kr);
#pragma unroll
                for (int uu = 0; uu < U; ++uu) {
                    const int gi = gi0 + 4 * uu;
                    float acc[G];
#pragma unroll
                    for (int t = 0; t < G; ++t) {
                        float x = 0.f;
#pragma unroll
                        for (int p = 0; p < P; ++p) x = dot16(kr[uu][p], qr[t][p], x, T());
                        acc[t] = x;
                    }
                    // Sum over the 8 lanes of the row, halving the queries per lane at each
                    // exchange while there are several.
                    float score;
                    if constexpr (G == 4) {
                        const bool hi = (lane & 4) != 0;
                        const float k0 = hi ? acc[2] : acc[0], s0 = hi ? acc[0] : acc[2];
                        const float k1 = hi ? acc[3] : acc[1], s1 = hi ? acc[1] : acc[3];
                        const float a0 = k0 + dpp_half_mirror(s0);
                        const float a1 = k1 + dpp_half_mirror(s1);
                        const bool hi1 = (lane & 2) != 0;
                        const float kk = hi1 ? a1 : a0, ss = hi1 ? a0 : a1;
                        const float b0 = kk + dpp_xor2(ss);
                        score = b0 + dpp_xor1(b0);
                    } else if constexpr (G == 2) {
                        const bool hi = (lane & 4) != 0;
                        const float kk = hi ? acc[1] : acc[0], ss = hi ? acc[0] : acc[1];
                        float a0 = kk + dpp_half_mirror(ss);
                        a0 += dpp_xor2(a0);
                        score = a0 + dpp_xor1(a0);
                    } else {
                        float a0 = acc[0] + dpp_half_mirror(acc[0]);
                        a0 += dpp_xor2(a0);
                        score = a0 + dpp_xor1(a0);
                    }
                    const int rr = gi * 8 + (lane >> 3);
                    if (writer && rr < nrows)
                        keys32[my_t * CH + rr] = (row0 + rr <= my_rlast) ? score_key(score) : 0u;
                }
            }
            __syncthreads();

            // Running-list update of query `wave`.
            if (w_query) {
                const int64_t vend = (rows_end < w_rlast + 1) ? rows_end : w_rlast + 1;
                const int nvalid = vend > row0 ? (int)(vend - row0) : 0;
                if (nvalid > 0) {
                    uint32_t thr = wave_max_u32_dpp(sl0 > sl1 ? sl0 : sl1);
                    thr = thr > tau_loc ? thr : tau_loc;
                    if (use_min_bound) {
                        const uint32_t mb = wave_min_u32_dpp(sb);
                        thr = thr > mb ? thr : mb;
                    }
                    const uint32_t *kq32 = keys32 + wave * CH;
                    int cnt = 0;
                    uint32_t bmax = 0u;
                    for (int e0 = 4 * lane; e0 < nvalid; e0 += 256) {
                        const uint4 v = *reinterpret_cast<const uint4 *>(kq32 + e0);
                        const uint32_t kv[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
                        for (int t4 = 0; t4 < 4; ++t4) {
                            const bool ok = e0 + t4 < nvalid && kv[t4] >= thr && kv[t4] != 0u;
                            cnt += ok;
                            bmax = (ok && kv[t4] > bmax) ? kv[t4] : bmax;
                        }
                    }
                    int tot;
                    int pos = rc + wave_excl_scan(cnt, &tot);
                    if (tot > 0) {
                        for (int e0 = 4 * lane; e0 < nvalid; e0 += 256) {
                            const uint4 v = *reinterpret_cast<const uint4 *>(kq32 + e0);
                            const uint32_t kv[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
                            for (int t4 = 0; t4 < 4; ++t4) {
                                if (e0 + t4 < nvalid && kv[t4] >= thr && kv[t4] != 0u) {
                                    w_run[pos] = make_rank_key(kv[t4], (uint32_t)(row0 + e0 + t4));
                                    ++pos;
                                }
                            }
                        }
                        rc += tot;
                        bmax = wave_max_u32_dpp(bmax);
                        best_loc = bmax > best_loc ? bmax : best_loc;
                        if (rc > cut_at) {  // cut back to the exact top-k
                            wave_sync();
                            uint64_t kk[RE];
#pragma unroll
                            for (int e = 0; e < RE; ++e) {
                                const int f = lane + 64 * e;
                                kk[e] = f < rc ? w_run[f] : 0ull;
                            }
                            tau_loc = wave_keep_top_u64(kk, a.topk, hist, w_run);
                            rc = a.topk;
                        }
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
                }
            }
            __syncthreads();  // keys32 is rewritten for the next chunk
            c = cn;
        }

        // Leave the keys that reach the best visible bound (at most k of them), and their
        // count, in this workgroup's segment of the query.
        if (w_query) {
            wave_sync();
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
            // A later unit of this workgroup rereads the slots of another query only.
        }
        __syncthreads();  // LDS is reused by the next unit
    }
}

}  // namespace

size_t topk_lds_bytes(const Plan &pl) {
    return (size_t)pl.G * pl.chunk * sizeof(uint32_t) + (size_t)pl.G * pl.rcap * sizeof(uint64_t) +
           4 * 320 * sizeof(uint32_t) + (size_t)pl.G * pl.d * (pl.dtype == 1 ? 2 : 4);
}

hipError_t launch_score_select(const Plan &pl, const void *q, const void *k, void *ws,
                               hipStream_t s) {
    uint32_t *tau = static_cast<uint32_t *>(ws);
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
    const size_t shmem = topk_lds_bytes(pl);
    dim3 grid((unsigned)pl.nwg), block(256);
#define CA_LAUNCH_TK(T, D, G)                                                                     \
    do {                                                                                          \
        if (pl.rcap == 512)                                                                       \
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
