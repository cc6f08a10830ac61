// Stage 1 of condensate attention for prefill-shaped problems with bf16 inputs on gfx950 (pages
// of "The Condensate Theorem", metaphor-xennon blog: section 2.1, S = QK^T / sqrt(d) and
// Definition 1, C_i = {0} u {i-W+1..i} u Top-k_i; section 2.2.3, the top-k part over the
// positions R_i = {1..i-W}).
//
// When many query vectors read the same KV head, their scores are a dense product, computed
// here on the matrix cores: v_mfma_f32_16x16x32_bf16 multiplies 16 key rows by 16 query vectors
// over 32 elements of d per instruction, accumulating in fp32. A workgroup takes 16*QB*NWV query
// vectors of one KV head (NWV wavefronts of 16*QB, whose slices stay in registers) and brings the
// key rows 0..max(i - W) through LDS in tiles of 64 rows: a ring of four tiles filled straight
// from memory (global_load_lds) three tiles ahead of their use, the 16-byte chunks of a row
// XOR-swizzled so that the operand reads of 16 rows hit distinct banks. The scores are
// the plain dot products: the positive factor 1/sqrt(d) changes no order.
//
// The exact top-k' of R_i (k' = min(k, |R_i|) <= 128) takes two passes over the same products
// (the same instruction sequence, hence bit-identical scores):
//   bound  For each query, one score of its candidate rows in each of 128 disjoint classes (a
//          row's place in its pair of tiles; the class maximum whenever the class holds a
//          non-negative score), so k' distinct rows reach the k'-th largest of those scores: a
//          lower bound of the query's k'-th score. The lower edge of the 16-bit radix bin that
//          holds it goes out as a score key. A bound from a subset of the rows is a lower bound
//          too, only a looser one: with k <= 64 the pass reads KEEP of every 4 tiles (2 for
//          k <= 32, 3 for k <= 64), trading its products for more appends in the next pass
//          (about 1.25 k * 4 / KEEP rows reach it, within the lists' 256 entries).
//   cand   Every candidate row whose score key reaches the bound is appended to the query's
//          list as a ranking key (about 1.25 k * 4 / KEEP of them on Gaussian data). A list that might
//          not take another tile is cut to its exact top-k' (wave_keep_top_u64); from then on
//          only keys above the k'-th kept one are appended, since later rows have larger
//          positions and rank lower on equal scores.
// The lists go out as the segments the finish kernel merges: [nqv][wpu][topk] ranking keys
// and [nqv][wpu] lengths, the list of a query filling its segments in order.
#include "ca_internal.h"
#include "device_utils.h"
#include "select_core.h"

namespace ca {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

constexpr int kTile = 64;      // key rows per LDS tile
constexpr int kBuf = 4;        // LDS ring of tiles: rows arrive three tiles ahead of their use
constexpr int kXcds = 8;       // workgroups are dealt to the XCDs in turn
constexpr int kMaxKeep = 128;  // largest k' of the path
constexpr int kLanesPerQuery = 4;  // lanes that hold one query's scores
constexpr int kCutE = kLanesPerQuery * kMfmaSeg / 64;  // keys per lane in a list cut
// A lane's list takes at most 16 keys per tile (4 blocks x 4 rows); it is cut before it might
// not, and a cut leaves at most kMaxKeep / 4 keys in each of a query's lists.
static_assert(kMaxKeep / kLanesPerQuery + 16 <= kMfmaSeg, "list room");

__device__ __forceinline__ int wave_of_thread() { return __builtin_amdgcn_readfirstlane(threadIdx.x >> 6); }

struct MfmaArgs {
    int64_t n, nq;
    int Hq, Hkv, g, W, topk;
    uint32_t nvec;         // query vectors per KV head (g * nq)
    uint32_t wg_per_unit;  // workgroups per (batch, KV head)
    uint32_t nwg;          // workgroups of the launch
    uint32_t *tau;         // [nqv] bound of each query (score key; 0xFFFFFFFF: no candidates)
    uint32_t *cnt;         // [nqv][4] list lengths
    uint64_t *lists;       // [nqv][4][kMfmaSeg] ranking keys: list g is kept by lane group g
    float scale_log2e;     // log2(e) / sqrt(d)
    float2 *zmass;         // bound pass with the mass diagnostic: [nqv] (m, l), l = sum over R_i
                           // of exp2((s - m) * scale_log2e), m within 64 / scale_log2e of the best s
};

// Running softmax sum over a lane's scores against a reference score m: l = sum of
// exp2((s - m) * c). The reference moves (and l is rescaled) only when a score passes it by more
// than 64 / c, so each term stays below 2^64 and most calls take one fma and one exponential per
// score. mc = m * c.
__device__ __forceinline__ void softmax_fold(float &m, float &mc, float &l, float bm, float c,
                                             const float (&s)[4], const bool (&ok)[4]) {
    if (bm > m + 64.f / c) {
        const float mn = bm;
        l = m == -INFINITY ? 0.f : l * __builtin_amdgcn_exp2f((m - mn) * c);
        m = mn;
        mc = mn * c;
    }
    float add = 0.f;
#pragma unroll
    for (int r = 0; r < 4; ++r) add += ok[r] ? __builtin_amdgcn_exp2f(__builtin_fmaf(s[r], c, -mc)) : 0.f;
    l += add;
}

// Inverse of score_key for the admission test in float: keys below every finite score give
// -inf, the "no candidates" key 0xFFFFFFFF gives +inf.
__device__ __forceinline__ float key_floor_float(uint32_t key) {
    if (key < 0x00800000u) return -INFINITY;
    if (key == 0xFFFFFFFFu) return INFINITY;
    return __uint_as_float(key & 0x80000000u ? key & 0x7FFFFFFFu : ~key);
}

// Sum over the four lanes col, col + 16, col + 32, col + 48 (the lanes that hold one query).
__device__ __forceinline__ uint32_t quad_sum_u32(uint32_t x) {
    const auto r16 = __builtin_amdgcn_permlane16_swap(x, x, false, false);
    x = r16[0] + r16[1];
    const auto r32 = __builtin_amdgcn_permlane32_swap(x, x, false, false);
    return r32[0] + r32[1];
}
// Float sum over the same four lanes (bits in, bits out), in a fixed order.
__device__ __forceinline__ uint32_t quad_sum_f32_bits(uint32_t x) {
    const auto r16 = __builtin_amdgcn_permlane16_swap(x, x, false, false);
    float y = __uint_as_float(r16[0]) + __uint_as_float(r16[1]);
    const auto r32 = __builtin_amdgcn_permlane32_swap(__float_as_uint(y), __float_as_uint(y), false, false);
    return __float_as_uint(__uint_as_float(r32[0]) + __uint_as_float(r32[1]));
}
// Float maximum over the same four lanes.
__device__ __forceinline__ float quad_max_f32(float x) {
    const auto r16 = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    const float y = fmaxf(__uint_as_float(r16[0]), __uint_as_float(r16[1]));
    const auto r32 = __builtin_amdgcn_permlane32_swap(__float_as_uint(y), __float_as_uint(y), false, false);
    return fmaxf(__uint_as_float(r32[0]), __uint_as_float(r32[1]));
}
__device__ __forceinline__ uint32_t quad_max_u32(uint32_t x) {
    const auto r16 = __builtin_amdgcn_permlane16_swap(x, x, false, false);
    x = r16[0] > r16[1] ? r16[0] : r16[1];
    const auto r32 = __builtin_amdgcn_permlane32_swap(x, x, false, false);
    return r32[0] > r32[1] ? r32[0] : r32[1];
}
__device__ __forceinline__ uint32_t quad_min_u32(uint32_t x) {
    const auto r16 = __builtin_amdgcn_permlane16_swap(x, x, false, false);
    x = r16[0] < r16[1] ? r16[0] : r16[1];
    const auto r32 = __builtin_amdgcn_permlane32_swap(x, x, false, false);
    return r32[0] < r32[1] ? r32[0] : r32[1];
}

// Chunk c of key row `row` of a tile sits at chunk (c ^ swizzle) of the row: 16 consecutive rows
// then cover 16 distinct 16-byte bank groups (rows of 256 bytes: row & 15; of 128 bytes, two
// rows share 256 bytes: (row >> 1) & 7).
template <int D>
__device__ __forceinline__ int chunk_swizzle(int row) {
    return D == 128 ? (row & 15) : ((row >> 1) & 7);
}
template <int D>
__device__ __forceinline__ int chunk_at(int row, int c) {
    return row * (D / 8) + (c ^ chunk_swizzle<D>(row));
}

template <int D, int QB, bool CAND, bool PRE, int NWV, bool MASS = false, int KEEP = 4>
__global__ __launch_bounds__(64 * NWV) void mfma_select_kernel(const __bf16 *__restrict__ q,
                                                          const __bf16 *__restrict__ k,
                                                          MfmaArgs a) {
    constexpr int KS = D / 32;                  // MFMA steps over d
    constexpr int CPR = D / 8;                  // 16-byte chunks per key row
    constexpr int NT = 64 * NWV;                // threads per workgroup
    constexpr int NCH = kTile * CPR / NT;       // chunks per thread per tile
    constexpr int QW = 16 * QB;                 // query vectors per wavefront
    constexpr int ROWS = NWV * QW;              // per workgroup
    static_assert(NCH >= 1 && NCH * NT == kTile * CPR, "tile");
    // s_waitcnt with vmcnt = the loads a wavefront issues for kBuf - 2 tiles (expcnt and
    // lgkmcnt at their maxima: no wait on them).
    constexpr int kAhead = NCH * (kBuf - 2);
    constexpr int kWaitAhead = (kAhead & 15) | (7 << 4) | (15 << 8) | ((kAhead >> 4) << 14);
    // One LDS object: the tile ring, then (candidate pass) per wavefront the histogram of a list
    // cut and the keys it keeps. (With several LDS objects the compiler waits for every tile in
    // flight before each operand read; the waits below are the ones needed.)
    constexpr int kCutWords = 320 + 2 * kMaxKeep;
    constexpr int kExtra = CAND ? NWV * kCutWords / 4 : 0;
    __shared__ uint4 smem[kBuf * kTile * CPR + kExtra];
    uint4 (*kt)[kTile * CPR] = reinterpret_cast<uint4 (*)[kTile * CPR]>(smem);
    uint32_t *cutw = reinterpret_cast<uint32_t *>(smem + kBuf * kTile * CPR) + wave_of_thread() * kCutWords;

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int col = lane & 15, grp = lane >> 4;
    // Consecutive logical workgroups (the query vectors of one KV head, which read the same
    // key rows) go to the same XCD and share its L2.
    const uint32_t bid = blockIdx.x, xcd = bid % kXcds;
    const uint32_t per = a.nwg / kXcds, rem = a.nwg % kXcds;
    const uint32_t L = xcd * per + (xcd < rem ? xcd : rem) + bid / kXcds;
    const uint32_t bk = L / a.wg_per_unit;             // b * Hkv + kvh
    const uint32_t part = L - bk * a.wg_per_unit;
    const uint32_t b = bk / (uint32_t)a.Hkv, kvh = bk - b * (uint32_t)a.Hkv;
    const uint32_t g = (uint32_t)a.g;
    const uint32_t idx_w = part * ROWS + wave * QW;    // first vector of this wavefront

    // Vector idx of the KV head is query head kvh*g + idx % g at row idx / g (position
    // n - nq + idx / g).
    auto vec_of = [&](uint32_t idx, uint32_t &qv, int &lim) {
        const uint32_t r = idx / g, hh = idx - r * g;
        qv = ((b * (uint32_t)a.Hq + kvh * g + hh) * (uint32_t)a.nq) + r;
        lim = (int)(a.n - a.nq + r) - a.W;  // last candidate row (< 1: none)
    };
    bf16x8_t qf[QB][KS];
    int lim[QB], kq[QB];
    uint32_t qvi[QB];
    int lim_lo = INT32_MAX, lim_hi = 0;
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
        const uint32_t idx = idx_w + qb * 16 + col;
        const bool valid = idx < a.nvec;
        int lm;
        vec_of(valid ? idx : 0u, qvi[qb], lm);
        lim[qb] = valid && lm >= 1 ? lm : -1;
        kq[qb] = lim[qb] >= 1 ? (a.topk < lim[qb] ? a.topk : lim[qb]) : 0;
        const uint4 *src = reinterpret_cast<const uint4 *>(q + (size_t)qvi[qb] * D);
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
            qf[qb][ks] = __builtin_bit_cast(bf16x8_t, valid ? src[ks * 4 + grp] : make_uint4(0, 0, 0, 0));
        if (kq[qb] > 0) {
            lim_lo = lim[qb] < lim_lo ? lim[qb] : lim_lo;
            lim_hi = lim[qb] > lim_hi ? lim[qb] : lim_hi;
        }
    }
    // Wave-uniform row range of the wavefront's queries with candidates: no row mask is needed
    // for tiles inside [1, lim_lo]; nothing to do past lim_hi.
    lim_lo = (int)wave_min_u32_dpp((uint32_t)lim_lo);
    lim_hi = (int)wave_max_u32_dpp((uint32_t)lim_hi);
    const int t_wave = lim_hi >= 1 ? lim_hi / kTile : -1;
    // Tiles of the workgroup: rows 0 .. the last vector's last candidate row.
    int jmax;
    {
        const uint32_t last = (part + 1) * ROWS < a.nvec ? (part + 1) * ROWS - 1 : a.nvec - 1;
        uint32_t qv_last;
        vec_of(last, qv_last, jmax);
    }
    const int ntiles = jmax >= 1 ? jmax / kTile + 1 : 0;
    // Step v takes tile tile_of(v): every tile, or (bound pass without the mass sum) the first
    // KEEP of every 4.
    constexpr int kKeep = !CAND && !MASS ? KEEP : 4;
    static_assert(kKeep >= 2 && kKeep <= 4, "keep");
    auto tile_of = [](int v) { return kKeep == 4 ? v : (v / kKeep) * 4 + v % kKeep; };
    const int nsteps = (ntiles / 4) * kKeep + (ntiles % 4 < kKeep ? ntiles % 4 : kKeep);

    // Candidate pass: admission key of each query (a score is appended when its key reaches
    // adm, tested first as a float against tf) and the length of this lane's list of it.
    float tf[QB];
    int32_t ti[QB];  // tf's bits when tf > 0, else INT32_MIN: the block pre-test below
    uint32_t adm[QB], lc[QB];
    uint64_t *lbase[QB];  // this lane's list of each query
    if constexpr (CAND) {
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) {
            adm[qb] = kq[qb] > 0 ? a.tau[qvi[qb]] : 0xFFFFFFFFu;
            tf[qb] = key_floor_float(adm[qb]);
            ti[qb] = tf[qb] > 0.f ? __float_as_int(tf[qb]) : INT32_MIN;
            lc[qb] = 0u;
            lbase[qb] = a.lists + ((size_t)qvi[qb] * kLanesPerQuery + grp) * kMfmaSeg;
        }
    }
    // [tile parity][16-row block][row of the lane][query]: per class, the largest score as a
    // signed integer over the float's bits. That order agrees with the float order for every
    // pair that holds a non-negative score, so a class with one gets its maximum; a class with
    // only negative scores gets one of them (the most negative) and one with none gets INT_MIN
    // (the bits of -0.0, read as "no row"). Every value kept is the score of a row of its class,
    // which is all the bound needs, and the maximum costs one integer instruction per score (a
    // float maximum would first quiet each product as a possible NaN).
    int32_t m[2][4][4][QB];
    // Mass diagnostic (bound pass): this lane's softmax sum over its candidate scores per query.
    float zm[QB], zmc[QB], zl[QB];
    if constexpr (MASS) {
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) {
            zm[qb] = -INFINITY;
            zmc[qb] = 0.f;
            zl[qb] = 0.f;
        }
    }
    if constexpr (!CAND) {
#pragma unroll
        for (int p = 0; p < 2; ++p)
#pragma unroll
            for (int kb = 0; kb < 4; ++kb)
#pragma unroll
                for (int r = 0; r < 4; ++r)
#pragma unroll
                    for (int qb = 0; qb < QB; ++qb) m[p][kb][r][qb] = INT32_MIN;
    }

    const __bf16 *kbase = k + (size_t)bk * (size_t)a.n * D;
    const int nlast = (int)a.n - 1;
    // The wavefronts' share of tile t, straight from memory into LDS buffer B: instruction u of
    // wavefront w fills chunks (NWV*u + w)*64 .. +63 of the tile, lane by lane (16 bytes each), so
    // lane l fetches the row chunk that the swizzle puts there: row lrow[u] of the tile, chunk
    // byte offset coff[u]. Rows past n - 1 are clamped. Addresses are the KV head's base plus a
    // 32-bit byte offset (the plan keeps a KV head's rows below 4 GiB).
    int lrow[NCH];
    uint32_t coff[NCH];
#pragma unroll
    for (int u = 0; u < NCH; ++u) {
        const int p = (u * NWV + wave) * 64 + lane;
        const int row = p / CPR, c = (p % CPR) ^ chunk_swizzle<D>(row);
        lrow[u] = row;
        coff[u] = (uint32_t)c * 16u;
    }
    const char *kbytes = reinterpret_cast<const char *>(kbase);
    auto issue = [&](int t, auto bufc) {
        constexpr int B = decltype(bufc)::value;
        const int j0 = tile_of(t) * kTile;
#pragma unroll
        for (int u = 0; u < NCH; ++u) {
            const int j = j0 + lrow[u];
            const uint32_t off = (uint32_t)(j < nlast ? j : nlast) * (uint32_t)(D * sizeof(__bf16)) + coff[u];
            __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void *)(kbytes + off),
                                             (__attribute__((address_space(3))) void *)&kt[B][(u * NWV + wave) * 64],
                                             16, 0, 0);
        }
    };

    // Cut of the four lists of query col c of block QBC (wavefront-uniform): the exact top-k'
    // of their keys so far (wave_keep_top_u64), dealt back to the lists in turn (key e to list
    // e mod 4). When k' keys are kept, a later row can only enter with a larger score: its
    // position is larger than theirs.
    auto cut_list = [&](auto qbc, int c) {
        constexpr int QBC = decltype(qbc)::value;
        const uint32_t qv = __builtin_amdgcn_readlane(qvi[QBC], c);
        const int lm = __builtin_amdgcn_readlane(lim[QBC], c);
        const int keep = a.topk < lm ? a.topk : lm;
        uint32_t n4[kLanesPerQuery];
        int total = 0;
#pragma unroll
        for (int gq = 0; gq < kLanesPerQuery; ++gq) {
            n4[gq] = __builtin_amdgcn_readlane(lc[QBC], c + 16 * gq);
            total += (int)n4[gq];
        }
        uint64_t *lst = a.lists + (size_t)qv * (kLanesPerQuery * kMfmaSeg);
        __threadfence_block();  // this wavefront's appends are visible to its loads
        uint64_t kr[kCutE];
#pragma unroll
        for (int e = 0; e < kCutE; ++e) {
            const int f = lane + 64 * e, gq = f / kMfmaSeg;
            kr[e] = (uint32_t)(f % kMfmaSeg) < n4[gq] ? lst[f] : 0ull;
        }
        uint64_t *kept = reinterpret_cast<uint64_t *>(cutw + 320);
        const uint32_t hi = wave_keep_top_u64(kr, keep, cutw, kept);
        const int nk = total < keep ? total : keep;
        for (int e = lane; e < nk; e += 64) lst[(e % kLanesPerQuery) * kMfmaSeg + e / kLanesPerQuery] = kept[e];
        __threadfence_block();
        if (col == c) {
            lc[QBC] = (uint32_t)((nk - grp + kLanesPerQuery - 1) / kLanesPerQuery);
            if (total >= keep) {
                adm[QBC] = hi + 1u > adm[QBC] ? hi + 1u : adm[QBC];
                tf[QBC] = key_floor_float(adm[QBC]);
                ti[QBC] = tf[QBC] > 0.f ? __float_as_int(tf[QBC]) : INT32_MIN;
            }
        }
    };

    // Products of tile t (LDS buffer B, t = B mod kBuf, so t & 1 = B & 1) with this wavefront's
    // queries: four blocks of 16 rows; the products of block kb + 1 are issued before block kb
    // is examined.
    auto compute = [&](int t, auto bufc) {
        constexpr int B = decltype(bufc)::value;
        constexpr int P = B & 1;
        const int j0 = tile_of(t) * kTile;
        const bool inner = j0 >= 1 && j0 + kTile - 1 <= lim_lo;
        // Operand rows of block kb from LDS. The bound pass issues them a block ahead of their
        // products, with a scheduling barrier that keeps the compiler from moving the products
        // above them (measured: bound pass -4%; the branchy candidate pass is faster in the
        // compiler's own order, reads next to their products).
        auto operands = [&](int kb, bf16x8_t (&af)[KS]) {
            const int row = kb * 16 + col;
#pragma unroll
            for (int ks = 0; ks < KS; ++ks)
                af[ks] = __builtin_bit_cast(bf16x8_t, kt[B][chunk_at<D>(row, ks * 4 + grp)]);
            if constexpr (!CAND) __builtin_amdgcn_sched_barrier(0);
        };
        auto products = [&](const bf16x8_t (&af)[KS], f32x4_t (&acc)[QB]) {
#pragma unroll
            for (int qb = 0; qb < QB; ++qb) acc[qb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ks = 0; ks < KS; ++ks)
#pragma unroll
                for (int qb = 0; qb < QB; ++qb)
                    acc[qb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[ks], qf[qb][ks], acc[qb], 0, 0, 0);
        };
        // acc[qb][r]: row jb + r of the tile for query qb*16 + col.
        auto examine = [&](auto kbc, const f32x4_t (&acc)[QB], auto innerc) {
            constexpr int kb = decltype(kbc)::value;
            constexpr bool INNER = decltype(innerc)::value;
            const int jb = j0 + kb * 16 + 4 * grp;
            if constexpr (!CAND) {
#pragma unroll
                for (int qb = 0; qb < QB; ++qb)
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        int32_t v = __float_as_int(acc[qb][r]);
                        if constexpr (!INNER) v = (jb + r >= 1 && jb + r <= lim[qb]) ? v : INT32_MIN;
                        m[P][kb][r][qb] = v > m[P][kb][r][qb] ? v : m[P][kb][r][qb];
                    }
                if constexpr (MASS) {
#pragma unroll
                    for (int qb = 0; qb < QB; ++qb) {
                        float sv[4];
                        bool ok[4];
                        float bm = -INFINITY;
#pragma unroll
                        for (int r = 0; r < 4; ++r) {
                            sv[r] = acc[qb][r];
                            ok[r] = INNER || (jb + r >= 1 && jb + r <= lim[qb]);
                            if (ok[r]) bm = fmaxf(bm, sv[r]);
                        }
                        softmax_fold(zm[qb], zmc[qb], zl[qb], bm, a.scale_log2e, sv, ok);
                    }
                }
            } else {
                // About 1.25 k * 4 / KEEP of a query's rows reach its bound, so a block of 16 rows
                // holds few of them. With PRE, per query block, a test of the largest of a
                // lane's four scores as signed integers over their bits (for tf > 0 the same
                // order as the float compare against tf; for other tf it lets everything
                // through): when no lane passes it, the block's 64 scores cost one branch. Then
                // each row slot with a score that passes in some lane appends it.
#pragma unroll
                for (int qb = 0; qb < QB; ++qb) {
                    if constexpr (PRE) {
                        const int32_t b01 = max(__float_as_int(acc[qb][0]), __float_as_int(acc[qb][1]));
                        const int32_t b23 = max(__float_as_int(acc[qb][2]), __float_as_int(acc[qb][3]));
                        if (__builtin_expect(__ballot(max(b01, b23) >= ti[qb]) == 0ull, 1)) continue;
                    }
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const float v = acc[qb][r];
                        bool h = v >= tf[qb];
                        if constexpr (!INNER) h = h && jb + r >= 1 && jb + r <= lim[qb];
                        // (v >= tf is key >= adm: score_key orders every non-NaN float as
                        // the float compare does, -0 and +0 alike.)
                        if (__builtin_expect(__ballot(h) != 0ull, 0) && h) {
                            lbase[qb][lc[qb]] = make_rank_key(score_key(v), (uint32_t)(jb + r));
                            ++lc[qb];
                        }
                    }
                }
                // (These stores may still be in flight at the next tile's wait: loads complete
                // in order among themselves, so the wait still covers the tile.)
            }
        };
        // Tiles inside every query's candidate rows need no row mask: a separate copy of the
        // code, so that no test is made per score.
        auto run = [&](auto innerc) {
            f32x4_t acc0[QB], acc1[QB];
            bf16x8_t a0[KS], a1[KS];
            if constexpr (CAND) {
                operands(0, a0);
                products(a0, acc0);
                operands(1, a1);
                products(a1, acc1);
                examine(std::integral_constant<int, 0>(), acc0, innerc);
                operands(2, a0);
                products(a0, acc0);
                examine(std::integral_constant<int, 1>(), acc1, innerc);
                operands(3, a1);
                products(a1, acc1);
            } else {
                operands(0, a0);
                operands(1, a1);
                products(a0, acc0);
                operands(2, a0);
                products(a1, acc1);
                operands(3, a1);
                examine(std::integral_constant<int, 0>(), acc0, innerc);
                products(a0, acc0);
                examine(std::integral_constant<int, 1>(), acc1, innerc);
                products(a1, acc1);
            }
            examine(std::integral_constant<int, 2>(), acc0, innerc);
            examine(std::integral_constant<int, 3>(), acc1, innerc);
        };
        if (inner) run(std::true_type());
        else run(std::false_type());
        if constexpr (CAND) {
            // Lists that might not take another tile are cut now.
            auto cut_full = [&](auto qbc) {
                constexpr int QBC = decltype(qbc)::value;
                const uint64_t bal = __ballot(lc[QBC] + 16u > (uint32_t)kMfmaSeg);
                uint32_t cols = (uint32_t)(bal | (bal >> 16) | (bal >> 32) | (bal >> 48)) & 0xFFFFu;
                while (cols) {
                    const int c = __builtin_ctz(cols);
                    cols &= cols - 1u;
                    cut_list(qbc, c);
                }
            };
            cut_full(std::integral_constant<int, 0>());
            if constexpr (QB > 1) cut_full(std::integral_constant<int, 1>());
            if constexpr (QB > 2) cut_full(std::integral_constant<int, 2>());
            if constexpr (QB > 3) cut_full(std::integral_constant<int, 3>());
        }
    };

    // One tile: wait for this wavefront's part of tile t (the loads of the kBuf - 2 tiles after
    // it may still fly), then for everyone's (the barrier also ends every use of the buffer that
    // the next issue refills), issue tile t + kBuf - 1, compute tile t.
    auto step = [&](int t, auto bufc) {
        constexpr int B = decltype(bufc)::value;
        // (A plain barrier: __syncthreads would also wait for the loads of the tiles ahead.)
        __builtin_amdgcn_s_waitcnt(kWaitAhead);
        asm volatile("s_barrier" ::: "memory");
        issue(t + kBuf - 1, std::integral_constant<int, (B + kBuf - 1) % kBuf>());
        if (tile_of(t) <= t_wave) compute(t, bufc);
    };
    // Tiles past the last one are fetched too (clamped rows, never read), so that every wait
    // counts the same loads.
    issue(0, std::integral_constant<int, 0>());
    issue(1, std::integral_constant<int, 1>());
    issue(2, std::integral_constant<int, 2>());
    static_assert(kBuf == 4, "ring");
    for (int t0 = 0; t0 < nsteps; t0 += kBuf) {
        step(t0, std::integral_constant<int, 0>());
        if (t0 + 1 < nsteps) step(t0 + 1, std::integral_constant<int, 1>());
        if (t0 + 2 < nsteps) step(t0 + 2, std::integral_constant<int, 2>());
        if (t0 + 3 < nsteps) step(t0 + 3, std::integral_constant<int, 3>());
    }
    // No LDS fill may outlive the workgroup.
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();

    if constexpr (!CAND) {
        // Bound of each query from its 128 class maxima (32 in each of its four lanes).
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) {
            uint32_t x[32];
            uint32_t nz = 0u, hmax = 0u, hmin = 0xFFFFFFFFu;
#pragma unroll
            for (int s = 0; s < 32; ++s) {
                const int32_t v = m[s / 16][(s / 4) % 4][s % 4][qb];
                x[s] = v != INT32_MIN ? score_key(__int_as_float(v)) : 0u;
                nz += x[s] != 0u;
                hmax = x[s] > hmax ? x[s] : hmax;
                hmin = x[s] != 0u && x[s] < hmin ? x[s] : hmin;
            }
            nz = quad_sum_u32(nz);
            hmax = quad_max_u32(hmax);
            hmin = quad_min_u32(hmin);
            uint32_t tau;
            if (kq[qb] == 0) {
                tau = 0xFFFFFFFFu;
            } else if (nz < (uint32_t)kq[qb]) {
                tau = 0u;  // (not reached: the first 128 candidate rows fill distinct classes)
            } else if (hmax == hmin) {
                tau = hmax;
            } else {
                const int hb = 31 - __builtin_clz(hmax ^ hmin);
                tau = hb >= 31 ? 0u : (hmax >> (hb + 1)) << (hb + 1);
#pragma unroll 1
                for (int it = 0; it < 16; ++it) {
                    const int bit = hb - it;
                    const uint32_t cand = tau | (bit >= 0 ? 1u << bit : 0u);
                    uint32_t c = 0u;
#pragma unroll
                    for (int s = 0; s < 32; ++s) c += x[s] >= cand ? 1u : 0u;
                    c = quad_sum_u32(c);
                    if (bit >= 0 && c >= (uint32_t)kq[qb]) tau = cand;
                }
            }
            if (grp == 0 && lim[qb] != -1) a.tau[qvi[qb]] = tau;
            if (grp == 0 && lim[qb] == -1 && idx_w + qb * 16 + col < a.nvec) a.tau[qvi[qb]] = 0xFFFFFFFFu;
            if constexpr (MASS) {
                // The query's four lanes merged: (largest reference score, sum relative to it)
                // over R_i.
                const float m4 = quad_max_f32(zm[qb]);
                const float l4 = __uint_as_float(quad_sum_f32_bits(__float_as_uint(
                    zm[qb] == -INFINITY ? 0.f : zl[qb] * exp2f((zm[qb] - m4) * a.scale_log2e))));
                if (grp == 0 && idx_w + qb * 16 + col < a.nvec) a.zmass[qvi[qb]] = make_float2(m4, l4);
            }
        }
    } else {
#pragma unroll
        for (int qb = 0; qb < QB; ++qb)
            if (idx_w + qb * 16 + col < a.nvec) a.cnt[(size_t)qvi[qb] * kLanesPerQuery + grp] = lc[qb];
    }
}

// Anchor-and-window softmax partials of the query vectors (pages of "The Condensate Theorem",
// metaphor-xennon blog: section 2.1 Definition 1, {0} u {i-W+1..i}; section 2.3, the softmax
// over C_i and its product with V). Consecutive positions share almost all of their window
// rows, so a workgroup takes 64 query vectors of one KV head (16 per wavefront) and brings the
// rows of their windows (and row 0) through LDS once, in tiles of 64 rows. Per tile and
// wavefront the scores are K . Q^T on the matrix cores (the layout of the selection passes:
// lane l holds query l % 16 and rows 4(l/16)..+3 of each block of 16), masked to each query's
// anchor and window, folded into a running softmax (largest score m, weight sum l), and the
// weights times V are accumulated as O^T += V^T P^T: the weights a lane holds for two blocks of
// 16 rows are exactly its B operand of one 32-row step (the same rows on both sides of the
// contraction), and V^T comes from a transposed copy of the tile in LDS. Each fp32 weight enters
// the product as the sum of two bf16 parts (two products per step), so the weights times V agree
// with the fp32 weight sum to about 2^-17 per weight; accumulation is fp32. Output per query
// vector: m, l and the weighted sum of V rows, the partial the finish kernel merges.
constexpr int kWinTile = 64;
// Query blocks of 16 per wavefront in the dense kernel, per d.
constexpr int kDenseQB128 = 2;
constexpr int kDenseQB64 = 4;
constexpr int kVtStride = kWinTile + 4;  // bf16 per transposed V row (padded against bank conflicts)

struct WinArgs {
    int64_t n, nq;
    int Hq, Hkv, g, W;
    uint32_t nvec, wg_per_unit, nwg;
    float scale_log2e;
    float *win;  // [nqv][D + 2] partials (window kernel)
    float *out;  // [nqv][D] normalised outputs (dense kernel)
};

// K and V rows base..base+63 of a tile (clamped to n - 1): 16-byte chunks, NCH per thread.
// (Native 4 x u32 vectors: arrays of HIP's uint4 struct filled from memory stay on the stack.)
// K: chunk c of row r per thread, D / 8 threads to a row. V: the same chunk of two consecutive
// rows per thread (rows 2p and 2p + 1), so that its transposed copy is written as 4-byte pairs.
// d = 128: p = lane % 32, chunk v_chunk(u), the two half-wavefronts two chunks (32 banks) apart;
// a wavefront's 2-byte stores of the K-like layout fell on 4 banks (dense kernel 3.50 -> 2.44 ms
// on the 4K x 32K chunk). d = 64: the 8 lanes of a group take the 8 chunks of one row pair, so a
// wavefront still reads whole rows (16 of them), with 2-way conflicts left (dense kernel on the
// 131K prefill 20.14 -> 19.79 ms).
typedef unsigned int win_u32x4 __attribute__((ext_vector_type(4)));

template <int D>
__device__ __forceinline__ int v_chunk(int u, int tid) {
    if constexpr (D == 128) return u + 2 * ((tid >> 5) & 1) + 4 * (tid >> 6);
    else return tid & 7;
}
template <int D>
__device__ __forceinline__ int v_pair(int tid) {
    if constexpr (D == 128) return tid & 31;
    else return ((tid & 63) >> 3) + 8 * (tid >> 6);
}

template <int D>
__device__ __forceinline__ void win_tile_load(win_u32x4 (&pk)[kWinTile * D / 8 / 256],
                                              win_u32x4 (&pv)[kWinTile * D / 8 / 256],
                                              const __bf16 *__restrict__ kb, const __bf16 *__restrict__ vb,
                                              int base, int nlast, int tid) {
    constexpr int CPR = D / 8, NCH = kWinTile * CPR / 256;
    // (Byte offsets from the KV head's first row in 32 bits: the plan keeps a head below 4 GiB.)
    const char *kc = reinterpret_cast<const char *>(kb), *vc = reinterpret_cast<const char *>(vb);
#pragma unroll
    for (int u = 0; u < NCH; ++u) {
        const int cid = tid + 256 * u, row = cid / CPR, c = cid % CPR;
        const int j = base + row < nlast ? base + row : nlast;
        const uint32_t off = (uint32_t)j * (uint32_t)(D * sizeof(__bf16)) + (uint32_t)c * 16u;
        pk[u] = *reinterpret_cast<const win_u32x4 *>(kc + off);
    }
#pragma unroll
    for (int u = 0; u < NCH; ++u) {
        const int row = 2 * v_pair<D>(tid) + (u & 1), c = v_chunk<D>(u >> 1, tid);
        const int j = base + row < nlast ? base + row : nlast;
        const uint32_t off = (uint32_t)j * (uint32_t)(D * sizeof(__bf16)) + (uint32_t)c * 16u;
        pv[u] = *reinterpret_cast<const win_u32x4 *>(vc + off);
    }
}
// The tile into LDS: K with swizzled chunks; V transposed ([d][row], bf16 bits), each element of
// the thread's two rows as one 4-byte word.
template <int D>
__device__ __forceinline__ void win_tile_store(const win_u32x4 (&pk)[kWinTile * D / 8 / 256],
                                               const win_u32x4 (&pv)[kWinTile * D / 8 / 256], uint4 *kt,
                                               uint16_t *vt, int tid) {
    constexpr int CPR = D / 8, NCH = kWinTile * CPR / 256;
#pragma unroll
    for (int u = 0; u < NCH; ++u) {
        const int cid = tid + 256 * u, row = cid / CPR, c = cid % CPR;
        reinterpret_cast<win_u32x4 *>(kt)[chunk_at<D>(row, c)] = pk[u];
    }
#pragma unroll
    for (int u = 0; u < NCH / 2; ++u) {
        const int row = 2 * v_pair<D>(tid), c = v_chunk<D>(u, tid);
        uint32_t *vd = reinterpret_cast<uint32_t *>(vt + (c * 8) * kVtStride + row);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const uint32_t a = pv[2 * u][e], b = pv[2 * u + 1][e];
            vd[(2 * e) * (kVtStride / 2)] = (a & 0xFFFFu) | (b << 16);
            vd[(2 * e + 1) * (kVtStride / 2)] = (a >> 16) | (b & 0xFFFF0000u);
        }
    }
}

template <int D>
__global__ __launch_bounds__(256) void mfma_window_kernel(const __bf16 *__restrict__ q,
                                                          const __bf16 *__restrict__ k,
                                                          const __bf16 *__restrict__ v, WinArgs a) {
    constexpr int KS = D / 32, CPR = D / 8, NCH = kWinTile * CPR / 256, DB = D / 16;
    static_assert(NCH * 256 == kWinTile * CPR, "tile");
    __shared__ uint4 kt[kWinTile * CPR];
    __shared__ alignas(16) uint16_t vt[D * kVtStride];  // bf16 bits
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int col = lane & 15, grp = lane >> 4;
    const uint32_t bid = blockIdx.x, xcd = bid % kXcds;
    const uint32_t per = a.nwg / kXcds, rem = a.nwg % kXcds;
    const uint32_t L = xcd * per + (xcd < rem ? xcd : rem) + bid / kXcds;
    const uint32_t bk = L / a.wg_per_unit, part = L - bk * a.wg_per_unit;
    const uint32_t b = bk / (uint32_t)a.Hkv, kvh = bk - b * (uint32_t)a.Hkv, g = (uint32_t)a.g;
    auto pos_of = [&](uint32_t idx) -> int { return (int)(a.n - a.nq + idx / g); };
    // This lane's query vector.
    const uint32_t idx = part * 64 + wave * 16 + col;
    const bool valid = idx < a.nvec;
    const uint32_t idxc = valid ? idx : a.nvec - 1;
    const uint32_t qv = (b * (uint32_t)a.Hq + kvh * g + idxc % g) * (uint32_t)a.nq + idxc / g;
    const int i = pos_of(idxc);
    const int wlo = i - a.W + 1 > 0 ? i - a.W + 1 : 0;
    uint4 qf[KS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) qf[ks] = reinterpret_cast<const uint4 *>(q + (size_t)qv * D)[ks * 4 + grp];
    // Rows of the workgroup: the windows of its first to last vector, and row 0 in a tile of
    // its own when no window reaches it.
    const int i_first = pos_of(part * 64);
    const uint32_t last = part * 64 + 63 < a.nvec ? part * 64 + 63 : a.nvec - 1;
    const int s_lo = i_first - a.W + 1 > 0 ? i_first - a.W + 1 : 0, s_hi = pos_of(last);
    const int anchor_tile = s_lo > 0 ? 1 : 0;
    const int ntiles = anchor_tile + (s_hi - s_lo + kWinTile) / kWinTile;
    const __bf16 *kb = k + (size_t)bk * (size_t)a.n * D, *vb = v + (size_t)bk * (size_t)a.n * D;
    const int nlast = (int)a.n - 1;

    float m = -INFINITY, lsum = 0.f;
    f32x4_t o[DB];
#pragma unroll
    for (int db = 0; db < DB; ++db) o[db] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    win_u32x4 pk[NCH], pv[NCH];
    // Tile t: rows base(t) + 0..63 (row 0 alone for the anchor tile).
    auto tile_base = [&](int t) { return t < anchor_tile ? 0 : s_lo + (t - anchor_tile) * kWinTile; };
    if (ntiles > 0) {
        win_tile_load<D>(pk, pv, kb, vb, tile_base(0), nlast, tid);
        win_tile_store<D>(pk, pv, kt, vt, tid);
    }
    __syncthreads();
    for (int t = 0; t < ntiles; ++t) {
        if (t + 1 < ntiles) win_tile_load<D>(pk, pv, kb, vb, tile_base(t + 1), nlast, tid);
        const int base = tile_base(t);
        const bool is_anchor = t < anchor_tile;
        // Scores of the tile's 64 rows for this wavefront's 16 queries.
        f32x4_t sc[4];
#pragma unroll
        for (int kbk = 0; kbk < 4; ++kbk) {
            bf16x8_t af[KS];
#pragma unroll
            for (int ks = 0; ks < KS; ++ks)
                af[ks] = __builtin_bit_cast(bf16x8_t, kt[chunk_at<D>(kbk * 16 + col, ks * 4 + grp)]);
            sc[kbk] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ks = 0; ks < KS; ++ks)
                sc[kbk] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[ks], __builtin_bit_cast(bf16x8_t, qf[ks]), sc[kbk], 0, 0, 0);
        }
        // Rows of C_i: row 0 (the anchor), and rows wlo..i (the window).
        float mt = -INFINITY;
        uint32_t inm = 0u;  // bit 4*kbk + r: row base + 16 kbk + 4 grp + r is in C_i
#pragma unroll
        for (int kbk = 0; kbk < 4; ++kbk)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int j = base + kbk * 16 + 4 * grp + r;
                const bool in = valid && (is_anchor ? j == 0 : (j == 0 || (j >= wlo && j <= i)));
                inm |= in ? 1u << (4 * kbk + r) : 0u;
                mt = in ? fmaxf(mt, sc[kbk][r]) : mt;
            }
        {
            const auto r16 = __builtin_amdgcn_permlane16_swap(__float_as_uint(mt), __float_as_uint(mt), false, false);
            mt = fmaxf(__uint_as_float(r16[0]), __uint_as_float(r16[1]));
            const auto r32 = __builtin_amdgcn_permlane32_swap(__float_as_uint(mt), __float_as_uint(mt), false, false);
            mt = fmaxf(__uint_as_float(r32[0]), __uint_as_float(r32[1]));
        }
        const float mn = fmaxf(m, mt);
        if (mn != -INFINITY) {  // same for the four lanes of a query
            const float alpha = m == -INFINITY ? 0.f : exp2f((m - mn) * a.scale_log2e);
            lsum *= alpha;
#pragma unroll
            for (int db = 0; db < DB; ++db) o[db] *= alpha;
            m = mn;
        }
        f32x4_t pw[4];
#pragma unroll
        for (int kbk = 0; kbk < 4; ++kbk)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                pw[kbk][r] = (inm >> (4 * kbk + r)) & 1u ? exp2f((sc[kbk][r] - m) * a.scale_log2e) : 0.f;
                lsum += pw[kbk][r];
            }
        // O^T += V^T P^T over two steps of 32 rows (blocks 0,1 and 2,3). Each fp32 weight enters
        // as two bf16 parts, w = hi + lo (hi = w rounded to bf16, lo = the rest rounded again),
        // in two products with the same V^T operand: the weights V is multiplied by agree with
        // the fp32 weights summed into lsum to about 2^-17 of each weight, as in the other
        // attend paths, instead of the 2^-9 of one bf16 rounding.
#pragma unroll
        for (int h2 = 0; h2 < 2; ++h2) {
            bf16x8_t pb_hi, pb_lo;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
#pragma unroll
                for (int half = 0; half < 2; ++half) {
                    const float w = pw[2 * h2 + half][r];
                    const __bf16 hi = (__bf16)w;
                    pb_hi[4 * half + r] = hi;
                    pb_lo[4 * half + r] = (__bf16)(w - (float)hi);
                }
            }
#pragma unroll
            for (int db = 0; db < DB; ++db) {
                const uint16_t *vr = vt + (db * 16 + col) * kVtStride + h2 * 32 + 4 * grp;
                const uint2 lo = *reinterpret_cast<const uint2 *>(vr);
                const uint2 hi = *reinterpret_cast<const uint2 *>(vr + 16);
                const bf16x8_t av = __builtin_bit_cast(bf16x8_t, make_uint4(lo.x, lo.y, hi.x, hi.y));
                o[db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, pb_hi, o[db], 0, 0, 0);
                o[db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, pb_lo, o[db], 0, 0, 0);
            }
        }
        __syncthreads();
        if (t + 1 < ntiles) win_tile_store<D>(pk, pv, kt, vt, tid);
        __syncthreads();
    }
    lsum = __uint_as_float(quad_sum_f32_bits(__float_as_uint(lsum)));
    if (valid) {
        float *out = a.win + (size_t)qv * (D + 2);
        if (grp == 0) { out[0] = m; out[1] = lsum; }
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
            for (int r = 0; r < 4; ++r) out[2 + db * 16 + 4 * grp + r] = o[db][r];
    }
}

// Dense causal attention (every j <= i), the denominator of the method's speedup (pages of "The
// Condensate Theorem", metaphor-xennon blog: section 2.1, softmax(S) V over all causal
// positions; section 5.1.2 compares against it). The layout of the window kernel, for long rows:
// each wavefront holds QB blocks of 16 query vectors, so every K and V^T fragment read from LDS
// feeds QB products; tiles wholly below the wavefront's first query position take no mask; the
// running output is rescaled only when some lane's maximum moved; the workgroups with the most
// rows (the last query positions) are dispatched first.
template <int D, int QB>
__global__ __launch_bounds__(256) void mfma_dense_kernel(const __bf16 *__restrict__ q,
                                                         const __bf16 *__restrict__ k,
                                                         const __bf16 *__restrict__ v, WinArgs a) {
    constexpr int KS = D / 32, CPR = D / 8, NCH = kWinTile * CPR / 256, DB = D / 16;
    constexpr int QW = 16 * QB, ROWS = 4 * QW;
    static_assert(NCH * 256 == kWinTile * CPR, "tile");
    __shared__ uint4 kt[kWinTile * CPR];
    __shared__ alignas(16) uint16_t vt[D * kVtStride];  // bf16 bits
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int col = lane & 15, grp = lane >> 4;
    const uint32_t bid = blockIdx.x, xcd = bid % kXcds;
    const uint32_t per = a.nwg / kXcds, rem = a.nwg % kXcds;
    const uint32_t L = xcd * per + (xcd < rem ? xcd : rem) + bid / kXcds;
    const uint32_t bk = L / a.wg_per_unit;
    const uint32_t part = a.wg_per_unit - 1 - (L - bk * a.wg_per_unit);  // most rows first
    const uint32_t b = bk / (uint32_t)a.Hkv, kvh = bk - b * (uint32_t)a.Hkv, g = (uint32_t)a.g;
    auto pos_of = [&](uint32_t idx) -> int { return (int)(a.n - a.nq + idx / g); };
    // This lane's query vectors (one per query block).
    bool valid[QB];
    uint32_t qv[QB];
    int qi[QB];
    bf16x8_t qf[QB][KS];
    int i_lo = INT32_MAX, i_hi = 0;
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
        const uint32_t idx = part * ROWS + wave * QW + qb * 16 + col;
        valid[qb] = idx < a.nvec;
        const uint32_t idxc = valid[qb] ? idx : a.nvec - 1;
        qv[qb] = (b * (uint32_t)a.Hq + kvh * g + idxc % g) * (uint32_t)a.nq + idxc / g;
        qi[qb] = pos_of(idxc);
        i_lo = qi[qb] < i_lo ? qi[qb] : i_lo;
        i_hi = qi[qb] > i_hi ? qi[qb] : i_hi;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
            qf[qb][ks] = __builtin_bit_cast(bf16x8_t, reinterpret_cast<const uint4 *>(q + (size_t)qv[qb] * D)[ks * 4 + grp]);
    }
    i_lo = (int)wave_min_u32_dpp((uint32_t)i_lo);
    i_hi = (int)wave_max_u32_dpp((uint32_t)i_hi);
    // Rows of the workgroup: 0 .. the position of its last vector.
    const uint32_t last = part * ROWS + ROWS - 1 < a.nvec ? part * ROWS + ROWS - 1 : a.nvec - 1;
    const int ntiles = pos_of(last) / kWinTile + 1;
    const __bf16 *kb = k + (size_t)bk * (size_t)a.n * D, *vb = v + (size_t)bk * (size_t)a.n * D;
    const int nlast = (int)a.n - 1;
    const float sc_l2 = a.scale_log2e;

    float m[QB], lsum[QB];  // running maximum of the raw scores, weight sum (this lane's rows)
    f32x4_t o[QB][DB];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
        m[qb] = -INFINITY;
        lsum[qb] = 0.f;
#pragma unroll
        for (int db = 0; db < DB; ++db) o[qb][db] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    }
    win_u32x4 pk[NCH], pv[NCH];
    win_tile_load<D>(pk, pv, kb, vb, 0, nlast, tid);
    win_tile_store<D>(pk, pv, kt, vt, tid);
    __syncthreads();
    for (int t = 0; t < ntiles; ++t) {
        if (t + 1 < ntiles) win_tile_load<D>(pk, pv, kb, vb, (t + 1) * kWinTile, nlast, tid);
        const int base = t * kWinTile;
        if (base <= i_hi) {  // wavefront-uniform: some query of the wavefront sees these rows
            const bool full = base + kWinTile - 1 <= i_lo;
            f32x4_t sc[4][QB];
#pragma unroll
            for (int kbk = 0; kbk < 4; ++kbk) {
                bf16x8_t af[KS];
#pragma unroll
                for (int ks = 0; ks < KS; ++ks)
                    af[ks] = __builtin_bit_cast(bf16x8_t, kt[chunk_at<D>(kbk * 16 + col, ks * 4 + grp)]);
#pragma unroll
                for (int qb = 0; qb < QB; ++qb) {
                    sc[kbk][qb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int ks = 0; ks < KS; ++ks)
                        sc[kbk][qb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[ks], qf[qb][ks], sc[kbk][qb], 0, 0, 0);
                }
            }
            if (!full) {  // rows past the query's position leave the softmax
#pragma unroll
                for (int kbk = 0; kbk < 4; ++kbk)
#pragma unroll
                    for (int qb = 0; qb < QB; ++qb)
#pragma unroll
                        for (int r = 0; r < 4; ++r)
                            sc[kbk][qb][r] = base + kbk * 16 + 4 * grp + r <= qi[qb] ? sc[kbk][qb][r] : -INFINITY;
            }
            bool moved = false;
            float alpha[QB];
#pragma unroll
            for (int qb = 0; qb < QB; ++qb) {
                float mt = fmaxf(fmaxf(fmaxf(sc[0][qb][0], sc[0][qb][1]), fmaxf(sc[0][qb][2], sc[0][qb][3])),
                                 fmaxf(fmaxf(sc[1][qb][0], sc[1][qb][1]), fmaxf(sc[1][qb][2], sc[1][qb][3])));
                mt = fmaxf(mt, fmaxf(fmaxf(fmaxf(sc[2][qb][0], sc[2][qb][1]), fmaxf(sc[2][qb][2], sc[2][qb][3])),
                                     fmaxf(fmaxf(sc[3][qb][0], sc[3][qb][1]), fmaxf(sc[3][qb][2], sc[3][qb][3]))));
                const auto r16 = __builtin_amdgcn_permlane16_swap(__float_as_uint(mt), __float_as_uint(mt), false, false);
                mt = fmaxf(__uint_as_float(r16[0]), __uint_as_float(r16[1]));
                const auto r32 = __builtin_amdgcn_permlane32_swap(__float_as_uint(mt), __float_as_uint(mt), false, false);
                mt = fmaxf(__uint_as_float(r32[0]), __uint_as_float(r32[1]));
                const float mn = fmaxf(m[qb], mt);  // finite: row 0 is in every tile 0
                alpha[qb] = mn > m[qb] ? __builtin_amdgcn_exp2f((m[qb] - mn) * sc_l2) : 1.f;
                moved = moved || mn > m[qb];
                m[qb] = mn;
            }
            if (__ballot(moved) != 0ull) {
#pragma unroll
                for (int qb = 0; qb < QB; ++qb) {
                    lsum[qb] *= alpha[qb];
#pragma unroll
                    for (int db = 0; db < DB; ++db) o[qb][db] *= alpha[qb];
                }
            }
            // Weights exp2((s - m) * scale) as bf16, blocks (0, 1) and (2, 3) forming the B
            // operand of the two 32-row steps of O^T += V^T P^T. (v_exp_f32 itself: weights
            // below 2^-126 of the largest are dropped, the rest keep its relative error.)
            bf16x8_t pb[2][QB];
#pragma unroll
            for (int qb = 0; qb < QB; ++qb) {
                const float mb = m[qb] * sc_l2;
#pragma unroll
                for (int h2 = 0; h2 < 2; ++h2)
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const float p0 = __builtin_amdgcn_exp2f(fmaf(sc[2 * h2][qb][r], sc_l2, -mb));
                        const float p1 = __builtin_amdgcn_exp2f(fmaf(sc[2 * h2 + 1][qb][r], sc_l2, -mb));
                        lsum[qb] += p0 + p1;
                        pb[h2][qb][r] = (__bf16)p0;
                        pb[h2][qb][4 + r] = (__bf16)p1;
                    }
            }
#pragma unroll
            for (int h2 = 0; h2 < 2; ++h2)
#pragma unroll
                for (int db = 0; db < DB; ++db) {
                    const uint16_t *vr = vt + (db * 16 + col) * kVtStride + h2 * 32 + 4 * grp;
                    const uint2 lo = *reinterpret_cast<const uint2 *>(vr);
                    const uint2 hi = *reinterpret_cast<const uint2 *>(vr + 16);
                    const bf16x8_t av = __builtin_bit_cast(bf16x8_t, make_uint4(lo.x, lo.y, hi.x, hi.y));
#pragma unroll
                    for (int qb = 0; qb < QB; ++qb)
                        o[qb][db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, pb[h2][qb], o[qb][db], 0, 0, 0);
                }
        }
        __syncthreads();
        if (t + 1 < ntiles) win_tile_store<D>(pk, pv, kt, vt, tid);
        __syncthreads();
    }
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
        const float l = __uint_as_float(quad_sum_f32_bits(__float_as_uint(lsum[qb])));
        if (valid[qb]) {
            float *out = a.out + (size_t)qv[qb] * D;
            const float inv = 1.f / l;
#pragma unroll
            for (int db = 0; db < DB; ++db)
#pragma unroll
                for (int r = 0; r < 4; ++r) out[db * 16 + 4 * grp + r] = o[qb][db][r] * inv;
        }
    }
}

}  // namespace

hipError_t launch_mfma_select(const Plan &pl, const void *q, const void *k, void *ws, hipStream_t s,
                              int pass, bool mass) {
    MfmaArgs a;
    a.n = pl.n; a.nq = pl.nq; a.Hq = pl.Hq; a.Hkv = pl.Hkv; a.g = pl.g; a.W = pl.W; a.topk = pl.topk;
    a.nvec = (uint32_t)(pl.g * pl.nq);
    char *w = static_cast<char *>(ws);
    a.tau = reinterpret_cast<uint32_t *>(w + pl.slots_offset);
    a.cnt = reinterpret_cast<uint32_t *>(w + pl.slots_offset) + 2 * pl.nqv * pl.wpu;
    a.lists = reinterpret_cast<uint64_t *>(w + pl.lists_offset);
    a.scale_log2e = (float)(1.4426950408889634 / __builtin_sqrt((double)pl.d));
    a.zmass = reinterpret_cast<float2 *>(w + pl.zmass_offset);
    const bool cand = pass != 0;
    const int qb_bound = pl.d == 128 ? kMfmaQBBound128 : kMfmaQBBound64;
    const int rows = 16 * kMfmaWaves * (cand ? kMfmaQBCand : qb_bound);
    a.wg_per_unit = (uint32_t)((a.nvec + rows - 1) / rows);
    a.nwg = (uint32_t)(pl.B * pl.Hkv) * a.wg_per_unit;
    const dim3 grid(a.nwg), block(64 * kMfmaWaves);
    const __bf16 *qt = static_cast<const __bf16 *>(q), *kt = static_cast<const __bf16 *>(k);
    // Candidate pass: the block pre-test pays when few blocks hold a candidate, i.e. when the
    // queries have many rows per kept key: about 1.25k of a query's rows pass the full bound, so a block of 16
    // rows x 16 queries holds one with probability about 320k / rows (measured: -13% with rows
    // averaging 64K and k = 32, +4% with 30K rows and k = 64). Rows: the mean over the queries.
    const int64_t mean_rows = pl.n - pl.nq / 2 - pl.W;
    const bool pre = mean_rows > 1024 * (int64_t)pl.topk;
    // Bound pass: tiles kept of every 4 (the mass sum needs every row).
    const int keep = pl.topk <= 32 ? 2 : (pl.topk <= 64 ? 3 : 4);
#define CA_MFMA_SELECT(D)                                                                          \
    do {                                                                                           \
        if (!cand && mass) hipLaunchKernelGGL((mfma_select_kernel<D, D == 128 ? kMfmaQBBound128 : kMfmaQBBound64, false, false, kMfmaWaves, true>), grid, block, 0, s, qt, kt, a); \
        else if (!cand && keep == 2) hipLaunchKernelGGL((mfma_select_kernel<D, D == 128 ? kMfmaQBBound128 : kMfmaQBBound64, false, false, kMfmaWaves, false, 2>), grid, block, 0, s, qt, kt, a); \
        else if (!cand && keep == 3) hipLaunchKernelGGL((mfma_select_kernel<D, D == 128 ? kMfmaQBBound128 : kMfmaQBBound64, false, false, kMfmaWaves, false, 3>), grid, block, 0, s, qt, kt, a); \
        else if (!cand) hipLaunchKernelGGL((mfma_select_kernel<D, D == 128 ? kMfmaQBBound128 : kMfmaQBBound64, false, false, kMfmaWaves>), grid, block, 0, s, qt, kt, a); \
        else if (pre) hipLaunchKernelGGL((mfma_select_kernel<D, kMfmaQBCand, true, true, kMfmaWaves>), grid, block, 0, s, qt, kt, a); \
        else hipLaunchKernelGGL((mfma_select_kernel<D, kMfmaQBCand, true, false, kMfmaWaves>), grid, block, 0, s, qt, kt, a); \
    } while (0)
    if (pl.d == 128) CA_MFMA_SELECT(128);
    else CA_MFMA_SELECT(64);
#undef CA_MFMA_SELECT
    return hipGetLastError();
}

hipError_t launch_mfma_window(const Plan &pl, const void *q, const void *k, const void *v, void *ws,
                              hipStream_t s) {
    WinArgs a;
    a.n = pl.n; a.nq = pl.nq; a.Hq = pl.Hq; a.Hkv = pl.Hkv; a.g = pl.g; a.W = pl.W;
    a.nvec = (uint32_t)(pl.g * pl.nq);
    a.wg_per_unit = (a.nvec + 63) / 64;
    a.nwg = (uint32_t)(pl.B * pl.Hkv) * a.wg_per_unit;
    a.scale_log2e = (float)(1.4426950408889634 / __builtin_sqrt((double)pl.d));
    a.win = reinterpret_cast<float *>(static_cast<char *>(ws) + pl.win_offset);
    a.out = nullptr;
    const __bf16 *qt = static_cast<const __bf16 *>(q), *kt = static_cast<const __bf16 *>(k),
                 *vt = static_cast<const __bf16 *>(v);
    if (pl.d == 128) hipLaunchKernelGGL((mfma_window_kernel<128>), dim3(a.nwg), dim3(256), 0, s, qt, kt, vt, a);
    else hipLaunchKernelGGL((mfma_window_kernel<64>), dim3(a.nwg), dim3(256), 0, s, qt, kt, vt, a);
    return hipGetLastError();
}

hipError_t launch_dense_attention(const Plan &pl, const void *q, const void *k, const void *v,
                                  float *out, hipStream_t s) {
    WinArgs a;
    a.n = pl.n; a.nq = pl.nq; a.Hq = pl.Hq; a.Hkv = pl.Hkv; a.g = pl.g;
    a.W = (int)pl.n;  // the window covers every causal position: C_i = {0..i}
    a.nvec = (uint32_t)(pl.g * pl.nq);
    const uint32_t rows = 64 * (pl.d == 128 ? kDenseQB128 : kDenseQB64);
    a.wg_per_unit = (a.nvec + rows - 1) / rows;
    a.nwg = (uint32_t)(pl.B * pl.Hkv) * a.wg_per_unit;
    a.scale_log2e = (float)(1.4426950408889634 / __builtin_sqrt((double)pl.d));
    a.win = nullptr;
    a.out = out;
    const __bf16 *qt = static_cast<const __bf16 *>(q), *kt = static_cast<const __bf16 *>(k),
                 *vt = static_cast<const __bf16 *>(v);
    if (pl.d == 128) hipLaunchKernelGGL((mfma_dense_kernel<128, kDenseQB128>), dim3(a.nwg), dim3(256), 0, s, qt, kt, vt, a);
    else hipLaunchKernelGGL((mfma_dense_kernel<64, kDenseQB64>), dim3(a.nwg), dim3(256), 0, s, qt, kt, vt, a);
    return hipGetLastError();
}

}  // namespace ca
