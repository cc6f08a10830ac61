// Stage 1 of condensate attention for prefill-shaped problems with bf16 inputs on gfx950 (pages
// of "The Condensate Theorem", metaphor-xennon blog: section 2.1, S = QK^T / sqrt(d) and
// Definition 1, C_i = {0} u {i-W+1..i} u Top-k_i; section 2.2.3, the top-k part over the
// positions R_i = {1..i-W}).
//
// When many query vectors read the same KV head, their scores are a dense product, computed
// here on the matrix cores: v_mfma_f32_16x16x32_bf16 multiplies 16 key rows by 16 query vectors
// over 32 elements of d per instruction, accumulating in fp32. A workgroup takes 64*QB query
// vectors of one KV head (4 wavefronts of 16*QB, whose slices stay in registers) and brings the
// key rows 0..max(i - W) through LDS in tiles of 64 rows: double-buffered, the 16-byte chunks
// of a row XOR-swizzled so that the operand reads of 16 rows hit distinct banks. The scores are
// the plain dot products: the positive factor 1/sqrt(d) changes no order.
//
// The exact top-k' of R_i (k' = min(k, |R_i|) <= 128) takes two passes over the same products
// (the same instruction sequence, hence bit-identical scores):
//   bound  For each query, the maxima of its candidate rows in the 128 classes j mod 128. The
//          classes are disjoint, so k' distinct rows reach the k'-th largest of those maxima: a
//          lower bound of the query's k'-th score. The lower edge of the 16-bit radix bin that
//          holds it goes out as a score key.
//   cand   Every candidate row whose score key reaches the bound is appended to the query's
//          list as a ranking key (about k + k/4 of them on Gaussian data). A list that might
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
constexpr int kXcds = 8;       // workgroups are dealt to the XCDs in turn
constexpr int kKeepE = 8;      // keys per lane in a list cut (lists of up to 512)

struct MfmaArgs {
    int64_t n, nq;
    int Hq, Hkv, g, W, topk;
    uint32_t nvec;         // query vectors per KV head (g * nq)
    uint32_t wg_per_unit;  // workgroups per (batch, KV head)
    uint32_t nwg;          // workgroups of the launch
    int wpu, lcap;         // segments per query, list capacity (wpu * topk)
    uint32_t *tau;         // [nqv] bound of each query (score key; 0xFFFFFFFF: no candidates)
    uint32_t *cnt;         // [nqv][wpu] segment lengths
    uint64_t *lists;       // [nqv][lcap] ranking keys
};

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
__device__ __forceinline__ int chunk_at(int row, int c) {
    constexpr int CPR = D / 8;
    return row * CPR + (c ^ (D == 128 ? (row & 15) : ((row >> 1) & 7)));
}

template <int D, int QB, bool CAND>
__global__ __launch_bounds__(256) void mfma_select_kernel(const __bf16 *__restrict__ q,
                                                          const __bf16 *__restrict__ k,
                                                          MfmaArgs a) {
    constexpr int KS = D / 32;                  // MFMA steps over d
    constexpr int CPR = D / 8;                  // 16-byte chunks per key row
    constexpr int NCH = kTile * CPR / 256;      // chunks per thread per tile
    constexpr int QW = 16 * QB;                 // query vectors per wavefront
    constexpr int ROWS = 4 * QW;                // per workgroup
    static_assert(NCH >= 1 && NCH * 256 == kTile * CPR, "tile");
    __shared__ uint4 kt[2][kTile * CPR];
    __shared__ uint32_t lcnt[CAND ? ROWS : 1], ladm[CAND ? ROWS : 1];
    __shared__ uint32_t hist[CAND ? 4 : 1][CAND ? 320 : 1];

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

    float tf[QB];
    if constexpr (CAND) {
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) {
            const uint32_t adm = kq[qb] > 0 ? a.tau[qvi[qb]] : 0xFFFFFFFFu;
            tf[qb] = key_floor_float(adm);
            if (grp == 0) {
                lcnt[wave * QW + qb * 16 + col] = 0u;
                ladm[wave * QW + qb * 16 + col] = adm;
            }
        }
    }
    float m[2][4][4][QB];  // [tile parity][16-row block][row of the lane][query]: class maxima
    if constexpr (!CAND) {
#pragma unroll
        for (int p = 0; p < 2; ++p)
#pragma unroll
            for (int kb = 0; kb < 4; ++kb)
#pragma unroll
                for (int r = 0; r < 4; ++r)
#pragma unroll
                    for (int qb = 0; qb < QB; ++qb) m[p][kb][r][qb] = -INFINITY;
    }

    const __bf16 *kbase = k + (size_t)bk * (size_t)a.n * D;
    const int nlast = (int)a.n - 1;
    uint4 pre[NCH];
    auto gload = [&](int t) {
#pragma unroll
        for (int u = 0; u < NCH; ++u) {
            const int cid = tid + 256 * u, row = cid / CPR, c = cid % CPR;
            const int j = t * kTile + row;
            pre[u] = reinterpret_cast<const uint4 *>(kbase + (size_t)(j < nlast ? j : nlast) * D)[c];
        }
    };
    auto lstore = [&](int buf) {
#pragma unroll
        for (int u = 0; u < NCH; ++u) {
            const int cid = tid + 256 * u, row = cid / CPR, c = cid % CPR;
            kt[buf][chunk_at<D>(row, c)] = pre[u];
        }
    };

    // Cut of list ql (wavefront-local) to its exact top-k'; returns nothing, updates LDS and tf.
    auto cut_list = [&](int ql) {
        uint32_t qv;
        int lm;
        vec_of(idx_w + (uint32_t)ql, qv, lm);
        const int keep = a.topk < lm ? a.topk : lm;
        const int row = wave * QW + ql;
        __threadfence_block();  // this wavefront's appends are visible to its loads
        const uint32_t c = lcnt[row];
        uint64_t *lst = a.lists + (size_t)qv * a.lcap;
        uint64_t kr[kKeepE];
#pragma unroll
        for (int e = 0; e < kKeepE; ++e) {
            const uint32_t f = lane + 64 * e;
            kr[e] = f < c ? lst[f] : 0ull;
        }
        const uint32_t hi = wave_keep_top_u64(kr, keep, hist[wave], lst);
        __threadfence_block();
        const uint32_t adm = hi + 1u > ladm[row] ? hi + 1u : ladm[row];
        if (lane == 0) { lcnt[row] = (uint32_t)keep; ladm[row] = adm; }
        const float f = key_floor_float(adm);
#pragma unroll
        for (int qb = 0; qb < QB; ++qb)
            if (qb * 16 + col == ql) tf[qb] = f;
    };

    // Products of tile t (LDS buffer buf) with this wavefront's queries; P = t & 1.
    auto compute = [&](int t, int buf, auto parity) {
        constexpr int P = decltype(parity)::value;
        const int j0 = t * kTile;
        const bool inner = j0 >= 1 && j0 + kTile - 1 <= lim_lo;
#pragma unroll
        for (int kb = 0; kb < 4; ++kb) {
            bf16x8_t af[KS];
            const int row = kb * 16 + col;
#pragma unroll
            for (int ks = 0; ks < KS; ++ks)
                af[ks] = __builtin_bit_cast(bf16x8_t, kt[buf][chunk_at<D>(row, ks * 4 + grp)]);
            f32x4_t acc[QB];
#pragma unroll
            for (int qb = 0; qb < QB; ++qb) acc[qb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ks = 0; ks < KS; ++ks)
#pragma unroll
                for (int qb = 0; qb < QB; ++qb)
                    acc[qb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[ks], qf[qb][ks], acc[qb], 0, 0, 0);
            // acc[qb][r]: row jb + r of the tile for query qb*16 + col.
            const int jb = j0 + kb * 16 + 4 * grp;
            if constexpr (!CAND) {
#pragma unroll
                for (int qb = 0; qb < QB; ++qb)
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        float v = acc[qb][r];
                        if (!inner) v = (jb + r >= 1 && jb + r <= lim[qb]) ? v : -INFINITY;
                        m[P][kb][r][qb] = fmaxf(m[P][kb][r][qb], v);
                    }
            } else {
                bool hit = false;
#pragma unroll
                for (int qb = 0; qb < QB; ++qb)
#pragma unroll
                    for (int r = 0; r < 4; ++r) hit |= acc[qb][r] >= tf[qb];
                if (__builtin_expect(__ballot(hit) != 0ull, 0)) {
#pragma unroll
                    for (int qb = 0; qb < QB; ++qb)
#pragma unroll
                        for (int r = 0; r < 4; ++r) {
                            const int j = jb + r;
                            const float v = acc[qb][r];
                            if (v >= tf[qb] && j >= 1 && j <= lim[qb]) {
                                const uint32_t key = score_key(v);
                                const int row = wave * QW + qb * 16 + col;
                                if (key >= ladm[row]) {
                                    const uint32_t pos = atomicAdd(&lcnt[row], 1u);
                                    a.lists[(size_t)qvi[qb] * a.lcap + pos] = make_rank_key(key, (uint32_t)j);
                                }
                            }
                        }
                }
            }
        }
        if constexpr (CAND) {
            // A list that might not take another tile (64 more rows) is cut now.
            const bool full = lane < QW && lcnt[wave * QW + lane] + kTile > (uint32_t)a.lcap;
            uint64_t bal = __ballot(full);
            while (bal) {
                const int ql = __builtin_ctzll(bal);
                bal &= bal - 1ull;
                cut_list(ql);
            }
        }
    };

    if (ntiles > 0) {
        gload(0);
        lstore(0);
    }
    __syncthreads();
    for (int t = 0; t < ntiles; ++t) {
        const int buf = t & 1;
        if (t + 1 < ntiles) gload(t + 1);
        if (t <= t_wave) {
            if (t & 1) compute(t, buf, std::integral_constant<int, 1>());
            else compute(t, buf, std::integral_constant<int, 0>());
        }
        if (t + 1 < ntiles) lstore(buf ^ 1);
        __syncthreads();
    }

    if constexpr (!CAND) {
        // Bound of each query from its 128 class maxima (32 in each of its four lanes).
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) {
            uint32_t x[32];
            uint32_t nz = 0u, hmax = 0u, hmin = 0xFFFFFFFFu;
#pragma unroll
            for (int s = 0; s < 32; ++s) {
                const float v = m[s / 16][(s / 4) % 4][s % 4][qb];
                x[s] = v > -INFINITY ? score_key(v) : 0u;
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
        }
    } else {
        if (lane < QW && idx_w + lane < a.nvec) {
            uint32_t qv;
            int lm;
            vec_of(idx_w + (uint32_t)lane, qv, lm);
            const int total = (int)lcnt[wave * QW + lane];
            for (int w = 0; w < a.wpu; ++w) {
                const int c = total - w * a.topk;
                a.cnt[(size_t)qv * a.wpu + w] = (uint32_t)(c < 0 ? 0 : (c > a.topk ? a.topk : c));
            }
        }
    }
}

}  // namespace

hipError_t launch_mfma_select(const Plan &pl, const void *q, const void *k, void *ws, hipStream_t s,
                              int pass) {
    MfmaArgs a;
    a.n = pl.n; a.nq = pl.nq; a.Hq = pl.Hq; a.Hkv = pl.Hkv; a.g = pl.g; a.W = pl.W; a.topk = pl.topk;
    a.nvec = (uint32_t)(pl.g * pl.nq);
    a.wpu = pl.wpu;
    a.lcap = (int)pl.lmax;
    char *w = static_cast<char *>(ws);
    a.tau = reinterpret_cast<uint32_t *>(w);
    a.cnt = reinterpret_cast<uint32_t *>(w) + 2 * pl.nqv * pl.wpu;
    a.lists = reinterpret_cast<uint64_t *>(w + pl.lists_offset);
    const bool cand = pass != 0;
    const int rows = 64 * (cand ? kMfmaQBCand : kMfmaQBBound);
    a.wg_per_unit = (uint32_t)((a.nvec + rows - 1) / rows);
    a.nwg = (uint32_t)(pl.B * pl.Hkv) * a.wg_per_unit;
    const dim3 grid(a.nwg), block(256);
    const __bf16 *qt = static_cast<const __bf16 *>(q), *kt = static_cast<const __bf16 *>(k);
    if (pl.d == 128) {
        if (cand) hipLaunchKernelGGL((mfma_select_kernel<128, kMfmaQBCand, true>), grid, block, 0, s, qt, kt, a);
        else hipLaunchKernelGGL((mfma_select_kernel<128, kMfmaQBBound, false>), grid, block, 0, s, qt, kt, a);
    } else {
        if (cand) hipLaunchKernelGGL((mfma_select_kernel<64, kMfmaQBCand, true>), grid, block, 0, s, qt, kt, a);
        else hipLaunchKernelGGL((mfma_select_kernel<64, kMfmaQBBound, false>), grid, block, 0, s, qt, kt, a);
    }
    return hipGetLastError();
}

}  // namespace ca
