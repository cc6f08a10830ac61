// decode_stream: the key stream of the decode path on gfx950 (pages of "The Condensate
// Theorem", metaphor-xennon blog: section 2.1, the scores q_i . k_j of every causal key; section
// 2.2.3, the candidates R_i of the top-k part). Every K row is read once and its keys staged in
// LDS; per block of 256 rows and query vector, 16 lanes reduce them to a 32-byte record: the
// block's four best rows as (key, offset), ties to the smaller offset, and X, the largest key of
// its other rows; with the mass diagnostic also the block's largest score m_b and the sum of
// exp2((s - m_b) * scale) over its candidate rows.
#include "attend_core.h"
#include "decode_core.h"

namespace ca {
namespace dec {
namespace {

// ---- anchor-and-window partials in the last workgroups of the grid ---------------------------
// Window workgroup b (< units * G * nch): chunk c = b % nch of query t = (b / nch) / units of unit
// (b / nch) % units, entries [c * kWinChunkRows, (c + 1) * kWinChunkRows) of the query's
// anchor-and-window list ({0} if the window does not reach it, then i - W + 1 .. i). Its eight
// wavefronts take their share (wave_partial) and the merged partial (m, l, acc[D],
// unnormalised) goes to a.win. They are dispatched after the key workgroups, into the CUs that
// the stream's last workgroups leave idle, so decode_finish only merges their partials.
template <typename T, int D, int G>
__device__ __forceinline__ void window_chunk(const T *__restrict__ q, const T *__restrict__ k,
                                             const T *__restrict__ v, const DecodeArgs &a, uint32_t blk,
                                             SoftmaxPartials<D, kWaves> &part) {
    using AS = AttendShape<D, T>;
    constexpr int UWIN = kWinChunkRows / (kWaves * AS::RPW) < 8 ? kWinChunkRows / (kWaves * AS::RPW) : 8;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const uint32_t c = blk % (uint32_t)a.nch, b = blk / (uint32_t)a.nch;
    const int t = (int)(b / a.units);
    const uint32_t uu = b - (uint32_t)t * a.units;
    const uint32_t ng = (uint32_t)a.groups;
    const uint32_t bk = uu / ng, grp = uu - bk * ng;
    const QInfo qi = query_info<G>(a, bk, grp, t);
    if (!qi.valid) return;  // (uniform: the whole workgroup)
    const size_t kv0 = (size_t)bk * (size_t)a.n * D;
    const T *kb = k + kv0, *vb = v + kv0;
    const int wn = qi.base + qi.wcount;
    const int c0 = (int)c * kWinChunkRows;
    const int cnt = wn - c0 < kWinChunkRows ? wn - c0 : kWinChunkRows;  // (may be <= 0)
    const uint4 qs = reinterpret_cast<const uint4 *>(q + (size_t)qi.qv * D)[lane % AS::LPR];
    auto row_at = [&](int e) -> size_t {
        const int f = c0 + e;
        return f < qi.base ? 0 : (size_t)(qi.wlo - qi.base + f);
    };
    if (cnt > 0) {
        wave_partial<D, T, UWIN>(qs, kb, vb, row_at, cnt, wave, kWaves, a.scale_log2e, part, wave);
    } else {
        for (int e = lane; e < D; e += 64) part.acc[wave][e] = 0.f;
        if (lane == 0) { part.m[wave] = -INFINITY; part.l[wave] = 0.f; }
    }
    __syncthreads();
    float *dst = a.win + ((size_t)qi.qv * a.nch + c) * (D + 2);
    float mx = -INFINITY;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) mx = fmaxf(mx, part.m[w]);
    float f[kWaves], l = 0.f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
        f[w] = part.m[w] == -INFINITY ? 0.f : exp2f((part.m[w] - mx) * a.scale_log2e);
        l += part.l[w] * f[w];
    }
    for (int e = tid; e < D; e += kNT) {
        float o = 0.f;
#pragma unroll
        for (int w = 0; w < kWaves; ++w) o = fmaf(part.acc[w][e], f[w], o);
        dst[2 + e] = o;
    }
    if (tid == 0) {
        dst[0] = mx;
        dst[1] = l;
    }
}

// ---- decode_stream: keys of two blocks into LDS, then the block records ---------------------
template <typename T, int D, int G, bool MASS>
__global__ __launch_bounds__(kNT) __attribute__((amdgpu_waves_per_eu(sizeof(T) == 2 ? 5 : 4))) void decode_stream_kernel(
    const T *__restrict__ q, const T *__restrict__ k, const T *__restrict__ v, DecodeArgs a) {
    __shared__ uint32_t kst[G][kBW * kRows];  // keys of the workgroup's rows, per query
    // The workgroups after the units' key workgroups make the anchor-and-window partials.
    const uint32_t nkey = a.units * (uint32_t)((a.nblk + kBW - 1) / kBW);
    if (blockIdx.x >= nkey) {
        __shared__ SoftmaxPartials<D, kWaves> wpart;
        if (a.win) window_chunk<T, D, G>(q, k, v, a, blockIdx.x - nkey, wpart);
        return;
    }
    // Key workgroup s: unit s % units, its part s / units.
    const uint32_t sblk = blockIdx.x;
    const uint32_t part = sblk / a.units;
    const uint32_t uu = sblk - part * a.units;
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
        // (Every term is at most 1: zm is the block's best score. The hardware exponential
        // flushes terms below 2^-126 to zero.)
        zm = k1 ? key_score(k1) : -INFINITY;
        const float zmc = k1 ? zm * a.scale_log2e : 0.f;
        float zsum = 0.f;
#pragma unroll
        for (int c = 0; c < 16; ++c)
            zsum += kk[c] ? __builtin_amdgcn_exp2f(__builtin_fmaf(key_score(kk[c]), a.scale_log2e, -zmc)) : 0.f;
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

}  // namespace
}  // namespace dec

hipError_t launch_decode_stream(const Plan &pl, const void *q, const void *k, const void *v, void *ws,
                                bool mass, bool attend, hipStream_t s) {
    using namespace dec;
    DecodeArgs a = decode_args(pl, ws, nullptr, nullptr, nullptr);
    if (!attend) a.win = nullptr;  // (no output: the window partials are not needed)
    const uint32_t wpb = (uint32_t)((pl.nblk + kBW - 1) / kBW);
    const uint64_t nwin = a.win ? (uint64_t)pl.units * pl.G * pl.win_chunks : 0;
    const dim3 grid((unsigned)((uint64_t)pl.units * wpb + nwin)), block(kNT);
#define CA_DS(T, D, G)                                                                                   \
    do {                                                                                                 \
        const T *qt = static_cast<const T *>(q), *kt = static_cast<const T *>(k), *vt = static_cast<const T *>(v); \
        if (mass) hipLaunchKernelGGL((decode_stream_kernel<T, D, G, true>), grid, block, 0, s, qt, kt, vt, a); \
        else hipLaunchKernelGGL((decode_stream_kernel<T, D, G, false>), grid, block, 0, s, qt, kt, vt, a);   \
    } while (0)
#define CA_DS_G(T, D)                                   \
    do {                                                \
        if (pl.G == 4) CA_DS(T, D, 4);                  \
        else if (pl.G == 2) CA_DS(T, D, 2);             \
        else CA_DS(T, D, 1);                            \
    } while (0)
    if (pl.dtype == 1) {
        if (pl.d == 128) CA_DS_G(__bf16, 128); else CA_DS_G(__bf16, 64);
    } else {
        if (pl.d == 128) CA_DS_G(float, 128); else CA_DS_G(float, 64);
    }
#undef CA_DS_G
#undef CA_DS
    return hipGetLastError();
}


}  // namespace ca
