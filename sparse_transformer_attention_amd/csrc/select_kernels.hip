// Stage 1 of condensate attention on gfx950: score every causal key and select the
// condensate set C_i = {0} u {i-W+1..i} u Top-k_i (pages of "The Condensate Theorem",
// metaphor-xennon blog, section 2.1 Definition 1 and section 2.2.3; the top-k part ranks the
// positions R_i = {1..i-W} outside the anchor and window, ties toward the smaller position).
//
// Two kernels:
//   score_select   one workgroup per (key chunk, query group, batch*kv_head). Streams the
//                  chunk's K rows once with 16-byte loads, computes fp32 dot products for up
//                  to G query vectors that share the KV head, keeps the chunk's order keys in
//                  LDS, and then each wavefront radix-selects the chunk-local exact top-k of
//                  one query and writes it to the candidate workspace.
//   merge_assemble one workgroup per query vector: exact top-k over the chunk candidates
//                  (radix select on 64-bit keys), then C_i in ascending order into out_idx.
//
// Ranking key of a candidate j with fp32 score s: (score_key(s) << 32) | ~j. The order is
// total, so the chunk-local top-k lists always contain the global top-k and the merge is exact.
#include "ca_internal.h"
#include "device_utils.h"

namespace ca {
namespace {

struct ScoreSelectArgs {
    int64_t n, nq;
    int Hq, Hkv, g, W, topk, chunk;
    int64_t groups, nchunks;
};

// One wavefront: exact top-kc of the nvalid keys keys[0..nvalid) (LDS), key order
// (key desc, position asc); the winners go to out[0..kc) as 64-bit ranking keys, in position
// order. hist is this wavefront's 256-entry LDS histogram.
__device__ void wave_select_emit(const uint32_t *keys, int nvalid, int kc, int64_t row0,
                                 uint32_t *hist, uint64_t *__restrict__ out) {
    const int lane = threadIdx.x & 63;
    uint32_t prefix = 0, mask = 0;
    int rem = kc;
    if (kc < nvalid) {
        // Most significant digit first: keep the digit holding the rem-th largest key.
        for (int shift = 24; shift >= 0; shift -= 8) {
            reinterpret_cast<uint4 *>(hist)[lane] = make_uint4(0, 0, 0, 0);
            wave_sync();
            for (int e = lane; e < nvalid; e += 64) {
                uint32_t key = keys[e];
                if ((key & mask) == prefix) atomicAdd(&hist[(key >> shift) & 255u], 1u);
            }
            wave_sync();
            const uint4 h = reinterpret_cast<const uint4 *>(hist)[lane];  // bins 4l..4l+3
            const uint32_t own = h.x + h.y + h.z + h.w;
            uint32_t incl = own;  // keys in bins >= 4*lane
#pragma unroll
            for (int off = 1; off < 64; off <<= 1) {
                uint32_t o = __shfl_down(incl, off);
                if (lane + off < 64) incl += o;
            }
            const uint32_t excl = incl - own;  // keys in bins >= 4*lane + 4
            const uint32_t c3 = excl + h.w, c2 = c3 + h.z, c1 = c2 + h.y, c0 = incl;
            const uint32_t r = (uint32_t)rem;
            const bool mine = (incl >= r) && (excl < r);
            const int u = (c3 >= r) ? 3 : (c2 >= r) ? 2 : (c1 >= r) ? 1 : 0;
            const uint32_t hd = (u == 3) ? h.w : (u == 2) ? h.z : (u == 1) ? h.y : h.x;
            const uint32_t cd = (u == 3) ? c3 : (u == 2) ? c2 : (u == 1) ? c1 : c0;
            const int src = __ffsll((unsigned long long)__ballot(mine)) - 1;
            const uint32_t digit = (uint32_t)__shfl(4 * lane + u, src);
            const uint32_t h_digit = (uint32_t)__shfl((int)hd, src);
            const uint32_t above = (uint32_t)__shfl((int)(cd - hd), src);
            rem -= (int)above;
            prefix |= digit << shift;
            mask |= 0xFFu << shift;
            wave_sync();
            if (h_digit == (uint32_t)rem) break;
        }
    }
    // Keys above the prefix are in; keys equal on the masked bits are in while fewer than rem
    // of them precede (smaller position wins a full tie).
    int tied_before = 0, written = 0;
    for (int e0 = 0; e0 < nvalid; e0 += 64) {
        const int e = e0 + lane;
        const bool valid = e < nvalid;
        const uint32_t key = valid ? keys[e] : 0u;
        const bool tied = valid && ((key & mask) == prefix);
        const uint64_t bt = __ballot(tied);
        const int rank = tied_before + lanes_below(bt);
        const bool sel = valid && (((key & mask) > prefix) || (tied && rank < rem));
        tied_before += __popcll(bt);
        const uint64_t bs = __ballot(sel);
        const int pos = written + lanes_below(bs);
        if (sel && pos < kc) {  // exactly kc are selected; the bound only guards the buffer
            const uint32_t j = (uint32_t)(row0 + e);
            out[pos] = ((uint64_t)key << 32) | (uint32_t)(~j);
        }
        written += __popcll(bs);
    }
}

template <typename T, int D, int G>
__global__ __launch_bounds__(256) void score_select_kernel(const T *__restrict__ q,
                                                           const T *__restrict__ k,
                                                           uint64_t *__restrict__ cand,
                                                           ScoreSelectArgs a) {
    extern __shared__ uint32_t smem[];  // [G][chunk] order keys, then [4][256] histograms
    constexpr int EB = sizeof(T);
    constexpr int RB = D * EB;          // bytes per key row
    constexpr int P = RB / 64;          // 16-byte loads per lane per row (4 lanes per row)
    constexpr int U = (P >= 8) ? 2 : (P == 4 ? 4 : 8);  // row groups in flight per wavefront
    static_assert(G == 1 || G == 2 || G == 4, "G");

    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int64_t lin = blockIdx.x;
    const int64_t c = lin % a.nchunks;
    const int64_t grp = (lin / a.nchunks) % a.groups;
    const int bk = (int)(lin / (a.nchunks * a.groups));  // b * Hkv + kvh
    const int kvh = bk % a.Hkv;
    const int b = bk / a.Hkv;
    const int64_t row0 = 1 + c * a.chunk;
    const int64_t nvec = (int64_t)a.g * a.nq;  // query vectors of this KV head

    // Last candidate row of each query of the group, -1 if the slot is empty.
    int64_t rlast[G];
    int64_t rl_max = -1;
#pragma unroll
    for (int t = 0; t < G; ++t) {
        const int64_t idx = grp * G + t;
        rlast[t] = -1;
        if (idx < nvec) {
            const int64_t r = idx / a.g;
            rlast[t] = (a.n - a.nq + r) - a.W;
            rl_max = rlast[t] > rl_max ? rlast[t] : rl_max;
        }
    }
    if (row0 > rl_max) return;  // no query of the group has candidates here
    const int64_t rows_end = (row0 + a.chunk < rl_max + 1) ? row0 + a.chunk : rl_max + 1;
    const int nrows = (int)(rows_end - row0);

    // Query slices: lane s = lane & 3 holds the 16-byte pieces p*64 + s*16 of each row.
    const int s = lane & 3;
    uint4 qr[G][P];
#pragma unroll
    for (int t = 0; t < G; ++t) {
        const int64_t idx = grp * G + t;
        if (idx < nvec) {
            const int64_t r = idx / a.g;
            const int h = kvh * a.g + (int)(idx % a.g);
            const uint4 *src = reinterpret_cast<const uint4 *>(q + (((int64_t)b * a.Hq + h) * a.nq + r) * D);
#pragma unroll
            for (int p = 0; p < P; ++p) qr[t][p] = src[p * 4 + s];
        } else {
#pragma unroll
            for (int p = 0; p < P; ++p) qr[t][p] = make_uint4(0, 0, 0, 0);
        }
    }

    // After the lane reduction each lane owns one query's score of its row (G == 4), lanes
    // with bit 0 clear own query (lane>>1)&1 (G == 2), or lane 0 of 4 owns query 0 (G == 1).
    const int my_t = (G == 4) ? (lane & 3) : (G == 2) ? ((lane >> 1) & 1) : 0;
    const bool writer = (G == 4) ? true : (G == 2) ? ((lane & 1) == 0) : ((lane & 3) == 0);
    int64_t my_rlast = rlast[0];
#pragma unroll
    for (int t = 1; t < G; ++t) my_rlast = (my_t == t) ? rlast[t] : my_rlast;
    uint32_t *my_keys = smem + my_t * a.chunk;

    const uint4 *kbase = reinterpret_cast<const uint4 *>(k + (int64_t)bk * a.n * D);
    const int ngroups = (nrows + 15) >> 4;  // 16 rows per wavefront step
    for (int gi0 = wave; gi0 < ngroups; gi0 += 4 * U) {
        uint4 kr[U][P];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int gi = gi0 + 4 * u;
            if (gi < ngroups) {
                int64_t row = row0 + gi * 16 + (lane >> 2);
                row = row < rows_end ? row : rows_end - 1;
                const uint4 *src = kbase + row * (RB / 16);
#pragma unroll
                for (int p = 0; p < P; ++p) kr[u][p] = src[p * 4 + s];
            }
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int gi = gi0 + 4 * u;
            if (gi >= ngroups) break;
            float acc[G];
#pragma unroll
            for (int t = 0; t < G; ++t) {
                float x = 0.f;
#pragma unroll
                for (int p = 0; p < P; ++p) x = dot16(kr[u][p], qr[t][p], x, T());
                acc[t] = x;
            }
            float score;
            if constexpr (G == 4) {
                const bool hi2 = (lane & 2) != 0;
                const float k0 = hi2 ? acc[2] : acc[0], s0 = hi2 ? acc[0] : acc[2];
                const float k1 = hi2 ? acc[3] : acc[1], s1 = hi2 ? acc[1] : acc[3];
                const float a0 = k0 + dpp_xor2(s0);
                const float a1 = k1 + dpp_xor2(s1);
                const bool hi1 = (lane & 1) != 0;
                const float kk = hi1 ? a1 : a0, ss = hi1 ? a0 : a1;
                score = kk + dpp_xor1(ss);
            } else if constexpr (G == 2) {
                const bool hi2 = (lane & 2) != 0;
                const float kk = hi2 ? acc[1] : acc[0], ss = hi2 ? acc[0] : acc[1];
                const float a0 = kk + dpp_xor2(ss);
                score = a0 + dpp_xor1(a0);
            } else {
                const float a0 = acc[0] + dpp_xor2(acc[0]);
                score = a0 + dpp_xor1(a0);
            }
            const int64_t row = row0 + gi * 16 + (lane >> 2);
            if (writer && row < rows_end)
                my_keys[row - row0] = (row <= my_rlast) ? score_key(score) : 0u;
        }
    }
    __syncthreads();

    // Chunk-local exact top-k, one query per wavefront.
    uint32_t *hist = smem + G * a.chunk + wave * 256;
    for (int t = wave; t < G; t += 4) {
        const int64_t idx = grp * G + t;
        if (idx >= nvec) continue;
        const int64_t r = idx / a.g;
        const int h = kvh * a.g + (int)(idx % a.g);
        const int64_t rl = (a.n - a.nq + r) - a.W;
        const int64_t vend = (rows_end < rl + 1) ? rows_end : rl + 1;
        const int nvalid = vend > row0 ? (int)(vend - row0) : 0;
        if (nvalid == 0) continue;
        const int kc = a.topk < nvalid ? a.topk : nvalid;
        const int64_t qv = ((int64_t)b * a.Hq + h) * a.nq + r;
        wave_select_emit(smem + t * a.chunk, nvalid, kc, row0, hist,
                         cand + (qv * a.nchunks + c) * a.topk);
    }
}

struct MergeArgs {
    int64_t n, nq, nchunks;
    int W, topk, chunk, cap;
};

// Keys (position-inverted low word) -> position.
__device__ __forceinline__ int32_t key_pos(uint64_t key) { return (int32_t)(~(uint32_t)key); }

__global__ __launch_bounds__(256) void merge_assemble_kernel(const uint64_t *__restrict__ cand,
                                                             int32_t *__restrict__ out_idx,
                                                             MergeArgs a) {
    extern __shared__ int32_t msm[];  // [topk] selected positions
    __shared__ uint32_t hist[256];
    __shared__ uint32_t wave_tot[4];
    __shared__ uint32_t pick[3];      // digit, count in digit, count above
    __shared__ int sel_count;

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int64_t qv = blockIdx.x;
    const int64_t r = qv % a.nq;
    const int64_t i = a.n - a.nq + r;
    const int64_t wlo = (i - a.W + 1 > 0) ? i - a.W + 1 : 0;
    const int64_t rl = i - a.W;
    const int64_t n_r = rl >= 1 ? rl : 0;
    const int kp = (int)(a.topk < n_r ? a.topk : n_r);
    int32_t *row = out_idx + qv * a.cap;

    if (kp > 0) {
        const uint64_t *keys = cand + qv * a.nchunks * a.topk;
        const int64_t nch = (n_r + a.chunk - 1) / a.chunk;  // chunks meeting R_i
        const int64_t slots = nch * a.topk;
        const int last_kc = (int)((n_r - (nch - 1) * a.chunk) < a.topk ? (n_r - (nch - 1) * a.chunk) : a.topk);
        const int full_kc = a.chunk < a.topk ? a.chunk : a.topk;
        const int64_t total = (nch - 1) * full_kc + last_kc;

        uint64_t prefix = 0, mask = 0;
        int rem = kp;
        if (kp < total) {
            for (int shift = 56; shift >= 0; shift -= 8) {
                hist[tid] = 0;
                __syncthreads();
                for (int64_t f = tid; f < slots; f += 256) {
                    const int64_t ch = f / a.topk;
                    const int sl = (int)(f - ch * a.topk);
                    if (sl >= (ch == nch - 1 ? last_kc : full_kc)) continue;
                    const uint64_t key = keys[f];
                    if ((key & mask) == prefix) atomicAdd(&hist[(uint32_t)(key >> shift) & 255u], 1u);
                }
                __syncthreads();
                // Suffix sums over the bins: incl = keys in bins >= tid.
                const uint32_t own = hist[tid];
                uint32_t incl = own;
#pragma unroll
                for (int off = 1; off < 64; off <<= 1) {
                    uint32_t o = __shfl_down(incl, off);
                    if (lane + off < 64) incl += o;
                }
                if (lane == 0) wave_tot[wave] = incl;
                __syncthreads();
                for (int w2 = wave + 1; w2 < 4; ++w2) incl += wave_tot[w2];
                if (incl >= (uint32_t)rem && incl - own < (uint32_t)rem) {
                    pick[0] = (uint32_t)tid;
                    pick[1] = own;
                    pick[2] = incl - own;
                }
                __syncthreads();
                const uint32_t digit = pick[0], h_digit = pick[1], above = pick[2];
                rem -= (int)above;
                prefix |= (uint64_t)digit << shift;
                mask |= (uint64_t)0xFF << shift;
                __syncthreads();  // pick[] and hist[] are rewritten next pass
                if (h_digit == (uint32_t)rem) break;
            }
        }
        // Keys are distinct, so exactly kp of them reach the prefix.
        if (tid == 0) sel_count = 0;
        __syncthreads();
        for (int64_t f = tid; f < slots; f += 256) {
            const int64_t ch = f / a.topk;
            const int sl = (int)(f - ch * a.topk);
            if (sl >= (ch == nch - 1 ? last_kc : full_kc)) continue;
            const uint64_t key = keys[f];
            if ((key & mask) >= prefix) {
                const int pos = atomicAdd(&sel_count, 1);
                if (pos < kp) msm[pos] = key_pos(key);  // exactly kp reach the prefix
            }
        }
        __syncthreads();
        // Ascending order by counting smaller positions. The anchor is separate here
        // (R_i non-empty means i - W + 1 >= 2), so the top-k part starts at slot 1.
        for (int t = tid; t < kp; t += 256) {
            const int32_t j = msm[t];
            int rank = 0;
            for (int u = 0; u < kp; ++u) rank += (msm[u] < j);
            row[1 + rank] = j;
        }
    }
    int64_t base = 0;
    if (wlo > 0) {
        if (tid == 0) row[0] = 0;
        base = 1 + kp;
    }
    const int64_t wcount = i - wlo + 1;
    for (int64_t t = tid; t < wcount; t += 256) row[base + t] = (int32_t)(wlo + t);
    for (int64_t t = base + wcount + tid; t < a.cap; t += 256) row[t] = -1;
}

}  // namespace

hipError_t launch_score_select(const Plan &pl, const void *q, const void *k, uint64_t *cand,
                               hipStream_t s) {
    ScoreSelectArgs a;
    a.n = pl.n; a.nq = pl.nq; a.Hq = pl.Hq; a.Hkv = pl.Hkv; a.g = pl.g; a.W = pl.W;
    a.topk = pl.topk; a.chunk = pl.chunk; a.groups = pl.groups; a.nchunks = pl.nchunks;
    const int64_t nblk = pl.nchunks * pl.groups * (int64_t)pl.B * pl.Hkv;
    const size_t shmem = ((size_t)pl.G * pl.chunk + 4 * 256) * sizeof(uint32_t);
    dim3 grid((unsigned)nblk), block(256);
#define CA_LAUNCH_SS(T, D, G)                                                                   \
    hipLaunchKernelGGL((score_select_kernel<T, D, G>), grid, block, shmem, s,                  \
                       static_cast<const T *>(q), static_cast<const T *>(k), cand, a)
#define CA_LAUNCH_SS_G(T, D)                         \
    do {                                             \
        if (pl.G == 4) CA_LAUNCH_SS(T, D, 4);        \
        else if (pl.G == 2) CA_LAUNCH_SS(T, D, 2);   \
        else CA_LAUNCH_SS(T, D, 1);                  \
    } while (0)
    if (pl.dtype == 1) {
        if (pl.d == 128) CA_LAUNCH_SS_G(__bf16, 128); else CA_LAUNCH_SS_G(__bf16, 64);
    } else {
        if (pl.d == 128) CA_LAUNCH_SS_G(float, 128); else CA_LAUNCH_SS_G(float, 64);
    }
#undef CA_LAUNCH_SS_G
#undef CA_LAUNCH_SS
    return hipGetLastError();
}

hipError_t launch_merge_assemble(const Plan &pl, const uint64_t *cand, int32_t *out_idx,
                                 hipStream_t s) {
    MergeArgs a;
    a.n = pl.n; a.nq = pl.nq; a.nchunks = pl.nchunks; a.W = pl.W; a.topk = pl.topk;
    a.chunk = pl.chunk; a.cap = pl.cap;
    const size_t shmem = (size_t)(pl.topk > 0 ? pl.topk : 1) * sizeof(int32_t);
    hipLaunchKernelGGL(merge_assemble_kernel, dim3((unsigned)pl.nqv), dim3(256), shmem, s, cand,
                       out_idx, a);
    return hipGetLastError();
}

}  // namespace ca
