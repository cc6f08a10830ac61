// Exact top-k' of a query's candidates over the whole workgroup, shared by the kernels that end
// the path (pages of "The Condensate Theorem", metaphor-xennon blog, section 2.2.3: the top-k
// part of C_i over R_i, ranked by score and, on equal scores, by the smaller position; ranking
// keys (score_key << 32) | ~position as in select_core.h).
#pragma once

#include "device_utils.h"
#include "select_core.h"

namespace ca {

constexpr int kGather = 1024;  // candidates gathered into LDS for the one-wavefront select
// Room for gathered candidates by workgroup size: 64- and 128-thread workgroups (the MFMA path)
// gather lists of at most 256 keys.
template <int NT>
constexpr int kGatherFor = NT <= 128 ? 256 : kGather;
constexpr int kMaxKeysPerThread = 16;  // candidate keys held in registers per thread

template <int NT>
struct SelectShared {
    uint32_t hist[NT / 64][320];  // words 256 + lane absorb keys outside the current prefix
    uint64_t red64[2][NT / 64];
    uint32_t wtot[NT / 64];
    uint32_t pick[3];
    int sel_count;
};

// Exact top-kp of one query's candidates, given as n keys gathered in LDS (gathered[0..n) when
// n <= kGatherFor<NT>) and as key_at(f) over f in [0, slots) (0 = no candidate): the distinct,
// non-zero ranking keys. The kp positions go to js[0..kp), ascending (js needs room for 2*kp),
// and with jk their score keys to jk[0..kp) in the same order (jk needs room for 2*kp too).
// Up to kGatherFor<NT> candidates are selected by wavefront 0 alone with the keys in registers; more
// by the whole workgroup, calling key_at on every radix pass.
template <int NT, typename KeyAt>
__device__ __forceinline__ void select_exact(int n, int64_t slots, KeyAt key_at, int kp, int32_t *js,
                                             uint64_t *sel, const uint64_t *gathered,
                                             SelectShared<NT> &sh, uint32_t *jk = nullptr) {
    constexpr int NW = NT / 64;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    if (n <= kGatherFor<NT>) {
        if (wave == 0) {
            uint64_t kk[kMaxKeysPerThread];
#pragma unroll
            for (int e = 0; e < kMaxKeysPerThread; ++e) {
                const int f = lane + 64 * e;
                kk[e] = f < n && f < kGatherFor<NT> ? gathered[f] : 0ull;
            }
            (void)wave_keep_top_u64(kk, kp, &sh.hist[0][0], sel);
        }
        __syncthreads();
        for (int t = tid; t < kp; t += NT) {
            js[t] = rank_key_pos(sel[t]);
            if (jk) jk[t] = (uint32_t)(sel[t] >> 32);
        }
    } else if constexpr (NT >= 256) {
        // (128-thread workgroups select from at most 256 keys: never here.)
        uint64_t kmax = 0ull, kmin = ~0ull;
        for (int64_t f = tid; f < slots; f += NT) {
            const uint64_t x = key_at(f);
            if (x) { kmax = x > kmax ? x : kmax; kmin = x < kmin ? x : kmin; }
        }
        kmax = wave_max_u64_dpp(kmax);
        kmin = wave_min_u64_dpp(kmin);
        if (lane == 0) { sh.red64[0][wave] = kmax; sh.red64[1][wave] = kmin; }
        __syncthreads();
        kmax = sh.red64[0][0];
        kmin = sh.red64[1][0];
#pragma unroll
        for (int w2 = 1; w2 < NW; ++w2) {
            kmax = sh.red64[0][w2] > kmax ? sh.red64[0][w2] : kmax;
            kmin = sh.red64[1][w2] < kmin ? sh.red64[1][w2] : kmin;
        }
        int hb = 63 - __builtin_clzll((kmax ^ kmin) | 1ull);
        uint64_t mask = hb >= 63 ? 0ull : (~0ull << (hb + 1));
        uint64_t prefix = kmax & mask;
        int rem = kp;
        if (kp >= n) { hb = -1; mask = 0ull; prefix = 0ull; }
        while (hb >= 0) {
            const int lb = hb >= 7 ? hb - 7 : 0;
            const uint32_t dmask = (2u << (hb - lb)) - 1u;
            for (int t = tid; t < NW * 320; t += NT) (&sh.hist[0][0])[t] = 0u;
            __syncthreads();
            for (int64_t f = tid; f < slots; f += NT) {
                const uint64_t x = key_at(f);
                const bool in = x && (x & mask) == prefix;
                atomicAdd(&sh.hist[wave][in ? (uint32_t)(x >> lb) & dmask : 256u + lane], 1u);
            }
            __syncthreads();
            uint32_t own = 0u, pre = 0u;
            if (tid < 256) {
#pragma unroll
                for (int w2 = 0; w2 < NW; ++w2) own += sh.hist[w2][tid];
                pre = wave_incl_scan_u32(own);
                if (lane == 63) sh.wtot[wave] = pre;
            }
            __syncthreads();
            if (tid < 256) {
                uint32_t before = 0u, all = 0u;
#pragma unroll
                for (int w2 = 0; w2 < 4; ++w2) {
                    before += w2 < wave ? sh.wtot[w2] : 0u;
                    all += sh.wtot[w2];
                }
                const uint32_t incl = all - (before + pre) + own;  // keys in bins >= tid
                if (incl >= (uint32_t)rem && incl - own < (uint32_t)rem) {  // exactly one bin
                    sh.pick[0] = (uint32_t)tid;
                    sh.pick[1] = own;
                    sh.pick[2] = incl - own;
                }
            }
            __syncthreads();
            const uint32_t digit = sh.pick[0], h_digit = sh.pick[1], above = sh.pick[2];
            rem -= (int)above;
            prefix |= (uint64_t)digit << lb;
            mask |= (uint64_t)dmask << lb;
            __syncthreads();
            if (h_digit == (uint32_t)rem) break;  // distinct keys: reached by the last digit
            hb = lb - 1;
        }
        if (tid == 0) sh.sel_count = 0;
        __syncthreads();
        for (int64_t f = tid; f < slots; f += NT) {
            const uint64_t x = key_at(f);
            if (x && (x & mask) >= prefix) {
                const int pos = atomicAdd(&sh.sel_count, 1);
                if (pos < kp) {
                    js[pos] = rank_key_pos(x);
                    if (jk) jk[pos] = (uint32_t)(x >> 32);
                }
            }
        }
    }
    __syncthreads();
    // Ascending order: each position's rank is the number of smaller ones; the sorted copy
    // goes to js[kp..2kp) and then back.
    for (int t0 = 0; t0 < kp; t0 += NT) {
        const int t = t0 + tid;
        if (t < kp) {
            const int32_t j = js[t];
            int rank = 0;
#pragma unroll 8
            for (int u = 0; u < kp; ++u) rank += js[u] < j;
            js[kp + rank] = j;
            if (jk) jk[kp + rank] = jk[t];
        }
    }
    __syncthreads();
    for (int t = tid; t < kp; t += NT) {
        js[t] = js[kp + t];
        if (jk) jk[t] = jk[kp + t];
    }
    __syncthreads();
}


}  // namespace ca
