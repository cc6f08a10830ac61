// Exact wavefront-level top-k selection on 64-bit ranking keys, shared by the score and finish
// kernels. A ranking key orders candidates the way the top-k part of the condensate set does
// (pages of "The Condensate Theorem", metaphor-xennon blog, section 2.2.3): higher score first,
// and on equal scores the smaller position first:
//     key = (score_key(s) << 32) | ~j,
// so keys of distinct positions are distinct and the order is total. 0 marks an empty slot
// (every real key has a high word >= 0x00800000).
#pragma once

#include "device_utils.h"

namespace ca {

// Exclusive prefix sum over the lanes of a wavefront; *total gets the wavefront sum.
__device__ __forceinline__ int wave_excl_scan(int x, int *total) {
    const uint32_t incl = wave_incl_scan_u32((uint32_t)x);
    *total = (int)__builtin_amdgcn_readlane(incl, 63);
    return (int)incl - x;
}

__device__ __forceinline__ uint64_t make_rank_key(uint32_t skey, uint32_t pos) {
    return ((uint64_t)skey << 32) | (uint32_t)(~pos);
}
__device__ __forceinline__ int32_t rank_key_pos(uint64_t key) { return (int32_t)(~(uint32_t)key); }

// One wavefront keeps the `keep` largest of the distinct non-zero keys kr[0..E) of its lanes
// (0 = empty) and writes them to dst[0..min(keep, count)) in any order. dst may be the keys'
// own source: every lane holds its keys in registers before anything is written. Radix select
// (8-bit digits, starting at the highest bit where the keys differ) with a 320-word LDS
// histogram per wavefront (words 256 + lane absorb keys outside the current prefix).
// Returns the high word of the smallest kept key (0xFFFFFFFF if none is kept). With
// dst == nullptr nothing is written: only that high word is computed.
template <int E>
__device__ __forceinline__ uint32_t wave_keep_top_u64(const uint64_t (&kr)[E], int keep,
                                                      uint32_t *hist, uint64_t *dst) {
    const int lane = threadIdx.x & 63;
    int nz = 0;
#pragma unroll
    for (int e = 0; e < E; ++e) nz += kr[e] != 0ull;
    int total;
    (void)wave_excl_scan(nz, &total);
    uint64_t prefix = 0ull, mask = 0ull;
    if (keep < total) {
        uint32_t hmax = 0u, hmin = 0xFFFFFFFFu;
#pragma unroll
        for (int e = 0; e < E; ++e) {
            const uint32_t hi = (uint32_t)(kr[e] >> 32);
            if (kr[e]) { hmax = hi > hmax ? hi : hmax; hmin = hi < hmin ? hi : hmin; }
        }
        hmax = wave_max_u32_dpp(hmax);
        hmin = wave_min_u32_dpp(hmin);
        int hb;
        uint32_t lmax = 0u;
        if (hmax != hmin) {
            hb = 32 + 31 - __builtin_clz(hmax ^ hmin);
        } else {
            uint32_t lmin = 0xFFFFFFFFu;
#pragma unroll
            for (int e = 0; e < E; ++e) {
                const uint32_t lo = (uint32_t)kr[e];
                if (kr[e]) { lmax = lo > lmax ? lo : lmax; lmin = lo < lmin ? lo : lmin; }
            }
            lmax = wave_max_u32_dpp(lmax);
            lmin = wave_min_u32_dpp(lmin);
            hb = 31 - __builtin_clz((lmax ^ lmin) | 1u);
        }
        // Bits above hb are common to every key. (A 64-bit shift by 64 is undefined: hb == 63
        // whenever the scores have both signs.)
        mask = hb >= 63 ? 0ull : (~0ull << (hb + 1));
        prefix = (((uint64_t)hmax << 32) | lmax) & mask;
        int rem = keep;
        while (hb >= 0) {
            const int lb = hb >= 7 ? hb - 7 : 0;
            const uint32_t dmask = (2u << (hb - lb)) - 1u;
            reinterpret_cast<uint4 *>(hist)[lane] = make_uint4(0, 0, 0, 0);
            wave_sync();
#pragma unroll
            for (int e = 0; e < E; ++e) {
                const uint64_t key = kr[e];
                const bool in = key != 0ull && (key & mask) == prefix;
                atomicAdd(&hist[in ? (uint32_t)(key >> lb) & dmask : 256u + lane], 1u);
            }
            wave_sync();
            const uint4 h = reinterpret_cast<const uint4 *>(hist)[lane];  // bins 4l..4l+3
            const uint32_t own = h.x + h.y + h.z + h.w;
            const uint32_t pre = wave_incl_scan_u32(own);
            const uint32_t all = __builtin_amdgcn_readlane(pre, 63);
            const uint32_t excl = all - pre, incl = excl + own;  // keys in bins >= 4l+4, >= 4l
            const uint32_t c3 = excl + h.w, c2 = c3 + h.z, c1 = c2 + h.y, c0 = incl;
            const uint32_t r = (uint32_t)rem;
            const bool mine = (incl >= r) && (excl < r);
            const int u = (c3 >= r) ? 3 : (c2 >= r) ? 2 : (c1 >= r) ? 1 : 0;
            const uint32_t hd = (u == 3) ? h.w : (u == 2) ? h.z : (u == 1) ? h.y : h.x;
            const uint32_t cd = (u == 3) ? c3 : (u == 2) ? c2 : (u == 1) ? c1 : c0;
            int src = __ffsll((unsigned long long)__ballot(mine)) - 1;
            src = src < 0 ? 0 : src;
            const uint32_t digit = __builtin_amdgcn_readlane((uint32_t)(4 * lane + u), src);
            const uint32_t h_digit = __builtin_amdgcn_readlane(hd, src);
            const uint32_t above = __builtin_amdgcn_readlane(cd - hd, src);
            rem -= (int)above;
            prefix |= (uint64_t)digit << lb;
            mask |= (uint64_t)dmask << lb;
            wave_sync();
            if (h_digit == (uint32_t)rem) break;  // distinct keys: reached by the last digit
            hb = lb - 1;
        }
    }
    const int lim = keep < total ? keep : total;
    int cnt = 0;
    uint32_t tmin = 0xFFFFFFFFu;
#pragma unroll
    for (int e = 0; e < E; ++e) {
        const bool sel = kr[e] != 0ull && (kr[e] & mask) >= prefix;
        cnt += sel;
        const uint32_t hi = (uint32_t)(kr[e] >> 32);
        tmin = (sel && hi < tmin) ? hi : tmin;
    }
    if (dst != nullptr) {
        int tot;
        int pos = wave_excl_scan(cnt, &tot);
        wave_sync();  // every lane holds its keys before dst (possibly their source) is written
#pragma unroll
        for (int e = 0; e < E; ++e) {
            if (kr[e] != 0ull && (kr[e] & mask) >= prefix) {
                if (pos < lim) dst[pos] = kr[e];
                ++pos;
            }
        }
        wave_sync();
    }
    return wave_min_u32_dpp(tmin);
}

// Maximum / minimum of 64-bit values over the lanes of a wavefront (uniform result).
__device__ __forceinline__ uint64_t wave_max_u64_dpp(uint64_t x) {
    const uint32_t hi = (uint32_t)(x >> 32);
    const uint32_t hmax = wave_max_u32_dpp(hi);
    const uint32_t lmax = wave_max_u32_dpp(hi == hmax ? (uint32_t)x : 0u);
    return ((uint64_t)hmax << 32) | lmax;
}
__device__ __forceinline__ uint64_t wave_min_u64_dpp(uint64_t x) {
    const uint32_t hi = (uint32_t)(x >> 32);
    const uint32_t hmin = wave_min_u32_dpp(hi);
    const uint32_t lmin = wave_min_u32_dpp(hi == hmin ? (uint32_t)x : 0xFFFFFFFFu);
    return ((uint64_t)hmin << 32) | lmin;
}

// A value T that exactly `keep` of the wavefront's distinct non-zero keys kr[0..E) reach (0 =
// empty; at least `keep` keys, keep >= 1): the keys >= T are the top `keep`. Found bit by bit
// from the highest bit where the keys differ, each step counting the keys that reach the
// candidate value with ballots (no LDS); it stops as soon as exactly `keep` reach it.
template <int E>
__device__ __forceinline__ uint64_t wave_kth_u64(const uint64_t (&kr)[E], int keep) {
    uint64_t mx = 0ull, mn = ~0ull;
#pragma unroll
    for (int e = 0; e < E; ++e) {
        if (kr[e]) { mx = kr[e] > mx ? kr[e] : mx; mn = kr[e] < mn ? kr[e] : mn; }
    }
    mx = wave_max_u64_dpp(mx);
    mn = wave_min_u64_dpp(mn);
    if (mx == mn) return mx;
    const int hb = 63 - __builtin_clzll(mx ^ mn);
    uint64_t t = hb >= 63 ? 0ull : (mx >> (hb + 1)) << (hb + 1);
    for (int bit = hb; bit >= 0; --bit) {
        const uint64_t c = t | (1ull << bit);
        int cnt = 0;
#pragma unroll
        for (int e = 0; e < E; ++e) cnt += __popcll(__ballot(kr[e] >= c));
        if (cnt >= keep) {
            t = c;
            if (cnt == keep) break;
        }
    }
    return t;
}

// A value t that at least `keep` of the wavefront's non-zero values v[0..E) reach (at least `keep`
// of them must be non-zero), found bit by bit from the highest bit where they differ; the
// search stops as soon as at most keep + slack values reach t, so without equal values near the
// keep-th largest that many at most reach it.
template <int E>
__device__ __forceinline__ uint32_t wave_loose_kth_u32(const uint32_t (&v)[E], int keep, int slack) {
    uint32_t mx = 0u, mn = 0xFFFFFFFFu;
#pragma unroll
    for (int e = 0; e < E; ++e) {
        if (v[e]) { mx = v[e] > mx ? v[e] : mx; mn = v[e] < mn ? v[e] : mn; }
    }
    mx = wave_max_u32_dpp(mx);
    mn = wave_min_u32_dpp(mn);
    if (mx == mn) return mx;
    const int hb = 31 - __builtin_clz(mx ^ mn);
    uint32_t t = hb >= 31 ? 0u : (mx >> (hb + 1)) << (hb + 1);
    for (int bit = hb; bit >= 0; --bit) {
        const uint32_t c = t | (1u << bit);
        int cnt = 0;
#pragma unroll
        for (int e = 0; e < E; ++e) cnt += __popcll(__ballot(v[e] >= c));
        if (cnt >= keep) {
            t = c;
            if (cnt <= keep + slack) break;
        }
    }
    return t;
}

// A value that at least `keep` of the wavefront's non-zero values v[0..E) reach, close to their
// keep-th largest: the largest P whose bits above the highest bit hb where the values differ are
// theirs, whose bits below lb = hb - 9 are 0, and which `keep` values reach (the lower edge of the
// 10-bit radix bin that holds the keep-th largest value). Found bit by bit from hb down, each
// step a count of the values that reach the candidate (compares and one DPP sum: no LDS, no
// atomics). 0 when there are fewer than `keep` values.
template <int E>
__device__ __forceinline__ uint32_t wave_bound_u32(const uint32_t (&v)[E], int keep) {
    int nz = 0;
    uint32_t hmax = 0u, hmin = 0xFFFFFFFFu;
#pragma unroll
    for (int e = 0; e < E; ++e) {
        if (v[e]) { ++nz; hmax = v[e] > hmax ? v[e] : hmax; hmin = v[e] < hmin ? v[e] : hmin; }
    }
    int total;
    (void)wave_excl_scan(nz, &total);
    if (keep < 1 || total < keep) return 0u;
    hmax = wave_max_u32_dpp(hmax);
    hmin = wave_min_u32_dpp(hmin);
    if (hmax == hmin) return hmax;
    const int hb = 31 - __builtin_clz(hmax ^ hmin);
    const int lb = hb >= 9 ? hb - 9 : 0;
    uint32_t p = hb >= 31 ? 0u : (hmax >> (hb + 1)) << (hb + 1);
    for (int bit = hb; bit >= lb; --bit) {
        const uint32_t cand = p | (1u << bit);
        uint32_t c = 0u;
#pragma unroll
        for (int e = 0; e < E; ++e) c += v[e] >= cand ? 1u : 0u;
        c = __builtin_amdgcn_readlane(wave_incl_scan_u32(c), 63);
        if (c >= (uint32_t)keep) p = cand;
    }
    return p;
}

// One wavefront thins its distinct non-zero keys kr[0..E) (0 = empty) to those whose high word
// reaches the 8-bit radix bin that holds the keep-th largest high word: at least `keep` keys,
// usually a few more. One histogram pass over the highest differing bits of the high words
// replaces the full select. The kept keys go to dst[0..count) in any order (dst may be their
// source). If the kept set would exceed `limit` keys, or every high word is the same, it falls
// back to the exact top-keep. Returns the number kept; *thr gets a high word that at least
// `keep` kept keys reach (0 when there are no more than `keep` keys).
template <int E>
__device__ __forceinline__ int wave_thin_u64(const uint64_t (&kr)[E], int keep, int limit, uint32_t *hist,
                                             uint64_t *dst, uint32_t *thr) {
    const int lane = threadIdx.x & 63;
    int nz = 0;
    uint32_t hmax = 0u, hmin = 0xFFFFFFFFu;
#pragma unroll
    for (int e = 0; e < E; ++e) {
        const uint32_t hi = (uint32_t)(kr[e] >> 32);
        if (kr[e]) { ++nz; hmax = hi > hmax ? hi : hmax; hmin = hi < hmin ? hi : hmin; }
    }
    int total;
    (void)wave_excl_scan(nz, &total);
    hmax = wave_max_u32_dpp(hmax);
    hmin = wave_min_u32_dpp(hmin);
    uint32_t t = 0u;
    if (total > keep) {
        if (hmax == hmin) {
            *thr = wave_keep_top_u64(kr, keep, hist, dst);
            return keep;
        }
        const int hb = 31 - __builtin_clz(hmax ^ hmin);
        const int lb = hb >= 7 ? hb - 7 : 0;
        const uint32_t dmask = (2u << (hb - lb)) - 1u;
        reinterpret_cast<uint4 *>(hist)[lane] = make_uint4(0, 0, 0, 0);
        wave_sync();
#pragma unroll
        for (int e = 0; e < E; ++e)
            if (kr[e]) atomicAdd(&hist[((uint32_t)(kr[e] >> 32) >> lb) & dmask], 1u);
        wave_sync();
        const uint4 h = reinterpret_cast<const uint4 *>(hist)[lane];  // bins 4l..4l+3
        const uint32_t own = h.x + h.y + h.z + h.w;
        const uint32_t pre = wave_incl_scan_u32(own);
        const uint32_t all = __builtin_amdgcn_readlane(pre, 63);
        const uint32_t excl = all - pre;  // keys in bins >= 4l+4
        const uint32_t c3 = excl + h.w, c2 = c3 + h.z, c1 = c2 + h.y, c0 = c1 + h.x;
        const uint32_t r = (uint32_t)keep;
        const bool mine = (c0 >= r) && (excl < r);
        const int u = (c3 >= r) ? 3 : (c2 >= r) ? 2 : (c1 >= r) ? 1 : 0;
        const uint32_t cd = (u == 3) ? c3 : (u == 2) ? c2 : (u == 1) ? c1 : c0;
        int src = __ffsll((unsigned long long)__ballot(mine)) - 1;
        src = src < 0 ? 0 : src;
        const uint32_t digit = __builtin_amdgcn_readlane((uint32_t)(4 * lane + u), src);
        const uint32_t kept = __builtin_amdgcn_readlane(cd, src);
        wave_sync();
        if ((int)kept > limit) {
            *thr = wave_keep_top_u64(kr, keep, hist, dst);
            return keep;
        }
        const uint32_t pfx = hb >= 31 ? 0u : (hmax >> (hb + 1)) << (hb + 1);
        t = pfx | (digit << lb);
    }
    int cnt = 0;
#pragma unroll
    for (int e = 0; e < E; ++e) cnt += kr[e] != 0ull && (uint32_t)(kr[e] >> 32) >= t;
    int tot;
    int pos = wave_excl_scan(cnt, &tot);
    wave_sync();  // every lane holds its keys before dst (possibly their source) is written
#pragma unroll
    for (int e = 0; e < E; ++e) {
        if (kr[e] != 0ull && (uint32_t)(kr[e] >> 32) >= t) {
            dst[pos] = kr[e];
            ++pos;
        }
    }
    wave_sync();
    *thr = t;
    return tot;
}

// ---- rank counting by groups of 8 lanes ----

// The number of keys y of list[0..n) with beats(y, s), s = 0 and 1, summed over
// the 8 lanes of each group (every lane of the group gets both): lane `part` of a group reads keys
// 16 i + 2 part and 16 i + 2 part + 1 (the group reads 128 contiguous bytes, four 16-byte reads
// in flight per lane). Reads reach list[64 ceil(n / 64) - 1]: the caller's storage must hold that
// much, 16-byte aligned; entries past n are not counted.
// Both counts come from the same reads (beats(y, 0) and beats(y, 1): two members per group).
template <typename Beats>
__device__ __forceinline__ uint2 group8_count(const uint64_t *list, int n, Beats beats) {
    const int part = threadIdx.x & 7;
    uint32_t r0 = 0u, r1 = 0u;
    for (int j0 = 0; j0 < n; j0 += 64) {
        uint4 x[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) x[e] = *reinterpret_cast<const uint4 *>(list + j0 + 16 * e + 2 * part);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int j = j0 + 16 * e + 2 * part;
            const uint64_t y0 = ((uint64_t)x[e].y << 32) | x[e].x, y1 = ((uint64_t)x[e].w << 32) | x[e].z;
            r0 += (j < n && beats(y0, 0)) ? 1u : 0u;
            r0 += (j + 1 < n && beats(y1, 0)) ? 1u : 0u;
            r1 += (j < n && beats(y0, 1)) ? 1u : 0u;
            r1 += (j + 1 < n && beats(y1, 1)) ? 1u : 0u;
        }
    }
    r0 += dpp_u32<0xB1>(0u, r0);   // lane ^ 1
    r1 += dpp_u32<0xB1>(0u, r1);
    r0 += dpp_u32<0x4E>(0u, r0);   // lane ^ 2
    r1 += dpp_u32<0x4E>(0u, r1);
    r0 += dpp_u32<0x141>(0u, r0);  // the mirrored lane of the group of 8: the other quad
    r1 += dpp_u32<0x141>(0u, r1);
    return make_uint2(r0, r1);
}

// As group8_count with four members per group (beats(y, s), s = 0..3) and no bounds test: the
// entries from n up to 64 ceil(n / 64) must be 0 keys, which beat no member under either use
// (y > x, and a position ~low word below p).
template <typename Beats>
__device__ __forceinline__ uint4 group8_count4(const uint64_t *list, int n, Beats beats) {
    const int part = threadIdx.x & 7;
    uint32_t r[4] = {0u, 0u, 0u, 0u};
    for (int j0 = 0; j0 < n; j0 += 64) {
        uint4 x[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) x[e] = *reinterpret_cast<const uint4 *>(list + j0 + 16 * e + 2 * part);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const uint64_t y0 = ((uint64_t)x[e].y << 32) | x[e].x, y1 = ((uint64_t)x[e].w << 32) | x[e].z;
#pragma unroll
            for (int s = 0; s < 4; ++s) r[s] += (beats(y0, s) ? 1u : 0u) + (beats(y1, s) ? 1u : 0u);
        }
    }
#pragma unroll
    for (int s = 0; s < 4; ++s) {
        r[s] += dpp_u32<0xB1>(0u, r[s]);
        r[s] += dpp_u32<0x4E>(0u, r[s]);
        r[s] += dpp_u32<0x141>(0u, r[s]);
    }
    return make_uint4(r[0], r[1], r[2], r[3]);
}

}  // namespace ca
