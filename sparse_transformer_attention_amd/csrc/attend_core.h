// Restricted softmax times V for one query vector, executed by one workgroup of NT threads
// (pages of "The Condensate Theorem", metaphor-xennon blog: section 2.3, Theorem 1's
// Attention_C; section 3.2.4, the output evaluated over C_i alone).
//
// The set is given as `count` positions js[0..count) in LDS. Every gathered row is loaded
// with 16-byte loads: K rows 4 lanes per row (P loads each) for the fp32 dot products, V rows
// LPR lanes per row for the accumulation. The V rows of the first block are requested before
// the scores are reduced, so the two gathers overlap. Softmax in fp32: m = max s, w = exp(s-m),
// l = sum w; out = sum w v / l. All reductions run in a fixed order (deterministic output).
#pragma once

#include "device_utils.h"

namespace ca {

template <int NT, int D, typename T>
struct AttendShape {
    static constexpr int NW = NT / 64;
    static constexpr int EB = sizeof(T);
    static constexpr int RB = D * EB;     // bytes per row
    static constexpr int P = RB / 64;     // scoring: 16-byte loads per lane, 4 lanes per row
    static constexpr int KSTEP = 16 * NW; // rows scored per workgroup step
    static constexpr int KU = P >= 8 ? 1 : 2;  // scoring steps in flight
    static constexpr int LPR = RB / 16;   // accumulation: lanes per row
    static constexpr int RPW = 64 / LPR;  // accumulation: rows per wavefront load
    static constexpr int EPL = 16 / EB;   // elements per 16-byte slice
    static constexpr int VU = NT >= 1024 ? 8 : 16;  // V loads in flight per lane
    static constexpr int VBLOCK = VU * NW * RPW;    // V rows per block
};

// LDS the attend core needs besides js[] and sc[] (both sized by the caller).
template <int NT, int D, typename T>
struct AttendShared {
    float red[AttendShape<NT, D, T>::NW];
    float part[AttendShape<NT, D, T>::NW][D];
};

__device__ __forceinline__ void accumulate16(float *acc, const uint4 &v, float w, __bf16) {
    const uint32_t wd[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        acc[2 * e] = fmaf(w, __uint_as_float(wd[e] << 16), acc[2 * e]);
        acc[2 * e + 1] = fmaf(w, __uint_as_float(wd[e] & 0xFFFF0000u), acc[2 * e + 1]);
    }
}
__device__ __forceinline__ void accumulate16(float *acc, const uint4 &v, float w, float) {
    acc[0] = fmaf(w, __uint_as_float(v.x), acc[0]);
    acc[1] = fmaf(w, __uint_as_float(v.y), acc[1]);
    acc[2] = fmaf(w, __uint_as_float(v.z), acc[2]);
    acc[3] = fmaf(w, __uint_as_float(v.w), acc[3]);
}

// qrow: this query's row; kbase/vbase: row 0 of its KV head in K and V (nrows rows); js/sc:
// LDS arrays of >= count entries (sc is overwritten); positions are clamped into [0, nrows) for
// addressing. Must be called by all NT threads, count uniform and >= 1.
template <int NT, int D, typename T>
__device__ __forceinline__ void attend_set(const T *__restrict__ qrow, const T *__restrict__ kbase,
                           const T *__restrict__ vbase, const int32_t *js, float *sc, int count,
                           int64_t nrows, float scale_log2e, float *__restrict__ out,
                           AttendShared<NT, D, T> &sh) {
    auto row_of = [&](int c) -> size_t {
        const uint32_t j = (uint32_t)js[c];
        return (size_t)(j < (uint64_t)nrows ? j : (uint32_t)(nrows - 1));
    };
    using S = AttendShape<NT, D, T>;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int s4 = lane & 3;
    const int slot = lane / S::LPR, cs = lane % S::LPR;

    uint4 qr[S::P];
    {
        const uint4 *qsrc = reinterpret_cast<const uint4 *>(qrow);
#pragma unroll
        for (int p = 0; p < S::P; ++p) qr[p] = qsrc[p * 4 + s4];
    }
    // V rows of the first block, requested now so that they arrive while scores are computed.
    uint4 vr[S::VU];
#pragma unroll
    for (int u = 0; u < S::VU; ++u) {
        const int c = (u * S::NW + wave) * S::RPW + slot;
        if (c < count) vr[u] = reinterpret_cast<const uint4 *>(vbase + row_of(c) * D)[cs];
    }

    // Scores: raw fp32 dot products, 4 lanes per row.
    for (int c0 = 0; c0 < count; c0 += S::KSTEP * S::KU) {
        uint4 kr[S::KU][S::P];
#pragma unroll
        for (int u = 0; u < S::KU; ++u) {
            int c = c0 + u * S::KSTEP + wave * 16 + (lane >> 2);
            c = c < count ? c : count - 1;
            const uint4 *src = reinterpret_cast<const uint4 *>(kbase + row_of(c) * D);
#pragma unroll
            for (int p = 0; p < S::P; ++p) kr[u][p] = src[p * 4 + s4];
        }
#pragma unroll
        for (int u = 0; u < S::KU; ++u) {
            float x = 0.f;
#pragma unroll
            for (int p = 0; p < S::P; ++p) x = dot16(kr[u][p], qr[p], x, T());
            x += dpp_xor2(x);
            x += dpp_xor1(x);
            const int c = c0 + u * S::KSTEP + wave * 16 + (lane >> 2);
            if (s4 == 0 && c < count) sc[c] = x;
        }
    }
    __syncthreads();

    // Softmax weights over the set.
    float m = -INFINITY;
    for (int c = tid; c < count; c += NT) m = fmaxf(m, sc[c]);
    m = wave_max_f32(m);
    if (lane == 0) sh.red[wave] = m;
    __syncthreads();
    m = sh.red[0];
#pragma unroll
    for (int w2 = 1; w2 < S::NW; ++w2) m = fmaxf(m, sh.red[w2]);
    __syncthreads();
    float l = 0.f;
    for (int c = tid; c < count; c += NT) {
        const float w = exp2f((sc[c] - m) * scale_log2e);
        sc[c] = w;
        l += w;
    }
    l = wave_sum_f32(l);
    if (lane == 0) sh.red[wave] = l;
    __syncthreads();
    l = 0.f;
#pragma unroll
    for (int w2 = 0; w2 < S::NW; ++w2) l += sh.red[w2];

    // sum_c w_c v_c, lane = (row slot, 16-byte column slice).
    float acc[S::EPL];
#pragma unroll
    for (int e = 0; e < S::EPL; ++e) acc[e] = 0.f;
#pragma unroll
    for (int u = 0; u < S::VU; ++u) {
        const int c = (u * S::NW + wave) * S::RPW + slot;
        if (c < count) accumulate16(acc, vr[u], sc[c], T());
    }
    for (int vb = S::VBLOCK; vb < count; vb += S::VBLOCK) {
#pragma unroll
        for (int u = 0; u < S::VU; ++u) {
            const int c = vb + (u * S::NW + wave) * S::RPW + slot;
            if (c < count) vr[u] = reinterpret_cast<const uint4 *>(vbase + row_of(c) * D)[cs];
        }
#pragma unroll
        for (int u = 0; u < S::VU; ++u) {
            const int c = vb + (u * S::NW + wave) * S::RPW + slot;
            if (c < count) accumulate16(acc, vr[u], sc[c], T());
        }
    }
#pragma unroll
    for (int off = S::LPR; off < 64; off <<= 1)
#pragma unroll
        for (int e = 0; e < S::EPL; ++e) acc[e] += __shfl_xor(acc[e], off);
    if (slot == 0)
#pragma unroll
        for (int e = 0; e < S::EPL; ++e) sh.part[wave][cs * S::EPL + e] = acc[e];
    __syncthreads();
    const float inv_l = 1.0f / l;
    for (int t = tid; t < D; t += NT) {
        float sum = 0.f;
#pragma unroll
        for (int w2 = 0; w2 < S::NW; ++w2) sum += sh.part[w2][t];
        out[t] = sum * inv_l;
    }
}

}  // namespace ca
