// Restricted softmax times V for one query vector on gfx950 (pages of "The Condensate Theorem",
// metaphor-xennon blog: section 2.3, Theorem 1's Attention_C; section 3.2.4, the output
// evaluated over C_i alone).
//
// The rows of a set are spread over wavefronts. A wavefront requests the K and V slices of its
// rows together (16-byte loads, LPR = row bytes / 16 lanes per row, RPW = 64 / LPR rows per
// load), computes the fp32 scores s = q . k_j, and keeps a partial result over its rows: the
// largest score m, l = sum of exp2((s - m) * scale * log2 e) and acc = the sum of those
// weights times the V rows. Partials of disjoint row subsets combine exactly: with M the largest
// m_p and f_p = exp2((m_p - M) * scale * log2 e), out = sum f_p acc_p / sum f_p l_p, the softmax
// over the union. Every sum runs in a fixed order (deterministic output, no atomics).
#pragma once

#include "device_utils.h"

namespace ca {

template <int D, typename T>
struct AttendShape {
    static constexpr int RB = D * (int)sizeof(T);  // bytes per row
    static constexpr int LPR = RB / 16;            // lanes per row, one 16-byte slice each
    static constexpr int RPW = 64 / LPR;           // rows per wavefront load
    static constexpr int EPL = 16 / (int)sizeof(T);  // elements per slice
    static_assert(LPR == 8 || LPR == 16 || LPR == 32, "row size");
};

// NP partial results in LDS: acc[p][0..D), the largest score m[p] (-inf: no rows) and the weight
// sum l[p]; f[p] is the merge factor.
template <int D, int NP>
struct SoftmaxPartials {
    float acc[NP][D];
    float m[NP], l[NP], f[NP];
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

// Sum over the LPR lanes of a row (every lane of the row gets it): DPP mirrors and quad
// exchanges inside rows of 16 lanes, the gfx950 permlane16 swap across two of them.
template <int LPR>
__device__ __forceinline__ float row_sum(float x) {
    if constexpr (LPR >= 16) x += dpp_mirror16(x);
    x += dpp_half_mirror(x);
    x += dpp_xor2(x);
    x += dpp_xor1(x);
    if constexpr (LPR == 32) {
        const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
        x = __uint_as_float(r[0]) + __uint_as_float(r[1]);
    }
    return x;
}

// K and V slices of U rows per lane: rows c = c0 + u*step + slot (slot = lane / LPR) of a row
// list row_at(c), c in [0, count); rows past the end are clamped to the last one (loaded,
// ignored: every load is unconditional, so that all are in flight together). Issued together,
// consumed by accumulate_rows.
template <int D, typename T, int U>
struct RowSlices {
    uint4 k[U], v[U];
};

template <int D, typename T, int U, typename RowAt>
__device__ __forceinline__ void load_rows(RowSlices<D, T, U> &rs, const T *__restrict__ kbase,
                                          const T *__restrict__ vbase, RowAt row_at, int count,
                                          int c0, int step) {
    using S = AttendShape<D, T>;
    const int lane = threadIdx.x & 63, slot = lane / S::LPR, cs = lane % S::LPR;
#pragma unroll
    for (int u = 0; u < U; ++u) {
        int c = c0 + u * step + slot;
        c = c < count ? c : count - 1;
        const size_t row = row_at(c);
        rs.k[u] = reinterpret_cast<const uint4 *>(kbase + row * D)[cs];
        rs.v[u] = reinterpret_cast<const uint4 *>(vbase + row * D)[cs];
    }
}

// Running softmax state of one row slot of a wavefront.
template <int D, typename T>
struct SlotState {
    float m = -INFINITY, l = 0.f, acc[AttendShape<D, T>::EPL] = {};
};

// Adds the rows of rs whose index passes use(c) to the slot state.
template <int D, typename T, int U, typename Use>
__device__ __forceinline__ void accumulate_rows(SlotState<D, T> &st, const RowSlices<D, T, U> &rs,
                                                const uint4 &qs, Use use, int c0, int step,
                                                float scale_log2e) {
    using S = AttendShape<D, T>;
    const int slot = (threadIdx.x & 63) / S::LPR;
    float s[U];
    bool ok[U];
    float mr = st.m;
#pragma unroll
    for (int u = 0; u < U; ++u) {
        s[u] = row_sum<S::LPR>(dot16(rs.k[u], qs, 0.f, T()));
        ok[u] = use(c0 + u * step + slot);
        if (ok[u]) mr = fmaxf(mr, s[u]);
    }
    // Rescale what the slot holds to the new maximum (nothing held: m = -inf).
    const float f = st.m == -INFINITY ? 0.f : exp2f((st.m - mr) * scale_log2e);
    st.l *= f;
#pragma unroll
    for (int e = 0; e < S::EPL; ++e) st.acc[e] *= f;
#pragma unroll
    for (int u = 0; u < U; ++u) {
        if (ok[u]) {
            const float w = exp2f((s[u] - mr) * scale_log2e);
            st.l += w;
            accumulate16(st.acc, rs.v[u], w, T());
        }
    }
    st.m = mr;
}

// Merges the row slots of a wavefront (lanes LPR apart) and writes the result to partial p
// (m = -inf, l = 0, acc = 0 when the wavefront had no rows). All 64 lanes, p uniform.
template <int D, typename T, int NP>
__device__ __forceinline__ void store_wave_partial(SlotState<D, T> st, float scale_log2e,
                                                   SoftmaxPartials<D, NP> &out, int p) {
    using S = AttendShape<D, T>;
    const int lane = threadIdx.x & 63, cs = lane % S::LPR;
    float mw = st.m;
    if constexpr (S::LPR <= 8) mw = lane_pair_max<8>(mw);
    if constexpr (S::LPR <= 16) mw = lane_pair_max<16>(mw);
    mw = lane_pair_max<32>(mw);
    const float f = st.m == -INFINITY ? 0.f : exp2f((st.m - mw) * scale_log2e);
    float l = st.l * f;
    float acc[S::EPL];
#pragma unroll
    for (int e = 0; e < S::EPL; ++e) acc[e] = st.acc[e] * f;
    if constexpr (S::LPR <= 8) {
        l = lane_pair_sum<8>(l);
#pragma unroll
        for (int e = 0; e < S::EPL; ++e) acc[e] = lane_pair_sum<8>(acc[e]);
    }
    if constexpr (S::LPR <= 16) {
        l = lane_pair_sum<16>(l);
#pragma unroll
        for (int e = 0; e < S::EPL; ++e) acc[e] = lane_pair_sum<16>(acc[e]);
    }
    l = lane_pair_sum<32>(l);
#pragma unroll
    for (int e = 0; e < S::EPL; ++e) acc[e] = lane_pair_sum<32>(acc[e]);
    if (lane < S::LPR) {
#pragma unroll
        for (int e = 0; e < S::EPL; ++e) out.acc[p][cs * S::EPL + e] = acc[e];
    }
    if (lane == 0) { out.m[p] = mw; out.l[p] = l; }
}

// Partial result of wavefront wv of nw over the rows row_at(c), c in [0, count): it takes rows
// c = wv*RPW + slot + r*nw*RPW, U of them per lane in flight (K and V requested together). qs is
// this lane's slice of the query (slice lane % LPR). kbase/vbase: row 0 of the KV head. The
// result goes to partial p of *out. Must be called by all 64 lanes, wv and p uniform.
template <int D, typename T, int U, int NP, typename RowAt>
__device__ __forceinline__ void wave_partial(const uint4 &qs, const T *__restrict__ kbase,
                                             const T *__restrict__ vbase, RowAt row_at, int count,
                                             int wv, int nw, float scale_log2e,
                                             SoftmaxPartials<D, NP> &out, int p) {
    using S = AttendShape<D, T>;
    SlotState<D, T> st;
    const int step = nw * S::RPW;
    auto use = [&](int c) { return c < count; };
    for (int c0 = wv * S::RPW; c0 < count; c0 += U * step) {
        RowSlices<D, T, U> rs;
        load_rows<D, T, U>(rs, kbase, vbase, row_at, count, c0, step);
        accumulate_rows<D, T, U>(st, rs, qs, use, c0, step, scale_log2e);
    }
    store_wave_partial<D, T>(st, scale_log2e, out, p);
}

// As wave_partial, with the scores given (score_at(c), the same for every lane of a row slot)
// instead of computed: only the V rows are read.
template <int D, typename T, int U, int NP, typename RowAt, typename ScoreAt>
__device__ __forceinline__ void wave_partial_scored(const T *__restrict__ vbase, RowAt row_at,
                                                    ScoreAt score_at, int count, int wv, int nw,
                                                    float scale_log2e, SoftmaxPartials<D, NP> &out, int p) {
    using S = AttendShape<D, T>;
    SlotState<D, T> st;
    const int step = nw * S::RPW;
    const int lane = threadIdx.x & 63, slot = lane / S::LPR, cs = lane % S::LPR;
    for (int c0 = wv * S::RPW; c0 < count; c0 += U * step) {
        uint4 vr[U];
        float s[U];
        bool ok[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int c = c0 + u * step + slot;
            ok[u] = c < count;
            const int cc = ok[u] ? c : count - 1;
            vr[u] = reinterpret_cast<const uint4 *>(vbase + row_at(cc) * D)[cs];
            s[u] = score_at(cc);
        }
        float mr = st.m;
#pragma unroll
        for (int u = 0; u < U; ++u)
            if (ok[u]) mr = fmaxf(mr, s[u]);
        // (The hardware exponential: a weight below 2^-126 of the largest counts as 0, which
        // no fp32 sum sees.)
        const float f = st.m == -INFINITY ? 0.f : __builtin_amdgcn_exp2f((st.m - mr) * scale_log2e);
        st.l *= f;
#pragma unroll
        for (int e = 0; e < S::EPL; ++e) st.acc[e] *= f;
#pragma unroll
        for (int u = 0; u < U; ++u) {
            if (ok[u]) {
                const float w = __builtin_amdgcn_exp2f((s[u] - mr) * scale_log2e);
                st.l += w;
                accumulate16(st.acc, vr[u], w, T());
            }
        }
        st.m = mr;
    }
    store_wave_partial<D, T>(st, scale_log2e, out, p);
}

// out[0..D) from partials p0..p1-1 (at most 64 of them, all written, at least one row in all),
// combined in index order: wavefront 0 turns their m[p], l[p] into normalised factors
// f[p] = exp2((m[p] - M) * scale_log2e) / L, then each column sums f[p] acc[p][t]. Called by all
// NT threads after the partials are visible.
template <int NT, int D, int NP>
__device__ __forceinline__ void merge_partials(SoftmaxPartials<D, NP> &ps, int p0, int p1,
                                               float scale_log2e, float *__restrict__ out) {
    static_assert(NP <= 64, "partials");
    const int tid = threadIdx.x, lane = tid & 63;
    if (tid < 64) {
        const int p = p0 + lane;
        const float m = p < p1 ? ps.m[p] : -INFINITY;
        const float l = p < p1 ? ps.l[p] : 0.f;
        const float mx = wave_max_f32_dpp(m);
        const float f = m == -INFINITY ? 0.f : exp2f((m - mx) * scale_log2e);
        const float lsum = wave_sum_f32_dpp(l * f);
        if (p < p1) ps.f[p] = f / lsum;
    }
    lds_barrier();
    for (int t = tid; t < D; t += NT) {
        float o = 0.f;
#pragma unroll 8
        for (int p = p0; p < p1; ++p) o = fmaf(ps.acc[p][t], ps.f[p], o);
        out[t] = o;
    }
}

}  // namespace ca
