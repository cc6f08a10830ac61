// Stage 2 of condensate attention on gfx950: softmax restricted to the condensate set, times V
// (pages of "The Condensate Theorem", metaphor-xennon blog: section 2.3, Theorem 1's
// Attention_C, and section 3.2.4, the output "computed only on C_i"; section 5.2.2 sketches it
// as flash_attention_on_subset(Q, K[C], V[C], C)).
//
// One workgroup (4 wavefronts) per query vector:
//   1. the valid entries of its index row are compacted in order into LDS;
//   2. the gathered K rows are scored in fp32 (4 lanes per row, 16-byte loads);
//   3. max and sum of exp over the set with wavefront reductions, in fp32;
//   4. the gathered V rows are accumulated with 16-byte loads per lane, one row slice per
//      lane, then reduced across row slots and wavefronts in a fixed order (deterministic).
#include "ca_internal.h"
#include "device_utils.h"

namespace ca {
namespace {

struct AttendArgs {
    int64_t n, nq;
    int Hq, Hkv, g, cap;
    float scale_log2e;  // log2(e) / sqrt(d)
};

__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) x = fmaxf(x, __shfl_xor(x, off));
    return x;
}
__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) x += __shfl_xor(x, off);
    return x;
}

template <typename T, int D>
__global__ __launch_bounds__(256) void attend_kernel(const T *__restrict__ q, const T *__restrict__ k,
                                                     const T *__restrict__ v,
                                                     const int32_t *__restrict__ idx,
                                                     float *__restrict__ out, AttendArgs a) {
    constexpr int EB = sizeof(T);
    constexpr int RB = D * EB;
    constexpr int P = RB / 64;       // scoring: 4 lanes per row, P 16-byte loads each
    constexpr int LPR = RB / 16;     // AV: lanes per row, one 16-byte slice each
    constexpr int RPW = 64 / LPR;    // AV: rows per wavefront step
    constexpr int EPL = 16 / EB;     // elements per 16-byte slice

    extern __shared__ int32_t asm_[];       // [cap] positions, then [cap] weights
    int32_t *js = asm_;
    float *ws = reinterpret_cast<float *>(asm_ + a.cap);
    __shared__ int wave_cnt[4];
    __shared__ float red[4];
    __shared__ float part[4][LPR][EPL];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int64_t qv = blockIdx.x;
    const int64_t r = qv % a.nq;
    const int64_t bh = qv / a.nq;
    const int h = (int)(bh % a.Hq);
    const int b = (int)(bh / a.Hq);
    const int kvh = h / a.g;
    const int64_t i = a.n - a.nq + r;
    const int32_t *row = idx + qv * a.cap;

    // 1. Ordered compaction of positions in 0..i.
    int count = 0;
    for (int base = 0; base < a.cap; base += 256) {
        const int c = base + tid;
        int32_t j = c < a.cap ? row[c] : -1;
        const bool ok = j >= 0 && j <= i;
        const uint64_t m = __ballot(ok);
        if (lane == 0) wave_cnt[wave] = __popcll(m);
        __syncthreads();
        int off = count;
        for (int w2 = 0; w2 < wave; ++w2) off += wave_cnt[w2];
        if (ok) js[off + lanes_below(m)] = j;
        count += wave_cnt[0] + wave_cnt[1] + wave_cnt[2] + wave_cnt[3];
        __syncthreads();
    }
    float *o = out + qv * D;
    if (count == 0) {
        for (int t = tid; t < D; t += 256) o[t] = 0.f;
        return;
    }

    const size_t kv_row0 = ((size_t)b * a.Hkv + kvh) * (size_t)a.n;

    // 2. Scores (raw fp32 dot products) of the gathered K rows.
    {
        const int s = lane & 3;
        const uint4 *qsrc = reinterpret_cast<const uint4 *>(q + qv * D);
        uint4 qr[P];
#pragma unroll
        for (int p = 0; p < P; ++p) qr[p] = qsrc[p * 4 + s];
        for (int c0 = wave * 16; c0 < count; c0 += 64) {
            const int c = c0 + (lane >> 2);
            const int cc = c < count ? c : count - 1;
            const uint4 *src = reinterpret_cast<const uint4 *>(k + (kv_row0 + js[cc]) * D);
            float x = 0.f;
#pragma unroll
            for (int p = 0; p < P; ++p) x = dot16(src[p * 4 + s], qr[p], x, T());
            x += dpp_xor2(x);
            x += dpp_xor1(x);
            if ((lane & 3) == 0 && c < count) ws[c] = x;
        }
    }
    __syncthreads();

    // 3. Softmax weights: w_c = exp((s_c - max s) / sqrt(d)), l = sum w_c.
    float m = -INFINITY;
    for (int c = tid; c < count; c += 256) m = fmaxf(m, ws[c]);
    m = wave_max(m);
    if (lane == 0) red[wave] = m;
    __syncthreads();
    m = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
    __syncthreads();
    float l = 0.f;
    for (int c = tid; c < count; c += 256) {
        const float w = exp2f((ws[c] - m) * a.scale_log2e);
        ws[c] = w;
        l += w;
    }
    l = wave_sum(l);
    if (lane == 0) red[wave] = l;
    __syncthreads();
    l = (red[0] + red[1]) + (red[2] + red[3]);

    // 4. sum_c w_c v_{j_c}: lane = (row slot, 16-byte column slice).
    const int slot = lane / LPR, cs = lane % LPR;
    float acc[EPL];
#pragma unroll
    for (int e = 0; e < EPL; ++e) acc[e] = 0.f;
    for (int c0 = wave * RPW; c0 < count; c0 += 4 * RPW) {
        const int c = c0 + slot;
        if (c < count) {
            const float w = ws[c];
            const uint4 vv = reinterpret_cast<const uint4 *>(v + (kv_row0 + js[c]) * D)[cs];
            if constexpr (EB == 2) {
                const uint32_t wd[4] = {vv.x, vv.y, vv.z, vv.w};
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    acc[2 * e] = fmaf(w, __uint_as_float(wd[e] << 16), acc[2 * e]);
                    acc[2 * e + 1] = fmaf(w, __uint_as_float(wd[e] & 0xFFFF0000u), acc[2 * e + 1]);
                }
            } else {
                acc[0] = fmaf(w, __uint_as_float(vv.x), acc[0]);
                acc[1] = fmaf(w, __uint_as_float(vv.y), acc[1]);
                acc[2] = fmaf(w, __uint_as_float(vv.z), acc[2]);
                acc[3] = fmaf(w, __uint_as_float(vv.w), acc[3]);
            }
        }
    }
    // Reduce the row slots of the wavefront (lanes cs, cs+LPR, ...), then the wavefronts.
#pragma unroll
    for (int off = LPR; off < 64; off <<= 1)
#pragma unroll
        for (int e = 0; e < EPL; ++e) acc[e] += __shfl_xor(acc[e], off);
    if (slot == 0)
#pragma unroll
        for (int e = 0; e < EPL; ++e) part[wave][cs][e] = acc[e];
    __syncthreads();
    const float inv_l = 1.0f / l;
    for (int t = tid; t < D; t += 256) {
        const int c2 = t / EPL, e = t % EPL;
        const float sum = (part[0][c2][e] + part[1][c2][e]) + (part[2][c2][e] + part[3][c2][e]);
        o[t] = sum * inv_l;
    }
}

}  // namespace

hipError_t launch_gather_softmax_av(const Plan &pl, const void *q, const void *k, const void *v,
                                    const int32_t *idx, float *out, hipStream_t s) {
    AttendArgs a;
    a.n = pl.n; a.nq = pl.nq; a.Hq = pl.Hq; a.Hkv = pl.Hkv; a.g = pl.g; a.cap = pl.cap;
    a.scale_log2e = (float)(1.4426950408889634 / __builtin_sqrt((double)pl.d));
    const size_t shmem = (size_t)pl.cap * (sizeof(int32_t) + sizeof(float));
    dim3 grid((unsigned)pl.nqv), block(256);
#define CA_LAUNCH_AT(T, D)                                                                      \
    hipLaunchKernelGGL((attend_kernel<T, D>), grid, block, shmem, s, static_cast<const T *>(q), \
                       static_cast<const T *>(k), static_cast<const T *>(v), idx, out, a)
    if (pl.dtype == 1) {
        if (pl.d == 128) CA_LAUNCH_AT(__bf16, 128); else CA_LAUNCH_AT(__bf16, 64);
    } else {
        if (pl.d == 128) CA_LAUNCH_AT(float, 128); else CA_LAUNCH_AT(float, 64);
    }
#undef CA_LAUNCH_AT
    return hipGetLastError();
}

}  // namespace ca
