// Device-side helpers for the gfx950 kernels: bf16 dot products, DPP lane exchanges,
// order-preserving score keys and wavefront-level synchronisation.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ca {

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

// acc + a.lo*b.lo + a.hi*b.hi for two packed bf16 pairs, fp32 accumulate (v_dot2c_f32_bf16).
__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float acc) {
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a),
                                           __builtin_bit_cast(bf16x2_t, b), acc, false);
}

// Dot product of one 16-byte slice of a key row with the matching slice of a query.
__device__ __forceinline__ float dot16(const uint4 &kv, const uint4 &qv, float acc, __bf16) {
    acc = dot2_bf16(kv.x, qv.x, acc);
    acc = dot2_bf16(kv.y, qv.y, acc);
    acc = dot2_bf16(kv.z, qv.z, acc);
    acc = dot2_bf16(kv.w, qv.w, acc);
    return acc;
}
__device__ __forceinline__ float dot16(const uint4 &kv, const uint4 &qv, float acc, float) {
    acc = fmaf(__uint_as_float(kv.x), __uint_as_float(qv.x), acc);
    acc = fmaf(__uint_as_float(kv.y), __uint_as_float(qv.y), acc);
    acc = fmaf(__uint_as_float(kv.z), __uint_as_float(qv.z), acc);
    acc = fmaf(__uint_as_float(kv.w), __uint_as_float(qv.w), acc);
    return acc;
}

// Lane exchanges inside each group of 4 lanes (DPP quad_perm): value of lane ^ 1, lane ^ 2.
__device__ __forceinline__ float dpp_xor1(float x) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0xB1, 0xF, 0xF, false));
}
__device__ __forceinline__ float dpp_xor2(float x) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x4E, 0xF, 0xF, false));
}
// Value of the lane at the mirrored position within each group of 8 (lane i <-> 7 - i), which
// always pairs a lane of the lower half of the group with one of the upper half.
__device__ __forceinline__ float dpp_half_mirror(float x) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x141, 0xF, 0xF, false));
}

// Value of the lane at the mirrored position within each group of 16 (lane i <-> 15 - i).
__device__ __forceinline__ float dpp_mirror16(float x) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x140, 0xF, 0xF, false));
}

// Maximum of x over lanes l and l ^ 8 (within rows of 16: DPP row_ror:8), l ^ 16 and l ^ 32
// (gfx950 permlane swaps: the pair they return holds both partners of every lane).
__device__ __forceinline__ uint32_t lane_max_xor8(uint32_t x) {
    const uint32_t o = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x128, 0xF, 0xF, false);
    return o > x ? o : x;
}
__device__ __forceinline__ uint32_t lane_max_xor16(uint32_t x) {
    const auto r = __builtin_amdgcn_permlane16_swap(x, x, false, false);
    return r[0] > r[1] ? r[0] : r[1];
}
__device__ __forceinline__ uint32_t lane_max_xor32(uint32_t x) {
    const auto r = __builtin_amdgcn_permlane32_swap(x, x, false, false);
    return r[0] > r[1] ? r[0] : r[1];
}
// Maximum over the lanes l, l + off, l + 2 off, ... (mod 64) for off = 8, 16 or 32.
template <int OFF>
__device__ __forceinline__ uint32_t lane_max_stride(uint32_t x) {
    static_assert(OFF == 8 || OFF == 16 || OFF == 32, "stride");
    if constexpr (OFF == 8) x = lane_max_xor8(x);
    if constexpr (OFF <= 16) x = lane_max_xor16(x);
    return lane_max_xor32(x);
}

// x(lane) op x(lane ^ OFF) for OFF = 8 (DPP row_ror:8 inside rows of 16 lanes), 16 or 32
// (gfx950 permlane swaps); every lane gets the result.
template <int OFF>
__device__ __forceinline__ void lane_pair(float x, float &a, float &b) {
    static_assert(OFF == 8 || OFF == 16 || OFF == 32, "offset");
    if constexpr (OFF == 8) {
        a = x;
        b = __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x128, 0xF, 0xF, false));
    } else if constexpr (OFF == 16) {
        const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
        a = __uint_as_float(r[0]);
        b = __uint_as_float(r[1]);
    } else {
        const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
        a = __uint_as_float(r[0]);
        b = __uint_as_float(r[1]);
    }
}
template <int OFF>
__device__ __forceinline__ float lane_pair_sum(float x) {
    float a, b;
    lane_pair<OFF>(x, a, b);
    return a + b;
}
template <int OFF>
__device__ __forceinline__ float lane_pair_max(float x) {
    float a, b;
    lane_pair<OFF>(x, a, b);
    return fmaxf(a, b);
}

// Order-preserving map of a float32 score to uint32 (larger score -> larger key); -0 is
// folded onto +0 so that equal scores give equal keys. Every finite score maps to a key
// >= 0x00800000, so 0 is free to mean "no candidate".
__device__ __forceinline__ uint32_t score_key(float s) {
    uint32_t u = __float_as_uint(s);
    u = (u == 0x80000000u) ? 0u : u;
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// The score a key of score_key stands for (any key >= 0x00800000).
__device__ __forceinline__ float key_score(uint32_t key) {
    return __uint_as_float((key & 0x80000000u) ? (key & 0x7FFFFFFFu) : ~key);
}

// Workgroup barrier for LDS traffic: waits for this wavefront's LDS operations, not for its
// vector memory loads in flight (__syncthreads waits for those as well).
__device__ __forceinline__ void lds_barrier() {
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0); vmcnt and expcnt not constrained
    asm volatile("s_barrier" ::: "memory");
}

// Count of set bits of `m` in lanes below this one.
__device__ __forceinline__ int lanes_below(uint64_t m) {
    return __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0));
}

// DPP lane move (gfx9 controls): row_shr:n = 0x110+n, row_ror:n = 0x120+n, row_bcast:15 = 0x142,
// row_bcast:31 = 0x143. Lanes of disabled rows, or reading outside their row, get `old`.
template <int CTRL, int ROW_MASK = 0xF, int BANK_MASK = 0xF>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t old, uint32_t x) {
    return (uint32_t)__builtin_amdgcn_update_dpp((int)old, (int)x, CTRL, ROW_MASK, BANK_MASK, false);
}

// Inclusive prefix sum over the 64 lanes, all in DPP (no LDS traffic).
__device__ __forceinline__ uint32_t wave_incl_scan_u32(uint32_t x) {
    x += dpp_u32<0x111>(0u, x);
    x += dpp_u32<0x112>(0u, x);
    x += dpp_u32<0x114>(0u, x);
    x += dpp_u32<0x118>(0u, x);
    x += dpp_u32<0x142, 0xA>(0u, x);
    x += dpp_u32<0x143, 0xC>(0u, x);
    return x;
}

// Maximum / minimum over the 64 lanes (result uniform), DPP within rows then 4 lane reads.
__device__ __forceinline__ uint32_t wave_max_u32_dpp(uint32_t x) {
    uint32_t o;
    o = dpp_u32<0x121>(x, x); x = o > x ? o : x;
    o = dpp_u32<0x122>(x, x); x = o > x ? o : x;
    o = dpp_u32<0x124>(x, x); x = o > x ? o : x;
    o = dpp_u32<0x128>(x, x); x = o > x ? o : x;
    const uint32_t a = __builtin_amdgcn_readlane(x, 0), b = __builtin_amdgcn_readlane(x, 16);
    const uint32_t c = __builtin_amdgcn_readlane(x, 32), d = __builtin_amdgcn_readlane(x, 48);
    const uint32_t ab = a > b ? a : b, cd = c > d ? c : d;
    return ab > cd ? ab : cd;
}
__device__ __forceinline__ uint32_t wave_min_u32_dpp(uint32_t x) {
    uint32_t o;
    o = dpp_u32<0x121>(x, x); x = o < x ? o : x;
    o = dpp_u32<0x122>(x, x); x = o < x ? o : x;
    o = dpp_u32<0x124>(x, x); x = o < x ? o : x;
    o = dpp_u32<0x128>(x, x); x = o < x ? o : x;
    const uint32_t a = __builtin_amdgcn_readlane(x, 0), b = __builtin_amdgcn_readlane(x, 16);
    const uint32_t c = __builtin_amdgcn_readlane(x, 32), d = __builtin_amdgcn_readlane(x, 48);
    const uint32_t ab = a < b ? a : b, cd = c < d ? c : d;
    return ab < cd ? ab : cd;
}

__device__ __forceinline__ uint32_t wave_max_u32(uint32_t x) {
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) { const uint32_t o = __shfl_xor(x, off); x = o > x ? o : x; }
    return x;
}
__device__ __forceinline__ uint32_t wave_min_u32(uint32_t x) {
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) { const uint32_t o = __shfl_xor(x, off); x = o < x ? o : x; }
    return x;
}
__device__ __forceinline__ uint64_t wave_max_u64(uint64_t x) {
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) {
        const uint64_t o = __shfl_xor((unsigned long long)x, off);
        x = o > x ? o : x;
    }
    return x;
}
__device__ __forceinline__ uint64_t wave_min_u64(uint64_t x) {
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) {
        const uint64_t o = __shfl_xor((unsigned long long)x, off);
        x = o < x ? o : x;
    }
    return x;
}
__device__ __forceinline__ float wave_max_f32(float x) {
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) x = fmaxf(x, __shfl_xor(x, off));
    return x;
}
__device__ __forceinline__ float wave_sum_f32(float x) {
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) x += __shfl_xor(x, off);
    return x;
}

// Maximum / sum of a float over the 64 lanes (result uniform): DPP rotations inside rows of 16,
// then the 4 row results.
__device__ __forceinline__ float wave_max_f32_dpp(float x) {
    x = fmaxf(x, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x121, 0xF, 0xF, false)));
    x = fmaxf(x, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x122, 0xF, 0xF, false)));
    x = fmaxf(x, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x124, 0xF, 0xF, false)));
    x = fmaxf(x, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x128, 0xF, 0xF, false)));
    const float r0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 0));
    const float r1 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 16));
    const float r2 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 32));
    const float r3 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 48));
    return fmaxf(fmaxf(r0, r1), fmaxf(r2, r3));
}
__device__ __forceinline__ float wave_sum_f32_dpp(float x) {
    x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x121, 0xF, 0xF, false));
    x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x122, 0xF, 0xF, false));
    x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x124, 0xF, 0xF, false));
    x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x128, 0xF, 0xF, false));
    const float r0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 0));
    const float r1 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 16));
    const float r2 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 32));
    const float r3 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 48));
    return (r0 + r1) + (r2 + r3);
}

// Orders LDS traffic between the lanes of one wavefront (no workgroup barrier).
__device__ __forceinline__ void wave_sync() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

}  // namespace ca
