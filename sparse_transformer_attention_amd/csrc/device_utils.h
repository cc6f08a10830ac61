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

// Order-preserving map of a float32 score to uint32 (larger score -> larger key); -0 is
// folded onto +0 so that equal scores give equal keys. Every finite score maps to a key
// >= 0x00800000, so 0 is free to mean "no candidate".
__device__ __forceinline__ uint32_t score_key(float s) {
    uint32_t u = __float_as_uint(s);
    u = (u == 0x80000000u) ? 0u : u;
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Count of set bits of `m` in lanes below this one.
__device__ __forceinline__ int lanes_below(uint64_t m) {
    return __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0));
}

// Orders LDS traffic between the lanes of one wavefront (no workgroup barrier).
__device__ __forceinline__ void wave_sync() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

}  // namespace ca
