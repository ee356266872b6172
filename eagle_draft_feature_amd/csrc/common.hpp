// Shared device helpers of the gfx950 kernels: bfloat16 bit tricks, the
// 16x16x32 bf16 MFMA operand types and wave64 reductions.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace e31 {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));  // register-friendly 16 bytes

constexpr int NORM_NONE = 0;
constexpr int NORM_LN = 1;
constexpr int NORM_RMS = 2;

// bfloat16 is the upper half of a float32: decoding is a shift or a mask.
__device__ __forceinline__ float bf_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
__device__ __forceinline__ float bf_one(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }

// Two float32 -> packed bf16x2 with round-to-nearest-even (v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack_bf2(float lo, float hi) {
    bf16x2 v = {(__bf16)lo, (__bf16)hi};
    return __builtin_bit_cast(uint32_t, v);
}

__device__ __forceinline__ f32x4 mfma16x16x32(const uint4& a, const uint4& b, const f32x4& c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

__device__ __forceinline__ f32x4 mfma16x16x32(const u32x4& a, const u32x4& b, const f32x4& c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

// Stores / loads performed at the device coherence point (agent-scope
// relaxed atomics), for values handed from one workgroup to another within a
// launch without writing back or invalidating a whole L2.
__device__ __forceinline__ void store_coherent(float* p, float v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float load_coherent(const float* p) {
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void store_coherent_u32(uint32_t* p, uint32_t v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint32_t load_coherent_u32(const uint32_t* p) {
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Cross-lane sums in registers (no LDS round trip); the whole wave must be
// active.  v plus the value of lane l ^ 16 (l ^ 32): a gfx950 permlane swap
// of v with itself hands every lane its own value and its partner's.
__device__ __forceinline__ float xor16_sum(float v) {
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float xor32_sum(float v) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
// v moved by one DPP control within each 16-lane row
template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) {
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xf, 0xf, false));
}
// v plus the value of lane l ^ 1, then of lane l ^ 2 (quad permutations):
// every lane of a quad ends with the quad's sum
__device__ __forceinline__ float quad_sum(float v) {
    v += dpp_f<0xb1>(v);  // quad_perm [1, 0, 3, 2]
    v += dpp_f<0x4e>(v);  // quad_perm [2, 3, 0, 1]
    return v;
}

// Sum over the wave, the butterfly over lane masks 32, 16, 8, 4, 2, 1 (every
// lane ends with the same bits).  Masks 32 and 16 are permlane swaps, mask 8
// the row rotation by 8; after those steps a lane's value depends on its
// index mod 8 only, so the rotations by 4, 2 and 1 reach a lane that holds the
// same value as lane l ^ 4, l ^ 2, l ^ 1: the adds are those of the butterfly.
__device__ __forceinline__ float wave_sum(float v) {
    v = xor32_sum(v);
    v = xor16_sum(v);
    v += dpp_f<0x128>(v);  // row_ror:8
    v += dpp_f<0x124>(v);  // row_ror:4
    v += dpp_f<0x122>(v);  // row_ror:2
    v += dpp_f<0x121>(v);  // row_ror:1
    return v;
}

// Sum over the four 16-lane groups (lanes l, l^16, l^32, l^48 share an MFMA row).
__device__ __forceinline__ float group4_sum(float v) { return xor32_sum(xor16_sum(v)); }

}  // namespace e31
