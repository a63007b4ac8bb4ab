// common.hpp -- device-side building blocks shared by the gfx950 kernels:
// vector types, MFMA wrappers, wavefront shuffles and bf16 conversion.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sap {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kWave = 64;

__device__ __forceinline__ bf16x8 as_bf16x8(uint4 v) { return __builtin_bit_cast(bf16x8, v); }

// D = A * B + C on a 16x16 tile with a 32-deep reduction.  Lane l holds
// A[m = l%16][k = 8(l/16) .. +7], B[k = 8(l/16) .. +7][n = l%16] and
// D[m = 4(l/16) + i][n = l%16] for i = 0..3.
__device__ __forceinline__ f32x4 mfma16x16x32(uint4 a, uint4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(a), as_bf16x8(b), c, 0, 0, 0);
}

// D = A * B + C on a 32x32 tile with a 16-deep reduction.  Lane l holds
// A[m = l%32][k = 8(l/32) .. +7], B[k = 8(l/32) .. +7][n = l%32] and
// D[m = 8(i/4) + 4(l/32) + i%4][n = l%32] for i = 0..15.
__device__ __forceinline__ f32x16 mfma32x32x16(uint4 a, uint4 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(a), as_bf16x8(b), c, 0, 0, 0);
}

__device__ __forceinline__ float shfl_xor(float v, int mask) { return __shfl_xor(v, mask, kWave); }
__device__ __forceinline__ int shfl_xor(int v, int mask) { return __shfl_xor(v, mask, kWave); }

// float -> bf16 bits, round to nearest even (hardware conversion)
__device__ __forceinline__ uint32_t bf16_bits(float x) {
    __bf16 b = (__bf16)x;
    return (uint32_t)__builtin_bit_cast(uint16_t, b);
}
// two floats -> packed bf16 pair (lo in bits 0-15), one v_cvt_pk_bf16_f32
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    typedef float f32x2 __attribute__((ext_vector_type(2)));
    const bf16x2 b = __builtin_convertvector((f32x2{lo, hi}), bf16x2);
    return __builtin_bit_cast(uint32_t, b);
}

// byte-select permute of two dwords: selector bytes 0-3 pick from `lo`,
// 4-7 from `hi`
__device__ __forceinline__ uint32_t perm(uint32_t hi, uint32_t lo, uint32_t sel) {
    return __builtin_amdgcn_perm(hi, lo, sel);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Inclusive prefix scan over the 64 lanes of a wave with DPP row shifts and
// row broadcasts (VALU only, no LDS crossbar): op is applied with identity
// `id` where a lane has no source.  The last lane holds the wave total.
template <class Op>
__device__ __forceinline__ uint32_t wave_scan_dpp(uint32_t v, uint32_t id, Op op) {
    v = op(v, (uint32_t)__builtin_amdgcn_update_dpp((int)id, (int)v, 0x111, 0xf, 0xf, false));  // row_shr:1
    v = op(v, (uint32_t)__builtin_amdgcn_update_dpp((int)id, (int)v, 0x112, 0xf, 0xf, false));  // row_shr:2
    v = op(v, (uint32_t)__builtin_amdgcn_update_dpp((int)id, (int)v, 0x114, 0xf, 0xf, false));  // row_shr:4
    v = op(v, (uint32_t)__builtin_amdgcn_update_dpp((int)id, (int)v, 0x118, 0xf, 0xf, false));  // row_shr:8
    v = op(v, (uint32_t)__builtin_amdgcn_update_dpp((int)id, (int)v, 0x142, 0xa, 0xf, false));  // row_bcast:15
    v = op(v, (uint32_t)__builtin_amdgcn_update_dpp((int)id, (int)v, 0x143, 0xc, 0xf, false));  // row_bcast:31
    return v;
}
__device__ __forceinline__ int wave_incl_sum(int v) {
    return (int)wave_scan_dpp((uint32_t)v, 0u, [](uint32_t a, uint32_t b) { return a + b; });
}
// value of lane 63, as a wave-uniform scalar
__device__ __forceinline__ uint32_t wave_last(uint32_t v) { return (uint32_t)__builtin_amdgcn_readlane((int)v, 63); }

}  // namespace sap
