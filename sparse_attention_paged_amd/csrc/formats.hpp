// formats.hpp -- the row loaders' decode steps: OCP e4m3 KV codes to bf16
// MFMA operands, and fp4_e8m0_b32 indexer key words (e2m1 codes with ue8m0
// block scales) to bf16 operands.  The debug table entry points run these
// same functions over every code.
#pragma once

#include "common.hpp"

namespace sap {

// e4m3 -> bf16.  Every finite OCP E4M3 value (|x| in [2^-9, 448]) is exactly
// a normal bf16, so the tile keeps the true value and the fold factor is 1:
// the per-row dequant scale is applied to the dot outputs and folded into the
// softmax weights instead ("Perf/kv fp8 read path", What this changes).
constexpr float kE4m3FoldFactor = 1.0f;

// Two codes in the low (HIGH = false) or high (HIGH = true) 16 bits of
// `codes` -> two bf16 in one dword (first code in the low half).
template <bool HIGH>
__device__ __forceinline__ uint32_t e4m3x2_to_bf16x2(uint32_t codes) {
    bf16x2 r = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(codes, 1.0f, HIGH);
    return __builtin_bit_cast(uint32_t, r);
}

// 8 codes (little-endian in two dwords) -> 8 bf16 (element e in half e%2 of dword e/2).
__device__ __forceinline__ uint4 e4m3x8_to_bf16x8(uint2 c) {
    uint4 r;
    r.x = e4m3x2_to_bf16x2<false>(c.x);
    r.y = e4m3x2_to_bf16x2<true>(c.x);
    r.z = e4m3x2_to_bf16x2<false>(c.y);
    r.w = e4m3x2_to_bf16x2<true>(c.y);
    return r;
}

// 8 codes -> 8 f16 (element e in half e%2 of dword e/2).  Every finite e4m3
// value (|x| in [2^-9, 448], 4 significant bits) is exactly an f16 as well.
__device__ __forceinline__ uint4 e4m3x8_to_f16x8(uint2 c) {
    uint4 r;
    r.x = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(c.x, 1.0f, false));
    r.y = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(c.x, 1.0f, true));
    r.z = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(c.y, 1.0f, false));
    r.w = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(c.y, 1.0f, true));
    return r;
}

// ---------------------------------------------------------------------------
// fp4_e8m0_b32 ("perf(kernel): read dsv41 indexer key rows as int32 words",
// Changes).  One key row is 17 int32 words: words 0..15 carry 128 e2m1 codes
// (element 2i is the low nibble of byte i), word 16 carries four ue8m0 scale
// bytes, byte j scaling elements 32j .. 32j+31 by 2^(byte - 127).  The
// dequantised element is the bf16 value e2m1 * scale; every such product with
// a finite scale is exactly representable in bf16 or overflows, so no
// rounding is ever needed.

// Exact integer construction of bf16(e2m1(nib) * 2^(e - 127)), valid for
// every scale byte, including e = 0 (2^-127), results in the bf16 subnormal
// range, overflow to infinity and e = 255 (NaN).  Code 0x8 is -0.0.
__device__ __forceinline__ uint32_t fp4_elem_exact(uint32_t nib, uint32_t e) {
    const uint32_t sign = (nib & 8u) << 12;
    const uint32_t c = nib & 7u;
    if (e == 255u) return 0x7FC0u | sign;
    if (c == 0u) return sign;
    // magnitude = (1 + mbit/2) * 2^u
    const uint32_t mbit = (c >= 2u) ? (c & 1u) : 0u;
    const int u = ((c >= 2u) ? (int)(c >> 1) - 1 : -1) + (int)e - 127;
    if (u > 127) return 0x7F80u | sign;
    if (u >= -126) return sign | ((uint32_t)(u + 127) << 7) | (mbit << 6);
    // subnormal: value / 2^-133 = (2 + mbit) * 2^(u + 132), an integer for u >= -128
    return sign | ((2u + mbit) << (u + 132));
}

// 8 e2m1 codes of one word times scale = 2^(e - 127) for a scale byte e in
// 2..252 (the caller has checked it), by the hardware scaled conversion,
// which is exact there.
__device__ __forceinline__ uint4 fp4x8_scaled_bf16x8(uint32_t word, float scale) {
    uint4 r;
    r.x = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(word, scale, 0));
    r.y = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(word, scale, 1));
    r.z = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(word, scale, 2));
    r.w = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(word, scale, 3));
    return r;
}

// 8 e2m1 codes of one word with one scale byte -> 8 bf16 (element e in half
// e%2 of dword e/2).  Scale bytes 2..252 keep every result a finite normal
// bf16; there the hardware scaled conversion is exact and is used.  Other
// scale bytes take the integer construction above.
__device__ __forceinline__ uint4 fp4x8_to_bf16x8(uint32_t word, uint32_t e) {
    uint4 r;
    if (e >= 2u && e <= 252u) {
        r = fp4x8_scaled_bf16x8(word, __uint_as_float(e << 23));   // 2^(e - 127)
    } else {
        uint32_t h[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) h[i] = fp4_elem_exact((word >> (4 * i)) & 0xFu, e);
        r.x = h[0] | (h[1] << 16);
        r.y = h[2] | (h[3] << 16);
        r.z = h[4] | (h[5] << 16);
        r.w = h[6] | (h[7] << 16);
    }
    return r;
}

}  // namespace sap
