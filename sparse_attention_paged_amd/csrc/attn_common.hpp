// attn_common.hpp -- device helpers shared by the attention kernels
// (attn.hip: every head_dim and row format; attn_d512.hip and attn_dec.hip:
// bf16 and e4m3 rows at head_dim 512).
#pragma once
#include "common.hpp"
#include "internal.hpp"

namespace sap {
namespace attn {

constexpr float kRescaleSlack = 32.0f; // log2 units: weights stay <= 2^32
constexpr int kIdxChunk = 2048;        // columns whose row indices are staged in LDS at a time

typedef short v4i16 __attribute__((ext_vector_type(4)));

// Tile row rho holds 16-byte chunk j at position j ^ rswz(rho).  rswz maps
// rows 0..7 to 8 distinct values (the S reads: 8 lanes, 8 rows, one chunk)
// and rows 4a .. 4a+3 to 4 distinct even-or-odd pairs (the transposed PV
// reads: 4 rows x 2 adjacent chunks), so both read patterns are free of LDS
// bank conflicts.
__device__ __forceinline__ int rswz(int rho) { return ((rho & 3) << 1) | ((rho >> 2) & 1); }

__device__ __forceinline__ uint4 lds_b128(const uint8_t *p) { return *(const uint4 *)p; }
__device__ __forceinline__ uint2 lds_tr16(const uint8_t *p)
{
    v4i16 r = __builtin_amdgcn_ds_read_tr16_b64_v4i16((v4i16 __attribute__((address_space(3))) *)p);
    return __builtin_bit_cast(uint2, r);
}

// An e4m3 tile (raw codes, 512 bytes per row): row rho holds 16-byte chunk j
// at slot j ^ eswz(rho).  16 consecutive rows take 16 distinct values (the S
// reads: 16 rows, one chunk), and so do rows {4a .. 4a+3, 16+4a .. 16+4a+3}
// and the 16 rows that two neighbouring 16-lane blocks of a transposed V^T
// read cover.
__device__ __forceinline__ int eswz(int rho) { return (rho & 7) | ((((rho >> 3) ^ (rho >> 4)) & 1) << 3); }

// ds_read_b64_tr_b8: in each 16-lane block, lane 8h + i receives byte i of
// the 8 bytes addressed by lanes 2k + h, k = 0..7 (byte k of the result)
__device__ __forceinline__ uint2 lds_tr8(const uint8_t *p)
{
    typedef int v2i __attribute__((ext_vector_type(2)));
    const v2i r = __builtin_amdgcn_ds_read_tr8_b64_v2i32((v2i __attribute__((address_space(3))) *)p);
    return __builtin_bit_cast(uint2, r);
}

// a, b -> two f16 terms each (round to nearest): hi = f16(a), lo =
// f16(a - hi); a - hi is exact in fp32 and |a - (hi + lo)| <= 2^-22 |a|
// above the f16 subnormal range (an absolute 2^-25 below it)
__device__ __forceinline__ void split_f16x2(float a, float b, uint32_t &hi, uint32_t &lo)
{
    typedef float f32x2 __attribute__((ext_vector_type(2)));
    typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
    const f16x2 h = __builtin_convertvector((f32x2{a, b}), f16x2);
    const f16x2 l = __builtin_convertvector((f32x2{a - (float)h[0], b - (float)h[1]}), f16x2);
    hi = __builtin_bit_cast(uint32_t, h);
    lo = __builtin_bit_cast(uint32_t, l);
}

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));

// a, b -> an f16 pair (round to nearest, a in bits 0-15)
__device__ __forceinline__ uint32_t pack_f16x2(float a, float b)
{
    typedef float f32x2 __attribute__((ext_vector_type(2)));
    typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
    return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2{a, b}), f16x2));
}
// the f16 in bits 0-15 / 16-31 of a word, widened (exactly)
__device__ __forceinline__ float f16_lo(uint32_t u) { return (float)__builtin_bit_cast(_Float16, (uint16_t)(u & 0xFFFFu)); }
__device__ __forceinline__ float f16_hi(uint32_t u) { return (float)__builtin_bit_cast(_Float16, (uint16_t)(u >> 16)); }

// max over the four lanes l, l^16, l^32, l^48 with the gfx950 row-swap
// permutes (VALU, no LDS round trip)
__device__ __forceinline__ float group4_max(float x)
{
    const uint32_t u = __float_as_uint(x);
    const auto a = __builtin_amdgcn_permlane16_swap(u, u, false, false);
    const float y = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
    const uint32_t v = __float_as_uint(y);
    const auto b = __builtin_amdgcn_permlane32_swap(v, v, false, false);
    return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}

// sum over the same four lanes
__device__ __forceinline__ float group4_sum(float x)
{
    const uint32_t u = __float_as_uint(x);
    const auto a = __builtin_amdgcn_permlane16_swap(u, u, false, false);
    const float y = __uint_as_float(a[0]) + __uint_as_float(a[1]);
    const uint32_t v = __float_as_uint(y);
    const auto b = __builtin_amdgcn_permlane32_swap(v, v, false, false);
    return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

// v *= a for an accumulator tile held in AGPRs, one element at a time through
// one temporary VGPR (the rescale is rare; this keeps it from needing a VGPR
// copy of the whole accumulator)
__device__ __forceinline__ void agpr_scale(f32x4 &v, float a)
{
    float x0 = v[0], x1 = v[1], x2 = v[2], x3 = v[3], tmp;
    asm volatile("v_accvgpr_read_b32 %4, %0\n\t"
                 "v_mul_f32 %4, %4, %5\n\t"
                 "v_accvgpr_write_b32 %0, %4\n\t"
                 "v_accvgpr_read_b32 %4, %1\n\t"
                 "v_mul_f32 %4, %4, %5\n\t"
                 "v_accvgpr_write_b32 %1, %4\n\t"
                 "v_accvgpr_read_b32 %4, %2\n\t"
                 "v_mul_f32 %4, %4, %5\n\t"
                 "v_accvgpr_write_b32 %2, %4\n\t"
                 "v_accvgpr_read_b32 %4, %3\n\t"
                 "v_mul_f32 %4, %4, %5\n\t"
                 "v_accvgpr_write_b32 %3, %4"
                 : "+a"(x0), "+a"(x1), "+a"(x2), "+a"(x3), "=&v"(tmp)
                 : "v"(a));
    v = f32x4{x0, x1, x2, x3};
}

// wait until at most N vector memory instructions of this wave are in flight
template <int N>
__device__ __forceinline__ void wait_vm() { asm volatile("s_waitcnt vmcnt(%0)" :: "n"(N) : "memory"); }

// 16 bytes per lane from global memory straight into LDS at lds_addr + 16 *
// lane (global_load_lds_dwordx4).  Issued from inline assembly, so the
// compiler neither tracks nor waits for it: the caller waits with wait_vm<N>()
// and publishes the tile with a barrier.
__device__ __forceinline__ void dma16(const void *src, uint32_t lds_addr)
{
    const uint32_t m = __builtin_amdgcn_readfirstlane(lds_addr);   // wave-uniform by construction
    asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off"
                 :: "v"(src), "s"(m) : "memory", "m0");
}

__device__ __forceinline__ uint32_t lds_offset(const void *p)
{
    return (uint32_t)(size_t)(const __attribute__((address_space(3))) uint8_t *)p;
}

}  // namespace attn
}  // namespace sap
