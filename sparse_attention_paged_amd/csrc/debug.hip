// debug.hip -- run the hot path's row decoders over every code, so the
// tests can compare them bit for bit with the format definitions
// ("perf(kernel): read dsv41 indexer key rows as int32 words", Correctness
// and tests: every code byte against every scale byte; "Perf/kv fp8 read
// path", Tests: all 256 e4m3 codes).
#include "common.hpp"
#include "formats.hpp"
#include "internal.hpp"

namespace sap {
namespace {

__global__ __launch_bounds__(64) void debug_e4m3_kernel(uint16_t *out, float *fold)
{
    // 8 codes per lane, converted exactly as the attention row loader does
    const int lane = threadIdx.x;
    if (lane >= 32) return;
    const uint32_t c0 = 8u * lane;
    uint2 codes;
    codes.x = c0 | ((c0 + 1) << 8) | ((c0 + 2) << 16) | ((c0 + 3) << 24);
    codes.y = (c0 + 4) | ((c0 + 5) << 8) | ((c0 + 6) << 16) | ((c0 + 7) << 24);
    const uint4 r = e4m3x8_to_bf16x8(codes);
    const uint32_t dw[4] = {r.x, r.y, r.z, r.w};
    for (int e = 0; e < 8; ++e) out[c0 + e] = (uint16_t)(dw[e >> 1] >> (16 * (e & 1)));
    if (lane == 0) *fold = kE4m3FoldFactor;
}

// the f16 widening of the one-pass kernel at head_dim 512 (its V^T operand)
__global__ __launch_bounds__(64) void debug_e4m3_f16_kernel(uint16_t *out)
{
    const int lane = threadIdx.x;
    if (lane >= 32) return;
    const uint32_t c0 = 8u * lane;
    uint2 codes;
    codes.x = c0 | ((c0 + 1) << 8) | ((c0 + 2) << 16) | ((c0 + 3) << 24);
    codes.y = (c0 + 4) | ((c0 + 5) << 8) | ((c0 + 6) << 16) | ((c0 + 7) << 24);
    const uint4 r = e4m3x8_to_f16x8(codes);
    const uint32_t dw[4] = {r.x, r.y, r.z, r.w};
    for (int e = 0; e < 8; ++e) out[c0 + e] = (uint16_t)(dw[e >> 1] >> (16 * (e & 1)));
}

__global__ __launch_bounds__(256) void debug_fp4_kernel(uint16_t *out)
{
    // one code byte per block, one scale byte per thread
    const uint32_t c = blockIdx.x, s = threadIdx.x;
    const uint4 r = fp4x8_to_bf16x8(c, s);     // byte 0 of the word is the code byte
    out[(c * 256 + s) * 2 + 0] = (uint16_t)(r.x & 0xFFFFu);
    out[(c * 256 + s) * 2 + 1] = (uint16_t)(r.x >> 16);
}

}  // namespace

hipError_t launch_debug_e4m3(uint16_t *out, float *fold, hipStream_t s)
{
    hipLaunchKernelGGL(debug_e4m3_kernel, dim3(1), dim3(64), 0, s, out, fold);
    return hipGetLastError();
}

hipError_t launch_debug_e4m3_f16(uint16_t *out, hipStream_t s)
{
    hipLaunchKernelGGL(debug_e4m3_f16_kernel, dim3(1), dim3(64), 0, s, out);
    return hipGetLastError();
}

hipError_t launch_debug_fp4(uint16_t *out, hipStream_t s)
{
    hipLaunchKernelGGL(debug_fp4_kernel, dim3(256), dim3(256), 0, s, out);
    return hipGetLastError();
}

}  // namespace sap
