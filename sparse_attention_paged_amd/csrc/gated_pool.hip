// gated_pool.hip -- the compressor's gated pool on gfx950.
//
// "perf(kernel): keep 16-byte kv loads in dsv4 sparse attention and unroll
// gated pool" (Call paths: the compressor's decode step calls gated_pool;
// Changes: it has a max loop and a second loop over R) prints no formula.
// Reading taken: channel d of the R raw rows of pool b is weighted by a
// softmax over R of its gate scores,
//   out[b, d] = sum_r e_r x[b, r, d] / sum_r e_r,
//   e_r = exp(g[b, r, d] - m),  m = max_r g[b, r, d],
// -inf gates contribute nothing and an all -inf column pools to 0.
//
// A workgroup takes 64 consecutive channels of one pool with 8 waves; lane
// = channel, wave w takes rows w, w + 8, ...  Each wave keeps (max, sum,
// weighted sum) per channel over its rows, taken in chunks of CH rows held in
// registers (the chunk's max, then one exp per element, merged into the
// running state), and the 8 partial states are combined in wave order
// through LDS.  Loads along a row are 64 consecutive channels (coalesced).
// CH = 16 for R > 32 (R = 128: one chunk, one memory round trip per wave),
// else 4 (R = 8: one row per wave, few loads past R).
#include "common.hpp"
#include "internal.hpp"

#include <math.h>
#include <type_traits>

namespace sap {
namespace {

constexpr int kPoolWaves = 8;
constexpr float kLog2e = 1.4426950408889634f;

__device__ __forceinline__ float load_f(const uint16_t *p) { return __uint_as_float((uint32_t)*p << 16); }
__device__ __forceinline__ float load_f(const float *p) { return *p; }
__device__ __forceinline__ void store_f(uint16_t *p, float v) { *p = (uint16_t)bf16_bits(v); }
__device__ __forceinline__ void store_f(float *p, float v) { *p = v; }

template <typename XT, typename GT, typename OT, int CH>
__global__ __launch_bounds__(kPoolWaves * 64) void gated_pool_kernel(GatedPoolParams p)
{
    __shared__ float part[3][kPoolWaves][64];
    const int b = blockIdx.y;
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int d = blockIdx.x * 64 + lane;
    const bool dok = d < p.D;
    const XT *xb = (const XT *)p.x + (int64_t)b * p.x_sb + (dok ? d : 0);
    const GT *gb = (const GT *)p.g + (int64_t)b * p.g_sb + (dok ? d : 0);

    float m = -INFINITY, s = 0.0f, a = 0.0f;   // running state, log2 domain for m
    for (int r0 = wave; r0 < p.R; r0 += kPoolWaves * CH) {
        float gv[CH], xv[CH];
        // every load is issued, from a row clamped into range, and the value
        // selected afterwards: loads inside a branch each got a wait of
        // their own, so the chunk took one memory round trip per row
#pragma unroll
        for (int i = 0; i < CH; ++i) {
            const int r = r0 + kPoolWaves * i;
            const int rc = r < p.R ? r : p.R - 1;
            const float gl = load_f(gb + (int64_t)rc * p.g_sr), xl = load_f(xb + (int64_t)rc * p.x_sr);
            const bool ok = dok && r < p.R;
            gv[i] = ok ? gl * kLog2e : -INFINITY;
            xv[i] = ok ? xl : 0.0f;
        }
        float cm = gv[0];
#pragma unroll
        for (int i = 1; i < CH; ++i) cm = fmaxf(cm, gv[i]);
        if (cm == -INFINITY) continue;   // nothing of weight in this chunk
        const float mn = fmaxf(m, cm);
        const float alpha = m == -INFINITY ? 0.0f : fast_exp2(m - mn);
        float cs = 0.0f, ca = 0.0f;
#pragma unroll
        for (int i = 0; i < CH; ++i) {
            const float e = gv[i] == -INFINITY ? 0.0f : fast_exp2(gv[i] - mn);
            cs += e;
            ca = fmaf(e, xv[i], ca);
        }
        s = fmaf(s, alpha, cs);
        a = fmaf(a, alpha, ca);
        m = mn;
    }
    part[0][wave][lane] = m;
    part[1][wave][lane] = s;
    part[2][wave][lane] = a;
    __syncthreads();
    if (wave != 0 || !dok) return;
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < kPoolWaves; ++w) M = fmaxf(M, part[0][w][lane]);
    float S = 0.0f, A = 0.0f;
    if (M != -INFINITY) {
#pragma unroll
        for (int w = 0; w < kPoolWaves; ++w) {
            const float mw = part[0][w][lane];
            const float f = mw == -INFINITY ? 0.0f : fast_exp2(mw - M);
            S = fmaf(part[1][w][lane], f, S);
            A = fmaf(part[2][w][lane], f, A);
        }
    }
    store_f((OT *)p.out + (int64_t)b * p.out_sb + d, S > 0.0f ? A / S : 0.0f);
}

template <typename XT, typename GT>
hipError_t launch_out(const GatedPoolParams &p, dim3 grid, hipStream_t s)
{
    auto go = [&](auto ch_tag) {
        constexpr int CH = decltype(ch_tag)::value;
        if (p.out_bf16)
            hipLaunchKernelGGL((gated_pool_kernel<XT, GT, uint16_t, CH>), grid, dim3(kPoolWaves * 64), 0, s, p);
        else
            hipLaunchKernelGGL((gated_pool_kernel<XT, GT, float, CH>), grid, dim3(kPoolWaves * 64), 0, s, p);
    };
    if (p.R > 32) go(std::integral_constant<int, 16>{});
    else go(std::integral_constant<int, 4>{});
    return hipGetLastError();
}

}  // namespace

hipError_t launch_gated_pool(const GatedPoolParams &p, hipStream_t s)
{
    const dim3 grid((unsigned)((p.D + 63) / 64), (unsigned)p.B);
    if (grid.x == 0 || grid.y == 0) return hipSuccess;
    if (p.x_bf16)
        return p.g_bf16 ? launch_out<uint16_t, uint16_t>(p, grid, s) : launch_out<uint16_t, float>(p, grid, s);
    return p.g_bf16 ? launch_out<float, uint16_t>(p, grid, s) : launch_out<float, float>(p, grid, s);
}

}  // namespace sap
