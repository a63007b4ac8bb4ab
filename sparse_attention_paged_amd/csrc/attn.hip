// attn.hip -- top-k sparse attention over a paged KV cache on gfx950.
//
// What is computed ("perf(kernel): keep 16-byte kv loads in dsv4 sparse
// attention and unroll gated pool", Call paths / Changes / Kernel time): for
// each query token t, its H query heads share one KV head and attend to the
// columns of idx[t, :]; column c reads one row from the window pool
// (c < n_win) or from the compressed pool, and that row serves as both key and
// value.  For e4m3 pools the per-row scale multiplies the dot outputs and is
// folded into the softmax weights for PV; the softmax denominator sums the
// unscaled weights ("Perf/kv fp8 read path", What this changes).
//
// One workgroup (4 waves) handles one token, a range of its columns and up to
// 64 heads; wave w owns heads 16w .. 16w+15.  Per tile of 32 columns:
//  1. gather: 32 rows are fetched with 16-byte loads (one wave instruction
//     reads one full 1 KiB bf16 row), written to LDS as a row-major K tile and,
//     after an 8x8 register transpose, as a V^T tile (columns contiguous per
//     head_dim element).  The next tile's loads are in flight while the
//     current tile computes; row indices are fetched one tile earlier still.
//  2. S^T = K Q^T on MFMA 16x16x32 bf16 (M = columns, N = 16 heads, K = D):
//     each lane ends up with 8 columns of one head.
//  3. online softmax per head in the log2 domain (max over the lane's 8
//     columns, then across the 4 lane groups with two xor shuffles).
//  4. O^T += V^T P^T on MFMA 16x16x32 bf16 (M = head_dim, N = heads, K = 32
//     columns); P^T is already in the B-operand layout, so P never goes
//     through LDS.  e4m3 pools feed P as a hi + lo pair of bf16 terms.
// With one split per token the output is normalised and stored; with several
// splits each workgroup stores (unnormalised O, running max, sum) and the
// merge kernel combines them in split order.
#include "common.hpp"
#include "formats.hpp"
#include "internal.hpp"

namespace sap {
namespace {

template <int D>
struct AttnShape {
    static constexpr int CH = D / 8;                            // 16-byte chunks per bf16 row
    static constexpr int KT_BYTES = kAttnTile * D * 2;          // K tile, row-major
    static constexpr int VT_BYTES = D * kAttnTile * 2;          // V^T tile
    static constexpr int META_BYTES = 2 * kAttnTile * 4;        // column bias + column scale
    static constexpr int BUF_BYTES = KT_BYTES + VT_BYTES + META_BYTES;
    static constexpr int GATHER_THREADS = (kAttnTile / 8) * CH; // one 8x8 block per thread
    static_assert(GATHER_THREADS <= 256, "tile too large for the workgroup");
};

// K tile: row rho (0..31) at rho * 2D bytes; 16-byte chunk j stored at
// position j ^ kswz(rho).  The S^T A-operand reads rows
// {0,1,2,3,8,9,10,11} (+4) with one chunk per 8-lane phase; kswz maps them to
// 8 distinct bank groups.
__device__ __forceinline__ int kswz(int rho) { return (rho & 3) | ((rho & 8) >> 1); }
template <int D>
__device__ __forceinline__ int kt_off(int rho, int chunk) { return rho * (2 * D) + 16 * (chunk ^ kswz(rho)); }

// V^T tile: head_dim element d owns 64 bytes (32 columns); 16-byte column
// chunk kc stored at position kc ^ vswz(d).  Reads take 8 consecutive d per
// phase (distinct via d & 1 and vswz); writes take d = 8j + e for 8
// consecutive j (2-way at worst).
__device__ __forceinline__ int vswz(int d) { return ((d >> 1) ^ (d >> 3)) & 3; }
__device__ __forceinline__ int vt_off(int d, int kc) { return d * 64 + 16 * (kc ^ vswz(d)); }

template <int KV> struct RawRow;
template <> struct RawRow<0> { using T = uint4; };   // 8 bf16
template <> struct RawRow<2> { using T = uint2; };   // 8 e4m3 codes

template <int D, int KV, int OUT>
__global__ __attribute__((amdgpu_flat_work_group_size(256, 256), amdgpu_waves_per_eu(1, 1)))
void attn_kernel(AttnParams p)
{
    using SH = AttnShape<D>;
    using Raw = typename RawRow<KV>::T;
    __shared__ __attribute__((aligned(16))) uint8_t smem[2 * SH::BUF_BYTES];

    // XCD-aware order: consecutive logical blocks (one token's splits, then
    // neighbouring tokens, which share window rows) stay on one XCD.
    int lb = blockIdx.x;
    {
        const int per = (int)gridDim.x >> 3;
        if (lb < (per << 3)) lb = (lb & 7) * per + (lb >> 3);
    }
    const int t = lb / p.num_splits;
    const int split = lb - t * p.num_splits;
    const int c_begin = split * p.cols_per_split;
    const int c_end = min(p.n_cols, c_begin + p.cols_per_split);
    const int n_tiles = c_end > c_begin ? (c_end - c_begin + kAttnTile - 1) / kAttnTile : 0;

    const int tid = threadIdx.x;
    const int wave = tid >> 6, lane = tid & 63, l16 = lane & 15, g = lane >> 4;
    const int head = blockIdx.y * kAttnHeadsPerBlock + wave * 16 + l16;
    const bool head_ok = head < p.H;

    // Q as the B operand of S^T: k-step s holds q[t, head, 32s + 8g .. +7].
    uint4 qf[D / 32];
    {
        const uint16_t *qrow = p.q + (int64_t)t * p.q_st + (int64_t)(head_ok ? head : 0) * p.q_sh;
#pragma unroll
        for (int s = 0; s < D / 32; ++s)
            qf[s] = head_ok ? *(const uint4 *)(qrow + 32 * s + 8 * g) : make_uint4(0, 0, 0, 0);
    }

    // gather role: row block gv (rows 8gv .. 8gv+7 of a tile), chunk gj
    const bool gthr = tid < SH::GATHER_THREADS;
    const int gv = tid / SH::CH;
    const int gj = tid - gv * SH::CH;
    const int32_t *idx_row = p.idx + (int64_t)t * p.idx_st;

    int ridx[8];     // row indices, one tile ahead of the row loads
    Raw raw[8];      // row data of the next tile to be written to LDS
    float rsc[8];    // their dequant scales (e4m3)
    bool rok[8];

    auto load_idx = [&](int tile) {
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int c = c_begin + tile * kAttnTile + 8 * gv + i;
            ridx[i] = (gthr && tile < n_tiles && c < c_end) ? idx_row[c] : -1;
        }
    };
    auto load_rows = [&](int tile) {
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int c = c_begin + tile * kAttnTile + 8 * gv + i;
            const int r = ridx[i];
            rok[i] = r >= 0;
            if (r >= 0) {
                const bool w = c < p.n_win;
                const uint8_t *base = w ? p.win : p.cmp;
                const int64_t rs = w ? p.win_rs : p.cmp_rs;
                raw[i] = *(const Raw *)(base + (int64_t)r * rs + (int64_t)gj * sizeof(Raw));
                if constexpr (KV == 2) rsc[i] = (w ? p.win_scale : p.cmp_scale)[r];
                else rsc[i] = 1.0f;
            } else {
                raw[i] = Raw{};
                rsc[i] = 0.0f;
            }
        }
    };
    auto write_tile = [&](uint8_t *buf) {
        if (!gthr) return;
        uint8_t *kt = buf;
        uint8_t *vt = buf + SH::KT_BYTES;
        float *meta = (float *)(buf + SH::KT_BYTES + SH::VT_BYTES);
        uint4 row[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            if constexpr (KV == 2) row[i] = e4m3x8_to_bf16x8(raw[i]);
            else row[i] = raw[i];
            *(uint4 *)(kt + kt_off<D>(8 * gv + i, gj)) = row[i];
        }
        // 8x8 transpose: element e of row i -> slot i of head_dim row 8gj + e
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const uint32_t sel = (e & 1) ? 0x07060302u : 0x05040100u;
            uint4 v;
            const int dw = e >> 1;
            auto pick = [&](const uint4 &u) { return dw == 0 ? u.x : dw == 1 ? u.y : dw == 2 ? u.z : u.w; };
            v.x = perm(pick(row[1]), pick(row[0]), sel);
            v.y = perm(pick(row[3]), pick(row[2]), sel);
            v.z = perm(pick(row[5]), pick(row[4]), sel);
            v.w = perm(pick(row[7]), pick(row[6]), sel);
            *(uint4 *)(vt + vt_off(8 * gj + e, gv)) = v;
        }
        if (gj == 0) {
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                meta[8 * gv + i] = rok[i] ? 0.0f : -INFINITY;
                meta[kAttnTile + 8 * gv + i] = rsc[i];
            }
        }
    };

    f32x4 acc[D / 16];
#pragma unroll
    for (int m = 0; m < D / 16; ++m) acc[m] = f32x4{0.f, 0.f, 0.f, 0.f};
    float m_run = -INFINITY, l_run = 0.0f;

    auto compute = [&](const uint8_t *buf) {
        const uint8_t *kt = buf;
        const uint8_t *vt = buf + SH::KT_BYTES;
        const float *meta = (const float *)(buf + SH::KT_BYTES + SH::VT_BYTES);
        f32x4 sacc[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
        const int rho0 = 8 * (l16 >> 2) + (l16 & 3);
#pragma unroll
        for (int s = 0; s < D / 32; ++s) {
#pragma unroll
            for (int mt = 0; mt < 2; ++mt) {
                const uint4 a = *(const uint4 *)(kt + kt_off<D>(rho0 + 4 * mt, 4 * s + g));
                sacc[mt] = mfma16x16x32(a, qf[s], sacc[mt]);
            }
        }
        // this lane: head `head`, columns rho = 8g + 4mt + i
        float x[8], csc[8];
        float tmax = -INFINITY;
#pragma unroll
        for (int mt = 0; mt < 2; ++mt)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int rho = 8 * g + 4 * mt + i;
                float v = sacc[mt][i] * p.sm_scale_log2;
                if constexpr (KV == 2) {
                    csc[4 * mt + i] = meta[kAttnTile + rho];
                    v *= csc[4 * mt + i];
                }
                v += meta[rho];
                x[4 * mt + i] = v;
                tmax = fmaxf(tmax, v);
            }
        tmax = fmaxf(tmax, shfl_xor(tmax, 16));
        tmax = fmaxf(tmax, shfl_xor(tmax, 32));
        const float m_new = fmaxf(m_run, tmax);
        const bool none = (m_new == -INFINITY);
        const float alpha = none ? 1.0f : fast_exp2(m_run - m_new);
        const float msub = none ? 0.0f : m_new;
        float pr[8], psum = 0.0f;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            pr[i] = fast_exp2(x[i] - msub);
            psum += pr[i];
        }
        l_run = l_run * alpha + psum;
        m_run = m_new;
#pragma unroll
        for (int m = 0; m < D / 16; ++m) acc[m] *= alpha;

        uint4 pb, pl;
        if constexpr (KV == 2) {
            float hi[8], lo[8];
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const float pp = pr[i] * csc[i];
                const uint32_t hb = bf16_bits(pp);
                hi[i] = pp;
                lo[i] = pp - __uint_as_float(hb << 16);
            }
            pb = make_uint4(pack_bf16x2(hi[0], hi[1]), pack_bf16x2(hi[2], hi[3]),
                            pack_bf16x2(hi[4], hi[5]), pack_bf16x2(hi[6], hi[7]));
            pl = make_uint4(pack_bf16x2(lo[0], lo[1]), pack_bf16x2(lo[2], lo[3]),
                            pack_bf16x2(lo[4], lo[5]), pack_bf16x2(lo[6], lo[7]));
        } else {
            pb = make_uint4(pack_bf16x2(pr[0], pr[1]), pack_bf16x2(pr[2], pr[3]),
                            pack_bf16x2(pr[4], pr[5]), pack_bf16x2(pr[6], pr[7]));
            pl = pb;
        }
#pragma unroll
        for (int md = 0; md < D / 16; ++md) {
            const int d = 16 * md + l16;
            const uint4 a = *(const uint4 *)(vt + vt_off(d, g));
            acc[md] = mfma16x16x32(a, pb, acc[md]);
            if constexpr (KV == 2) acc[md] = mfma16x16x32(a, pl, acc[md]);
        }
    };

    if (n_tiles > 0) {
        load_idx(0);
        load_rows(0);
        load_idx(1);
        write_tile(smem);
        __syncthreads();
        load_rows(1);
        load_idx(2);
        for (int it = 0; it < n_tiles; ++it) {
            compute(smem + (it & 1) * SH::BUF_BYTES);
            if (it + 1 < n_tiles) {
                write_tile(smem + ((it + 1) & 1) * SH::BUF_BYTES);
                load_rows(it + 2);
                load_idx(it + 3);
            }
            __syncthreads();
        }
    }

    float l_tot = l_run + shfl_xor(l_run, 16);
    l_tot += shfl_xor(l_tot, 32);
    if (!head_ok) return;

    if (p.num_splits == 1) {
        const float inv = l_tot > 0.0f ? 1.0f / l_tot : 0.0f;
        if constexpr (OUT == 1) {
            float *o = (float *)p.out + (int64_t)t * p.out_st + (int64_t)head * p.out_sh;
#pragma unroll
            for (int md = 0; md < D / 16; ++md) {
                const f32x4 v = acc[md] * inv;
                *(float4 *)(o + 16 * md + 4 * g) = make_float4(v[0], v[1], v[2], v[3]);
            }
        } else {
            uint16_t *o = (uint16_t *)p.out + (int64_t)t * p.out_st + (int64_t)head * p.out_sh;
#pragma unroll
            for (int md = 0; md < D / 16; ++md) {
                const f32x4 v = acc[md] * inv;
                *(uint2 *)(o + 16 * md + 4 * g) = make_uint2(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]));
            }
        }
    } else {
        const int64_t slot = ((int64_t)t * p.num_splits + split) * p.H + head;
        float *o = p.part_o + slot * D;
#pragma unroll
        for (int md = 0; md < D / 16; ++md)
            *(float4 *)(o + 16 * md + 4 * g) = make_float4(acc[md][0], acc[md][1], acc[md][2], acc[md][3]);
        if (g == 0) *(float2 *)(p.part_ml + slot * 2) = make_float2(m_run, l_tot);
    }
}

// out[t, h, :] = sum_j 2^(m_j - M) O_j / sum_j 2^(m_j - M) l_j over the splits
// j in order; zero when every split was empty.
template <int D, int OUT>
__global__ __launch_bounds__(128) void attn_merge_kernel(AttnParams p)
{
    const int t = blockIdx.x, head = blockIdx.y, tid = threadIdx.x;
    if (4 * tid >= D) return;
    const int S = p.num_splits;
    const int64_t slot0 = ((int64_t)t * S) * p.H + head;
    float M = -INFINITY;
    for (int j = 0; j < S; ++j) M = fmaxf(M, p.part_ml[(slot0 + (int64_t)j * p.H) * 2]);
    float4 o = make_float4(0.f, 0.f, 0.f, 0.f);
    float L = 0.0f;
    if (M != -INFINITY) {
        for (int j = 0; j < S; ++j) {
            const int64_t slot = slot0 + (int64_t)j * p.H;
            const float2 ml = *(const float2 *)(p.part_ml + slot * 2);
            const float w = fast_exp2(ml.x - M);
            L += w * ml.y;
            const float4 v = *(const float4 *)(p.part_o + slot * D + 4 * tid);
            o.x += w * v.x; o.y += w * v.y; o.z += w * v.z; o.w += w * v.w;
        }
    }
    const float inv = L > 0.0f ? 1.0f / L : 0.0f;
    if constexpr (OUT == 1) {
        float *dst = (float *)p.out + (int64_t)t * p.out_st + (int64_t)head * p.out_sh + 4 * tid;
        *(float4 *)dst = make_float4(o.x * inv, o.y * inv, o.z * inv, o.w * inv);
    } else {
        uint16_t *dst = (uint16_t *)p.out + (int64_t)t * p.out_st + (int64_t)head * p.out_sh + 4 * tid;
        *(uint2 *)dst = make_uint2(pack_bf16x2(o.x * inv, o.y * inv), pack_bf16x2(o.z * inv, o.w * inv));
    }
}

template <int D, int KV, int OUT>
hipError_t launch_attn_t(const AttnParams &p, hipStream_t s)
{
    const dim3 grid((unsigned)(p.T * p.num_splits), (unsigned)((p.H + kAttnHeadsPerBlock - 1) / kAttnHeadsPerBlock));
    hipLaunchKernelGGL((attn_kernel<D, KV, OUT>), grid, dim3(256), 0, s, p);
    return hipGetLastError();
}

template <int D>
hipError_t launch_attn_d(const AttnParams &p, int kv, int out, hipStream_t s)
{
    if (kv == 0) return out == 1 ? launch_attn_t<D, 0, 1>(p, s) : launch_attn_t<D, 0, 0>(p, s);
    return out == 1 ? launch_attn_t<D, 2, 1>(p, s) : launch_attn_t<D, 2, 0>(p, s);
}

template <int D>
hipError_t launch_merge_d(const AttnParams &p, int out, hipStream_t s)
{
    const dim3 grid((unsigned)p.T, (unsigned)p.H);
    if (out == 1) hipLaunchKernelGGL((attn_merge_kernel<D, 1>), grid, dim3(128), 0, s, p);
    else hipLaunchKernelGGL((attn_merge_kernel<D, 0>), grid, dim3(128), 0, s, p);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_attn(const AttnParams &p, int D, int kv, int out, hipStream_t s)
{
    switch (D) {
    case 64: return launch_attn_d<64>(p, kv, out, s);
    case 128: return launch_attn_d<128>(p, kv, out, s);
    case 256: return launch_attn_d<256>(p, kv, out, s);
    case 512: return launch_attn_d<512>(p, kv, out, s);
    default: return hipErrorInvalidValue;
    }
}

hipError_t launch_attn_merge(const AttnParams &p, int D, int out, hipStream_t s)
{
    switch (D) {
    case 64: return launch_merge_d<64>(p, out, s);
    case 128: return launch_merge_d<128>(p, out, s);
    case 256: return launch_merge_d<256>(p, out, s);
    case 512: return launch_merge_d<512>(p, out, s);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace sap
