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
// One workgroup = 4 waves = up to 64 heads of one token over a range of its
// columns.  Wave (hh, dh) owns heads 32hh .. 32hh+31 (two 16-head MFMA tiles,
// so each K or V fragment read from LDS feeds two MFMAs) and head_dim half
// dh.  Per tile of 32 columns:
//  1. gather: each 16-byte chunk of the 32 rows goes straight from HBM into
//     LDS (global_load_lds_dwordx4; at D = 512 one wave instruction moves one
//     1 KiB row), XOR-swizzled per row.  The next tile is in flight while the
//     current one computes (two LDS arrays); e4m3 rows go through registers
//     and are widened to bf16 on the way.
//  2. S^T = K Q^T on MFMA 16x16x32 bf16 (M = columns, N = heads) over the
//     wave's half of head_dim; the two halves swap fp32 partial scores
//     through LDS and add them (a + b on one side, b + a on the other: the
//     same bits), so both waves hold the full scores of their 32 heads.
//  3. online softmax per head in the log2 domain; the running max is only
//     raised (and O rescaled) when a tile's max exceeds it by more than 8, so
//     the weights stay <= 2^8 and the rescale is rare.
//  4. O^T += V^T P^T on MFMA 16x16x32 bf16 (M = head_dim, N = heads, K = 32
//     columns) for the wave's head_dim half.  P^T leaves step 3 already in the
//     B-operand layout; the V^T A-operand is read from the same row-major
//     tile with ds_read_b64_tr_b16 (within 16 lanes, lane i receives element
//     i%4 of the 8 bytes addressed by lanes i/4 + 4r, r = 0..3).  e4m3 pools
//     feed P as a hi + lo pair of bf16 terms.
// With one split per token the output is normalised and stored; with several
// splits each workgroup stores (unnormalised O, running max, sum) and the
// merge kernel combines them in split order.
#include "common.hpp"
#include "formats.hpp"
#include "internal.hpp"

namespace sap {
namespace {

constexpr int kThreads = 256;          // 4 waves
constexpr float kRescaleSlack = 8.0f;  // log2 units

typedef short v4i16 __attribute__((ext_vector_type(4)));

template <int D>
struct AttnShape {
    static constexpr int CH = D / 8;                    // 16-byte chunks per bf16 row
    static constexpr int RPI = 64 / CH;                 // rows per 1 KiB wave instruction
    static constexpr int NQ = D / 64;                   // gather instructions per wave per tile
    static constexpr int SK = D / 64;                   // S k-steps per wave (its head_dim half)
    static constexpr int PM = D / 32;                   // PV head_dim tiles per wave
    static constexpr int KT_BYTES = kAttnTile * D * 2;  // K tile, row-major (= 1 KiB * D / 32)
    static constexpr int BUF_BYTES = KT_BYTES;
};

// K tile row rho (0..31) holds 16-byte chunk j at position j ^ kswz(rho): the
// S^T A-operand reads rows {0-3, 8-11} (+4) of one chunk per 8-lane phase and
// kswz sends them to 8 distinct bank groups.
__device__ __forceinline__ int kswz(int rho) { return (rho & 3) | ((rho & 8) >> 1); }

template <int KV> struct RawRow;
template <> struct RawRow<0> { using T = uint4; };   // 8 bf16
template <> struct RawRow<2> { using T = uint2; };   // 8 e4m3 codes

__device__ __forceinline__ uint4 lds_b128(const uint8_t *p) { return *(const uint4 *)p; }
__device__ __forceinline__ uint2 lds_tr16(const uint8_t *p)
{
    v4i16 r = __builtin_amdgcn_ds_read_tr16_b64_v4i16((v4i16 __attribute__((address_space(3))) *)p);
    return __builtin_bit_cast(uint2, r);
}

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

template <int D, int KV, int OUT>
__global__ __attribute__((amdgpu_flat_work_group_size(kThreads, kThreads), amdgpu_waves_per_eu(1, 1)))
void attn_kernel(AttnParams p)
{
    using SH = AttnShape<D>;
    using Raw = typename RawRow<KV>::T;
    // two distinct arrays (not halves of one) so the compiler can tell the
    // in-flight gather into one buffer from the reads of the other
    __shared__ __attribute__((aligned(1024))) uint8_t bufA[SH::BUF_BYTES];
    __shared__ __attribute__((aligned(1024))) uint8_t bufB[SH::BUF_BYTES];
    // per-column bias (0 or -inf) and dequant scale of each buffer, kept out of
    // the gather targets so writing them never waits on an in-flight gather
    __shared__ float metaA[2 * kAttnTile], metaB[2 * kAttnTile];
    __shared__ __attribute__((aligned(16))) float4 xch[4][4][64];   // [wave][j][lane] partial scores

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
    const int hh = wave >> 1, dh = wave & 1;
    const int hbase = blockIdx.y * kAttnHeadsPerBlock + hh * 32;

    // Q as the B operand of S^T over this wave's head_dim half:
    // qf[nt][s] = q[t, hbase + 16nt + l16, 32(dh*SK + s) + 8g .. +7]
    uint4 qf[2][SH::SK];
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) {
        const int head = hbase + 16 * nt + l16;
        const bool ok = head < p.H;
        const uint16_t *qrow = p.q + (int64_t)t * p.q_st + (int64_t)(ok ? head : 0) * p.q_sh;
#pragma unroll
        for (int s = 0; s < SH::SK; ++s)
            qf[nt][s] = ok ? *(const uint4 *)(qrow + 32 * (dh * SH::SK + s) + 8 * g) : make_uint4(0, 0, 0, 0);
    }
    // finite data that invalid columns load instead of a pool row (their
    // scores are masked to -inf and their weights are 0)
    const uint8_t *safe_src = (const uint8_t *)(p.q + (int64_t)t * p.q_st);

    // gather role: instruction q of this wave covers tile rows
    // 8*wave + q*RPI .. + RPI-1; this lane reads row grow(q), chunk slot gpos
    const int32_t *idx_row = p.idx + (int64_t)t * p.idx_st;
    const int gpos = lane % SH::CH;
    auto grow = [&](int q) { return 8 * wave + q * SH::RPI + lane / SH::CH; };
    int ridx[SH::NQ];      // row indices of the next tile to be issued
    Raw raw[SH::NQ];       // e4m3 only: codes of the next tile, widened when written
    float rsc[SH::NQ];

    auto load_idx = [&](int tile) {
#pragma unroll
        for (int q = 0; q < SH::NQ; ++q) {
            const int c = c_begin + tile * kAttnTile + grow(q);
            ridx[q] = (tile < n_tiles && c < c_end) ? idx_row[c] : -1;
        }
    };
    // issue the tile whose indices sit in ridx into buffer `bf`
    auto issue = [&](uint8_t *bf, float *meta, int tile) {
#pragma unroll
        for (int q = 0; q < SH::NQ; ++q) {
            const int rho = grow(q);
            const int c = c_begin + tile * kAttnTile + rho;
            // one row per instruction: the index is wave-uniform, use an SGPR
            const int r = SH::RPI == 1 ? __builtin_amdgcn_readfirstlane(ridx[q]) : ridx[q];
            const bool w = c < p.n_win;
            const uint8_t *base = w ? p.win : p.cmp;
            const int64_t rs = w ? p.win_rs : p.cmp_rs;
            const int j = gpos ^ kswz(rho);
            if constexpr (KV == 0) {
                const uint8_t *src = r >= 0 ? base + (int64_t)r * rs + 16 * j : safe_src + 16 * gpos;
                __builtin_amdgcn_global_load_lds(
                    (const void *)src,
                    (__attribute__((address_space(3))) void *)(bf + (8 * wave + q * SH::RPI) * 2 * D), 16, 0, 0);
            } else {
                // unused columns: load the stand-in bytes but keep zero codes,
                // since arbitrary bytes read as e4m3 may be NaN encodings
                const uint8_t *src = r >= 0 ? base + (int64_t)r * rs + 8 * j : safe_src + 8 * gpos;
                const Raw v = *(const Raw *)src;
                raw[q] = r >= 0 ? v : Raw{0u, 0u};
                rsc[q] = r >= 0 ? (w ? p.win_scale : p.cmp_scale)[r] : 0.0f;
            }
            if (gpos == 0) meta[rho] = r >= 0 ? 0.0f : -INFINITY;
        }
    };
    // e4m3: widen the registers of the issued tile into the buffer (after the
    // current tile's compute, so the loads had that long to arrive)
    auto land = [&](uint8_t *bf, float *meta) {
        if constexpr (KV == 2) {
            float *scl = meta + kAttnTile;
#pragma unroll
            for (int q = 0; q < SH::NQ; ++q) {
                *(uint4 *)(bf + (8 * wave + q * SH::RPI) * 2 * D + 16 * lane) = e4m3x8_to_bf16x8(raw[q]);
                if (gpos == 0) scl[grow(q)] = rsc[q];
            }
        }
    };

    f32x4 acc[SH::PM][2];
#pragma unroll
    for (int m = 0; m < SH::PM; ++m) acc[m][0] = acc[m][1] = f32x4{0.f, 0.f, 0.f, 0.f};
    float m_run[2] = {-INFINITY, -INFINITY}, l_run[2] = {0.0f, 0.0f};

    auto compute = [&](const uint8_t *bf, const float *meta) {
        const float *bias = meta;
        const float *scl = meta + kAttnTile;
        // --- S^T partial over this wave's head_dim half; rows
        //     a(mt, m) = 8(m>>2) + 4mt + (m&3) of the tile
        f32x4 sacc[2][2];
#pragma unroll
        for (int mt = 0; mt < 2; ++mt) sacc[mt][0] = sacc[mt][1] = f32x4{0.f, 0.f, 0.f, 0.f};
        {
            const int rho0 = 8 * (l16 >> 2) + (l16 & 3);
            const uint8_t *k0 = bf + rho0 * 2 * D, *k1 = bf + (rho0 + 4) * 2 * D;
            const int ks0 = kswz(rho0), ks1 = kswz(rho0 + 4);
            auto kfrag = [&](int s, int mt) {
                const int chunk = 4 * (dh * SH::SK + s) + g;
                return mt ? lds_b128(k1 + 16 * (chunk ^ ks1)) : lds_b128(k0 + 16 * (chunk ^ ks0));
            };
            uint4 f0[3], f1[3];   // fragments for k-steps s, s+1, s+2 (ring)
            f0[0] = kfrag(0, 0);
            f1[0] = kfrag(0, 1);
            if (SH::SK > 1) {
                f0[1] = kfrag(1, 0);
                f1[1] = kfrag(1, 1);
            }
#pragma unroll
            for (int s = 0; s < SH::SK; ++s) {
                if (s + 2 < SH::SK) {
                    f0[(s + 2) % 3] = kfrag(s + 2, 0);
                    f1[(s + 2) % 3] = kfrag(s + 2, 1);
                }
                __builtin_amdgcn_sched_barrier(0);
                sacc[0][0] = mfma16x16x32(f0[s % 3], qf[0][s], sacc[0][0]);
                sacc[0][1] = mfma16x16x32(f0[s % 3], qf[1][s], sacc[0][1]);
                sacc[1][0] = mfma16x16x32(f1[s % 3], qf[0][s], sacc[1][0]);
                sacc[1][1] = mfma16x16x32(f1[s % 3], qf[1][s], sacc[1][1]);
                __builtin_amdgcn_sched_barrier(0);
            }
        }
        // --- swap partial scores with the other head_dim half
        {
            float4 *mine = xch[wave][0];
            mine[0 * 64 + lane] = make_float4(sacc[0][0][0], sacc[0][0][1], sacc[0][0][2], sacc[0][0][3]);
            mine[1 * 64 + lane] = make_float4(sacc[0][1][0], sacc[0][1][1], sacc[0][1][2], sacc[0][1][3]);
            mine[2 * 64 + lane] = make_float4(sacc[1][0][0], sacc[1][0][1], sacc[1][0][2], sacc[1][0][3]);
            mine[3 * 64 + lane] = make_float4(sacc[1][1][0], sacc[1][1][1], sacc[1][1][2], sacc[1][1][3]);
            __syncthreads();
            const float4 *other = xch[wave ^ 1][0];
            float4 o[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) o[j] = other[j * 64 + lane];
            // dh 0 adds mine + other, dh 1 adds other + mine: identical sums
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                f32x4 &sv = sacc[j >> 1][j & 1];
                const f32x4 ov = f32x4{o[j].x, o[j].y, o[j].z, o[j].w};
                sv = dh == 0 ? sv + ov : ov + sv;
            }
        }
        // --- softmax; this lane: head hbase + 16nt + l16, columns 8g + k (k = 4mt + i)
        float bb[8], csc[8];
        {
            const float4 b0 = *(const float4 *)(bias + 8 * g), b1 = *(const float4 *)(bias + 8 * g + 4);
            bb[0] = b0.x; bb[1] = b0.y; bb[2] = b0.z; bb[3] = b0.w;
            bb[4] = b1.x; bb[5] = b1.y; bb[6] = b1.z; bb[7] = b1.w;
            if constexpr (KV == 2) {
                const float4 s0 = *(const float4 *)(scl + 8 * g), s1 = *(const float4 *)(scl + 8 * g + 4);
                csc[0] = s0.x; csc[1] = s0.y; csc[2] = s0.z; csc[3] = s0.w;
                csc[4] = s1.x; csc[5] = s1.y; csc[6] = s1.z; csc[7] = s1.w;
            }
        }
        // scores in log2 units; recomputed from sacc where needed instead of kept
        auto score = [&](int nt, int k) {
            float v = sacc[k >> 2][nt][k & 3] * p.sm_scale_log2;
            if constexpr (KV == 2) v *= csc[k];
            return v + bb[k];
        };
        float tmax[2];
#pragma unroll
        for (int nt = 0; nt < 2; ++nt) {
            tmax[nt] = -INFINITY;
#pragma unroll
            for (int k = 0; k < 8; ++k) tmax[nt] = fmaxf(tmax[nt], score(nt, k));
        }
        tmax[0] = group4_max(tmax[0]);
        tmax[1] = group4_max(tmax[1]);
        const bool raise0 = tmax[0] > m_run[0] + kRescaleSlack;
        const bool raise1 = tmax[1] > m_run[1] + kRescaleSlack;
        if (__builtin_amdgcn_ballot_w64(raise0 || raise1) != 0) {
#pragma unroll
            for (int nt = 0; nt < 2; ++nt) {
                const bool raise = nt ? raise1 : raise0;
                const float m_new = raise ? tmax[nt] : m_run[nt];
                const float alpha = raise ? fast_exp2(m_run[nt] - m_new) : 1.0f;
                m_run[nt] = m_new;
                l_run[nt] *= alpha;
#pragma unroll
                for (int m = 0; m < SH::PM; ++m) agpr_scale(acc[m][nt], alpha);
            }
        }
        uint4 pb[2], pl[2];
#pragma unroll
        for (int nt = 0; nt < 2; ++nt) {
            const float msub = m_run[nt] == -INFINITY ? 0.0f : m_run[nt];
            float pr[8], psum = 0.0f;
#pragma unroll
            for (int k = 0; k < 8; ++k) {
                pr[k] = fast_exp2(score(nt, k) - msub);
                psum += pr[k];
            }
            l_run[nt] += psum;
            if constexpr (KV == 2) {
                float hi[8], lo[8];
#pragma unroll
                for (int k = 0; k < 8; ++k) {
                    const float pp = pr[k] * csc[k];
                    hi[k] = pp;
                    lo[k] = pp - __uint_as_float(bf16_bits(pp) << 16);
                }
                pb[nt] = make_uint4(pack_bf16x2(hi[0], hi[1]), pack_bf16x2(hi[2], hi[3]),
                                    pack_bf16x2(hi[4], hi[5]), pack_bf16x2(hi[6], hi[7]));
                pl[nt] = make_uint4(pack_bf16x2(lo[0], lo[1]), pack_bf16x2(lo[2], lo[3]),
                                    pack_bf16x2(lo[4], lo[5]), pack_bf16x2(lo[6], lo[7]));
            } else {
                pb[nt] = make_uint4(pack_bf16x2(pr[0], pr[1]), pack_bf16x2(pr[2], pr[3]),
                                    pack_bf16x2(pr[4], pr[5]), pack_bf16x2(pr[6], pr[7]));
                pl[nt] = pb[nt];
            }
        }
        // --- O^T += V^T P^T over this wave's head_dim half: A-operand rows
        //     8g + 4h + (l16>>2), head_dim 16md + 4(l16&3)
        {
            const int trow0 = 8 * g + (l16 >> 2);
            const uint8_t *va0 = bf + trow0 * 2 * D, *va1 = bf + (trow0 + 4) * 2 * D;
            const int vs0 = kswz(trow0), vs1 = kswz(trow0 + 4);
            const int dsub = 4 * (l16 & 3);
            auto vfrag = [&](int m) {
                const int d = 16 * (dh * SH::PM + m) + dsub;
                const uint2 v0 = lds_tr16(va0 + 16 * ((d >> 3) ^ vs0) + 2 * (d & 7));
                const uint2 v1 = lds_tr16(va1 + 16 * ((d >> 3) ^ vs1) + 2 * (d & 7));
                return make_uint4(v0.x, v0.y, v1.x, v1.y);
            };
            uint4 vr[3];
            vr[0] = vfrag(0);
            if (SH::PM > 1) vr[1] = vfrag(1);
#pragma unroll
            for (int m = 0; m < SH::PM; ++m) {
                if (m + 2 < SH::PM) vr[(m + 2) % 3] = vfrag(m + 2);
                __builtin_amdgcn_sched_barrier(0);
                const uint4 a = vr[m % 3];
                acc[m][0] = mfma16x16x32(a, pb[0], acc[m][0]);
                acc[m][1] = mfma16x16x32(a, pb[1], acc[m][1]);
                if constexpr (KV == 2) {
                    acc[m][0] = mfma16x16x32(a, pl[0], acc[m][0]);
                    acc[m][1] = mfma16x16x32(a, pl[1], acc[m][1]);
                }
                __builtin_amdgcn_sched_barrier(0);
            }
        }
    };

    // wait until this wave's gathers for the next tile have landed in LDS
    auto wait_gather = [&]() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); };

    if (n_tiles > 0) {
        load_idx(0);
        issue(bufA, metaA, 0);
        land(bufA, metaA);
        load_idx(1);
        wait_gather();
        __syncthreads();
        for (int it = 0; it < n_tiles; it += 2) {
            // tile it is in bufA; tile it+1 goes to bufB
            if (it + 1 < n_tiles) {
                issue(bufB, metaB, it + 1);
                load_idx(it + 2);
            }
            compute(bufA, metaA);
            if (it + 1 < n_tiles) land(bufB, metaB);
            wait_gather();
            __syncthreads();
            if (it + 1 >= n_tiles) break;
            // tile it+1 is in bufB; tile it+2 goes to bufA
            if (it + 2 < n_tiles) {
                issue(bufA, metaA, it + 2);
                load_idx(it + 3);
            }
            compute(bufB, metaB);
            if (it + 2 < n_tiles) land(bufA, metaA);
            wait_gather();
            __syncthreads();
        }
    }

#pragma unroll
    for (int nt = 0; nt < 2; ++nt) {
        const int head = hbase + 16 * nt + l16;
        const float l_tot = group4_sum(l_run[nt]);
        if (head >= p.H) continue;
        const int d0 = 16 * dh * SH::PM + 4 * g;
        if (p.num_splits == 1) {
            const float inv = l_tot > 0.0f ? 1.0f / l_tot : 0.0f;
            if constexpr (OUT == 1) {
                float *o = (float *)p.out + (int64_t)t * p.out_st + (int64_t)head * p.out_sh + d0;
#pragma unroll
                for (int m = 0; m < SH::PM; ++m) {
                    const f32x4 v = acc[m][nt] * inv;
                    *(float4 *)(o + 16 * m) = make_float4(v[0], v[1], v[2], v[3]);
                }
            } else {
                uint16_t *o = (uint16_t *)p.out + (int64_t)t * p.out_st + (int64_t)head * p.out_sh + d0;
#pragma unroll
                for (int m = 0; m < SH::PM; ++m) {
                    const f32x4 v = acc[m][nt] * inv;
                    *(uint2 *)(o + 16 * m) = make_uint2(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]));
                }
            }
        } else {
            const int64_t slot = ((int64_t)t * p.num_splits + split) * p.H + head;
            float *o = p.part_o + slot * D + d0;
#pragma unroll
            for (int m = 0; m < SH::PM; ++m)
                *(float4 *)(o + 16 * m) = make_float4(acc[m][nt][0], acc[m][nt][1], acc[m][nt][2], acc[m][nt][3]);
            if (g == 0 && dh == 0) *(float2 *)(p.part_ml + slot * 2) = make_float2(m_run[nt], l_tot);
        }
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
    hipLaunchKernelGGL((attn_kernel<D, KV, OUT>), grid, dim3(kThreads), 0, s, p);
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
