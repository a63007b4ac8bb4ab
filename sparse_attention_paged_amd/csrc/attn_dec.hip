// attn_dec.hip -- split-K sparse attention for decode batches at head_dim 512.
//
// What is computed is the same as in attn.hip ("perf(kernel): keep 16-byte kv
// loads in dsv4 sparse attention and unroll gated pool", Call paths / Kernel
// time): query token t's H heads share one KV head and attend to the columns
// of idx[t, :]; column c reads one row of the window pool (c < n_win) or of
// the compressed pool, and that row is both key and value.  For e4m3 pools
// the per-row scale multiplies the dot outputs and is folded into the
// softmax weights for PV; the denominator sums the unscaled weights ("Perf/kv
// fp8 read path", What this changes).
//
// Decode has few tokens, so the work of one token is spread over many
// workgroups, and what they write for the merge should not outweigh the rows
// they read.  One workgroup = 4 waves = 16 heads of one token over a range of
// its columns taken in rounds of 128 (32 per wave); a split's partial output
// is then 16 heads x 512 f16 = 16 KiB (bf16 rows; e4m3 rows: fp32, 32 KiB),
// the size of 16 (32) rows, for the 128 rows (and more) it summarises:
//  - gather: wave w moves its 32 rows from HBM straight into its own LDS tile
//    (global_load_lds_dwordx4: one 1 KiB row per wave instruction, 16-byte
//    loads; e4m3 rows: the raw codes, two 512-byte rows per instruction);
//  - S^T = K Q^T for the wave's 32 columns and the 16 heads over all 512
//    dims on MFMA 16x16x32 bf16 (M = columns, N = heads): the wave's own rows
//    and its own copy of Q, so no partial score crosses waves;
//  - online softmax (log2 domain): the waves exchange their 16 tile maxima
//    through LDS (one barrier), so every wave rescales against the same
//    running max; the weights stay in the MFMA output layout, which is the
//    PV B-operand layout under the column order kk = 8g + 4c + i <-> column
//    16c + 4g + i;
//  - O^T += V^T P^T: wave w owns head_dim 128w .. 128w+127 for the 16 heads
//    over all 128 columns of the round (the other waves' weights come through
//    LDS, one barrier); V^T fragments are read from the four row-major tiles
//    with ds_read_b64_tr_b16.
// e4m3 rows: K fragments are widened to bf16 in registers (exact); the row
// scale s = mu * 2^e multiplies the scores and e joins the log2 score, V^T
// comes from ds_read_b64_tr_b8 widened to f16 (exact), and the weights
// p * s = mu * exp2(x + e - m) (below 1: the running max is exact here)
// enter PV as two f16 terms; the sums take p = 2^-e exp2(x + e - m).
// One split per token stores the normalised output; several splits store
// (unnormalised O, running max, sum) and attn_dec_merge_kernel combines them
// in split order; for bf16 rows O is stored in f16, each head's three values
// scaled by one power of two so that its O fits f16.  All workgroups of one
// token -- its splits and head groups -- are placed on one XCD, so a
// gathered row and the q rows come from HBM once and the other head groups
// find them in that XCD's L2.
#include "common.hpp"
#include "formats.hpp"
#include "internal.hpp"
#include "attn_common.hpp"

#include <type_traits>

namespace sap {
namespace {

using namespace attn;

constexpr int kD = 512;                 // head_dim
constexpr int kWv = 4;                  // waves per workgroup
constexpr int kCW = 32;                 // columns per wave per round
constexpr int kRows = kDecRound;        // columns per round (kWv * kCW)
constexpr int kPM = kD / (16 * kWv);    // PV m-steps over a wave's head_dim quarter

// what unused columns of an e4m3 tile gather: zeros (any other stand-in's
// bytes could hold the e4m3 NaN codes, and a zero weight times NaN is NaN)
__device__ __attribute__((aligned(16))) uint8_t g_dec_pad_row[kD];

static_assert(kRows == kWv * kCW, "a round is one tile per wave");

// lane l moves 16 bytes from base + voff into LDS at lds + 16 l, base a
// wave-uniform 64-bit address in scalar registers (taken with v_readlane,
// so the wait states a vector memory instruction needs after a VALU write
// of its scalar operand are inserted here: the compiler does not see into
// the assembly)
__device__ __forceinline__ void dma_row(uint64_t base, uint32_t voff, uint32_t lds)
{
    asm volatile("s_mov_b32 m0, %2\n\t"
                 "s_nop 4\n\t"
                 "global_load_lds_dwordx4 %0, %1"
                 :: "v"(voff), "s"(base), "s"(lds) : "memory", "m0");
}

// workgroup -> (unit u = token * splits + split, head group g); blocks whose
// token is past the end exit at once.  Block b runs on XCD b % 8 (workgroups
// are dealt to the eight XCDs in turn): token t's splits and head groups all
// run on XCD t % 8, so its q rows come from memory once, and its merge
// workgroups (placed the same way) read the partials through the same L2.
struct DecSlot {
    int u, g;
    bool valid;
};
__device__ __forceinline__ DecSlot dec_slot(int b, int G, int S, int T)
{
    const int x = b & 7, r = b >> 3;
    const int k = r / (S * G), rem = r - k * (S * G);
    const int t = 8 * k + x;
    return DecSlot{t * S + rem / G, rem % G, t < T};
}

template <int KV, int OUT>
__global__ __attribute__((amdgpu_flat_work_group_size(64 * kWv, 64 * kWv), amdgpu_waves_per_eu(1, 1)))
void attn_dec_kernel(AttnParams p)
{
    constexpr bool E4 = KV == 2;
    // PV weight terms: e4m3 weights carry the row scale and must be held to
    // fp32-like precision (outputs reach ~1e3 against an absolute bar), so
    // they enter as two f16 terms, hi + lo
    constexpr int NP = E4 ? 2 : 1;
    constexpr int kRB = E4 ? kD : 2 * kD;   // bytes of one tile row
    __shared__ __attribute__((aligned(1024))) uint8_t tiles[kWv][kCW * kRB];
    __shared__ __attribute__((aligned(1024))) uint8_t qs[kDecHeads * kD * 2];
    __shared__ __attribute__((aligned(16))) uint4 xp[NP][kWv][64];   // weights of each wave's columns
    __shared__ __attribute__((aligned(16))) float meta[kWv][2][kCW]; // per column: bias (0 / -inf), scale
    __shared__ float xm[kWv][kDecHeads];                            // tile maxima
    __shared__ float xl[kWv][kDecHeads];                            // softmax sums
    __shared__ float xa[kWv][kDecHeads];                            // largest |O| per head_dim quarter

    const int G = p.hgroups;
    const DecSlot sl = dec_slot((int)blockIdx.x, G, p.num_splits, p.T);
    if (!sl.valid) return;
    const int t = sl.u / p.num_splits, split = sl.u - t * p.num_splits;
    const int hbase = sl.g * kDecHeads;
    const int c_begin = split * p.cols_per_split;
    const int c_end = min(p.n_cols, c_begin + p.cols_per_split);

    const int tid = threadIdx.x;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63, l16 = lane & 15, g = lane >> 4;

    // q rows of the 16 heads -> qs, 16-byte chunk c of head h at slot c ^ h
    // (the fragment reads below are then free of bank conflicts); rows past
    // H load head hbase as a finite stand-in
#pragma unroll
    for (int k = 0; k < kDecHeads / kWv; ++k) {
        const int h = (kDecHeads / kWv) * w + k;
        const int head = hbase + h < p.H ? hbase + h : hbase;
        dma16(p.q + (int64_t)t * p.q_st + (int64_t)head * p.q_sh + 8 * (lane ^ h), lds_offset(qs + h * kD * 2));
    }
    // finite data that invalid columns load instead of a pool row
    const uint8_t *safe_src = (const uint8_t *)(p.q + (int64_t)t * p.q_st);
    const int32_t *idx_row = p.idx + (int64_t)t * p.idx_st;
    const float sl2 = p.sm_scale_log2;

    // LDS byte offsets: S reads chunk 4s + g of row 16c + l16 (swizzled by
    // rswz(row), the same for both column halves); PV reads rows 4g + l16/4
    // (+16) at head_dim 128w + 16m + 4(l16 % 4)
    const int ksw = rswz(l16);
    const int kb0 = l16 * kD * 2 + 16 * ((0 + g) ^ ksw), kb1 = l16 * kD * 2 + 16 * ((4 + g) ^ ksw);
    int vb[4];
    {
        const int r = 4 * g + (l16 >> 2), vs = rswz(r);
#pragma unroll
        for (int mm = 0; mm < 4; ++mm) {
            const int d = 128 * w + 16 * mm + 4 * (l16 & 3);
            vb[mm] = r * kD * 2 + 16 * ((d >> 3) ^ vs) + 2 * (d & 7);
        }
    }
    // e4m3 tiles: read u of column half c is chunk 4u + g (dims 16(4u + g)
    // .. +15, the K fragments of k-steps 2u and 2u + 1) of row 16c + l16, at
    // slot (4u + g) ^ eswz(row) = 16(u / 4) + (4(u % 4) ^ g ^ l16 ^ 8c).
    // V^T (ds_read_b64_tr_b8): lane l16 of block g addresses row R = 4g +
    // l16/2 (l16 < 8) or 16 + 4g + l16/2 - 4, bytes 8(l16 % 2) .. +7 of chunk
    // 8w + m at slot vy ^ m; result byte k is column R(2k) at head_dim 128w +
    // 16m + l16, the columns of the weights' B-operand layout
    int kbe[2][4], vrow = 0, vy = 0;
    if constexpr (E4) {
#pragma unroll
        for (int c = 0; c < 2; ++c)
#pragma unroll
            for (int u = 0; u < 4; ++u) kbe[c][u] = (16 * c + l16) * kRB + 16 * ((4 * u) ^ g ^ l16 ^ (8 * c));
        const int k = l16 >> 1;
        const int R = k < 4 ? 4 * g + k : 16 + 4 * g + (k - 4);
        vrow = R * kRB + 8 * (l16 & 1);
        vy = (8 * w) ^ eswz(R);
    }

    f32x4 acc[kPM];
#pragma unroll
    for (int m = 0; m < kPM; ++m) acc[m] = f32x4{0.f, 0.f, 0.f, 0.f};
    float m_run = -INFINITY;   // running max of head l16 (the same in every wave)
    float l_run = 0.0f;        // sum of this lane's weights of head l16
    uint4 qf[kD / 32];         // Q as the B operand of S: head l16, dims 32s + 8g .. +7

    uint8_t *const mytile = tiles[w];
    bool first = true;
    // the row indices of this wave's 32 columns (lane < 32 owns column cw +
    // lane); each round's indices load during the round before
    int e_next = -1;
    if (lane < kCW && c_begin + kCW * w + lane < c_end) e_next = idx_row[c_begin + kCW * w + lane];
    for (int c0 = c_begin; c0 < c_end; c0 += kRows) {
        const int cw = c0 + kCW * w;
        const int e = e_next;
        const bool win = cw + lane < p.n_win;
        if (!first) __syncthreads();   // every wave has finished PV of the previous round
        if (lane < kCW) meta[w][0][lane] = e >= 0 ? 0.0f : -INFINITY;
        // gathers: row r of the tile is column cw + r.  Lane r forms the row's
        // address (a stand-in row for an unused column), and each row goes out
        // with that address as a scalar base; chunk j of the row goes to slot
        // j ^ rswz(r).  e4m3: gather q moves rows 2q (lanes 0-31) and 2q + 1
        // (lanes 32-63), lane L filling slot L % 32 of its row, i.e. loading
        // chunk (L % 32) ^ eswz(row)
        const uint8_t *rsrc = E4 ? g_dec_pad_row : safe_src;
        if (e >= 0) rsrc = (win ? p.win : p.cmp) + (int64_t)e * (win ? p.win_rs : p.cmp_rs);
        const uint32_t alo = (uint32_t)(uintptr_t)rsrc, ahi = (uint32_t)((uintptr_t)rsrc >> 32);
        if constexpr (!E4) {
#pragma unroll
            for (int r = 0; r < kCW; ++r) {
                const uint64_t rb = ((uint64_t)(uint32_t)__builtin_amdgcn_readlane((int)ahi, r) << 32) |
                                    (uint32_t)__builtin_amdgcn_readlane((int)alo, r);
                dma_row(rb, 16 * (lane ^ rswz(r)), lds_offset(mytile + r * kD * 2));
            }
        } else {
            const bool hi_half = lane >= 32;
            const int ez = (lane & 31) ^ (lane >> 5);
#pragma unroll
            for (int q = 0; q < kCW / 2; ++q) {
                const uint32_t lo0 = (uint32_t)__builtin_amdgcn_readlane((int)alo, 2 * q);
                const uint32_t hi0 = (uint32_t)__builtin_amdgcn_readlane((int)ahi, 2 * q);
                const uint32_t lo1 = (uint32_t)__builtin_amdgcn_readlane((int)alo, 2 * q + 1);
                const uint32_t hi1 = (uint32_t)__builtin_amdgcn_readlane((int)ahi, 2 * q + 1);
                const uint64_t b = ((uint64_t)(hi_half ? hi1 : hi0) << 32) | (hi_half ? lo1 : lo0);
                const int sw = eswz(2 * q) & ~1;   // eswz(2q + h) = sw ^ h
                dma16((const void *)(b + 16u * (uint32_t)(ez ^ sw)), lds_offset(mytile + 2 * q * kRB));
            }
        }
        // e4m3: the row scales (unused columns 0), loaded after the gathers
        // so the wait for q below counts them out
        float scl = 0.0f;
        if constexpr (E4) {
            if (lane < kCW && e >= 0) scl = (win ? p.win_scale : p.cmp_scale)[e];
        }
        e_next = -1;
        if (lane < kCW && cw + kRows + lane < c_end) e_next = idx_row[cw + kRows + lane];
        if (first) {
            // q has landed in every wave (each waits for its own DMAs, the
            // barrier publishes them); read the fragments while the rows fly.
            // e4m3: step s = 2u + h takes dims 16(4u + g) + 8h .. +7 (the
            // order of the K reads), chunk 8u + 2g + h of the q row
            if constexpr (!E4) wait_vm<kCW>();
            else wait_vm<kCW / 2>();
            __syncthreads();
            const uint8_t *qrow = qs + l16 * kD * 2;
#pragma unroll
            for (int s = 0; s < kD / 32; ++s) {
                const int qc = E4 ? 8 * (s >> 1) + 2 * g + (s & 1) : 4 * s + g;
                qf[s] = lds_b128(qrow + 16 * (qc ^ l16));
            }
            first = false;
        }
        wait_vm<0>();
        if constexpr (E4) {
            if (lane < kCW) meta[w][1][lane] = scl;
        }

        // S^T of the wave's columns 16c + 4g + i, heads hbase + l16
        f32x4 sacc[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
        if constexpr (!E4) {
#pragma unroll
            for (int s = 0; s < kD / 32; ++s) {
                const int off = 128 * (s >> 1) + ((s & 1) ? kb1 : kb0);
                const uint4 k0 = lds_b128(mytile + off), k1 = lds_b128(mytile + 16 * kD * 2 + off);
                sacc[0] = mfma16x16x32(k0, qf[s], sacc[0]);
                sacc[1] = mfma16x16x32(k1, qf[s], sacc[1]);
            }
        } else {
#pragma unroll
            for (int u = 0; u < kD / 64; ++u) {
                const uint4 r0 = lds_b128(mytile + kbe[0][u & 3] + 256 * (u >> 2));
                const uint4 r1 = lds_b128(mytile + kbe[1][u & 3] + 256 * (u >> 2));
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    const uint4 k0 = e4m3x8_to_bf16x8(h ? make_uint2(r0.z, r0.w) : make_uint2(r0.x, r0.y));
                    const uint4 k1 = e4m3x8_to_bf16x8(h ? make_uint2(r1.z, r1.w) : make_uint2(r1.x, r1.y));
                    sacc[0] = mfma16x16x32(k0, qf[2 * u + h], sacc[0]);
                    sacc[1] = mfma16x16x32(k1, qf[2 * u + h], sacc[1]);
                }
            }
        }
        // scores (log2 domain; e4m3: + e of the column's scale s = mu * 2^e)
        float x[2][4], cmu[2][4];
        int cne[2][4];
        float mx = -INFINITY;
#pragma unroll
        for (int c = 0; c < 2; ++c) {
            const float4 b4 = *(const float4 *)&meta[w][0][16 * c + 4 * g];
            const float bb[4] = {b4.x, b4.y, b4.z, b4.w};
            float ss[4] = {1.0f, 1.0f, 1.0f, 1.0f};
            if constexpr (E4) {
                const float4 s4 = *(const float4 *)&meta[w][1][16 * c + 4 * g];
                ss[0] = s4.x; ss[1] = s4.y; ss[2] = s4.z; ss[3] = s4.w;
            }
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                float v = sacc[c][i] * sl2;
                if constexpr (E4) {
                    const int ex = __builtin_amdgcn_frexp_expf(ss[i]);
                    cmu[c][i] = __builtin_amdgcn_frexp_mantf(ss[i]);
                    cne[c][i] = -ex;
                    v = __builtin_fmaf(sacc[c][i], ss[i] * sl2, (float)ex);
                }
                x[c][i] = v + bb[i];
                mx = fmaxf(mx, x[c][i]);
            }
        }
        mx = group4_max(mx);
        if (g == 0) xm[w][l16] = mx;
        __syncthreads();   // maxima and every wave's rows published
        const float mt = fmaxf(fmaxf(xm[0][l16], xm[1][l16]), fmaxf(xm[2][l16], xm[3][l16]));
        const float m_new = fmaxf(m_run, mt);
        const float alpha = m_new == m_run ? 1.0f : fast_exp2(m_run - m_new);   // m_run = -inf: 0
        const float msub = m_new == -INFINITY ? 0.0f : m_new;
        m_run = m_new;
        float pr[2][4], psum = 0.0f;
#pragma unroll
        for (int c = 0; c < 2; ++c)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                pr[c][i] = fast_exp2(x[c][i] - msub);
                psum += E4 ? __builtin_amdgcn_ldexpf(pr[c][i], cne[c][i]) : pr[c][i];
            }
        l_run = l_run * alpha + psum;
        if (__builtin_amdgcn_ballot_w64(alpha != 1.0f) != 0) {
#pragma unroll
            for (int m = 0; m < kPM; ++m) acc[m] *= alpha;
        }
        // this wave's weights in the B-operand layout: element 4c + i of lane
        // (g, l16) is column 16c + 4g + i (e4m3: mu exp2(x - m) = p * s as
        // two f16 terms)
        if constexpr (!E4) {
            xp[0][w][lane] = make_uint4(pack_bf16x2(pr[0][0], pr[0][1]), pack_bf16x2(pr[0][2], pr[0][3]),
                                        pack_bf16x2(pr[1][0], pr[1][1]), pack_bf16x2(pr[1][2], pr[1][3]));
        } else {
            uint32_t hi[4], lo[4];
#pragma unroll
            for (int c = 0; c < 2; ++c)
#pragma unroll
                for (int h = 0; h < 2; ++h)
                    split_f16x2(pr[c][2 * h] * cmu[c][2 * h], pr[c][2 * h + 1] * cmu[c][2 * h + 1], hi[2 * c + h],
                                lo[2 * c + h]);
            xp[0][w][lane] = make_uint4(hi[0], hi[1], hi[2], hi[3]);
            xp[1][w][lane] = make_uint4(lo[0], lo[1], lo[2], lo[3]);
        }
        __syncthreads();   // every wave's weights published
        // O^T[128w + 16m + 4g + i][head l16] += sum over the round's 128 columns
#pragma unroll
        for (int wb = 0; wb < kWv; ++wb) {
            uint4 pb[NP];
#pragma unroll
            for (int ep = 0; ep < NP; ++ep) pb[ep] = xp[ep][wb][lane];
            const uint8_t *bt = tiles[wb];
#pragma unroll
            for (int m = 0; m < kPM; ++m) {
                if constexpr (!E4) {
                    const uint2 v0 = lds_tr16(bt + vb[m & 3] + 128 * (m >> 2));
                    const uint2 v1 = lds_tr16(bt + vb[m & 3] + 16 * kD * 2 + 128 * (m >> 2));
                    const uint4 a = make_uint4(v0.x, v0.y, v1.x, v1.y);
                    acc[m] = mfma16x16x32(a, pb[0], acc[m]);
                } else {
                    const uint4 a = e4m3x8_to_f16x8(lds_tr8(bt + vrow + 16 * (vy ^ m)));
                    const f16x8 av = __builtin_bit_cast(f16x8, a);
                    acc[m] = __builtin_amdgcn_mfma_f32_16x16x32_f16(av, __builtin_bit_cast(f16x8, pb[0]), acc[m], 0, 0, 0);
                    acc[m] = __builtin_amdgcn_mfma_f32_16x16x32_f16(av, __builtin_bit_cast(f16x8, pb[1]), acc[m], 0, 0, 0);
                }
            }
        }
    }

    // softmax sums: over the lane groups, then over the waves in a fixed order
    {
        const float ls = group4_sum(l_run);
        if (g == 0) xl[w][l16] = ls;
    }
    if (!E4 && p.num_splits > 1) {
        // a split's partial goes out in f16 scaled by a power of two: the
        // largest |O| of each head (over the waves' head_dim quarters)
        float mx = 0.0f;
#pragma unroll
        for (int m = 0; m < kPM; ++m)
            mx = fmaxf(fmaxf(mx, fmaxf(fabsf(acc[m][0]), fabsf(acc[m][1]))), fmaxf(fabsf(acc[m][2]), fabsf(acc[m][3])));
        mx = group4_max(mx);
        if (g == 0) xa[w][l16] = mx;
    }
    __syncthreads();
    const float l_tot = (xl[0][l16] + xl[1][l16]) + (xl[2][l16] + xl[3][l16]);
    const int head = hbase + l16;
    if (head >= p.H) return;
    const int d0 = 128 * w + 4 * g;
    if (p.num_splits == 1) {
        const float inv = l_tot > 0.0f ? 1.0f / l_tot : 0.0f;
        if constexpr (OUT == 1) {
            float *o = (float *)p.out + (int64_t)t * p.out_st + (int64_t)head * p.out_sh + d0;
#pragma unroll
            for (int m = 0; m < kPM; ++m) {
                const f32x4 v = acc[m] * inv;
                *(float4 *)(o + 16 * m) = make_float4(v[0], v[1], v[2], v[3]);
            }
        } else {
            uint16_t *o = (uint16_t *)p.out + (int64_t)t * p.out_st + (int64_t)head * p.out_sh + d0;
#pragma unroll
            for (int m = 0; m < kPM; ++m) {
                const f32x4 v = acc[m] * inv;
                *(uint2 *)(o + 16 * m) = make_uint2(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]));
            }
        }
    } else if constexpr (!E4) {
        // bf16 rows: partial outputs in f16, in the accumulators' own layout
        // [unit][head group][w][m][lane] x 4 halves (each store instruction
        // writes 512 consecutive bytes).  The head's O and sum are scaled by
        // 2^sh and its max lowered by sh, which leaves every merge weight
        // 2^(m - M) O and 2^(m - M) l unchanged: sh puts the largest |O| in
        // [2^14, 2^15) (f16 keeps 11 significant bits of it, normal down to
        // 2^-28 of it) unless the scaled sum would pass 2^120 or sh would
        // pass 100 (O that small is below anything its f16 terms could
        // matter for).  The f16 rounding, at most 8 in those units (2^-11 of
        // the head's largest |O|), is below that of the bf16 weights (2^-9
        // of each).
        const float mx = fmaxf(fmaxf(xa[0][l16], xa[1][l16]), fmaxf(xa[2][l16], xa[3][l16]));
        const int sh = min(min(15 - __builtin_amdgcn_frexp_expf(mx), 120 - __builtin_amdgcn_frexp_expf(l_tot)), 100);
        const int64_t pb = ((int64_t)sl.u * G + sl.g) * kWv + w;
        uint16_t *po = (uint16_t *)p.part_o;
#pragma unroll
        for (int m = 0; m < kPM; ++m)
            *(uint2 *)(po + ((pb * kPM + m) * 64 + lane) * 4) =
                make_uint2(pack_f16x2(__builtin_amdgcn_ldexpf(acc[m][0], sh), __builtin_amdgcn_ldexpf(acc[m][1], sh)),
                           pack_f16x2(__builtin_amdgcn_ldexpf(acc[m][2], sh), __builtin_amdgcn_ldexpf(acc[m][3], sh)));
        if (w == 0 && g == 0)
            *(float2 *)(p.part_ml + ((int64_t)sl.u * p.H + head) * 2) =
                make_float2(m_run - (float)sh, __builtin_amdgcn_ldexpf(l_tot, sh));
    } else {
        // e4m3 rows: partial outputs in fp32 (their values reach 448 times
        // the largest scale, where f16's 11 bits would not meet an absolute
        // bound), same layout with 4 floats per lane (1 KiB per store)
        const int64_t pb = ((int64_t)sl.u * G + sl.g) * kWv + w;
#pragma unroll
        for (int m = 0; m < kPM; ++m)
            *(float4 *)(p.part_o + ((pb * kPM + m) * 64 + lane) * 4) =
                make_float4(acc[m][0], acc[m][1], acc[m][2], acc[m][3]);
        if (w == 0 && g == 0) *(float2 *)(p.part_ml + ((int64_t)sl.u * p.H + head) * 2) = make_float2(m_run, l_tot);
    }
}

// out[t, h, :] = sum_j 2^(m_j - M) O_j / sum_j 2^(m_j - M) l_j over the splits
// j in order; zero when every split was empty.  One wave takes one (token,
// head group, w, m) group of the partial layout: lane l owns head 16g + l%16
// and head_dim 128w + 16m + 4(l/16) .. +3, so its partial loads are 512
// bytes (f16) or 1 KiB (fp32) contiguous per split; the loads of U splits go
// out before any is used.
template <int OUT, int U, int WPB, bool H16>   // WPB waves per workgroup; H16: f16 partials (bf16 rows)
__global__ __launch_bounds__(64 * WPB) void attn_dec_merge_kernel(AttnParams p, int nb)
{
    // block b -> (token t, block y of the token's nb): token t on XCD t % 8,
    // where its partials were written
    const int x = (int)blockIdx.x & 7, r = (int)blockIdx.x >> 3;
    const int t = 8 * (r / nb) + x;
    if (t >= p.T) return;
    const int grp = (r % nb) * WPB + (threadIdx.x >> 6), lane = threadIdx.x & 63;
    const int G = p.hgroups;
    if (grp >= G * kWv * kPM) return;
    const int m = grp % kPM, w = (grp / kPM) % kWv, hg = grp / (kPM * kWv);
    const int head = hg * kDecHeads + (lane & 15);
    if (head >= p.H) return;
    const int d = 128 * w + 16 * m + 4 * (lane >> 4);
    const int S = p.num_splits;
    const int64_t pstride = (int64_t)G * kWv * kPM * 64;   // 4-value slots per unit
    const int64_t po0 = ((int64_t)t * S) * pstride + (int64_t)grp * 64 + lane;
    const float2 *pml = (const float2 *)p.part_ml + ((int64_t)t * S) * p.H + head;
    float M = -INFINITY, L = 0.0f;
    float4 o = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int j0 = 0; j0 < S; j0 += U) {
        float2 ml[U];
        float4 v[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int js = min(j0 + u, S - 1);
            ml[u] = pml[(int64_t)js * p.H];
            if constexpr (H16) {
                const uint2 h = ((const uint2 *)p.part_o)[po0 + (int64_t)js * pstride];
                v[u] = make_float4(f16_lo(h.x), f16_hi(h.x), f16_lo(h.y), f16_hi(h.y));
            } else {
                v[u] = ((const float4 *)p.part_o)[po0 + (int64_t)js * pstride];
            }
        }
        float Mb = M;
#pragma unroll
        for (int u = 0; u < U; ++u) Mb = fmaxf(Mb, ml[u].x);   // repeats of split S-1 change nothing
        if (Mb == -INFINITY) continue;                         // every split so far empty
        const float r = M == -INFINITY ? 0.0f : fast_exp2(M - Mb);
        L *= r;
        o.x *= r; o.y *= r; o.z *= r; o.w *= r;
#pragma unroll
        for (int u = 0; u < U; ++u) {
            if (j0 + u < S) {
                const float wt = fast_exp2(ml[u].x - Mb);
                L += wt * ml[u].y;
                o.x += wt * v[u].x; o.y += wt * v[u].y; o.z += wt * v[u].z; o.w += wt * v[u].w;
            }
        }
        M = Mb;
    }
    const float inv = L > 0.0f ? 1.0f / L : 0.0f;
    if constexpr (OUT == 1) {
        float *dst = (float *)p.out + (int64_t)t * p.out_st + (int64_t)head * p.out_sh + d;
        *(float4 *)dst = make_float4(o.x * inv, o.y * inv, o.z * inv, o.w * inv);
    } else {
        uint16_t *dst = (uint16_t *)p.out + (int64_t)t * p.out_st + (int64_t)head * p.out_sh + d;
        *(uint2 *)dst = make_uint2(pack_bf16x2(o.x * inv, o.y * inv), pack_bf16x2(o.z * inv, o.w * inv));
    }
}

template <int KV, int OUT>
hipError_t launch_dec_t(const AttnParams &p, hipStream_t s)
{
    const int64_t blocks = 8 * (int64_t)p.num_splits * p.hgroups * ((p.T + 7) / 8);
    hipLaunchKernelGGL((attn_dec_kernel<KV, OUT>), dim3((unsigned)blocks), dim3(64 * kWv), 0, s, p);
    return hipGetLastError();
}

template <int OUT, bool H16>
hipError_t launch_dec_merge_t(const AttnParams &p, hipStream_t s)
{
    const int groups = p.hgroups * kWv * kPM;
    // a launch of at most one wave per CU takes one-wave workgroups (its
    // waves land on as many CUs), larger ones four waves per workgroup
    const bool one = (int64_t)p.T * groups <= 256;
    const int nb = one ? groups : (groups + 3) / 4;   // workgroups per token
    const dim3 grid((unsigned)(8 * (int64_t)nb * ((p.T + 7) / 8)));
    auto go = [&](auto u_tag) {
        constexpr int U = decltype(u_tag)::value;
        if (one) hipLaunchKernelGGL((attn_dec_merge_kernel<OUT, U, 1, H16>), grid, dim3(64), 0, s, p, nb);
        else hipLaunchKernelGGL((attn_dec_merge_kernel<OUT, U, 4, H16>), grid, dim3(256), 0, s, p, nb);
    };
    const int S = p.num_splits;
    if (S <= 2) go(std::integral_constant<int, 2>{});
    else if (S <= 4) go(std::integral_constant<int, 4>{});
    else if (S <= 8) go(std::integral_constant<int, 8>{});
    else go(std::integral_constant<int, 16>{});
    return hipGetLastError();
}

}  // namespace

hipError_t launch_attn_dec(const AttnParams &p, int kv, int out, hipStream_t s)
{
    if (kv == 0) return out == 1 ? launch_dec_t<0, 1>(p, s) : launch_dec_t<0, 0>(p, s);
    return out == 1 ? launch_dec_t<2, 1>(p, s) : launch_dec_t<2, 0>(p, s);
}

hipError_t launch_attn_dec_merge(const AttnParams &p, int kv, int out, hipStream_t s)
{
    if (kv == 0) return out == 1 ? launch_dec_merge_t<1, true>(p, s) : launch_dec_merge_t<0, true>(p, s);
    return out == 1 ? launch_dec_merge_t<1, false>(p, s) : launch_dec_merge_t<0, false>(p, s);
}

}  // namespace sap
