// attn_d512.hip -- top-k sparse attention over bf16 or e4m3 pools at
// head_dim 512, one workgroup barrier per 32-column tile.
//
// What is computed is the same as in attn.hip ("perf(kernel): keep 16-byte kv
// loads in dsv4 sparse attention and unroll gated pool", Call paths / Kernel
// time): query token t's H heads share one KV head and attend to the columns
// of idx[t, :]; column c reads one row of the window pool (c < n_win) or of
// the compressed pool, and that row is both key and value.
//
// One workgroup = 4 waves, one per SIMD with up to 512 registers each, =
// up to 64 heads of one token over all of its columns (one split per token:
// the prefill launch), in tiles of 32 columns:
//  - S: wave w = (hg, cs) = (w & 1, w >> 1) computes S^T = K Q^T for columns
//    16cs .. 16cs+15 and heads 32hg .. 32hg+31 over all 512 dims on MFMA
//    16x16x32 bf16; its 32 heads' Q fragments stay in 128 registers, so no
//    partial score crosses waves.
//  - softmax (log2 domain): the same wave owns those scores.  Its weights go
//    to LDS as bf16 in the PV B-operand layout, double-buffered by tile
//    parity.  The running max of a head only moves when a tile's max exceeds
//    it by more than 32 (weights stay <= 2^32); the first tile of a column
//    range, and any later tile whose max went past the slack, take a slow
//    path in which every wave agrees on the new maxima, O and the sums are
//    rescaled and the weights of that tile are rewritten.
//  - PV: wave w computes O^T = V^T P^T for head_dim 128w .. 128w+127 and all
//    64 heads (128 accumulators); the V^T operand is read from the row-major
//    tile with ds_read_b64_tr_b16.
//  - pipeline: iteration i issues the gathers of tile i+3, computes S of tile
//    i+1, then PV of tile i with the softmax of tile i+1 cut into pieces of a
//    few VALU cycles, one after each PV MFMA (one wave per SIMD issues in
//    order: a piece issues while the MFMA before it runs), and ends with the one barrier that publishes tile i+1's weights
//    and tile i+2's rows.  Tile i's slow path, when taken, runs at the start
//    of iteration i (after the first K reads of S are issued), so PV's
//    weights and first V^T fragments can be read under the last S steps.
//  - gathers: each wave moves 8 rows of a tile straight into LDS
//    (global_load_lds_dwordx4 with a scalar row base and a per-lane 32-bit
//    offset; one instruction = one 1 KiB row); the 8 row bases come from one
//    LDS read and a few vector instructions per tile.
//
// e4m3 rows (E4; "Perf/kv fp8 read path", What this changes): the tiles hold
// the raw codes (512 B per row, two rows per gather instruction, and one
// more instruction per wave and tile brings the rows' fp32 scales).  S widens
// each K fragment to bf16 in registers (exact) and multiplies the scores by
// the row scale; PV reads V^T fragments with ds_read_b64_tr_b8 and widens
// them to f16 (exact).  The scaled weights p * s enter PV as two f16 terms
// (hi + lo, relative error about 2^-22): with s = mu * 2^e (|mu| in
// [0.5, 1)), e is added to the log2 score, so the running max bounds every
// |p * s| by 2^kE4Slack whatever the scale, and the softmax sum takes
// p = exp2(x + e - m) * 2^-e exactly.
#include "common.hpp"
#include "internal.hpp"
#include "attn_common.hpp"
#include "formats.hpp"

#include <type_traits>
#include <utility>

namespace sap {
namespace {

using namespace attn;

constexpr int kD = 512;
constexpr int kNW = 4;                        // waves
constexpr int kNT = 64 * kNW;                 // threads
constexpr int kDepth = 4;                     // LDS tiles: PV(i), S(i+1), tile i+2 landing, tile i+3 gathering
constexpr int kRW = kAttnTile / kNW;          // gather rows per wave per tile
constexpr int kSK = kD / 32;                  // S k-steps over the full head_dim
constexpr int kPM = kD / (16 * kNW);          // PV m-steps over a wave's head_dim quarter
// e4m3 rows: the weights' f16 terms stay below 2^kE4Slack in magnitude,
// inside the f16 range
constexpr float kE4Slack = 12.0f;

// what padding columns of e4m3 tiles gather instead of a pool row (and its
// scale): zeros, so their values are finite (another stand-in's bytes, read
// as e4m3, could hold the NaN codes, and a zero weight times NaN is NaN)
__device__ __attribute__((aligned(16))) uint8_t g_e4m3_pad_row[kD];

// bytes of one LDS row and tile, and gather instructions per wave and tile
template <bool E4> constexpr int row_bytes() { return E4 ? kD : 2 * kD; }
template <bool E4> constexpr int tile_bytes() { return kAttnTile * row_bytes<E4>(); }
template <bool E4> constexpr int gathers_per_tile() { return E4 ? kRW / 2 + 1 : kRW; }

// lane l moves 16 bytes from base + voff into LDS at lds + 16 l.  The scalar
// base may come from v_readlane, so the wait states a vector memory
// instruction needs after a VALU write of its scalar operand are inserted
// here (the compiler does not see into the assembly).
__device__ __forceinline__ void dma_row(uint64_t base, uint32_t voff, uint32_t lds)
{
    asm volatile("s_mov_b32 m0, %2\n\t"
                 "s_nop 4\n\t"
                 "global_load_lds_dwordx4 %0, %1"
                 :: "v"(voff), "s"(base), "s"(lds) : "memory", "m0");
}

// 4 bytes per lane from global memory into LDS at lds_addr + 4 * lane
// (global_load_lds_dword), untracked like dma16
__device__ __forceinline__ void dma4(const void *src, uint32_t lds_addr)
{
    const uint32_t m = __builtin_amdgcn_readfirstlane(lds_addr);
    asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dword %0, off"
                 :: "v"(src), "s"(m) : "memory", "m0");
}

// MFMA 16x16x32 bf16 with the register classes pinned: O's 128 accumulators
// in AGPRs, the 128 registers of Q (the B operand of S) in AGPRs, everything
// the VALU touches in VGPRs.  Left to the register allocator, both O and Q
// compete for the AGPRs and values are copied back and forth around every
// MFMA.  The compiler's hazard tracking does not see into these statements,
// so: operands come straight from LDS loads (waited for by the compiler); the
// first S step of a chain starts from 0 rather than from a register the VALU
// wrote; the VALU reads S only after explicit wait states (s_wait_mfma); and
// O is read only after the tile loop, behind explicit wait states.
__device__ __forceinline__ void mfma_acc(f32x4 &c, const uint4 &a, const uint4 &b)
{
    asm("v_mfma_f32_16x16x32_bf16 %0, %1, %2, %0" : "+a"(c) : "v"(as_bf16x8(a)), "v"(as_bf16x8(b)));
}
__device__ __forceinline__ f32x4 mfma_s_first(const uint4 &a, const bf16x8 &b)
{
    f32x4 c;
    asm("v_mfma_f32_16x16x32_bf16 %0, %1, %2, 0" : "=&v"(c) : "v"(as_bf16x8(a)), "a"(b));
    return c;
}
__device__ __forceinline__ void mfma_s(f32x4 &c, const uint4 &a, const bf16x8 &b)
{
    asm("v_mfma_f32_16x16x32_bf16 %0, %1, %2, %0" : "+v"(c) : "v"(as_bf16x8(a)), "a"(b));
}
// the e4m3 PV step: O (AGPRs) += V^T (f16) P^T (one f16 term of the weights).
// V^T comes from a VALU conversion, made a whole m-step (eight MFMAs) before
// the MFMAs that read it.
__device__ __forceinline__ void mfma_acc_f16(f32x4 &c, const uint4 &a, const uint4 &b)
{
    asm("v_mfma_f32_16x16x32_f16 %0, %1, %2, %0"
        : "+a"(c) : "v"(__builtin_bit_cast(f16x8, a)), "v"(__builtin_bit_cast(f16x8, b)));
}
// a 4-byte global load the compiler does not track (it issues no wait for
// it): the value is only read through vm_wait4 below
__device__ __forceinline__ int gload_untracked(const int32_t *src)
{
    int v;
    asm volatile("global_load_dword %0, %1, off" : "=v"(v) : "v"(src) : "memory");
    return v;
}
// at most N vector memory operations in flight, then the four values loaded
// by gload_untracked are ready (they pass through this statement, so no use
// can be scheduled above it)
template <int N>
__device__ __forceinline__ void vm_wait4(int (&v)[4])
{
    asm volatile("s_waitcnt vmcnt(%4)" : "+v"(v[0]), "+v"(v[1]), "+v"(v[2]), "+v"(v[3]) : "n"(N) : "memory");
}

// 16 bytes from LDS at addr + OFF straight into AGPRs (Q); the caller waits
// with s_waitcnt lgkmcnt(0) before the first use
template <int OFF>
__device__ __forceinline__ bf16x8 lds_b128_agpr(uint32_t addr)
{
    bf16x8 v;
    asm volatile("ds_read_b128 %0, %1 offset:%2" : "=a"(v) : "v"(addr), "n"(OFF) : "memory");
    return v;
}
// x, opaque to the compiler: values derived from it inside a loop are formed
// there instead of being hoisted out and kept live across the loop
__device__ __forceinline__ int opaque(int x)
{
    asm volatile("" : "+v"(x));
    return x;
}
// Q fragments s of head rows 32hg + 16jj + l16 (jj = 0, 1): qa[s % 4] + the
// immediate offset of head tile jj and of chunk group s / 4
template <size_t... S>
__device__ __forceinline__ void load_q_frags(bf16x8 (&qf)[2][kSK], const uint32_t (&qa)[4], std::index_sequence<S...>)
{
    ((qf[0][S] = lds_b128_agpr<256 * (S / 4)>(qa[S % 4])), ...);
    ((qf[1][S] = lds_b128_agpr<16 * 2 * kD + 256 * (S / 4)>(qa[S % 4])), ...);
}
// v, materialised here: a conversion that produces an MFMA operand is kept
// where it is written instead of being sunk (or recomputed) next to the
// inline-assembly MFMA that reads it, whose hazard the compiler cannot see
__device__ __forceinline__ void pin(uint4 &v)
{
    asm volatile("" : "+v"(v.x), "+v"(v.y), "+v"(v.z), "+v"(v.w));
}

// wait states between an MFMA's last write of a VGPR and a VALU read of it
__device__ __forceinline__ void s_wait_mfma() { asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 3" ::: "memory"); }


template <int OUT, bool E4>
__global__ __attribute__((amdgpu_flat_work_group_size(kNT, kNT), amdgpu_waves_per_eu(1, 1)))
void attn_d512_kernel(AttnParams p)
{
    constexpr int kRB = row_bytes<E4>(), kTB = tile_bytes<E4>(), kGI = gathers_per_tile<E4>();
    constexpr float kSlack = E4 ? kE4Slack : kRescaleSlack;
    // sizes of the e4m3-only arrays below (one element for bf16 rows)
    constexpr int kQS = E4 ? kAttnHeadsPerBlock * 2 * kD : 16, kSC = E4 ? kDepth : 1, kXQ = E4 ? 2 : 1;
    __shared__ __attribute__((aligned(1024))) uint8_t tiles[kDepth][kTB];
    // e4m3: the q rows' own staging area (bf16: tiles 2 and 3)
    __shared__ __attribute__((aligned(1024))) uint8_t qsep[kQS];
    // e4m3: each tile's row scales; wave w's area holds rows 8w .. 8w+7,
    // eight times over (one dword per lane of its scale gather)
    __shared__ __attribute__((aligned(16))) float sc[kSC][kNW][64];
    __shared__ __attribute__((aligned(16))) int sidx[kIdxChunk];
    __shared__ int xscan[kNW];
    // weights by [tile parity][head tile][column half][lane]: lane l of
    // column half c holds columns 16c + 4(l/16) .. +3 of head 16 j + l%16, so a
    // PV lane reads its B operand (8 columns) with one ds_read2_b64.  bf16
    // weights, or for e4m3 rows the high f16 terms of p * s (xq: the low ones)
    __shared__ uint2 xp[2][4][2][64];
    __shared__ uint2 xq[kXQ][4][2][64];
    // per tile (ring of 3): some wave saw a max beyond the slack.  Tile k's
    // word is set during iteration k-1, read in iteration k and cleared in
    // iteration k+1, before tile k+3 uses it again.
    __shared__ int xf[3];
    __shared__ float xm[kNW][32];     // tile maxima of each wave's 32 heads (slow path)
    __shared__ float xl[kNW][32];     // softmax sums at the end

    // Tokens of this workgroup (all of a token's columns, one head block).
    // A grid of fewer workgroups than tokens is persistent and XCD-aware:
    // the grid takes the tokens in rounds of gridDim.x, and in each round
    // XCD x = blockIdx.x % 8 takes the 1/8 block of consecutive tokens
    // x per .. x per + per - 1 (per = its workgroup count), so consecutive
    // tokens (which share window rows) run at the same time on one XCD's
    // L2, and every XCD gets tokens from the whole range (early tokens have
    // fewer columns: contiguous eighths of the range left the XCD with the
    // last eighth working longest).
    int t0 = blockIdx.x, tstep = 1, tend = blockIdx.x + 1;
    if ((int)gridDim.x < p.T) {
        const int x = blockIdx.x & 7, per = (int)gridDim.x >> 3;
        t0 = x * per + (blockIdx.x >> 3);
        tend = p.T;
        tstep = (int)gridDim.x;
    }
    const int c_begin = 0, c_end = p.n_cols;

    const int tid = threadIdx.x;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63, l16 = lane & 15, g = lane >> 4;
    const int hg = w & 1, cs = w >> 1;
    const int hbase = blockIdx.y * kAttnHeadsPerBlock;
    const uint32_t tiles_lds = lds_offset(&tiles[0][0]);

    // The block's 64 q rows land in tiles 2 and 3 (e4m3: in qsep) with
    // whole-row LDS DMA (16-byte chunk c of head row h at slot c ^ (h & 15));
    // tiles 0 and 1 stay free for the first gathers.
    uint8_t *const qstage = E4 ? &qsep[0] : &tiles[2][0];
    // (h & 15 takes four values per wave, so four per-lane offsets serve
    // all 16 heads of a wave)
    auto stage_q = [&](int tq) __attribute__((always_inline)) {
        const int ln = opaque(lane);
        uint32_t voff[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) voff[k] = 16u * (uint32_t)(ln ^ (kNW * k + w));
#pragma unroll
        for (int k = 0; k < kAttnHeadsPerBlock / kNW; ++k) {
            const int h = kNW * k + w;
            const int head = hbase + h < p.H ? hbase + h : hbase;   // rows past H: finite stand-in
            const uint64_t src = (uint64_t)(p.q + (int64_t)tq * p.q_st + (int64_t)head * p.q_sh);
            dma_row(src, voff[k & 3], lds_offset(qstage + 1024 * h));
        }
    };

    const uint8_t *const win_pool = p.win, *const cmp_pool = p.cmp;
    const int64_t win_rs = p.win_rs, cmp_rs = p.cmp_rs;
    const int n_win = p.n_win;
    const float sl2 = p.sm_scale_log2;
    // finite bytes that padding columns of bf16 tiles load instead of a pool
    // row (their scores are -inf and their weights 0; e4m3 tiles take
    // g_e4m3_pad_row)
    int t = t0;
    uint64_t safe_src = 0;
    const int32_t *idx_row = nullptr;

    // Column staging: a chunk's valid columns are packed to the front of sidx
    // in column order; each entry is its pool row, bit 31 set for the
    // compressed pool; -1 pads the last tile.  4 consecutive columns per
    // thread per batch.
    int nval = 0, n_tiles = 0;
    auto load4 = [&](int cbase, int cn, int i0, int (&iv)[4]) __attribute__((always_inline)) {
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int i = i0 + 4 * tid + u;
            iv[u] = i < cn ? idx_row[cbase + i] : -1;
        }
    };
    auto stage4 = [&](int cbase, int i0, const int (&iv)[4]) __attribute__((always_inline)) {
        int cnt = 0;
#pragma unroll
        for (int u = 0; u < 4; ++u) cnt += iv[u] >= 0 ? 1 : 0;
        const int incl = wave_incl_sum(cnt);
        if (lane == 63) xscan[w] = incl;
        __syncthreads();
        int before = 0, tot = 0;
#pragma unroll
        for (int k = 0; k < kNW; ++k) {
            const int v = xscan[k];
            before += k < w ? v : 0;
            tot += v;
        }
        int at = nval + before + incl - cnt;
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            if (iv[u] >= 0) {
                const bool win = cbase + i0 + 4 * tid + u < n_win;
                sidx[at++] = win ? iv[u] : (int)((uint32_t)iv[u] | 0x80000000u);
            }
        }
        nval += tot;
        __syncthreads();   // xscan is rewritten by the next batch
    };
    auto pad = [&]() __attribute__((always_inline)) {
        n_tiles = (nval + kAttnTile - 1) / kAttnTile;
        for (int i = nval + tid; i < n_tiles * kAttnTile; i += kNT) sidx[i] = -1;
    };

    // gathers of a tile: lane k < 8 resolves the wave's row 8w + k from its
    // staged entry (row_bases), then each row goes out as one instruction
    // (gather_row).  Tile row rho holds chunk j at slot j ^ rswz(rho), and
    // rswz(8w + q) = rswz(q).
    struct RowBases {
        int lo, hi;
    };
    auto row_entry = [&](int tile) __attribute__((always_inline)) {
        return sidx[tile * kAttnTile + kRW * w + (lane & 7)];
    };
    auto row_bases = [&](int e) __attribute__((always_inline)) {
        const bool ok = e != -1, win = e >= 0;
        const uint64_t r = (uint32_t)e & 0x7FFFFFFFu;
        const uint64_t rb = (uint64_t)(win ? win_pool : cmp_pool) + r * (uint64_t)(win ? win_rs : cmp_rs);
        const uint64_t base = ok ? rb : E4 ? (uint64_t)&g_e4m3_pad_row[0] : safe_src;
        return RowBases{(int)(uint32_t)base, (int)(uint32_t)(base >> 32)};
    };
    // e4m3: gather q moves rows 2q (lanes 0-31) and 2q+1 (lanes 32-63) of
    // the wave's 8; lane L fills slot L % 32 of its row, so it loads chunk
    // (L % 32) ^ eswz(row) = ez ^ 2q
    const bool hi_half = lane >= 32;
    const int ez = (lane & 31) ^ (lane >> 5) ^ (((w ^ (w >> 1)) & 1) << 3);
    auto gather_row = [&](const RowBases &rb, int buf, int q) __attribute__((always_inline)) {
        if constexpr (!E4) {
            const uint64_t b = ((uint64_t)(uint32_t)__builtin_amdgcn_readlane(rb.hi, q) << 32) |
                               (uint32_t)__builtin_amdgcn_readlane(rb.lo, q);
            dma_row(b, 16u * (uint32_t)(lane ^ rswz(q)), tiles_lds + (uint32_t)(buf * kTB + (kRW * w + q) * kRB));
        } else {
            const uint32_t lo0 = (uint32_t)__builtin_amdgcn_readlane(rb.lo, 2 * q);
            const uint32_t hi0 = (uint32_t)__builtin_amdgcn_readlane(rb.hi, 2 * q);
            const uint32_t lo1 = (uint32_t)__builtin_amdgcn_readlane(rb.lo, 2 * q + 1);
            const uint32_t hi1 = (uint32_t)__builtin_amdgcn_readlane(rb.hi, 2 * q + 1);
            const uint64_t b = ((uint64_t)(hi_half ? hi1 : hi0) << 32) | (hi_half ? lo1 : lo0);
            dma16((const void *)(b + 16u * (uint32_t)(ez ^ (2 * q))),
                  tiles_lds + (uint32_t)(buf * kTB + (kRW * w + 2 * q) * kRB));
        }
    };
    // e4m3: lane L brings the scale of the wave's row L % 8 (entry e)
    auto gather_scales = [&](int e, int buf) __attribute__((always_inline)) {
        const bool ok = e != -1, win = e >= 0;
        const float *sp = (win ? p.win_scale : p.cmp_scale) + ((uint32_t)e & 0x7FFFFFFFu);
        dma4(ok ? (const void *)sp : (const void *)&g_e4m3_pad_row[0], lds_offset(&sc[buf][w][0]));
    };
    auto gather = [&](int buf, int tile) __attribute__((always_inline)) {
        const int e = row_entry(tile);
        const RowBases rb = row_bases(e);
        if constexpr (!E4) {
#pragma unroll
            for (int q = 0; q < kRW; ++q) gather_row(rb, buf, q);
        } else {
#pragma unroll
            for (int q = 0; q < kRW / 2; ++q) gather_row(rb, buf, q);
            gather_scales(e, buf);
        }
    };

    // S^T k-step s of this wave: row 16cs + l16, 16-byte chunk 4s + g.
    // e4m3: one 16-byte read u = chunk 4u + g (dims 16(4u + g) .. +15) holds
    // the K fragments of k-steps 2u and 2u + 1; its slot is (4u + g) ^
    // eswz(row) = 16(u / 4) + (4(u % 4) ^ g ^ l16 ^ 8cs)
    int kb[E4 ? 4 : 2];
    if constexpr (!E4) {
        const int rho = 16 * cs + l16, sw = rswz(rho);
#pragma unroll
        for (int e = 0; e < 2; ++e) kb[e] = rho * 2 * kD + 16 * ((4 * e + g) ^ sw);
    } else {
        const int rho = 16 * cs + l16, X = g ^ l16 ^ (8 * cs);
#pragma unroll
        for (int u = 0; u < 4; ++u) kb[u] = rho * kRB + 16 * ((4 * u) ^ X);
    }
    // V^T fragments of PV m-step m: rows 4g + l16/4 (+16) at head_dim
    // 128w + 16m + 4(l16 % 4).  e4m3 (ds_read_b64_tr_b8): lane l16 of block
    // g addresses row R = 4g + l16/2 (l16 < 8) or 16 + 4g + l16/2 - 4, bytes
    // 8(l16 % 2) .. +7 of chunk 8w + m, whose slot is vy ^ m; result byte k
    // is then column R(2k) at head_dim 128w + 16m + l16
    int vb[E4 ? 1 : 4];
    int vrow = 0, vy = 0;
    if constexpr (!E4) {
        const int dsub = 4 * (l16 & 3);
        const int r = 4 * g + (l16 >> 2), vs = rswz(r);
#pragma unroll
        for (int mm = 0; mm < 4; ++mm) {
            const int d = (kD / kNW) * w + 16 * mm + dsub;
            vb[mm] = r * 2 * kD + 16 * ((d >> 3) ^ vs) + 2 * (d & 7);
        }
    } else {
        const int k = l16 >> 1;
        const int R = k < 4 ? 4 * g + k : 16 + 4 * g + (k - 4);
        vrow = R * kRB + 8 * (l16 & 1);
        vy = (8 * w) ^ eswz(R);
        vb[0] = 0;
    }

    // O^T accumulators: acc[m][j] = O^T[d = 128w + 16m + 4g + i][head 16j + l16]
    f32x4 acc[kPM][4];
#pragma unroll
    for (int m = 0; m < kPM; ++m)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[m][j] = f32x4{0.f, 0.f, 0.f, 0.f};
    // running max of heads 16J + l16 (the same in every wave), the maxima of
    // the owned head tiles 2hg + jj, this lane's sums over its columns of the
    // owned heads, and the sums of the last softmax not yet added
    f32x4 m_run = {-INFINITY, -INFINITY, -INFINITY, -INFINITY};
    float m_own[2] = {-INFINITY, -INFINITY}, l_run[2] = {0.f, 0.f}, psum[2] = {0.f, 0.f};
    float x[2][4];   // scores of the last softmax'd tile (log2 domain; -inf for padding)
    // e4m3: the row scale s of each of those columns as s = mu * 2^e (mu 0
    // for padding); x holds score + e, and the weight p * s = exp2(x - m) * mu
    float cmu[E4 ? 4 : 1];
    int cne[E4 ? 4 : 1];   // -e
    // e4m3: the scales of this lane's four columns in tile buffer buf
    auto col_scales = [&](int buf) __attribute__((always_inline)) {
        return *(const float4 *)&sc[buf][2 * cs + (g >> 1)][4 * (g & 1)];
    };
    // e4m3: column i's mu and -e (from its scale sv, 0 for padding); returns
    // the factor and offset of its scores, x = S * sv * sl2 + e
    auto col_prep = [&](float sv, bool ok, int i, float &ks, float &ef) __attribute__((always_inline)) {
        const float sm = ok ? sv : 0.0f;
        const int e = __builtin_amdgcn_frexp_expf(sm);
        cmu[i] = __builtin_amdgcn_frexp_mantf(sm);
        cne[i] = -e;
        ks = sm * sl2;
        ef = (float)e;
    };

    // softmax pieces.  Scores of tile `tile` from the S accumulators
    // (column 16cs + 4g + i of the tile is valid iff i < vmax):
    auto scores = [&](const f32x4 (&sa)[2][2], int tile) __attribute__((always_inline)) {
        const int vmax = nval - tile * kAttnTile - 16 * cs - 4 * g;
        if constexpr (!E4) {
#pragma unroll
            for (int jj = 0; jj < 2; ++jj)
#pragma unroll
                for (int i = 0; i < 4; ++i) x[jj][i] = i < vmax ? (sa[jj][0][i] + sa[jj][1][i]) * sl2 : -INFINITY;
        } else {
            const float4 s4 = col_scales(tile & 3);
            const float sv[4] = {s4.x, s4.y, s4.z, s4.w};
            float ks[4], ef[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) col_prep(sv[i], i < vmax, i, ks[i], ef[i]);
#pragma unroll
            for (int jj = 0; jj < 2; ++jj)
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    x[jj][i] = i < vmax ? __builtin_fmaf(sa[jj][0][i] + sa[jj][1][i], ks[i], ef[i]) : -INFINITY;
        }
    };
    // weights of head tile jj against its owned max: bf16, or for e4m3 rows
    // the f16 terms of p * s (pl: the low terms); psum gets the sum of p
    auto weights_of = [&](int jj, uint2 &pk, uint2 &pl) __attribute__((always_inline)) {
        const float msub = m_own[jj] == -INFINITY ? 0.0f : m_own[jj];
        float pr[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) pr[i] = fast_exp2(x[jj][i] - msub);
        if constexpr (!E4) {
            psum[jj] = (pr[0] + pr[1]) + (pr[2] + pr[3]);
            pk = make_uint2(pack_bf16x2(pr[0], pr[1]), pack_bf16x2(pr[2], pr[3]));
        } else {
            float pp[4], ws[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                pp[i] = __builtin_amdgcn_ldexpf(pr[i], cne[i]);
                ws[i] = pr[i] * cmu[i];
            }
            psum[jj] = (pp[0] + pp[1]) + (pp[2] + pp[3]);
            split_f16x2(ws[0], ws[1], pk.x, pl.x);
            split_f16x2(ws[2], ws[3], pk.y, pl.y);
        }
    };
    auto put_weights = [&](int par, const uint2 (&pk)[2], const uint2 (&pl)[2]) __attribute__((always_inline)) {
#pragma unroll
        for (int jj = 0; jj < 2; ++jj) {
            xp[par][2 * hg + jj][cs][lane] = pk[jj];
            if constexpr (E4) xq[par][2 * hg + jj][cs][lane] = pl[jj];
        }
    };
    auto weights = [&](int par) __attribute__((always_inline)) {
        uint2 pk[2], pl[2];
        weights_of(0, pk[0], pl[0]);
        weights_of(1, pk[1], pl[1]);
        put_weights(par, pk, pl);
    };
    // slow path for the tile whose weights are in xp[par]: every wave agrees
    // on the new maxima, O and the sums are rescaled, the weights rewritten
    auto slow = [&](int par) __attribute__((always_inline)) {
#pragma unroll
        for (int jj = 0; jj < 2; ++jj) {
            const float tm = group4_max(fmaxf(fmaxf(x[jj][0], x[jj][1]), fmaxf(x[jj][2], x[jj][3])));
            if (g == 0) xm[w][16 * jj + l16] = tm;
        }
        __syncthreads();
        float alpha[4];
#pragma unroll
        for (int J = 0; J < 4; ++J) {
            const int o = 16 * (J & 1) + l16;
            const float mt = fmaxf(xm[J >> 1][o], xm[(J >> 1) + 2][o]);
            const float mr = m_run[J];
            const bool up = mt > mr + kSlack;   // also from -inf
            const float mn = up ? mt : mr;
            alpha[J] = up ? fast_exp2(mr - mn) : 1.0f;   // 0 from -inf: O and the sums are still zero
            m_run[J] = mn;
            // (from -inf O is zero: nothing to rescale)
            if (__builtin_amdgcn_ballot_w64(alpha[J] != 1.0f && mr != -INFINITY) != 0) {
#pragma unroll
                for (int m = 0; m < kPM; ++m) agpr_scale(acc[m][J], alpha[J]);
            }
        }
#pragma unroll
        for (int jj = 0; jj < 2; ++jj) {
            const float a = hg ? alpha[2 + jj] : alpha[jj];
            l_run[jj] *= a;
            m_own[jj] = hg ? m_run[2 + jj] : m_run[jj];
        }
        weights(par);
        __syncthreads();
    };

    // Q fragments of S: qf[jj][s] = q[hbase + 32hg + 16jj + l16, 32s + 8g .. +7]
    bf16x8 qf[2][kSK];
    // S^T of the tile in LDS tile `buf`: sa[jj][e] = partial S^T[column 16cs +
    // 4g + i][head 32hg + 16jj + l16] over the k-steps s with s % 2 == e
    // (K fragments are read KD steps ahead; hook(s) runs between the MFMAs)
    auto s_tile = [&](int buf, f32x4 (&sa)[2][2], auto before, auto hook) __attribute__((always_inline)) {
        const uint8_t *bf = &tiles[buf][0];
        if constexpr (!E4) {
            auto kfrag = [&](int s) __attribute__((always_inline)) { return lds_b128(bf + kb[s & 1] + 128 * (s >> 1)); };
            constexpr int KD = 6;
            uint4 f[KD];
#pragma unroll
            for (int s = 0; s + 1 < KD; ++s) f[s] = kfrag(s);
            before();
#pragma unroll
            for (int s = 0; s < kSK; ++s) {
                if (s + KD - 1 < kSK) f[(s + KD - 1) % KD] = kfrag(s + KD - 1);
                __builtin_amdgcn_sched_barrier(0);
                if (s < 2) {
                    sa[0][s] = mfma_s_first(f[s % KD], qf[0][s]);
                    sa[1][s] = mfma_s_first(f[s % KD], qf[1][s]);
                } else {
                    mfma_s(sa[0][s & 1], f[s % KD], qf[0][s]);
                    mfma_s(sa[1][s & 1], f[s % KD], qf[1][s]);
                }
                hook(s);
                __builtin_amdgcn_sched_barrier(0);
            }
        } else {
            // raw reads (two k-steps each) KD - 1 ahead; each step's
            // fragment is widened to bf16 before the MFMAs of the step
            // before it, so its VALU writes lie well ahead of its MFMAs
            auto kraw = [&](int u) __attribute__((always_inline)) { return lds_b128(bf + kb[u & 3] + 256 * (u >> 2)); };
            auto widen = [](const uint4 &r, int h) __attribute__((always_inline)) {
                return e4m3x8_to_bf16x8(h ? make_uint2(r.z, r.w) : make_uint2(r.x, r.y));
            };
            constexpr int KD = 3;
            uint4 f[KD];
#pragma unroll
            for (int u = 0; u + 1 < KD; ++u) f[u] = kraw(u);
            before();
            uint4 a = widen(f[0], 0);
            pin(a);
#pragma unroll
            for (int s = 0; s < kSK; ++s) {
                const int u = s >> 1;
                if ((s & 1) == 0 && u + KD - 1 < kSK / 2) f[(u + KD - 1) % KD] = kraw(u + KD - 1);
                uint4 an = a;
                if (s + 1 < kSK) {
                    an = widen(f[((s + 1) >> 1) % KD], (s + 1) & 1);
                    pin(an);
                }
                __builtin_amdgcn_sched_barrier(0);
                if (s < 2) {
                    sa[0][s] = mfma_s_first(a, qf[0][s]);
                    sa[1][s] = mfma_s_first(a, qf[1][s]);
                } else {
                    mfma_s(sa[0][s & 1], a, qf[0][s]);
                    mfma_s(sa[1][s & 1], a, qf[1][s]);
                }
                hook(s);
                __builtin_amdgcn_sched_barrier(0);
                a = an;
            }
        }
    };
    // O^T += V^T P^T for the tile in LDS tile `buf` with the weights in xp[par].
    // The weights and the first VD - 1 V^T fragments are read ahead (pv_pre,
    // under the MFMAs of the S before it); later V^T fragments are read VD - 1
    // steps ahead; hook(m) runs between the MFMAs.
    constexpr int VD = 3;
    struct PvPre {
        uint4 pb[4];
        uint4 pl[E4 ? 4 : 1];        // e4m3: the low f16 terms
        uint4 vr[E4 ? 1 : VD - 1];   // bf16 V^T fragments
        uint2 vw[E4 ? VD - 1 : 1];   // e4m3 V^T codes
    };
    auto vfrag = [&](int buf, int m) __attribute__((always_inline)) {
        const uint8_t *bf = &tiles[buf][0];
        const uint2 v0 = lds_tr16(bf + vb[m & 3] + 128 * (m >> 2));
        const uint2 v1 = lds_tr16(bf + vb[m & 3] + 16 * 2 * kD + 128 * (m >> 2));
        return make_uint4(v0.x, v0.y, v1.x, v1.y);
    };
    auto vfrag8 = [&](int buf, int m) __attribute__((always_inline)) {
        return lds_tr8(&tiles[buf][0] + vrow + 16 * (vy ^ m));
    };
    auto load_pb = [&](int par, PvPre &pre) __attribute__((always_inline)) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const uint2 a = xp[par][j][0][lane], b = xp[par][j][1][lane];
            pre.pb[j] = make_uint4(a.x, a.y, b.x, b.y);
            if constexpr (E4) {
                const uint2 c = xq[par][j][0][lane], d = xq[par][j][1][lane];
                pre.pl[j] = make_uint4(c.x, c.y, d.x, d.y);
            }
        }
    };
    auto pv_pre = [&](int buf, int par, PvPre &pre) __attribute__((always_inline)) {
        load_pb(par, pre);
        if constexpr (!E4) {
#pragma unroll
            for (int m = 0; m + 1 < VD; ++m) pre.vr[m] = vfrag(buf, m);
        } else {
#pragma unroll
            for (int m = 0; m + 1 < VD; ++m) pre.vw[m] = vfrag8(buf, m);
        }
    };
    auto pv = [&](int buf, const PvPre &pre, auto hook) __attribute__((always_inline)) {
        if constexpr (!E4) {
            uint4 vr[VD];
#pragma unroll
            for (int m = 0; m + 1 < VD; ++m) vr[m] = pre.vr[m];
#pragma unroll
            for (int m = 0; m < kPM; ++m) {
                if (m + VD - 1 < kPM) vr[(m + VD - 1) % VD] = vfrag(buf, m + VD - 1);
                __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    mfma_acc(acc[m][j], vr[m % VD], pre.pb[j]);
                    hook(4 * m + j);
                    __builtin_amdgcn_sched_barrier(0);
                }
            }
        } else {
            // each m-step: the high terms (with the hook pieces between
            // them), then the low terms; the next m-step's V^T is widened to
            // f16 before this one's MFMAs
            uint2 vw[VD];
#pragma unroll
            for (int m = 0; m + 1 < VD; ++m) vw[m] = pre.vw[m];
            uint4 a = e4m3x8_to_f16x8(vw[0]);
            pin(a);
#pragma unroll
            for (int m = 0; m < kPM; ++m) {
                if (m + VD - 1 < kPM) vw[(m + VD - 1) % VD] = vfrag8(buf, m + VD - 1);
                uint4 an = a;
                if (m + 1 < kPM) {
                    an = e4m3x8_to_f16x8(vw[(m + 1) % VD]);
                    pin(an);
                }
                __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    mfma_acc_f16(acc[m][j], a, pre.pb[j]);
                    hook(4 * m + j);
                    __builtin_amdgcn_sched_barrier(0);
                }
#pragma unroll
                for (int j = 0; j < 4; ++j) mfma_acc_f16(acc[m][j], a, pre.pl[j]);
                __builtin_amdgcn_sched_barrier(0);
                a = an;
            }
        }
    };

    // one chunk of columns whose indices are staged in sidx: prologue (tiles
    // 0 .. 2 in flight, S of tile 0), then the tile loop.  Tiles 0 and 1 may
    // have been issued already.
    // full: tiles 0 and 1 were issued before the previous token's 32 output
    // stores and the next token's 4 index loads (the waits for tiles 0 and 1
    // then leave those in flight)
    auto run_chunk = [&](bool issued01, bool full) __attribute__((always_inline)) {
        const int n = n_tiles;
        if (!issued01) {
            gather(0, 0);
            if (n > 1) gather(1, 1);
        }
        if (n > 2) gather(2, 2);
        if (tid < 3) xf[tid] = 0;
        constexpr int kAfter = kPM * 4 + 4;   // stores and index loads after tile 1
        if (full && n > 2) wait_vm<2 * kGI + kAfter>();
        else if (full) wait_vm<kGI + kAfter>();
        else if (n > 2) wait_vm<2 * kGI>();
        else if (n > 1) wait_vm<kGI>();
        else wait_vm<0>();
        __syncthreads();
        {
            f32x4 sa[2][2];
            s_tile(0, sa, [] {}, [](int) {});
            s_wait_mfma();
            scores(sa, 0);   // its maxima are agreed on in the slow path below
        }
        if (full && n > 2) wait_vm<kGI + kAfter>();
        else if (full) wait_vm<kAfter>();
        else if (n > 2) wait_vm<kGI>();
        else wait_vm<0>();
        __syncthreads();
        int f0 = 0, f1 = 1, f2 = 2;   // flag slots of tiles i, i+1, i+2
        // iteration i; G3: tile i+3 exists (its gathers go out), MORE: tile
        // i+1 exists (its S and softmax run).  Peeled so the steady-state
        // iterations have no branches besides the slow path.
        auto body = [&](int i, auto g3_tag, auto more_tag) __attribute__((always_inline)) {
            constexpr bool G3 = decltype(g3_tag)::value, MORE = decltype(more_tag)::value;
            const int fw = xf[f0];
            if (tid == 0) xf[f2] = 0;   // tile i-1's word: tile i+2 sets it next iteration
            // tile i: the first of the chunk, or a max beyond the slack (the
            // slow path rewrites its weights before PV reads them)
            auto check = [&]() __attribute__((always_inline)) {
                const int any = i == 0 ? 1 : __builtin_amdgcn_readfirstlane(fw);
                if (any) slow(i & 1);
            };
            int e3 = -1;
            if constexpr (G3) e3 = row_entry(i + 3);
            f32x4 sa[2][2];
            PvPre pre;
            RowBases rb3{0, 0};
            if constexpr (MORE) {
                // S of tile i+1; the row bases of tile i+3 are resolved after
                // the first k-step and its 8 rows go out spread over S and PV
                // (one every 4 k-steps, then one every 8 PV MFMAs; e4m3: the
                // four row pairs during S, the scales early in PV); PV's
                // first operands are read during the last steps
                s_tile((i + 1) & 3, sa, check, [&](int s) __attribute__((always_inline)) {
                    if constexpr (G3) {
                        if (s == 1) rb3 = row_bases(e3);
                        if ((s & 3) == 2) gather_row(rb3, (i + 3) & 3, s >> 2);
                    }
                    if (s == kSK - 3) pv_pre(i & 3, i & 1, pre);
                });
            } else {
                check();
                pv_pre(i & 3, i & 1, pre);
            }
            l_run[0] += psum[0];
            l_run[1] += psum[1];
            // PV of tile i with the softmax of tile i+1 cut into pieces of a
            // few VALU cycles, one after each MFMA (the pieces issue while
            // the MFMA runs)
            uint2 pk[2], pl[2];
            int fl = 0, vmax = 0;
            float tm[2], msub[2], pr[2][4];
            float4 s4;                    // e4m3: the scales of tile i+1's columns
            float ks[4], ef[4], ws[2][4];
            pv(i & 3, pre, [&](int k) __attribute__((always_inline)) {
                if constexpr (G3) {
                    if constexpr (!E4) {
                        if ((k & 7) == 2) gather_row(rb3, (i + 3) & 3, 4 + (k >> 3));
                    } else {
                        if (k == 2) gather_scales(e3, (i + 3) & 3);
                    }
                }
                if constexpr (MORE) {
                    if constexpr (E4) {
                        if (k == 0) s4 = col_scales((i + 1) & 3);
                    }
                    if (k == 1) {
                        s_wait_mfma();
                        vmax = nval - (i + 1) * kAttnTile - 16 * cs - 4 * g;
                    }
                    if (k >= 1 && k <= 8) {   // scores (log2 domain)
                        const int jj = (k - 1) >> 2, e = (k - 1) & 3;
                        if constexpr (!E4) {
                            x[jj][e] = e < vmax ? (sa[jj][0][e] + sa[jj][1][e]) * sl2 : -INFINITY;
                        } else {
                            if (jj == 0) {
                                const float sv = e == 0 ? s4.x : e == 1 ? s4.y : e == 2 ? s4.z : s4.w;
                                col_prep(sv, e < vmax, e, ks[e], ef[e]);
                            }
                            x[jj][e] = e < vmax ? __builtin_fmaf(sa[jj][0][e] + sa[jj][1][e], ks[e], ef[e]) : -INFINITY;
                        }
                    }
                    if (k == 9 || k == 12) {   // tile maxima and the slack check
                        const int jj = (k - 9) / 3;
                        tm[jj] = fmaxf(fmaxf(x[jj][0], x[jj][1]), fmaxf(x[jj][2], x[jj][3]));
                    }
                    if (k == 10 || k == 13) {
                        const int jj = (k - 10) / 3;
                        const uint32_t u = __float_as_uint(tm[jj]);
                        const auto a = __builtin_amdgcn_permlane16_swap(u, u, false, false);
                        tm[jj] = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
                    }
                    if (k == 11 || k == 14) {
                        const int jj = (k - 11) / 3;
                        const uint32_t u = __float_as_uint(tm[jj]);
                        const auto b = __builtin_amdgcn_permlane32_swap(u, u, false, false);
                        tm[jj] = fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
                        fl |= tm[jj] > m_own[jj] + kSlack ? 1 : 0;
                    }
                    if (k >= 15 && k <= 22) {   // weights against the owned max
                        const int jj = (k - 15) >> 2, e = (k - 15) & 3;
                        if (e == 0) msub[jj] = m_own[jj] == -INFINITY ? 0.0f : m_own[jj];
                        pr[jj][e] = fast_exp2(x[jj][e] - msub[jj]);
                        if constexpr (!E4) {
                            if (e == 3) {
                                psum[jj] = (pr[jj][0] + pr[jj][1]) + (pr[jj][2] + pr[jj][3]);
                                pk[jj] = make_uint2(pack_bf16x2(pr[jj][0], pr[jj][1]), pack_bf16x2(pr[jj][2], pr[jj][3]));
                            }
                        } else {
                            // p = 2^-e exp2(x - m) for the sum, p * s = mu exp2(x - m) for PV
                            ws[jj][e] = pr[jj][e] * cmu[e];
                            pr[jj][e] = __builtin_amdgcn_ldexpf(pr[jj][e], cne[e]);
                            if (e == 3) psum[jj] = (pr[jj][0] + pr[jj][1]) + (pr[jj][2] + pr[jj][3]);
                        }
                    }
                    // the flag: a ballot over the whole wave (every head of
                    // its two tiles), taken before lane 0 alone publishes it
                    if constexpr (!E4) {
                        if (k == 23) {
                            put_weights((i + 1) & 1, pk, pl);
                            const bool raise = __builtin_amdgcn_ballot_w64(fl != 0) != 0;
                            if (lane == 0 && raise) atomicOr(&xf[f1], 1);
                        }
                    } else {
                        if (k >= 23 && k <= 26) {   // the f16 terms, two weights at a time
                            const int jj = (k - 23) >> 1, h = (k - 23) & 1;
                            if (h == 0) split_f16x2(ws[jj][0], ws[jj][1], pk[jj].x, pl[jj].x);
                            else split_f16x2(ws[jj][2], ws[jj][3], pk[jj].y, pl[jj].y);
                        }
                        if (k == 27) {
                            put_weights((i + 1) & 1, pk, pl);
                            const bool raise = __builtin_amdgcn_ballot_w64(fl != 0) != 0;
                            if (lane == 0 && raise) atomicOr(&xf[f1], 1);
                        }
                    }
                }
            });
            if constexpr (G3) wait_vm<kGI>();
            else wait_vm<0>();
            __syncthreads();
            const int ft = f0;
            f0 = f1;
            f1 = f2;
            f2 = ft;
        };
        using T_ = std::integral_constant<bool, true>;
        using F_ = std::integral_constant<bool, false>;
        int i = 0;
        for (; i + 3 < n; ++i) body(i, T_{}, T_{});
        for (; i + 1 < n; ++i) body(i, F_{}, T_{});
        body(i, F_{}, F_{});   // the last tile (n >= 1)
    };
    // stage a chunk's indices; iv0: its first batch, already loaded
    auto stage_chunk = [&](int cc, const int (&iv0)[4]) __attribute__((always_inline)) {
        const int cn = min(c_end - cc, kIdxChunk);
        nval = 0;
        stage4(cc, 0, iv0);
        for (int i0 = 4 * kNT; i0 < cn; i0 += 4 * kNT) {
            int iv[4];
            load4(cc, cn, i0, iv);
            stage4(cc, i0, iv);
        }
        pad();
        __syncthreads();
    };

    // A token's first index batch is loaded while the token before it runs
    // its tiles (untracked loads: the compiler would otherwise wait for them
    // at once; the tile loop's waits are stronger than theirs).  After that
    // token's last tile, the token's q rows go out, its indices are staged
    // and its first two tiles go out, and only then does the previous token
    // write its output, so those loads land while the stores drain.
    int iv0[4];
    const int cn0 = min(c_end - c_begin, kIdxChunk);
    const bool cols = c_end > c_begin;
    auto load_idx0 = [&](int tq) __attribute__((always_inline)) {
        const int32_t *row = p.idx + (int64_t)tq * p.idx_st + c_begin;
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int i = 4 * tid + u;
            iv0[u] = gload_untracked(row + (i < cn0 ? i : 0));
        }
    };
    // token tq's indices are in iv0: stage them and send its first two tiles
    auto begin_token = [&](int tq) __attribute__((always_inline)) {
        idx_row = p.idx + (int64_t)tq * p.idx_st;
        safe_src = (uint64_t)(p.q + (int64_t)tq * p.q_st);
#pragma unroll
        for (int u = 0; u < 4; ++u) iv0[u] = 4 * tid + u < cn0 ? iv0[u] : -1;
        stage_chunk(c_begin, iv0);
        if (n_tiles > 0) gather(0, 0);
        if (n_tiles > 1) gather(1, 1);
    };
    if (t < tend && cols) {
        stage_q(t);
        load_idx0(t);
        vm_wait4<0>(iv0);
        begin_token(t);
    }
    for (bool later = false; t < tend; t += tstep, later = true) {
        const int tn = t + tstep;
        const bool next = tn < tend && cols;
        // the loads issued since this token's q rows: its first two tiles
        // (and no further index batch), the previous token's 32 output
        // stores (the first token has none) and the next token's 4 index
        // loads; otherwise wait for all
        const bool full = later && n_tiles > 1 && cn0 <= 4 * kNT && hbase + kAttnHeadsPerBlock <= p.H && next;
        if (next) load_idx0(tn);
#pragma unroll
        for (int m = 0; m < kPM; ++m)
#pragma unroll
            for (int j = 0; j < 4; ++j) acc[m][j] = f32x4{0.f, 0.f, 0.f, 0.f};
        // the zeros are written here: the MFMAs that accumulate onto them
        // are inline assembly, so the compiler would not keep the wait states
        // a vector write needs before an MFMA reads it if it moved (or
        // rematerialised) these writes next to the first PV
#pragma unroll
        for (int m = 0; m < kPM; ++m) asm volatile("" : "+a"(acc[m][0]), "+a"(acc[m][1]), "+a"(acc[m][2]), "+a"(acc[m][3]));
        m_run = f32x4{-INFINITY, -INFINITY, -INFINITY, -INFINITY};
        m_own[0] = m_own[1] = -INFINITY;
        l_run[0] = l_run[1] = psum[0] = psum[1] = 0.0f;
        if (cols) {
            // the first chunk is staged and its first two tiles are in
            // flight; the q rows must have landed before their fragments are
            // read
            const int n0 = n_tiles;
            if (full) wait_vm<2 * kGI + kPM * 4 + 4>();
            else wait_vm<0>();
            // (rows past H read the finite stand-in row staged for them; their
            // scores are never used)
            // fragment s of head row 32hg + 16jj + l16 sits at chunk
            // (4s + g) ^ l16 = 16(s / 4) + ((4(s % 4) + g) ^ l16): four
            // per-lane bases and immediate offsets.  e4m3 (the order of its
            // K reads): dims 16(4u + g) + 8h .. +7 for step s = 2u + h, chunk
            // 8u + 2g + h = 16(s / 4) + 8((s / 2) % 2) + 2g + s % 2
            {
                const int ln = opaque(lane), q16 = ln & 15, qg = ln >> 4;
                uint32_t qa[4];
#pragma unroll
                for (int u = 0; u < 4; ++u) {
                    const int c = E4 ? 8 * (u >> 1) + 2 * qg + (u & 1) : 4 * u + qg;
                    qa[u] = lds_offset(qstage) + (uint32_t)((32 * hg + q16) * 2 * kD + 16 * (c ^ q16));
                }
                load_q_frags(qf, qa, std::make_index_sequence<kSK>{});
            }
            asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
            __syncthreads();   // tiles 2 and 3 (q) are free
            if (n0 > 0) run_chunk(true, full);
            for (int cc = c_begin + kIdxChunk; cc < c_end; cc += kIdxChunk) {
                int iv[4];
                load4(cc, min(c_end - cc, kIdxChunk), 0, iv);
                stage_chunk(cc, iv);
                if (n_tiles > 0) run_chunk(false, false);
            }
        }
        // no transfer into LDS is left (and none outlives the workgroup); the
        // next token's first indices have landed
        vm_wait4<0>(iv0);
        // wait states between the last accumulating MFMA (inline assembly, which
        // the compiler's hazard tracking does not see) and the reads of O below
        asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory");
        // every wave is past its last read of the tiles and of sidx: the next
        // token's q rows and first two tiles go out now
        __syncthreads();
        if (next) {
            stage_q(tn);
            begin_token(tn);
        }
        // softmax sums: owners reduce over their columns, everyone adds the two
        // column halves of each head in a fixed order
#pragma unroll
        for (int jj = 0; jj < 2; ++jj) {
            const float ls = group4_sum(l_run[jj]);
            if (g == 0) xl[w][16 * jj + l16] = ls;
        }
        __syncthreads();
        // (the output strides pass through an empty statement so that the
        // per-lane row offsets are formed here, not kept live across the
        // token loop)
        int64_t out_st = p.out_st, out_sh = p.out_sh;
        asm volatile("" : "+s"(out_st), "+s"(out_sh));
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int head = hbase + 16 * j + l16;
            const int o = 16 * (j & 1) + l16;
            const float l_tot = xl[j >> 1][o] + xl[(j >> 1) + 2][o];
            if (head >= p.H) continue;
            const int d0 = (kD / kNW) * w + 4 * g;
            const float inv = l_tot > 0.0f ? 1.0f / l_tot : 0.0f;
            if constexpr (OUT == 1) {
                float *dst = (float *)p.out + (int64_t)t * out_st + (int64_t)head * out_sh + d0;
#pragma unroll
                for (int m = 0; m < kPM; ++m) {
                    const f32x4 v = acc[m][j] * inv;
                    *(float4 *)(dst + 16 * m) = make_float4(v[0], v[1], v[2], v[3]);
                }
            } else {
                uint16_t *dst = (uint16_t *)p.out + (int64_t)t * out_st + (int64_t)head * out_sh + d0;
#pragma unroll
                for (int m = 0; m < kPM; ++m) {
                    const f32x4 v = acc[m][j] * inv;
                    *(uint2 *)(dst + 16 * m) = make_uint2(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]));
                }
            }
        }
    }
}// workgroups per head block: one per CU (a workgroup takes most of a CU's
// LDS), rounded down to a multiple of the 8 XCDs, at most one per token
int persistent_blocks(int T)
{
    static int cus[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return T;
    if (cus[dev] == 0) {
        int n = 0;
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n < 8) return T;
        cus[dev] = n & ~7;
    }
    return T < cus[dev] ? T : cus[dev];
}

template <int OUT, bool E4>
hipError_t launch_t(const AttnParams &p, hipStream_t s)
{
    const dim3 grid((unsigned)persistent_blocks(p.T), (unsigned)((p.H + kAttnHeadsPerBlock - 1) / kAttnHeadsPerBlock));
    hipLaunchKernelGGL((attn_d512_kernel<OUT, E4>), grid, dim3(kNT), 0, s, p);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_attn_d512(const AttnParams &p, int kv, int out, hipStream_t s)
{
    if (p.num_splits != 1) return hipErrorInvalidValue;   // one split per token only
    if (kv == 2) return out == 1 ? launch_t<1, true>(p, s) : launch_t<0, true>(p, s);
    if (kv != 0) return hipErrorInvalidValue;
    return out == 1 ? launch_t<1, false>(p, s) : launch_t<0, false>(p, s);
}

}  // namespace sap
