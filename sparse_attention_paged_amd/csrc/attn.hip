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
// columns, taken in tiles of 32 columns.  The split of work between the waves
// is chosen so that every operand a wave reads from LDS feeds four MFMAs
// (64 heads as the MFMA N dimension) and every score is exponentiated once:
//  - gather: each wave moves 8 of the tile's 32 rows straight from HBM into
//    LDS (global_load_lds_dwordx4, 16 bytes per lane; one wave instruction
//    moves one 1 KiB row at D = 512), chunk-swizzled per row.  bf16: four LDS
//    tiles rotate and the gathers of tile t+3 are spread over the S, softmax
//    and PV phases of tiles t+1 and t; e4m3: three tiles, rows go through
//    registers and are widened to bf16 on the way.
//  - S^T = K Q^T on MFMA 16x16x32 bf16 (M = columns, N = heads): wave
//    (dq, ch) = (w & 1, w >> 1) takes columns 16ch .. 16ch+15, all 64 heads,
//    head_dim half dq.  The two head_dim halves of a column half add their
//    partial scores through LDS: each keeps the 32 heads whose softmax it
//    owns (32dq .. 32dq+31) and receives the partner's partial for them.
//  - online softmax in the log2 domain over the owned 32 heads x 16 columns
//    (8 scores per lane), placed between the MFMAs of the next tile's S
//    (software pipelined).  The running max only moves when a tile's max
//    exceeds it by more than 32 (weights stay <= 2^32); a head's first max
//    needs no rescale of O.  A later move beyond the slack (rare) leaves the
//    fast tile loop for a second loop that rescales O after all waves agree
//    on the new maxima, so the fast loop does no VALU work on the
//    accumulators.
//  - O^T += V^T P^T on MFMA 16x16x32 bf16 (M = head_dim, N = heads, K = the
//    32 columns): wave w owns head_dim quarter w for all 64 heads.  P^T is
//    read back from LDS in the B-operand layout; the V^T A-operand is read
//    from the row-major tile with ds_read_b64_tr_b16 (within 16 lanes, lane i
//    receives element i%4 of the 8 bytes addressed by lanes i/4 + 4r,
//    r = 0..3).  e4m3 pools feed P as hi + mid + lo bf16 terms.
// The PV reduction index kk = 8g + 4c + i stands for tile column
// 16c + 4g + i, which lets each lane take its own 4 weights of column half c
// straight from the softmax layout.
// With one split per token the output is normalised and stored; with several
// splits each workgroup stores (unnormalised O, running max, sum) and the
// merge kernel combines them in split order.
#include "common.hpp"
#include "formats.hpp"
#include "internal.hpp"
#include "attn_common.hpp"

#include <type_traits>

namespace sap {
namespace {

using namespace attn;

constexpr int kThreads = 256;          // 4 waves
template <int D>
struct AttnShape {
    static constexpr int CH = D / 8;                    // 16-byte chunks per bf16 row
    static constexpr int RPI = 64 / CH;                 // rows per 1 KiB wave instruction
    static constexpr int NQ = D / 64;                   // gather instructions per wave per tile
    static constexpr int SK = D / 64;                   // S k-steps (32 deep) over a head_dim half
    static constexpr int PM = D / 64;                   // PV m-tiles (16 rows) over a head_dim quarter
    static constexpr int TILE_BYTES = kAttnTile * D * 2;
};

template <int KV> struct RawRow;
template <> struct RawRow<0> { using T = uint4; };   // 8 bf16
template <> struct RawRow<2> { using T = uint2; };   // 8 e4m3 codes

// NW = 4: one wave per SIMD (the roles below), the shape the launches use;
// the code also covers NW = 8 (two head groups of four waves for S and the
// softmax, each wave holding half the Q operand and half the O accumulators,
// two waves per SIMD, D >= 128), which served head_dim 512 before the
// dedicated one-pass and decode kernels of attn_d512.hip and attn_dec.hip.
template <int D, int KV, int OUT, int NW>
__global__ __attribute__((amdgpu_flat_work_group_size(64 * NW, 64 * NW), amdgpu_waves_per_eu(NW / 4, NW / 4)))
void attn_kernel(AttnParams p)
{
    using SH = AttnShape<D>;
    static_assert(NW == 4 || (NW == 8 && D >= 128), "eight waves need at least two gather rows per wave");
    constexpr int NT = 64 * NW;            // threads
    constexpr int G = NW / 4;              // head groups of S / softmax
    constexpr int JS = 4 / G;              // 16-head tiles a wave computes S for
    constexpr int JO = JS / 2;             // 16-head tiles whose softmax a wave owns
    constexpr int RW = kAttnTile / NW;     // gather rows per wave per tile
    constexpr int NQW = SH::NQ * 4 / NW;   // gather instructions per wave per tile
    constexpr int PMW = D / (16 * NW);     // PV m-steps over this wave's head_dim range
    using Raw = typename RawRow<KV>::T;
    // bf16 terms per PV weight: e4m3 weights carry the row scale and PV must
    // hold them to fp32-like precision (outputs reach ~1e3 against an
    // absolute bar), so they go in as hi + mid + lo (relative error ~2^-25)
    constexpr int NP = KV == 2 ? 3 : 1;
    // rotating tiles (bf16: 4, the gathers of tile t+3 are issued while tile
    // t computes; e4m3: 3, rows pass through registers), each tile's
    // per-column bias (0 or -inf) and dequant scale, and the row indices of
    // the current chunk of columns
    constexpr int DEPTH = KV == 0 ? 4 : 3;
    // bf16: the gather instructions of tile u are spread over three phases
    // so that the four waves never issue them in one burst: rows [0, GA)
    // during PV(u-3), rows [GA, GA+GB) during S(u-2), the rest during the
    // softmax of u-2.  Tile u's buffer held tile u-4, free after B1(u-3).
    constexpr int GA = NQW * 3 / 8, GB = NQW * 3 / 8;
    static_assert(GA <= PMW && GB <= SH::SK, "every gather row needs a PV or S step");
    __shared__ __attribute__((aligned(1024))) uint8_t tiles[DEPTH][SH::TILE_BYTES];
    __shared__ __attribute__((aligned(16))) float metas[DEPTH][2 * kAttnTile];
    __shared__ __attribute__((aligned(16))) int sidx[kIdxChunk];
    __shared__ int xscan[NW];                // wave totals of the column compaction
    __shared__ float4 xs[NW][JO][64];        // partial scores for the partner wave
    // bf16 P by [term][head tile][ch][lane]: the two column halves of one
    // head tile sit 512 bytes apart, so a lane reads its B operand with one
    // ds_read2_b64
    __shared__ uint2 xp[NP][4][2][64];
    __shared__ uint2 xq[NP][4][2][64];       // the same after a max change
    __shared__ float xm[NW][16 * JO];        // tile max of each owned head
    __shared__ float xl[NW][16 * JO];        // softmax sums at the end
    __shared__ __attribute__((aligned(16))) int xf[NW];   // bit 0: a first max, bit 1: a larger max

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

    const int tid = threadIdx.x;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63, l16 = lane & 15, g = lane >> 4;
    // S / softmax role: head group gr, head_dim half dq, column half ch
    const int gr = w >> 2, dq = w & 1, ch = (w >> 1) & 1;
    const int hbase = blockIdx.y * kAttnHeadsPerBlock;

    // The block's 64 q rows are staged in the (still unused) first two tiles
    // with whole-row LDS DMA (each instruction moves 1 KiB; 16-byte chunk c
    // of row h lands in slot c ^ (h & 15), or h & 7 at D = 64), then each wave reads its
    // fragments: loading the MFMA operand layout straight from memory would
    // touch 16 rows per instruction and fetch every row twice.
    // (bf16: tiles 2 and 3, so the first two tiles' gathers can go out
    // while the fragments are read)
    uint8_t *const qstage = KV == 0 ? &tiles[2][0] : &tiles[0][0];
    constexpr int QSW = D >= 128 ? 15 : 7;   // chunk swizzle mask (a row has D/8 chunks)
    {
        constexpr int QI = 64 * 2 * D / 1024 / NW;   // DMA instructions per wave
#pragma unroll
        for (int k = 0; k < QI; ++k) {
            const int u = NW * k + w;                 // 1 KiB block of the staging area
            const int f = 1024 * u + 16 * lane;       // byte of the staging area this lane fills
            const int h = f / (2 * D), c = (f % (2 * D)) / 16;
            const int head = hbase + h < p.H ? hbase + h : hbase;   // rows past H: finite stand-in
            const uint16_t *src = p.q + (int64_t)t * p.q_st + (int64_t)head * p.q_sh + 8 * (c ^ (h & QSW));
            dma16(src, lds_offset(qstage + 1024 * u));
        }
    }
    // finite data that invalid columns load instead of a pool row (their
    // scores are masked to -inf and their weights are 0)
    const uint8_t *safe_src = (const uint8_t *)(p.q + (int64_t)t * p.q_st);

    // kernel arguments the lambdas below use, as plain scalars (capturing the
    // argument struct by reference would place it in scratch memory)
    const uint8_t *const win_pool = p.win, *const cmp_pool = p.cmp;
    const int64_t win_rs = p.win_rs, cmp_rs = p.cmp_rs;
    const float *const win_scale = p.win_scale, *const cmp_scale = p.cmp_scale;
    const int n_win = p.n_win;
    const float sl2 = p.sm_scale_log2;

    // gather role: instruction q of this wave covers tile rows
    // 8w + q*RPI .. + RPI-1; this lane reads row grow(q), chunk slot gpos
    const int32_t *idx_row = p.idx + (int64_t)t * p.idx_st;
    const int gpos = lane % SH::CH;
    auto grow = [&](int q) __attribute__((always_inline)) { return RW * w + q * SH::RPI + lane / SH::CH; };
    Raw raw[NQW];          // e4m3 only: codes of the issued tile, widened when landed
    float rsc[NQW];
    int cc = c_begin;      // first column of the current chunk
    int n_tiles = 0;       // tiles of the current chunk

    // Column staging: a chunk's valid columns are packed to the front of sidx
    // in column order, so tiles of unused (-1) columns are never gathered or
    // scored; each entry is its pool row, with bit 31 set for the compressed
    // pool, and -1 pads the last tile.  Each thread takes 4 consecutive
    // columns per batch of 4 NT.
    int nval = 0;   // columns of the current chunk staged so far
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
        for (int k = 0; k < NW; ++k) {
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
        for (int i = nval + tid; i < n_tiles * kAttnTile; i += NT) sidx[i] = -1;
    };
    // the first batch of the first chunk loads while q lands
    const int cn0 = min(c_end - c_begin, kIdxChunk);
    {
        int iv[4];
        load4(c_begin, cn0, 0, iv);
        wait_vm<0>();
        stage4(c_begin, 0, iv);
        if (cn0 <= 4 * NT) pad();   // the whole first chunk is staged
    }
    __syncthreads();
    // Q as the B operand of S^T over head_dim half dq, read from the staging
    // area below: qf[j][s] = q[t, hbase + 16(JS gr + j) + l16, D/2*dq + 32s + 8g .. +7]
    uint4 qf[JS][SH::SK];

    // issue gather instruction q of tile `tile` (of the current chunk) into
    // buffer `bf`; the row index comes from the staged chunk
    // rr: the row index when one instruction moves one row (RPI == 1, taken
    // from registers filled ahead of time, so issuing never waits on an LDS
    // read); otherwise each lane reads its own row's index here
    auto issue_row = [&](uint8_t *bf, float *meta, int tile, int q, int rr) __attribute__((always_inline)) {
        const int rho = grow(q);
        const int e = SH::RPI == 1 ? rr : sidx[tile * kAttnTile + rho];   // staged entry
        const bool ok = e != -1;
        const bool win = e >= 0;
        const int r = e & 0x7FFFFFFF;
        const uint8_t *base = win ? win_pool : cmp_pool;
        const int64_t rs = win ? win_rs : cmp_rs;
        const int j = gpos ^ rswz(rho);
        if constexpr (KV == 0) {
            const uint8_t *src = ok ? base + (int64_t)r * rs + 16 * j : safe_src + 16 * gpos;
            dma16(src, lds_offset(bf + (RW * w + q * SH::RPI) * 2 * D));
        } else {
            // unused columns: load the stand-in bytes but keep zero codes,
            // since arbitrary bytes read as e4m3 may be NaN encodings
            const uint8_t *src = ok ? base + (int64_t)r * rs + 8 * j : safe_src + 8 * gpos;
            const Raw v = *(const Raw *)src;
            raw[q] = ok ? v : Raw{0u, 0u};
            rsc[q] = ok ? (win ? win_scale : cmp_scale)[r] : 0.0f;
        }
        if (gpos == 0) meta[rho] = ok ? 0.0f : -INFINITY;
    };
    // the row indices of this wave's 8 rows of a tile, wave-uniform (RPI == 1)
    struct Rows {
        int r[NQW];
    };
    auto rows_of = [&](int tile, Rows &rw) __attribute__((always_inline)) {
        if constexpr (SH::RPI == 1) {
            // 16-byte LDS reads of the wave's RW indices (wave-uniform address)
            const int4 *src = (const int4 *)(sidx + tile * kAttnTile + RW * w);
#pragma unroll
            for (int h = 0; h < RW / 4; ++h) {
                const int4 a = src[h];
                const int v[4] = {a.x, a.y, a.z, a.w};
#pragma unroll
                for (int q = 0; q < 4; ++q) rw.r[4 * h + q] = __builtin_amdgcn_readfirstlane(v[q]);
            }
        }
    };
    auto issue = [&](uint8_t *bf, float *meta, int tile) __attribute__((always_inline)) {
        Rows rw;
        rows_of(tile, rw);
#pragma unroll
        for (int q = 0; q < NQW; ++q) issue_row(bf, meta, tile, q, rw.r[q]);
    };
    // e4m3: widen the registers of the issued tile into its buffer
    auto land = [&](uint8_t *bf, float *meta) __attribute__((always_inline)) {
        if constexpr (KV == 2) {
            float *scl = meta + kAttnTile;
#pragma unroll
            for (int q = 0; q < NQW; ++q) {
                *(uint4 *)(bf + (RW * w + q * SH::RPI) * 2 * D + 16 * lane) = e4m3x8_to_bf16x8(raw[q]);
                if (gpos == 0) scl[grow(q)] = rsc[q];
            }
        }
    };

    // O^T accumulators: acc[m][j] = O^T[d = D/NW*w + 16m + 4g + i][head 16j + l16]
    f32x4 acc[PMW][4];
#pragma unroll
    for (int m = 0; m < PMW; ++m)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[m][j] = f32x4{0.f, 0.f, 0.f, 0.f};
    // running max of heads 16j + l16 (identical in every wave), and the sum
    // over this lane's columns of the owned heads: tile J = JS gr + JO dq + nt
    // (a vector value, not an array: no access can turn into an address)
    f32x4 m_run = {-INFINITY, -INFINITY, -INFINITY, -INFINITY};
    float l_run[JO];
#pragma unroll
    for (int nt = 0; nt < JO; ++nt) l_run[nt] = 0.0f;
    // the head tile of owned tile nt, and the waves owning head tile j
    auto own_tile = [&](int nt) __attribute__((always_inline)) { return JS * gr + JO * dq + nt; };
    auto owner = [](int j) { return 4 * (j / JS) + (j % JS) / JO; };   // its ch = 0 wave; ch = 1 is +2
    // m_run of the wave-uniform tile index J, through selects of its
    // elements (an array indexed at run time would live in scratch memory)
    auto m_of = [&](int J) __attribute__((always_inline)) {
        float r = m_run[0];
#pragma unroll
        for (int k = 1; k < 4; ++k) r = J == k ? m_run[k] : r;
        return r;
    };

    // LDS byte offsets within a tile.  S reads chunk (D/16)dq + 4s + g of row
    // 16ch + l16; PV reads rows 16h + 4g + l16/4 at head_dim D/4*w + 16m +
    // 4(l16%4).  The swizzle only touches the low 3 chunk bits, so each read
    // is one of a few per-lane bases plus a constant.
    int kb[2];
    {
        const int rho = 16 * ch + l16, sw = rswz(rho);
#pragma unroll
        for (int e = 0; e < 2; ++e) kb[e] = rho * 2 * D + 16 * (((D / 16) * dq + 4 * e + g) ^ sw);
    }
    // (rows r and r + 16 have the same swizzle, so the second PV row is the
    // first plus a constant)
    constexpr int VB = PMW < 4 ? PMW : 4;
    int vb[VB];
    {
        const int dsub = 4 * (l16 & 3);
        const int r = 4 * g + (l16 >> 2), vs = rswz(r);
#pragma unroll
        for (int mm = 0; mm < VB; ++mm) {
            const int d = (D / NW) * w + 16 * mm + dsub;
            vb[mm] = r * 2 * D + 16 * ((d >> 3) ^ vs) + 2 * (d & 7);
        }
    }

    // --- S^T over head_dim half dq for columns 16ch .. 16ch+15:
    //     sacc[j] = S^T[col 16ch + 4g + i][head 16(JS gr + j) + l16] (partial)
    auto s_part = [&](const uint8_t *bf, f32x4 (&sacc)[JS], int dma_tile, uint8_t *nb2, float *nm2, const Rows &r2,
                      auto hook) __attribute__((always_inline)) {
#pragma unroll
        for (int j = 0; j < JS; ++j) sacc[j] = f32x4{0.f, 0.f, 0.f, 0.f};
        auto kfrag = [&](int s) __attribute__((always_inline)) { return lds_b128(bf + kb[s & 1] + 128 * (s >> 1)); };
        uint4 f[2];   // fragment ring: step s+1 is read while step s multiplies
        f[0] = kfrag(0);
#pragma unroll
        for (int s = 0; s < SH::SK; ++s) {
            if (s + 1 < SH::SK) f[(s + 1) % 2] = kfrag(s + 1);
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int j = 0; j < JS; ++j) sacc[j] = mfma16x16x32(f[s % 2], qf[j][s], sacc[j]);
            if constexpr (KV == 0) {
                // GB gathers of tile t+2, at k-steps spread over the loop
                constexpr int STEP = GB > 0 ? SH::SK / GB : 1;   // GB <= SK: rows at s = STEP-1, 2 STEP-1, ...
                if (GB > 0 && s % STEP == STEP - 1 && s / STEP < GB && dma_tile >= 0 && dma_tile < n_tiles)
                    issue_row(nb2, nm2, dma_tile, GA + s / STEP, r2.r[GA + s / STEP]);
            }
            // VALU work of the previous tile runs while these MFMAs execute
            hook(s);
            __builtin_amdgcn_sched_barrier(0);
        }
    };

    // weights of the owned heads against the current max: per head tile nt,
    // 4 columns packed as bf16 (e4m3: NP terms, each the bf16 rounding of
    // what the previous terms left)
    auto weights = [&](const float (&x)[JO][4], const float (&csc)[4], float (&pr)[JO][4],
                       uint2 (&pt)[NP][JO]) __attribute__((always_inline)) {
#pragma unroll
        for (int nt = 0; nt < JO; ++nt) {
            const float mr = m_of(own_tile(nt));
            const float msub = mr == -INFINITY ? 0.0f : mr;
#pragma unroll
            for (int i = 0; i < 4; ++i) pr[nt][i] = fast_exp2(x[nt][i] - msub);
            if constexpr (KV == 2) {
                float r[4];
#pragma unroll
                for (int i = 0; i < 4; ++i) r[i] = pr[nt][i] * csc[i];
#pragma unroll
                for (int e = 0; e < NP; ++e) {
                    pt[e][nt] = make_uint2(pack_bf16x2(r[0], r[1]), pack_bf16x2(r[2], r[3]));
#pragma unroll
                    for (int i = 0; i < 4; ++i) r[i] -= __uint_as_float(bf16_bits(r[i]) << 16);
                }
            } else {
                pt[0][nt] = make_uint2(pack_bf16x2(pr[nt][0], pr[nt][1]), pack_bf16x2(pr[nt][2], pr[nt][3]));
            }
        }
    };
    auto put_p = [&](uint2 (*px)[4][2][64], const uint2 (&pt)[NP][JO]) __attribute__((always_inline)) {
#pragma unroll
        for (int e = 0; e < NP; ++e)
#pragma unroll
            for (int nt = 0; nt < JO; ++nt) px[e][own_tile(nt)][ch][lane] = pt[e][nt];
    };

    // --- O^T += V^T P^T for head_dim range w (D/NW wide); P^T of head tile j
    //     comes from its two column-half owners
    auto pv = [&](const uint8_t *bf, const uint2 (*px)[4][2][64], int dma_tile, uint8_t *nb3, float *nm3,
                  const Rows &r3) __attribute__((always_inline)) {
        uint4 pb[NP][4];
#pragma unroll
        for (int e = 0; e < NP; ++e)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const uint2 a = px[e][j][0][lane], b = px[e][j][1][lane];
                pb[e][j] = make_uint4(a.x, a.y, b.x, b.y);
            }
        auto vfrag = [&](int m) __attribute__((always_inline)) {
            const uint2 v0 = lds_tr16(bf + vb[m & 3] + 128 * (m >> 2));
            const uint2 v1 = lds_tr16(bf + vb[m & 3] + 16 * 2 * D + 128 * (m >> 2));
            return make_uint4(v0.x, v0.y, v1.x, v1.y);
        };
        uint4 vr[3];
        vr[0] = vfrag(0);
        if (PMW > 1) vr[1] = vfrag(1);
#pragma unroll
        for (int m = 0; m < PMW; ++m) {
            if (m + 2 < PMW) vr[(m + 2) % 3] = vfrag(m + 2);
            __builtin_amdgcn_sched_barrier(0);
            const uint4 a = vr[m % 3];
#pragma unroll
            for (int j = 0; j < 4; ++j) acc[m][j] = mfma16x16x32(a, pb[0][j], acc[m][j]);
#pragma unroll
            for (int e = 1; e < NP; ++e)
#pragma unroll
                for (int j = 0; j < 4; ++j) acc[m][j] = mfma16x16x32(a, pb[e][j], acc[m][j]);
            // bf16: the remaining gather instructions of tile t+3, one per
            // m-step, so the memory pipeline fills while the MFMAs run
            if constexpr (KV == 0) {
                // GA gathers of tile t+3, at m-steps spread over the loop
                constexpr int STEP = GA > 0 ? PMW / GA : 1;   // GA <= PMW
                if (GA > 0 && m % STEP == STEP - 1 && m / STEP < GA && dma_tile < n_tiles)
                    issue_row(nb3, nm3, dma_tile, m / STEP, r3.r[m / STEP]);
            }
            __builtin_amdgcn_sched_barrier(0);
        }
    };

    // softmax inputs of the current tile, kept between the two halves of a step
    struct Soft {
        float x[JO][4], csc[4], psum[JO];   // scores, e4m3 scales, sums of this lane's weights
    };

    // --- softmax of the owned heads (tiles JS gr + JO dq + nt), columns
    //     16ch + 4g + i, in three pieces so they can be placed between the
    //     MFMAs of the next tile's S
    // (a) the partner's partial scores and the tile's bias / scales -> scores
    auto soft_a = [&](const float *cm, const f32x4 (&mine)[JO], Soft &st) __attribute__((always_inline)) {
        const float4 b4 = *(const float4 *)(cm + 16 * ch + 4 * g);
        const float bb[4] = {b4.x, b4.y, b4.z, b4.w};
        if constexpr (KV == 2) {
            const float4 s4 = *(const float4 *)(cm + kAttnTile + 16 * ch + 4 * g);
            st.csc[0] = s4.x; st.csc[1] = s4.y; st.csc[2] = s4.z; st.csc[3] = s4.w;
        }
#pragma unroll
        for (int nt = 0; nt < JO; ++nt) {
            const float4 o4 = xs[w ^ 1][nt][lane];
            const float ov[4] = {o4.x, o4.y, o4.z, o4.w};
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                float v = (mine[nt][i] + ov[i]) * sl2;
                if constexpr (KV == 2) v *= st.csc[i];
                st.x[nt][i] = v + bb[i];
            }
        }
    };
    // (b) tile maxima of the owned heads and the flags (bit 0: a first
    //     valid column, bit 1: a max beyond the slack)
    auto soft_b = [&](const Soft &st, float (&tmax)[JO]) __attribute__((always_inline)) {
        int flag = 0;
#pragma unroll
        for (int nt = 0; nt < JO; ++nt) {
            tmax[nt] = group4_max(fmaxf(fmaxf(st.x[nt][0], st.x[nt][1]), fmaxf(st.x[nt][2], st.x[nt][3])));
            const float mr = m_of(own_tile(nt));
            if (mr == -INFINITY) flag |= tmax[nt] > -INFINITY ? 1 : 0;
            else flag |= tmax[nt] > mr + kRescaleSlack ? 2 : 0;
        }
        return flag;
    };
    // (c) weights against the current max, published with the maxima and flags
    auto soft_c = [&](Soft &st, const float (&tmax)[JO], int flag) __attribute__((always_inline)) {
        uint2 pt[NP][JO];
        float pr[JO][4];
        weights(st.x, st.csc, pr, pt);
#pragma unroll
        for (int nt = 0; nt < JO; ++nt) st.psum[nt] = (pr[nt][0] + pr[nt][1]) + (pr[nt][2] + pr[nt][3]);
        put_p(xp, pt);
        if (g == 0) {
#pragma unroll
            for (int nt = 0; nt < JO; ++nt) xm[w][16 * nt + l16] = tmax[nt];
        }
        const int wf = (__builtin_amdgcn_ballot_w64((flag & 1) != 0) ? 1 : 0) |
                       (__builtin_amdgcn_ballot_w64((flag & 2) != 0) ? 2 : 0);
        if (lane == 0) xf[w] = wf;
    };

    // S^T partials of a tile: send the partner's heads, keep mine (register
    // arrays are only indexed by constants; the wave-uniform choice is a select)
    auto send_scores = [&](const f32x4 (&sacc)[JS], f32x4 (&mine)[JO]) __attribute__((always_inline)) {
#pragma unroll
        for (int nt = 0; nt < JO; ++nt) {
            mine[nt] = dq ? sacc[JO + nt] : sacc[nt];
            const f32x4 th = dq ? sacc[nt] : sacc[JO + nt];
            xs[w][nt][lane] = make_float4(th[0], th[1], th[2], th[3]);
        }
    };

    // One tile t, software pipelined: S of tile t+1 on the MFMAs while the
    // softmax of tile t runs on the VALU between them; then the second
    // barrier, the partial scores of tile t+1 (their buffer is free: every
    // wave has read tile t's), and (back) PV of tile t.  Tile t's partial
    // scores were exchanged before the first barrier of tile t (tail of the
    // previous tile).  Gathers: all of tile t+3 (bf16) or tile t+2 (e4m3).
    // Returns the workgroup's combined flags.
    auto front = [&](int tile, const float *cm, const uint8_t *nb1, uint8_t *nb2, float *nm2, uint8_t *nb3,
                     float *nm3, Soft &st, f32x4 (&mine)[JO], Rows &r3) __attribute__((always_inline)) {
        const bool more1 = tile + 1 < n_tiles;
        if constexpr (KV == 0) {
            if (tile + 3 < n_tiles) rows_of(tile + 3, r3);
        } else {
            if (tile + 2 < n_tiles) issue(nb2, nm2, tile + 2);   // into registers; landed at the tail
        }
        float tmax[JO];
        int flag = 0;
        auto hook = [&](int s) __attribute__((always_inline)) {
            constexpr int SK = SH::SK;
            if (s == 0) {
                soft_a(cm, mine, st);
                if constexpr (KV == 0) {
                    // the last gathers of tile t+3 (the rest go out in S and PV)
                    if (tile + 3 < n_tiles) {
#pragma unroll
                        for (int q = GA + GB; q < NQW; ++q) issue_row(nb3, nm3, tile + 3, q, r3.r[q]);
                    }
                }
            }
            if (s == (SK - 1) / 2) flag = soft_b(st, tmax);
            if (s == SK - 1) soft_c(st, tmax, flag);
        };
        f32x4 sacc[JS];
        if (more1) {
            s_part(nb1, sacc, tile + 3, nb3, nm3, r3, hook);
        } else {
#pragma unroll
            for (int s = 0; s < SH::SK; ++s) hook(s);   // the same pieces, no S
        }
        __syncthreads();
        // the waves' flags in 16-byte reads
        int any = 0;
#pragma unroll
        for (int k = 0; k < NW / 4; ++k) {
            const int4 f4 = ((const int4 *)xf)[k];
            any |= f4.x | f4.y | f4.z | f4.w;
        }
        any = __builtin_amdgcn_readfirstlane(any);
        if (more1) send_scores(sacc, mine);
        return any;
    };
    // tail of tile t: tile t+2 has landed, the partial scores of tile t+1 are
    // published (first barrier of tile t+1)
    auto tail = [&](int tile, uint8_t *nb2, float *nm2) __attribute__((always_inline)) {
        if (tile + 1 >= n_tiles) return;
        if constexpr (KV == 0) {
            // only the gathers of tile t+3 (all issued after those of t+2)
            // may stay in flight
            if (tile + 3 < n_tiles) wait_vm<NQW>();
            else wait_vm<0>();
        } else {
            wait_vm<0>();
            if (tile + 2 < n_tiles) land(nb2, nm2);
        }
        __syncthreads();
    };

    // second half: agree on new maxima if any head needs one (RESCALE: also
    // from a finite max, which rescales O and the sums), then PV
    auto back = [&](auto rescale_tag, int any, const uint8_t *cb, Soft &st, int dma_tile, uint8_t *nb3, float *nm3,
                    const Rows &r3) __attribute__((always_inline)) {
        constexpr bool RESCALE = decltype(rescale_tag)::value;
        if (any) {
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int ow = owner(j), oi = 16 * ((j % JS) % JO) + l16;
                const float mt = fmaxf(xm[ow][oi], xm[ow + 2][oi]);
                const float mr = m_run[j];
                if constexpr (RESCALE) {
                    const bool up = mt > mr + kRescaleSlack;   // also from -inf
                    const float m_new = up ? mt : mr;
                    const float alpha = up ? fast_exp2(mr - m_new) : 1.0f;
                    m_run[j] = m_new;
                    if (__builtin_amdgcn_ballot_w64(up && mr != -INFINITY) != 0) {
#pragma unroll
                        for (int m = 0; m < PMW; ++m) acc[m][j] *= alpha;
                    }
#pragma unroll
                    for (int nt = 0; nt < JO; ++nt)
                        if (own_tile(nt) == j) l_run[nt] *= alpha;
                } else {
                    // only first maxima here: O and the sums of such a head
                    // are still zero, nothing to rescale
                    if (mr == -INFINITY && mt > -INFINITY) m_run[j] = mt;
                }
            }
            uint2 pt[NP][JO];
            float pr[JO][4];
            weights(st.x, st.csc, pr, pt);
#pragma unroll
            for (int nt = 0; nt < JO; ++nt) st.psum[nt] = (pr[nt][0] + pr[nt][1]) + (pr[nt][2] + pr[nt][3]);
            put_p(xq, pt);
            __syncthreads();
        }
        pv(cb, any ? xq : xp, dma_tile, nb3, nm3, r3);
#pragma unroll
        for (int nt = 0; nt < JO; ++nt) l_run[nt] += st.psum[nt];
    };

    // bf16: the first chunk's first two tiles go out now; their gathers are
    // in flight while the q fragments are read
    const bool early = KV == 0 && c_end > c_begin && cn0 <= 4 * NT && n_tiles > 0;
    if (early) {
        issue(tiles[0], metas[0], 0);
        if (n_tiles > 1) issue(tiles[1], metas[1], 1);
    }
#pragma unroll
    for (int j = 0; j < JS; ++j) {
        const int hr = 16 * (JS * gr + j) + l16;   // staging row (head within the block)
        const bool ok = hbase + hr < p.H;
        const uint8_t *row = qstage + hr * 2 * D;
#pragma unroll
        for (int s = 0; s < SH::SK; ++s) {
            const int c = (D / 16) * dq + 4 * s + g;
            qf[j][s] = ok ? *(const uint4 *)(row + 16 * (c ^ (hr & QSW))) : make_uint4(0, 0, 0, 0);
        }
    }

    using Fast = std::integral_constant<bool, false>;
    using Slow = std::integral_constant<bool, true>;
    // columns are taken in chunks whose row indices are staged in LDS
    for (; cc < c_end; cc += kIdxChunk) {
        const int cn = min(c_end - cc, kIdxChunk);
        const bool first = cc == c_begin;
        __syncthreads();   // the previous chunk's indices are no longer read
        if (!first) nval = 0;
        // (the first 4 NT columns of the first chunk were staged with q)
        for (int i0 = first ? 4 * NT : 0; i0 < cn; i0 += 4 * NT) {
            int iv[4];
            load4(cc, cn, i0, iv);
            stage4(cc, i0, iv);
        }
        if (!(first && cn <= 4 * NT)) pad();
        // a wait the compiler sees: Q and the index loads are complete, so no
        // wait for them is left inside the tile loops (s_waitcnt vmcnt(0))
        __builtin_amdgcn_s_waitcnt(0x0F70);
        __syncthreads();
        if (n_tiles == 0) continue;   // no valid column in this chunk
        // prologue: tiles 0 and 1 in LDS (bf16: tile 2 too), S of tile 0 and
        // its partial-score exchange (the first chunk's tiles 0 and 1 went
        // out with the q fragments; the barrier above also freed tile 2,
        // which held q)
        const bool issued = early && cc == c_begin;
        if (!issued) issue(tiles[0], metas[0], 0);
        if constexpr (KV == 2) {
            wait_vm<0>();
            land(tiles[0], metas[0]);
        }
        if (!issued && n_tiles > 1) issue(tiles[1], metas[1], 1);
        if constexpr (KV == 2) {
            wait_vm<0>();
            if (n_tiles > 1) land(tiles[1], metas[1]);
        } else {
            if (n_tiles > 2) issue(tiles[2], metas[2], 2);
            wait_vm<0>();
        }
        __syncthreads();
        f32x4 mine[JO];
        {
            Rows none;
            f32x4 sacc[JS];
            s_part(tiles[0], sacc, -1, tiles[0], metas[0], none, [](int) {});
            send_scores(sacc, mine);
        }
        __syncthreads();
        int bi[DEPTH];
#pragma unroll
        for (int k = 0; k < DEPTH; ++k) bi[k] = k;
        auto rotate = [&]() __attribute__((always_inline)) {
            const int b0 = bi[0];
#pragma unroll
            for (int k = 0; k + 1 < DEPTH; ++k) bi[k] = bi[k + 1];
            bi[DEPTH - 1] = b0;
        };
        Rows r3;   // row indices of tile t+3 (bf16)
        auto fr = [&](int it, Soft &st) __attribute__((always_inline)) {
            return front(it, metas[bi[0]], tiles[bi[1]], tiles[bi[2]], metas[bi[2]], tiles[bi[DEPTH - 1]],
                         metas[bi[DEPTH - 1]], st, mine, r3);
        };
        auto bk = [&](auto tag, int any, int it, Soft &st) __attribute__((always_inline)) {
            back(tag, any, tiles[bi[0]], st, it + 3, tiles[bi[DEPTH - 1]], metas[bi[DEPTH - 1]], r3);
            tail(it, tiles[bi[2]], metas[bi[2]]);
            rotate();
        };
        Soft st;
        int it = 0, any = 0;
        // fast loop: no rescale of O in its body (a max that grows by more
        // than the slack is rare and leaves for the loop below)
        for (; it < n_tiles; ++it) {
            any = fr(it, st);
            if (any & 2) break;
            bk(Fast{}, any, it, st);
        }
        if (it < n_tiles) {
            bk(Slow{}, any, it, st);
            for (++it; it < n_tiles; ++it) {
                any = fr(it, st);
                bk(Slow{}, any, it, st);
            }
        }
    }

    // softmax sums: owners reduce over their columns, everyone adds the two
    // column halves of each head in a fixed order
#pragma unroll
    for (int nt = 0; nt < JO; ++nt) {
        const float ls = group4_sum(l_run[nt]);
        if (g == 0) xl[w][16 * nt + l16] = ls;
    }
    __syncthreads();
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int head = hbase + 16 * j + l16;
        const int ow = owner(j), oi = 16 * ((j % JS) % JO) + l16;
        const float l_tot = xl[ow][oi] + xl[ow + 2][oi];
        if (head >= p.H) continue;
        const int d0 = (D / NW) * w + 4 * g;
        if (p.num_splits == 1) {
            const float inv = l_tot > 0.0f ? 1.0f / l_tot : 0.0f;
            if constexpr (OUT == 1) {
                float *o = (float *)p.out + (int64_t)t * p.out_st + (int64_t)head * p.out_sh + d0;
#pragma unroll
                for (int m = 0; m < PMW; ++m) {
                    const f32x4 v = acc[m][j] * inv;
                    *(float4 *)(o + 16 * m) = make_float4(v[0], v[1], v[2], v[3]);
                }
            } else {
                uint16_t *o = (uint16_t *)p.out + (int64_t)t * p.out_st + (int64_t)head * p.out_sh + d0;
#pragma unroll
                for (int m = 0; m < PMW; ++m) {
                    const f32x4 v = acc[m][j] * inv;
                    *(uint2 *)(o + 16 * m) = make_uint2(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]));
                }
            }
        } else {
            // partial outputs in the accumulators' own layout
            // [t][split][head block][w][m][j][lane] x 4 floats: each store
            // instruction writes 1 KiB of consecutive bytes
            const int64_t slot = ((int64_t)t * p.num_splits + split) * p.H + head;
            const int64_t pb = (((int64_t)t * p.num_splits + split) * gridDim.y + blockIdx.y) * NW + w;
#pragma unroll
            for (int m = 0; m < PMW; ++m)
                *(float4 *)(p.part_o + (((pb * PMW + m) * 4 + j) * 64 + lane) * 4) =
                    make_float4(acc[m][j][0], acc[m][j][1], acc[m][j][2], acc[m][j][3]);
            if (g == 0 && w == 0) *(float2 *)(p.part_ml + slot * 2) = make_float2(m_run[j], l_tot);
        }
    }
}

// out[t, h, :] = sum_j 2^(m_j - M) O_j / sum_j 2^(m_j - M) l_j over the splits
// j in order; zero when every split was empty.  The partial outputs are in
// the split kernel's accumulator layout [t][split][head block][w][m][j][lane]
// x 4 floats (NW split-kernel waves): one wave of this kernel takes one
// (head block, w, m, j) group, lane l owning head 16j + l%16 and head_dim
// 16m + 4(l/16) .. +3 of the split wave's range w,
// so its partial loads are 1 KiB contiguous per split.  The loads of U splits
// are issued before any is used: one memory round trip when the launch picks
// a U of at least the split count (up to kMergeSplits).
template <int D, int OUT, int NW, int U, int WPB>   // WPB waves per workgroup
__global__ __launch_bounds__(64 * WPB) void attn_merge_kernel(AttnParams p)
{
    constexpr int PM = D / (16 * NW);   // the split kernel's m-steps per wave
    const int t = blockIdx.x;
    const int grp = blockIdx.y * WPB + (threadIdx.x >> 6), lane = threadIdx.x & 63;
    const int HB = (p.H + kAttnHeadsPerBlock - 1) / kAttnHeadsPerBlock;
    if (grp >= HB * NW * PM * 4) return;
    const int j = grp % 4, m = (grp / 4) % PM, w = (grp / (4 * PM)) % NW, hb = grp / (4 * NW * PM);
    const int head = hb * kAttnHeadsPerBlock + 16 * j + (lane & 15);
    if (head >= p.H) return;
    const int d = (D / NW) * w + 16 * m + 4 * (lane >> 4);
    const int S = p.num_splits;
    const int64_t pstride = (int64_t)HB * NW * PM * 4 * 64;   // float4 slots per split
    const float4 *po = (const float4 *)p.part_o + ((int64_t)t * S) * pstride + (int64_t)grp * 64 + lane;
    const float2 *pml = (const float2 *)p.part_ml + ((int64_t)t * S) * p.H + head;
    // one pass: each batch's (max, sum) and partial loads go out together and
    // the running result is rescaled when a later batch raises the max
    float M = -INFINITY, L = 0.0f;
    float4 o = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int j0 = 0; j0 < S; j0 += U) {
        float2 ml[U];
        float4 v[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int js = min(j0 + u, S - 1);
            ml[u] = pml[(int64_t)js * p.H];
            v[u] = po[(int64_t)js * pstride];
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

template <int D, int KV, int OUT>
hipError_t launch_attn_t(const AttnParams &p, hipStream_t s)
{
    constexpr int NW = kAttnWaves;
    const dim3 grid((unsigned)(p.T * p.num_splits), (unsigned)((p.H + kAttnHeadsPerBlock - 1) / kAttnHeadsPerBlock));
    hipLaunchKernelGGL((attn_kernel<D, KV, OUT, NW>), grid, dim3(64 * NW), 0, s, p);
    return hipGetLastError();
}

template <int D>
hipError_t launch_attn_d(const AttnParams &p, int kv, int out, hipStream_t s)
{
    // head_dim 512: one split per token runs the one-barrier kernel of
    // attn_d512.hip; its split plans run attn_dec.hip (the plan never sends
    // head_dim 512 splits here)
    if constexpr (D == 512) {
        return p.num_splits == 1 ? launch_attn_d512(p, kv, out, s) : hipErrorInvalidValue;
    } else {
        if (kv == 0) return out == 1 ? launch_attn_t<D, 0, 1>(p, s) : launch_attn_t<D, 0, 0>(p, s);
        return out == 1 ? launch_attn_t<D, 2, 1>(p, s) : launch_attn_t<D, 2, 0>(p, s);
    }
}

template <int D, int NW>
hipError_t launch_merge_t(const AttnParams &p, int out, hipStream_t s)
{
    // one wave per (head block, w, m, j) group of the partial layout
    const int HB = (p.H + kAttnHeadsPerBlock - 1) / kAttnHeadsPerBlock;
    // (HB * NW * PMW * 4 groups, 4 per workgroup; NW * PMW = D / 16)
    // a launch of at most one wave per CU takes one-wave workgroups (its
    // waves land on as many CUs), larger ones four waves per workgroup
    const bool one = (int64_t)p.T * HB * (D / 16) * 4 <= 256;
    const dim3 grid((unsigned)p.T, (unsigned)(HB * (D / 16) * (one ? 4 : 1)));
    // the smallest batch of the split count (unused slots of a batch repeat
    // the last split's loads)
    auto go = [&](auto u_tag) {
        constexpr int U = decltype(u_tag)::value;
        if (one) {
            if (out == 1) hipLaunchKernelGGL((attn_merge_kernel<D, 1, NW, U, 1>), grid, dim3(64), 0, s, p);
            else hipLaunchKernelGGL((attn_merge_kernel<D, 0, NW, U, 1>), grid, dim3(64), 0, s, p);
        } else {
            if (out == 1) hipLaunchKernelGGL((attn_merge_kernel<D, 1, NW, U, 4>), grid, dim3(256), 0, s, p);
            else hipLaunchKernelGGL((attn_merge_kernel<D, 0, NW, U, 4>), grid, dim3(256), 0, s, p);
        }
    };
    const int S = p.num_splits;
    if (S <= 4) go(std::integral_constant<int, 4>{});
    else if (S <= 8) go(std::integral_constant<int, 8>{});
    else if (S <= 12) go(std::integral_constant<int, 12>{});
    else if (S <= 16) go(std::integral_constant<int, 16>{});
    else if (S <= 20) go(std::integral_constant<int, 20>{});
    else go(std::integral_constant<int, kMergeSplits>{});
    return hipGetLastError();
}

template <int D>
hipError_t launch_merge_d(const AttnParams &p, int, int out, hipStream_t s)
{
    // head_dim 512 splits are merged by attn_dec.hip's merge kernel
    if constexpr (D == 512) return hipErrorInvalidValue;
    else return launch_merge_t<D, kAttnWaves>(p, out, s);
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

hipError_t launch_attn_merge(const AttnParams &p, int D, int kv, int out, hipStream_t s)
{
    switch (D) {
    case 64: return launch_merge_d<64>(p, kv, out, s);
    case 128: return launch_merge_d<128>(p, kv, out, s);
    case 256: return launch_merge_d<256>(p, kv, out, s);
    case 512: return launch_merge_d<512>(p, kv, out, s);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace sap
