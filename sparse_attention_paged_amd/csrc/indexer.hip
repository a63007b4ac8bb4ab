// indexer.hip -- indexer logits over fp4_e8m0_b32 packed key rows on gfx950.
//
// logits[b, n] = sum_h w[b, h] * max(0, q[b, h, :] . k_n) for n < n_keys[b],
// -inf beyond.  Key rows are 17 int32 words ("perf(kernel): read dsv41
// indexer key rows as int32 words", Changes): 16 words of e2m1 codes and one
// word of four ue8m0 block-32 scales.
//
// Each wave streams tiles of 64 keys: the tile's 64 x 17 words are read with
// coalesced dword loads (consecutive lanes, consecutive words) into a
// wave-private LDS area with a 17-word row pitch (odd, so the 32 rows read in
// one phase hit 32 distinct banks), the next tile's loads are in flight while
// the current one is scored.  In the MFMA 32x32x16 B-operand layout one lane
// needs exactly one word (8 consecutive head_dim elements of one key) per
// reduction step, decoded to 8 bf16 with the word's block scale.  The 32
// index heads are the M dimension, keys the N dimension; each lane ends with
// 16 heads of one key, applies ReLU and the head weights and adds the other
// half-wave's 16 heads.
#include "common.hpp"
#include "formats.hpp"
#include "internal.hpp"

#include <type_traits>

namespace sap {
namespace {

constexpr int kKeyTile = 64;
constexpr int kRowWords = 17;
constexpr int kTileWords = kKeyTile * kRowWords;         // 1088
constexpr int kWordsPerLane = kTileWords / kWave;         // 17

__device__ __forceinline__ void wave_lds_sync()
{
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// NWI waves per workgroup (1 or 4).  VEC: the host has checked that every
// tile is a whole one inside one page of 17-word rows on a 16-byte aligned
// pool (N a multiple of 64, pages a multiple of 64 rows or no page table), so
// every tile below the valid-key count loads as one contiguous block; the
// per-word path (and its registers) is compiled out.
template <int NWI, bool VEC>
__global__ __launch_bounds__(64 * NWI) void indexer_kernel(IndexerParams p)
{
    __shared__ __attribute__((aligned(16))) uint32_t stage[NWI][kTileWords];
    const int b = blockIdx.y;
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int l32 = lane & 31, hh = lane >> 5;
    const int n_tiles = (p.N + kKeyTile - 1) / kKeyTile;
    const int tile0 = (blockIdx.x * NWI + wave) * p.tiles_per_wave;
    // A tile of 64 keys starting at a multiple of 64 lies inside one page
    // when the page size is a multiple of 64: one (wave-uniform) page-table
    // read gives the pool row of its first key and the rest follow it.
    const bool page_tiles = p.pt == nullptr || p.page % kKeyTile == 0;
    // the first tile's page-table entry loads together with the valid-key
    // count (the page table holds an entry for every page below N), so the
    // key rows are one memory round trip after them, not two
    // (so is the second tile's: its rows then go out without waiting for a
    // page-table read)
    int pte0 = 0, pte1 = 0;
    if (p.pt && page_tiles && tile0 < n_tiles) pte0 = p.pt[(int64_t)b * p.pt_sb + tile0 * kKeyTile / p.page];
    if (p.pt && page_tiles && p.tiles_per_wave > 1 && tile0 + 1 < n_tiles)
        pte1 = p.pt[(int64_t)b * p.pt_sb + (tile0 + 1) * kKeyTile / p.page];
    const int nk = p.n_keys ? min(p.n_keys[b], p.N) : p.N;

    // q as the A operand: k-step s holds q[b, head l32, 16s + 8hh .. +7]
    uint4 qa[8];
    {
        const bool hok = l32 < p.Hi;
        const uint16_t *qr = p.q + (int64_t)b * p.q_sb + (int64_t)(hok ? l32 : 0) * 128;
#pragma unroll
        for (int s = 0; s < 8; ++s)
            qa[s] = hok ? *(const uint4 *)(qr + 16 * s + 8 * hh) : make_uint4(0, 0, 0, 0);
    }
    // head weights of this lane's 16 output rows: head = 8(i/4) + 4hh + i%4;
    // the 32 weights are wave-uniform loads, the half-wave picks its own
    float wv[16];
    {
        const float *wr = p.w + (int64_t)b * p.w_sb;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const int h0 = 8 * (i >> 2) + (i & 3), h1 = h0 + 4;
            const float w0 = h0 < p.Hi ? wr[h0] : 0.0f;
            const float w1 = h1 < p.Hi ? wr[h1] : 0.0f;
            wv[i] = hh ? w1 : w0;
        }
    }

    uint32_t *st = stage[wave];
    uint32_t regs[kWordsPerLane];
    // a full tile of 17-word rows is one contiguous 4352-byte block: 16-byte
    // loads (4 per lane) plus one word per lane instead of 17 word loads
    const bool vec_ok = VEC || (page_tiles && p.row_words == kRowWords && (reinterpret_cast<uintptr_t>(p.pool) & 15u) == 0);
    bool vec = false;   // layout of regs for the tile in flight (wave-uniform)
    auto load_tile = [&](int kt) {
        const int key0 = kt * kKeyTile;
        int64_t row0 = (int64_t)b * p.N + key0;
        if (p.pt && page_tiles) {
            const int pg = key0 / p.page;
            const int e = kt == tile0 ? pte0 : kt == tile0 + 1 ? pte1 : p.pt[(int64_t)b * p.pt_sb + pg];
            row0 = (int64_t)e * p.page + (key0 - pg * p.page);
        }
        // (VEC: a tile that holds the last valid key loads whole: its page
        // is a valid one and its rows exist; the keys past the count are
        // masked when the logits are written)
        vec = VEC ? key0 < nk : vec_ok && key0 + kKeyTile <= nk;
        if (vec) {
            const uint32_t *tp = (const uint32_t *)p.pool + row0 * kRowWords;
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                const uint4 v = *(const uint4 *)(tp + 4 * (lane + kWave * k));
                regs[4 * k] = v.x;
                regs[4 * k + 1] = v.y;
                regs[4 * k + 2] = v.z;
                regs[4 * k + 3] = v.w;
            }
            regs[16] = tp[4 * 4 * kWave + lane];
            return;
        }
        if constexpr (VEC) {
            // a tile past the valid keys: nothing is read, its logits are -inf
#pragma unroll
            for (int k = 0; k < kWordsPerLane; ++k) regs[k] = 0u;
            return;
        }
#pragma unroll
        for (int k = 0; k < kWordsPerLane; ++k) {
            const int i = lane + kWave * k;
            const int row = i / kRowWords;
            const int wd = i - row * kRowWords;
            const int n = key0 + row;
            uint32_t v = 0;
            if (n < nk) {
                int64_t prow = row0 + row;
                if (!page_tiles) prow = (int64_t)p.pt[(int64_t)b * p.pt_sb + n / p.page] * p.page + n % p.page;
                v = (uint32_t)p.pool[prow * p.row_words + wd];
            }
            regs[k] = v;
        }
    };

    if (tile0 < n_tiles) load_tile(tile0);
    for (int it = 0; it < p.tiles_per_wave; ++it) {
        const int kt = tile0 + it;
        if (kt >= n_tiles) break;
        if (vec) {
#pragma unroll
            for (int k = 0; k < 4; ++k)
                *(uint4 *)(st + 4 * (lane + kWave * k)) = make_uint4(regs[4 * k], regs[4 * k + 1], regs[4 * k + 2], regs[4 * k + 3]);
            st[4 * 4 * kWave + lane] = regs[16];
        } else {
#pragma unroll
            for (int k = 0; k < kWordsPerLane; ++k) st[lane + kWave * k] = regs[k];
        }
        wave_lds_sync();
        if (it + 1 < p.tiles_per_wave && kt + 1 < n_tiles) load_tile(kt + 1);

#pragma unroll
        for (int nt = 0; nt < 2; ++nt) {
            const uint32_t *r = st + (nt * 32 + l32) * kRowWords;
            const uint32_t sw = r[16];
            f32x16 acc = {};
            // the row's four scale bytes: when every lane's lie in 2..252 the
            // hardware scaled conversion is exact for all of them
            const uint32_t e0 = sw & 0xFFu, e1 = (sw >> 8) & 0xFFu, e2 = (sw >> 16) & 0xFFu, e3 = sw >> 24;
            const uint32_t emin = min(min(e0, e1), min(e2, e3)), emax = max(max(e0, e1), max(e2, e3));
            if (__builtin_amdgcn_ballot_w64(emin < 2u || emax > 252u) == 0) {
                const float sc[4] = {__uint_as_float(e0 << 23), __uint_as_float(e1 << 23), __uint_as_float(e2 << 23),
                                     __uint_as_float(e3 << 23)};
#pragma unroll
                for (int s = 0; s < 8; ++s) acc = mfma32x32x16(qa[s], fp4x8_scaled_bf16x8(r[2 * s + hh], sc[s >> 1]), acc);
            } else {
#pragma unroll
                for (int s = 0; s < 8; ++s) {
                    const uint32_t word = r[2 * s + hh];
                    const uint32_t e = (sw >> (8 * (s >> 1))) & 0xFFu;
                    acc = mfma32x32x16(qa[s], fp4x8_to_bf16x8(word, e), acc);
                }
            }
            float part = 0.0f;
#pragma unroll
            for (int i = 0; i < 16; ++i) part += wv[i] * fmaxf(acc[i], 0.0f);
            part += shfl_xor(part, 32);
            const int n = kt * kKeyTile + nt * 32 + l32;
            if (hh == 0 && n < p.N) p.logits[(int64_t)b * p.logits_sb + n] = n < nk ? part : -INFINITY;
        }
        wave_lds_sync();
    }
}

// ---------------------------------------------------------------------------
// Candidate and prefill modes.  Both read key rows straight into registers
// with a permuted reduction order: in MFMA step s, lane half hh covers
// head_dim elements 64hh + 8s .. 64hh + 8s + 7 (the sum over head_dim does not
// depend on the order).  A lane's B operands over the 8 steps are then the
// code words 8hh .. 8hh+7 of one key row (two 16-byte loads) with scale bytes
// 2hh and 2hh+1 of word 16, and its A operands the q elements 64hh .. 64hh+63
// of one head.

typedef uint32_t u32x4_a4 __attribute__((ext_vector_type(4), aligned(4)));

// raw words of one lane's half of a key row
struct KeyHalf {
    u32x4_a4 lo, hi;
    uint32_t sc;
};

__device__ __forceinline__ void load_key_half(const int32_t *row, int hh, KeyHalf &k)
{
    const u32x4_a4 *p = reinterpret_cast<const u32x4_a4 *>(row + 8 * hh);
    k.lo = p[0];
    k.hi = p[1];
    k.sc = (uint32_t)row[16];
}

__device__ __forceinline__ void zero_key_half(KeyHalf &k)
{
    k.lo = u32x4_a4{0, 0, 0, 0};
    k.hi = u32x4_a4{0, 0, 0, 0};
    k.sc = 0x7F7F7F7Fu;   // scale 1: zero codes decode to +0 on the fast path
}

// B operands of the 8 steps: word 8hh + s with scale byte 2hh + s/4.  When
// every lane's two scale bytes lie in 2..252 (the usual case) the hardware
// scaled conversion is exact and is used directly, else each word takes the
// general decode.
__device__ __forceinline__ void decode_key_half(const KeyHalf &k, int hh, uint4 (&b)[8])
{
    const uint32_t e0 = (k.sc >> (16 * hh)) & 0xFFu, e1 = (k.sc >> (16 * hh + 8)) & 0xFFu;
    const bool fast = e0 - 2u <= 250u && e1 - 2u <= 250u;
    if (__builtin_amdgcn_ballot_w64(!fast) == 0) {
        const float s0 = __uint_as_float(e0 << 23), s1 = __uint_as_float(e1 << 23);
        const uint32_t w[8] = {k.lo.x, k.lo.y, k.lo.z, k.lo.w, k.hi.x, k.hi.y, k.hi.z, k.hi.w};
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const float sc = i < 4 ? s0 : s1;
            b[i].x = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w[i], sc, 0));
            b[i].y = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w[i], sc, 1));
            b[i].z = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w[i], sc, 2));
            b[i].w = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w[i], sc, 3));
        }
        return;
    }
    b[0] = fp4x8_to_bf16x8(k.lo.x, e0);
    b[1] = fp4x8_to_bf16x8(k.lo.y, e0);
    b[2] = fp4x8_to_bf16x8(k.lo.z, e0);
    b[3] = fp4x8_to_bf16x8(k.lo.w, e0);
    b[4] = fp4x8_to_bf16x8(k.hi.x, e1);
    b[5] = fp4x8_to_bf16x8(k.hi.y, e1);
    b[6] = fp4x8_to_bf16x8(k.hi.z, e1);
    b[7] = fp4x8_to_bf16x8(k.hi.w, e1);
}

// the logit of this lane's key (column l32 of a 32x32 score block): its own
// 16 heads 8(i/4) + 4hh + i%4 plus the other half's 16
__device__ __forceinline__ float head_sum(const f32x16 &acc, const float (&wv)[16])
{
    float part = 0.0f;
#pragma unroll
    for (int i = 0; i < 16; ++i) part = fmaf(wv[i], fmaxf(acc[i], 0.0f), part);
    const uint32_t u = __float_as_uint(part);
    const auto x = __builtin_amdgcn_permlane32_swap(u, u, false, false);
    return __uint_as_float(x[0]) + __uint_as_float(x[1]);
}

// weights of the lane's 16 output heads, from a token's 32 weights
__device__ __forceinline__ void lane_weights(const float *wr, int Hi, int hh, float (&wv)[16])
{
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        const int h0 = 8 * (i >> 2) + (i & 3), h1 = h0 + 4;
        const float w0 = h0 < Hi ? wr[h0] : 0.0f;
        const float w1 = h1 < Hi ? wr[h1] : 0.0f;
        wv[i] = hh ? w1 : w0;
    }
}

// Candidate mode: one query token per blockIdx.y, scoring the keys listed in
// its candidate row.  Each wave takes a run of 64-candidate tiles; the pool
// rows of up to kCandChunk tiles are resolved first (all candidate loads,
// then all page-table loads: two memory round trips per chunk), then the
// tiles stream through registers with the next tile's rows in flight while
// the current one is scored.
constexpr int kCandChunk = 8;

// page-table entries of one sequence staged in LDS by the candidate kernel
constexpr int kCandPtLds = 4096;

__global__ __launch_bounds__(256) void indexer_cand_kernel(IndexerParams p)
{
    __shared__ int rowtab[4][kCandChunk * kKeyTile];
    __shared__ int ptab[kCandPtLds];
    const int t = blockIdx.y;
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int l32 = lane & 31, hh = lane >> 5;
    const int nk = p.n_keys ? p.n_keys[t] : 0x7FFFFFFF;

    uint4 qa[8];
    {
        const bool hok = l32 < p.Hi;
        const uint16_t *qr = p.q + (int64_t)t * p.q_sb + (int64_t)(hok ? l32 : 0) * 128 + 64 * hh;
#pragma unroll
        for (int s = 0; s < 8; ++s) qa[s] = hok ? *(const uint4 *)(qr + 8 * s) : make_uint4(0, 0, 0, 0);
    }
    float wv[16];
    lane_weights(p.w + (int64_t)t * p.w_sb, p.Hi, hh, wv);

    const int n_tiles = (p.N + kKeyTile - 1) / kKeyTile;
    const int tile0 = (blockIdx.x * 4 + wave) * p.tiles_per_wave;
    const int tile_end = min(tile0 + p.tiles_per_wave, n_tiles);
    const int32_t *cr = p.cand + (int64_t)t * p.cand_sb;
    float *out = p.logits + (int64_t)t * p.logits_sb;
    int *rt = rowtab[wave];

    // candidate positions of chunk c0: (c0 + j) * 64 + lane, -1 = none
    int cv[kCandChunk];
    auto load_cand = [&](int c0) __attribute__((always_inline)) {
        const int nc = min(kCandChunk, tile_end - c0);
#pragma unroll
        for (int j = 0; j < kCandChunk; ++j) {
            const int c = (c0 + j) * kKeyTile + lane;
            cv[j] = (j < nc && c < p.N) ? cr[c] : -1;
        }
    };
    // The first chunk's candidates and, when the sequence's pages are known
    // (n_keys), few enough and fewer than the workgroup's candidates, its
    // page-table entries go out in the same memory round trip; rows are then
    // found from LDS.
    if (tile0 < tile_end) load_cand(tile0);
    const int *pt_row = p.pt ? p.pt + (int64_t)t * p.pt_sb : nullptr;
    const int64_t npg = p.pt && p.n_keys ? ((int64_t)max(nk, 0) + p.page - 1) / p.page : 0;
    // (only when the workgroup's candidates outnumber the pages: a workgroup
    // of a few tiles reads fewer entries looking each one up)
    const bool pt_lds = p.pt && p.n_keys && npg <= kCandPtLds &&
                        (int64_t)p.tiles_per_wave * kKeyTile * 4 >= npg;   // uniform over the workgroup
    if (pt_lds) {
        // every load goes out before any is written (a loop that waited for
        // each load in turn made one round trip per entry group)
        constexpr int PPT = kCandPtLds / 256;
        int pv[PPT];
#pragma unroll
        for (int k = 0; k < PPT; ++k) {
            const int i = (int)threadIdx.x + 256 * k;
            pv[k] = i < (int)npg ? pt_row[i] : 0;
        }
#pragma unroll
        for (int k = 0; k < PPT; ++k) {
            const int i = (int)threadIdx.x + 256 * k;
            if (i < (int)npg) ptab[i] = pv[k];
        }
        __syncthreads();
    }
    const int psh = (p.page & (p.page - 1)) == 0 ? 31 - __builtin_clz((uint32_t)p.page) : -1;

    for (int c0 = tile0; c0 < tile_end; c0 += kCandChunk) {
        const int nc = min(kCandChunk, tile_end - c0);
        if (c0 != tile0) load_cand(c0);
#pragma unroll
        for (int j = 0; j < kCandChunk; ++j) {
            const int n = cv[j];
            int r = -1;
            if (n >= 0 && n < nk) {
                if (!p.pt) r = n;
                else {
                    const int pg = psh >= 0 ? n >> psh : n / p.page;
                    const int off = psh >= 0 ? n & (p.page - 1) : n - pg * p.page;
                    r = (pt_lds ? ptab[pg] : pt_row[pg]) * p.page + off;
                }
            }
            rt[j * kKeyTile + lane] = r;
        }
        wave_lds_sync();
        KeyHalf kh[2];
        auto load = [&](int j) __attribute__((always_inline)) {
#pragma unroll
            for (int nt = 0; nt < 2; ++nt) {
                const int r = rt[j * kKeyTile + 32 * nt + l32];
                if (r >= 0) load_key_half(p.pool + (int64_t)r * p.row_words, hh, kh[nt]);
                else zero_key_half(kh[nt]);
            }
        };
        load(0);
        for (int j = 0; j < nc; ++j) {
            uint4 kb[2][8];
            decode_key_half(kh[0], hh, kb[0]);
            decode_key_half(kh[1], hh, kb[1]);
            const int r0 = rt[j * kKeyTile + l32], r1 = rt[j * kKeyTile + 32 + l32];
            if (j + 1 < nc) load(j + 1);
#pragma unroll
            for (int nt = 0; nt < 2; ++nt) {
                f32x16 acc = {};
#pragma unroll
                for (int s = 0; s < 8; ++s) acc = mfma32x32x16(qa[s], kb[nt][s], acc);
                const float logit = head_sum(acc, wv);
                const int c = (c0 + j) * kKeyTile + 32 * nt + l32;
                if (hh == 0 && c < p.N) out[c] = (nt ? r1 : r0) >= 0 ? logit : -INFINITY;
            }
        }
        wave_lds_sync();   // the row table is rewritten by the next chunk
    }
}

// Prefill mode: a workgroup takes kPfTok consecutive query tokens of one
// sequence and a chunk of kc keys.  The tokens' q (64 KiB, 16-byte chunks
// swizzled by head so the A-operand reads are conflict-free) and weights are
// staged in LDS once; each wave decodes a 64-key sub-tile into registers and
// scores it for every token of the workgroup (16 MFMAs per token), so a key
// is decoded once per 8 tokens; the next sub-tile's rows load meanwhile and
// each token's epilogue overlaps the next token's MFMAs.  Keys at or beyond a token's visible count
// are -inf (the causal mask); sub-tiles beyond every token's count are only
// filled with -inf.
constexpr int kPfTok = 8;
constexpr int kPfPass = 4 * kKeyTile;

__global__ __launch_bounds__(256, 2) void indexer_prefill_kernel(IndexerPrefillParams p)
{
    __shared__ __attribute__((aligned(16))) uint4 qs[kPfTok][32][16];
    __shared__ __attribute__((aligned(16))) float ws[kPfTok][32];
    __shared__ int nks[kPfTok];
    const int sq = blockIdx.z;
    const int ta = p.tok_start[sq], tb = p.tok_start[sq + 1];
    // token tiles with the most visible keys are dispatched first
    const int t0 = ta + ((int)gridDim.y - 1 - (int)blockIdx.y) * kPfTok;
    if (t0 >= tb) return;
    const int ntok = min(kPfTok, tb - t0);
    const int k0 = blockIdx.x * p.kc, k1 = min(p.N, k0 + p.kc);
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int l32 = lane & 31, hh = lane >> 5;

    for (int i = tid; i < kPfTok * 32 * 16; i += 256) {
        const int j = i >> 9, h = (i >> 4) & 31, c = i & 15;
        uint4 v = make_uint4(0, 0, 0, 0);
        if (j < ntok && h < p.Hi) v = *(const uint4 *)(p.q + (int64_t)(t0 + j) * p.q_st + h * 128 + 8 * c);
        qs[j][h][c ^ (h & 15)] = v;
    }
    {
        const int j = tid >> 5, h = tid & 31;
        ws[j][h] = (j < ntok && h < p.Hi) ? p.w[(int64_t)(t0 + j) * p.w_st + h] : 0.0f;
    }
    if (tid < kPfTok) {
        int v = 0;
        if (tid < ntok) v = min(max(p.n_keys ? p.n_keys[t0 + tid] : p.N, 0), p.N);
        nks[tid] = v;
    }
    __syncthreads();
    int nk[kPfTok];
    int kmax = 0;
#pragma unroll
    for (int j = 0; j < kPfTok; ++j) {
        nk[j] = __builtin_amdgcn_readfirstlane(nks[j]);
        kmax = max(kmax, nk[j]);
    }
    const int32_t *ptr = p.pt ? p.pt + (int64_t)sq * p.pt_ss : nullptr;
    const bool page_tiles = ptr == nullptr || p.page % kKeyTile == 0;

    // raw rows of keys kb0 + 32 nt + l32 (zero beyond kmax)
    auto load_keys = [&](int kb0, KeyHalf (&kh)[2]) __attribute__((always_inline)) {
        int64_t row0 = (int64_t)sq * p.N + kb0;
        if (ptr && page_tiles) {
            const int pg = kb0 / p.page;
            row0 = (int64_t)ptr[pg] * p.page + (kb0 - pg * p.page);
        }
#pragma unroll
        for (int nt = 0; nt < 2; ++nt) {
            const int n = kb0 + 32 * nt + l32;
            if (n < kmax) {
                int64_t row = row0 + 32 * nt + l32;
                if (!page_tiles) row = (int64_t)ptr[n / p.page] * p.page + n % p.page;
                load_key_half(p.pool + row * p.row_words, hh, kh[nt]);
            } else {
                zero_key_half(kh[nt]);
            }
        }
    };
    // this wave's sub-tile of the next pass is in flight while the current
    // one is scored
    KeyHalf kh[2];
    if (k0 + kKeyTile * wave < min(k1, kmax)) load_keys(k0 + kKeyTile * wave, kh);

    for (int pb = k0; pb < k1; pb += kPfPass) {
        const int kb0 = pb + kKeyTile * wave;
        if (kb0 >= k1) break;
        const int kend = min(kb0 + kKeyTile, k1);
        if (kb0 >= kmax) {
            // no token of the tile sees these keys
            for (int j = 0; j < ntok; ++j)
                if (kb0 + lane < kend) p.logits[(int64_t)(t0 + j) * p.logits_st + kb0 + lane] = -INFINITY;
            continue;
        }
        uint4 kb[2][8];
        decode_key_half(kh[0], hh, kb[0]);
        decode_key_half(kh[1], hh, kb[1]);
        if (kb0 + kPfPass < min(k1, kmax)) load_keys(kb0 + kPfPass, kh);

        // every token slot of the tile is scored (q and w are zero for absent
        // tokens, whose stores are skipped); the MFMAs of token j+1 go out
        // ahead of the epilogue of token j
        f32x16 acc[2][2];
        auto mm = [&](int j, f32x16 (&a2)[2]) __attribute__((always_inline)) {
            a2[0] = f32x16{};
            a2[1] = f32x16{};
#pragma unroll
            for (int s = 0; s < 8; ++s) {
                const uint4 a = qs[j][l32][(8 * hh + s) ^ (l32 & 15)];
                a2[0] = mfma32x32x16(a, kb[0][s], a2[0]);
                a2[1] = mfma32x32x16(a, kb[1][s], a2[1]);
            }
        };
        mm(0, acc[0]);
#pragma unroll
        for (int j = 0; j < kPfTok; ++j) {
            if (j + 1 < kPfTok) mm(j + 1, acc[(j + 1) & 1]);
            float wv[16];
#pragma unroll
            for (int m = 0; m < 4; ++m) {
                const float4 w4 = *(const float4 *)&ws[j][8 * m + 4 * hh];
                wv[4 * m] = w4.x;
                wv[4 * m + 1] = w4.y;
                wv[4 * m + 2] = w4.z;
                wv[4 * m + 3] = w4.w;
            }
            const float g0 = head_sum(acc[j & 1][0], wv), g1 = head_sum(acc[j & 1][1], wv);
            const int n0 = kb0 + l32, n1 = kb0 + 32 + l32;
            float *orow = p.logits + (int64_t)(t0 + j) * p.logits_st;
            if (hh == 0 && j < ntok) {
                if (n0 < kend) orow[n0] = n0 < nk[j] ? g0 : -INFINITY;
                if (n1 < kend) orow[n1] = n1 < nk[j] ? g1 : -INFINITY;
            }
        }
    }
}

}  // namespace

int indexer_prefill_chunk(int S, int max_tokens, int N)
{
    // about 2048 workgroups (8 per CU): split the keys into chunks of whole
    // 256-key passes
    const int64_t tiles = (int64_t)S * ((max_tokens + kPfTok - 1) / kPfTok);
    const int64_t passes = ((int64_t)N + kPfPass - 1) / kPfPass;
    if (tiles <= 0 || passes <= 0) return kPfPass;
    int64_t chunks = (2048 + tiles - 1) / tiles;
    if (chunks > passes) chunks = passes;
    if (chunks < 1) chunks = 1;
    return (int)((passes + chunks - 1) / chunks) * kPfPass;
}

hipError_t launch_indexer_prefill(const IndexerPrefillParams &p, hipStream_t s)
{
    const unsigned gx = (unsigned)((p.N + p.kc - 1) / p.kc);
    const unsigned gy = (unsigned)((p.max_tokens + kPfTok - 1) / kPfTok);
    if (gx == 0 || gy == 0 || p.S == 0) return hipSuccess;
    hipLaunchKernelGGL(indexer_prefill_kernel, dim3(gx, gy, (unsigned)p.S), dim3(256), 0, s, p);
    return hipGetLastError();
}

hipError_t launch_indexer_candidates(const IndexerParams &p, hipStream_t s)
{
    const int n_tiles = (p.N + kKeyTile - 1) / kKeyTile;
    const int waves = (n_tiles + p.tiles_per_wave - 1) / p.tiles_per_wave;
    const unsigned gx = (unsigned)((waves + 3) / 4);
    if (gx == 0 || p.B == 0) return hipSuccess;
    hipLaunchKernelGGL(indexer_cand_kernel, dim3(gx, (unsigned)p.B), dim3(256), 0, s, p);
    return hipGetLastError();
}

hipError_t launch_indexer(const IndexerParams &p, hipStream_t s)
{
    const int n_tiles = (p.N + kKeyTile - 1) / kKeyTile;
    const int waves = (n_tiles + p.tiles_per_wave - 1) / p.tiles_per_wave;
    if (waves == 0 || p.B == 0) return hipSuccess;
    // a launch of at most one wave per CU spreads its waves over as many CUs
    // (decode B1 over 8192 keys: 4.35 us against 4.7 with four-wave
    // workgroups); larger launches keep four waves per workgroup
    const bool vec = p.N % kKeyTile == 0 && p.row_words == kRowWords &&
                     (reinterpret_cast<uintptr_t>(p.pool) & 15u) == 0 && (p.pt == nullptr || p.page % kKeyTile == 0);
    auto go = [&](auto vec_tag) {
        constexpr bool V = decltype(vec_tag)::value;
        if ((int64_t)waves * p.B <= 256) {
            hipLaunchKernelGGL((indexer_kernel<1, V>), dim3((unsigned)waves, (unsigned)p.B), dim3(64), 0, s, p);
        } else {
            const unsigned gx = (unsigned)((waves + 3) / 4);
            hipLaunchKernelGGL((indexer_kernel<4, V>), dim3(gx, (unsigned)p.B), dim3(256), 0, s, p);
        }
    };
    if (vec) go(std::true_type{});
    else go(std::false_type{});
    return hipGetLastError();
}

}  // namespace sap
