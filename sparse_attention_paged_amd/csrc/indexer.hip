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

__global__ __launch_bounds__(256) void indexer_kernel(IndexerParams p)
{
    __shared__ __attribute__((aligned(16))) uint32_t stage[4][kTileWords];
    const int b = blockIdx.y;
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int l32 = lane & 31, hh = lane >> 5;
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

    const int n_tiles = (p.N + kKeyTile - 1) / kKeyTile;
    const int tile0 = (blockIdx.x * 4 + wave) * p.tiles_per_wave;
    uint32_t *st = stage[wave];
    uint32_t regs[kWordsPerLane];

    // A tile of 64 keys starting at a multiple of 64 lies inside one page
    // when the page size is a multiple of 64: one (wave-uniform) page-table
    // read gives the pool row of its first key and the rest follow it.
    const bool page_tiles = p.pt == nullptr || p.page % kKeyTile == 0;
    // a full tile of 17-word rows is one contiguous 4352-byte block: 16-byte
    // loads (4 per lane) plus one word per lane instead of 17 word loads
    const bool vec_ok = page_tiles && p.row_words == kRowWords && (reinterpret_cast<uintptr_t>(p.pool) & 15u) == 0;
    bool vec = false;   // layout of regs for the tile in flight (wave-uniform)
    auto load_tile = [&](int kt) {
        const int key0 = kt * kKeyTile;
        int64_t row0 = (int64_t)b * p.N + key0;
        if (p.pt && page_tiles) {
            const int pg = key0 / p.page;
            row0 = (int64_t)p.pt[(int64_t)b * p.pt_sb + pg] * p.page + (key0 - pg * p.page);
        }
        vec = vec_ok && key0 + kKeyTile <= nk;
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
#pragma unroll
            for (int s = 0; s < 8; ++s) {
                const uint32_t word = r[2 * s + hh];
                const uint32_t e = (sw >> (8 * (s >> 1))) & 0xFFu;
                acc = mfma32x32x16(qa[s], fp4x8_to_bf16x8(word, e), acc);
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

}  // namespace

hipError_t launch_indexer(const IndexerParams &p, hipStream_t s)
{
    const int n_tiles = (p.N + kKeyTile - 1) / kKeyTile;
    const int waves = (n_tiles + p.tiles_per_wave - 1) / p.tiles_per_wave;
    const unsigned gx = (unsigned)((waves + 3) / 4);
    if (gx == 0 || p.B == 0) return hipSuccess;
    hipLaunchKernelGGL(indexer_kernel, dim3(gx, (unsigned)p.B), dim3(256), 0, s, p);
    return hipGetLastError();
}

}  // namespace sap
