// internal.hpp -- parameter blocks and launchers shared between the C-ABI
// layer (sap_abi.hip) and the kernel translation units.  Not installed.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace sap {

constexpr int kAttnTile = 32;        // gathered columns per LDS tile
constexpr int kAttnHeadsPerBlock = 64;

struct AttnParams {
    const uint16_t *q;               // bf16 [T, H, D]
    int64_t q_st, q_sh;              // element strides
    const uint8_t *win;              // pool bases and row strides (bytes)
    const uint8_t *cmp;
    int64_t win_rs, cmp_rs;
    const float *win_scale, *cmp_scale;
    const int32_t *idx;
    int64_t idx_st;
    int n_win, n_cols;
    void *out;
    int64_t out_st, out_sh;
    int T, H;
    float sm_scale_log2;             // sm_scale * log2(e)
    int num_splits, cols_per_split;  // cols_per_split: multiple of kAttnTile (decode kernel: of kDecRound)
    float *part_o;                   // [T, S, H, D] unnormalised partial outputs (decode kernel: its own layout, f16 for bf16 rows)
    float *part_ml;                  // [T, S, H, 2] running max (log2 domain), sum
    int hgroups;                     // decode kernel: head groups of kDecHeads
};

// decode kernel (attn_dec.hip, head_dim 512): heads per workgroup and
// columns per round (32 per wave)
constexpr int kDecHeads = 16;
constexpr int kDecRound = 128;

// splits whose partial outputs the merge reads in one memory round trip
// (more take further passes)
constexpr int kMergeSplits = 24;

// kv: 0 = bf16, 2 = e4m3.  out: 0 = bf16, 1 = f32.
hipError_t launch_attn(const AttnParams &p, int D, int kv, int out_dtype, hipStream_t s);
hipError_t launch_attn_merge(const AttnParams &p, int D, int kv, int out_dtype, hipStream_t s);
// bf16 or e4m3 rows (kv 0 or 2) at head_dim 512 with one split per token
// (attn_d512.hip); launch_attn dispatches to it
hipError_t launch_attn_d512(const AttnParams &p, int kv, int out_dtype, hipStream_t s);
// split-K decode at head_dim 512 (attn_dec.hip) and its merge
hipError_t launch_attn_dec(const AttnParams &p, int kv, int out_dtype, hipStream_t s);
hipError_t launch_attn_dec_merge(const AttnParams &p, int kv, int out_dtype, hipStream_t s);
// waves per workgroup of the tiled attention kernel (head_dims below 512),
// whose layout its split partials follow
constexpr int kAttnWaves = 4;

struct IndexerParams {
    const uint16_t *q;               // bf16 [B, Hi, 128]
    int64_t q_sb;
    const float *w;
    int64_t w_sb;
    const int32_t *pool;
    int64_t row_words;
    const int32_t *pt;               // may be null
    int64_t pt_sb;
    int page;
    const int32_t *n_keys;           // may be null
    float *logits;
    int64_t logits_sb;
    int B, Hi, N;
    int tiles_per_wave;
    const int32_t *cand;             // candidate mode: [B, N] logical key positions (-1 = none)
    int64_t cand_sb;
};
hipError_t launch_indexer(const IndexerParams &p, hipStream_t s);
hipError_t launch_indexer_candidates(const IndexerParams &p, hipStream_t s);

struct IndexerPrefillParams {
    const uint16_t *q;               // bf16 [T, Hi, 128]
    int64_t q_st;
    const float *w;                  // [T, Hi]
    int64_t w_st;
    const int32_t *pool;
    int64_t row_words;
    const int32_t *pt;               // [S, pages] (may be null: rows s * N + n)
    int64_t pt_ss;
    int page;
    const int32_t *tok_start;        // [S + 1]
    const int32_t *n_keys;           // [T] visible keys per token (may be null: N)
    float *logits;                   // [T, N]
    int64_t logits_st;
    int S, max_tokens, Hi, N;
    int kc;                          // keys per workgroup (multiple of 256)
};
int indexer_prefill_chunk(int S, int max_tokens, int N);

struct GatedPoolParams {
    const void *x;                   // [B, R, D] bf16 or fp32, element strides
    int64_t x_sb, x_sr;
    const void *g;                   // gate scores [B, R, D] bf16 or fp32
    int64_t g_sb, g_sr;
    void *out;                       // [B, D] bf16 or fp32
    int64_t out_sb;
    int B, R, D;
    int x_bf16, g_bf16, out_bf16;
};
hipError_t launch_gated_pool(const GatedPoolParams &p, hipStream_t s);
hipError_t launch_indexer_prefill(const IndexerPrefillParams &p, hipStream_t s);

struct TopkParams {
    const float *x;
    int64_t x_sb;
    const int32_t *n_valid;
    int B, N, k;
    int32_t *out;
    int64_t out_sb;
    void *workspace;                 // topk_workspace_bytes(B, N, k) bytes
    // fused index build (idx != null): row b of idx [B, n_win + k] receives
    // the window rows of position pos[b] and the selected entries mapped
    // through page table row seq[b] (out is unused)
    int32_t *idx;
    int64_t idx_st;
    const int32_t *pos, *seq;
    int n_win, page;
    const int32_t *win_pt, *cmp_pt;
    int64_t win_pt_sb, cmp_pt_sb;
};
size_t topk_workspace_bytes(int B, int N, int k);
hipError_t launch_topk(const TopkParams &p, hipStream_t s);

struct IdxBuildParams {
    const int32_t *pos, *seq;
    int T, n_win;
    const int32_t *win_pt;
    int64_t win_pt_sb;
    int page;
    const int32_t *cmp_logical;
    int64_t cmp_logical_st;
    int n_cmp;
    const int32_t *cmp_pt;
    int64_t cmp_pt_sb;
    int32_t *idx;
    int64_t idx_st;
};
hipError_t launch_build_idx(const IdxBuildParams &p, hipStream_t s);

hipError_t launch_debug_e4m3(uint16_t *out, float *fold, hipStream_t s);
hipError_t launch_debug_e4m3_f16(uint16_t *out, hipStream_t s);
hipError_t launch_debug_fp4(uint16_t *out, hipStream_t s);

}  // namespace sap
