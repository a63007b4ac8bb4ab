// sap_abi.hip -- the C ABI declared in include/sap.h: argument validation
// (every check runs on the host before any HIP call, so a rejected call
// launches nothing and touches no device), split planning, workspace sizing
// and kernel dispatch onto the caller's stream.
#include "sap.h"

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <mutex>

#include "internal.hpp"

namespace {

inline bool aligned(const void *p, uintptr_t a) { return ((uintptr_t)p & (a - 1)) == 0; }
inline size_t align256(size_t x) { return (x + 255) / 256 * 256; }
inline int dtype_size(int dt) { return dt == SAP_BF16 ? 2 : dt == SAP_F32 ? 4 : dt == SAP_FP8_E4M3 ? 1 : 0; }

// How a sparse attention call runs:
//  - ONEPASS: one pass per token (the prefill launch): at head_dim 512 with
//    bf16 rows the persistent one-barrier kernel, else the tiled kernel;
//  - DEC: the decode kernel at head_dim 512 (16 heads per workgroup, rounds
//    of 128 columns), `splits` column ranges per token, merged when > 1;
//  - SPLITK: other head_dims with several splits: the tiled kernel per
//    split, then its merge.
enum PlanKind { PLAN_ONEPASS = 0, PLAN_DEC = 1, PLAN_SPLITK = 2 };

struct SplitPlan {
    int kind;
    int splits;
    int cols_per_split;
};

// Decode workgroups hold 149 KiB of LDS each, so one fits on a CU: a launch
// of more than 256 runs the rest only as the first ones finish.  The split
// count keeps T * head groups * splits within kDecResident; a batch with at
// least kDecOnePass token x head-group pairs runs the one-pass kernel.
constexpr int kDecResident = 256;
constexpr int kDecOnePass = 512;

// Splitting a token's columns buys parallelism for decode, where a few tokens
// would otherwise occupy a few CUs; each split costs a partial output of H*D
// floats, so prefill-sized batches keep one split.
SplitPlan plan_splits(int T, int H, int D, int n_cols, int requested)
{
    SplitPlan p;
    if (D == 512 && requested != 1) {
        const int G = (H + sap::kDecHeads - 1) / sap::kDecHeads;
        const int rounds = n_cols > 0 ? (n_cols + sap::kDecRound - 1) / sap::kDecRound : 1;
        const int64_t tg = (int64_t)T * G;
        int s;
        if (requested >= 2) {
            s = requested;
        } else {
            // a batch that fills the GPU with one split per token runs the
            // one-pass kernel; smaller ones split the columns so the launch
            // has up to kDecResident workgroups (all resident at once), one
            // round each while that fits
            if (tg >= kDecOnePass) {
                p.kind = PLAN_ONEPASS;
                p.splits = 1;
                p.cols_per_split = n_cols;
                return p;
            }
            s = (int)(kDecResident / tg);
        }
        if (s > rounds) s = rounds;
        if (s < 1) s = 1;
        const int rps = (rounds + s - 1) / s;
        p.kind = PLAN_DEC;
        p.cols_per_split = rps * sap::kDecRound;
        p.splits = n_cols > 0 ? (n_cols + p.cols_per_split - 1) / p.cols_per_split : 1;
        return p;
    }
    const int tiles = n_cols > 0 ? (n_cols + sap::kAttnTile - 1) / sap::kAttnTile : 1;
    int s;
    if (requested >= 1) {
        s = requested;
    } else {
        const int hb = (H + sap::kAttnHeadsPerBlock - 1) / sap::kAttnHeadsPerBlock;
        const int64_t wgs = (int64_t)T * hb;
        // one 32-column tile per split while the launch stays within about
        // 128 workgroups and the merge reads every split in one round trip;
        // past that, the fewest tiles per split that keep within both
        s = wgs >= 128 ? 1 : (int)(128 / wgs);
        if (s > sap::kMergeSplits) s = sap::kMergeSplits;
    }
    if (s > tiles) s = tiles;
    if (s < 1) s = 1;
    const int tiles_per = (tiles + s - 1) / s;
    p.cols_per_split = tiles_per * sap::kAttnTile;
    p.splits = n_cols > 0 ? (n_cols + p.cols_per_split - 1) / p.cols_per_split : 1;
    p.kind = p.splits > 1 ? PLAN_SPLITK : PLAN_ONEPASS;
    if (p.kind == PLAN_ONEPASS) p.cols_per_split = n_cols;
    return p;
}

// partial-output bytes of a plan, then (max, sum) per head
size_t attn_ws_bytes(int T, int H, int D, const SplitPlan &sp)
{
    if (sp.splits <= 1) return 0;
    const size_t slots = (size_t)T * sp.splits * H;
    size_t oslots;
    if (sp.kind == PLAN_DEC)
        oslots = (size_t)T * sp.splits * ((H + sap::kDecHeads - 1) / sap::kDecHeads) * sap::kDecHeads;
    else
        oslots = (size_t)T * sp.splits * ((H + sap::kAttnHeadsPerBlock - 1) / sap::kAttnHeadsPerBlock) *
                 sap::kAttnHeadsPerBlock;
    return align256(oslots * D * 4) + align256(slots * 2 * 4);
}

inline int launched(hipError_t e) { return e == hipSuccess ? SAP_OK : SAP_ERR_LAUNCH; }

// waves a full-mode indexer launch is sized to (four per SIMD of 256 CUs)
#ifndef SAP_INDEXER_WAVES
#define SAP_INDEXER_WAVES 4096
#endif
constexpr int64_t kIndexerWaves = SAP_INDEXER_WAVES;

// The allocation-free entry point keeps its split partials in this array
// (each GPU the library runs on holds its own copy until the process ends).
// Host code must not use the array's name as a device address: its device
// address comes from hipGetSymbolAddress, taken once per device.
constexpr size_t kScratchBytes = (size_t)32 << 20;
constexpr int kMaxDevices = 64;

}  // namespace

static __device__ __align__(256) uint8_t scratch[kScratchBytes];

namespace {

std::mutex scratch_mu;
void *scratch_ptr[kMaxDevices];

// this device's address of `scratch`, looked up on its first use (with the
// device current); NULL if the runtime refuses
void *device_scratch()
{
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
    std::lock_guard<std::mutex> lock(scratch_mu);
    if (!scratch_ptr[dev]) {
        void *ptr = nullptr;
        if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) return nullptr;
        scratch_ptr[dev] = ptr;
    }
    return scratch_ptr[dev];
}

}  // namespace

extern "C" {

int sap_version(void) { return 100; }

const char *sap_status_string(int status)
{
    switch (status) {
    case SAP_OK: return "ok";
    case SAP_ERR_NULL: return "a required pointer is NULL";
    case SAP_ERR_ALIGN: return "a base address or row stride breaks the alignment contract";
    case SAP_ERR_SHAPE: return "a size, stride or count is out of range";
    case SAP_ERR_DTYPE: return "unsupported element type";
    case SAP_ERR_WORKSPACE: return "workspace missing or too small";
    case SAP_ERR_LAUNCH: return "kernel launch failed";
    case SAP_ERR_SCRATCH: return "the call needs more scratch memory than the allocation-free entry point holds";
    default: return "unknown status";
    }
}

int sap_build_sparse_idx(const int32_t *pos, const int32_t *seq, int T, int n_win,
                         const int32_t *win_pt, int64_t win_pt_stride, int page,
                         const int32_t *cmp_logical, int64_t cmp_logical_stride, int n_cmp,
                         const int32_t *cmp_pt, int64_t cmp_pt_stride,
                         int32_t *idx, int64_t idx_stride, sap_stream_t stream)
{
    if (T < 0 || n_win < 0 || n_cmp < 0 || page <= 0) return SAP_ERR_SHAPE;
    if ((int64_t)n_win + n_cmp > (1 << 20)) return SAP_ERR_SHAPE;
    if (T == 0 || n_win + n_cmp == 0) return SAP_OK;
    if (!pos || !seq || !idx) return SAP_ERR_NULL;
    if (n_win > 0 && !win_pt) return SAP_ERR_NULL;
    if (n_cmp > 0 && (!cmp_logical || !cmp_pt)) return SAP_ERR_NULL;
    if (idx_stride < n_win + n_cmp || win_pt_stride < 0 || cmp_pt_stride < 0) return SAP_ERR_SHAPE;
    if (n_cmp > 0 && cmp_logical_stride < n_cmp) return SAP_ERR_SHAPE;
    sap::IdxBuildParams p{};
    p.pos = pos;
    p.seq = seq;
    p.T = T;
    p.n_win = n_win;
    p.win_pt = win_pt;
    p.win_pt_sb = win_pt_stride;
    p.page = page;
    p.cmp_logical = cmp_logical;
    p.cmp_logical_st = cmp_logical_stride;
    p.n_cmp = n_cmp;
    p.cmp_pt = cmp_pt;
    p.cmp_pt_sb = cmp_pt_stride;
    p.idx = idx;
    p.idx_st = idx_stride;
    return launched(sap::launch_build_idx(p, (hipStream_t)stream));
}

int sap_sparse_attn_num_splits(int T, int H, int D, int n_cols, int num_splits)
{
    (void)D;
    if (T < 0 || H < 1 || n_cols < 0 || num_splits < 0) return SAP_ERR_SHAPE;
    return plan_splits(T, H, D, n_cols, num_splits).splits;
}

size_t sap_sparse_attn_workspace_bytes(int T, int H, int D, int n_cols, int num_splits)
{
    if (T <= 0 || H < 1 || D < 1 || n_cols < 0 || num_splits < 0) return 0;
    return attn_ws_bytes(T, H, D, plan_splits(T, H, D, n_cols, num_splits));
}

}  // extern "C"

namespace {

// Argument checks, split plan and launch of the sparse attention.  With
// `scratch_dev` the workspace is the library's own device array (the
// allocation-free entry point): `workspace` is then ignored and a call whose
// plan needs more than kScratchBytes is refused.
int attn_call(const void *q, sap_dtype q_dtype, int64_t q_stride_t, int64_t q_stride_h,
              const void *win_pool, int64_t win_row_stride_bytes,
              const void *cmp_pool, int64_t cmp_row_stride_bytes,
              sap_dtype kv_dtype,
              const int32_t *idx, int64_t idx_stride, int n_win, int n_cmp,
              const float *win_scale, const float *cmp_scale,
              void *out, sap_dtype out_dtype, int64_t out_stride_t, int64_t out_stride_h,
              int T, int H, int D, float sm_scale, int num_splits,
              void *workspace, size_t workspace_bytes, bool scratch_dev, sap_stream_t stream)
{
    if (T < 0 || H < 1 || n_win < 0 || n_cmp < 0 || num_splits < 0) return SAP_ERR_SHAPE;
    if (D != 64 && D != 128 && D != 256 && D != 512) return SAP_ERR_SHAPE;
    const int C = n_win + n_cmp;
    if (C > 65536) return SAP_ERR_SHAPE;
    if (q_dtype != SAP_BF16) return SAP_ERR_DTYPE;
    if (kv_dtype != SAP_BF16 && kv_dtype != SAP_FP8_E4M3) return SAP_ERR_DTYPE;
    if (out_dtype != SAP_F32 && out_dtype != SAP_BF16) return SAP_ERR_DTYPE;
    if (T == 0) return SAP_OK;
    if (!q || !out) return SAP_ERR_NULL;
    if (C > 0 && !idx) return SAP_ERR_NULL;
    if (n_win > 0 && !win_pool) return SAP_ERR_NULL;
    if (n_cmp > 0 && !cmp_pool) return SAP_ERR_NULL;
    if (kv_dtype == SAP_FP8_E4M3 && ((n_win > 0 && !win_scale) || (n_cmp > 0 && !cmp_scale))) return SAP_ERR_NULL;
    if (C > 0 && idx_stride < C) return SAP_ERR_SHAPE;
    if (q_stride_t < 0 || q_stride_h < 0 || out_stride_t < 0 || out_stride_h < 0) return SAP_ERR_SHAPE;
    const int kvb = dtype_size(kv_dtype), ob = dtype_size(out_dtype);
    // 16-byte vector loads and stores of q, out and pool rows
    if (!aligned(q, 16) || (q_stride_t * 2) % 16 || (q_stride_h * 2) % 16) return SAP_ERR_ALIGN;
    if (!aligned(out, 16) || (out_stride_t * ob) % 16 || (out_stride_h * ob) % 16) return SAP_ERR_ALIGN;
    if (n_win > 0) {
        if (!aligned(win_pool, 16) || win_row_stride_bytes % 16) return SAP_ERR_ALIGN;
        if (win_row_stride_bytes < (int64_t)D * kvb) return SAP_ERR_SHAPE;
    }
    if (n_cmp > 0) {
        if (!aligned(cmp_pool, 16) || cmp_row_stride_bytes % 16) return SAP_ERR_ALIGN;
        if (cmp_row_stride_bytes < (int64_t)D * kvb) return SAP_ERR_SHAPE;
    }
    const SplitPlan sp = plan_splits(T, H, D, C, num_splits);
    if ((int64_t)T * sp.splits >= (int64_t)1 << 31) return SAP_ERR_SHAPE;
    const size_t need = attn_ws_bytes(T, H, D, sp);
    if (scratch_dev && need > 0) {
        if (need > kScratchBytes) return SAP_ERR_SCRATCH;
        workspace = device_scratch();
        if (!workspace) return SAP_ERR_LAUNCH;
        workspace_bytes = kScratchBytes;
    }
    if (need > 0 && (!workspace || workspace_bytes < need || !aligned(workspace, 256))) return SAP_ERR_WORKSPACE;

    sap::AttnParams p{};
    p.q = (const uint16_t *)q;
    p.q_st = q_stride_t;
    p.q_sh = q_stride_h;
    p.win = (const uint8_t *)win_pool;
    p.cmp = (const uint8_t *)(n_cmp > 0 ? cmp_pool : win_pool);
    p.win_rs = win_row_stride_bytes;
    p.cmp_rs = n_cmp > 0 ? cmp_row_stride_bytes : win_row_stride_bytes;
    p.win_scale = win_scale;
    p.cmp_scale = cmp_scale;
    p.idx = idx;
    p.idx_st = idx_stride;
    p.n_win = n_win;
    p.n_cols = C;
    p.out = out;
    p.out_st = out_stride_t;
    p.out_sh = out_stride_h;
    p.T = T;
    p.H = H;
    p.sm_scale_log2 = sm_scale * 1.4426950408889634f;
    p.num_splits = sp.splits;
    p.cols_per_split = sp.cols_per_split;
    p.hgroups = (H + sap::kDecHeads - 1) / sap::kDecHeads;
    if (sp.splits > 1) {
        const size_t ml_off = attn_ws_bytes(T, H, D, sp) - align256((size_t)T * sp.splits * H * 2 * 4);
        p.part_o = (float *)workspace;
        p.part_ml = (float *)((uint8_t *)workspace + ml_off);
    }
    const int kv = kv_dtype == SAP_FP8_E4M3 ? 2 : 0;
    const int od = out_dtype == SAP_F32 ? 1 : 0;
    hipError_t e;
    if (sp.kind == PLAN_DEC) {
        e = sap::launch_attn_dec(p, kv, od, (hipStream_t)stream);
        if (e == hipSuccess && sp.splits > 1) e = sap::launch_attn_dec_merge(p, kv, od, (hipStream_t)stream);
    } else {
        e = sap::launch_attn(p, D, kv, od, (hipStream_t)stream);
        if (e == hipSuccess && sp.splits > 1) e = sap::launch_attn_merge(p, D, kv, od, (hipStream_t)stream);
    }
    return launched(e);
}

}  // namespace

extern "C" {

int sap_sparse_attn_paged(const void *q, sap_dtype q_dtype, int64_t q_stride_t, int64_t q_stride_h,
                          const void *win_pool, int64_t win_row_stride_bytes,
                          const void *cmp_pool, int64_t cmp_row_stride_bytes,
                          sap_dtype kv_dtype,
                          const int32_t *idx, int64_t idx_stride, int n_win, int n_cmp,
                          const float *win_scale, const float *cmp_scale,
                          void *out, sap_dtype out_dtype, int64_t out_stride_t, int64_t out_stride_h,
                          int T, int H, int D, float sm_scale, int num_splits,
                          void *workspace, size_t workspace_bytes, sap_stream_t stream)
{
    return attn_call(q, q_dtype, q_stride_t, q_stride_h, win_pool, win_row_stride_bytes, cmp_pool,
                     cmp_row_stride_bytes, kv_dtype, idx, idx_stride, n_win, n_cmp, win_scale, cmp_scale, out,
                     out_dtype, out_stride_t, out_stride_h, T, H, D, sm_scale, num_splits, workspace,
                     workspace_bytes, false, stream);
}

size_t sap_sparse_attn_noalloc_max_bytes(void) { return kScratchBytes; }

int sap_sparse_attn_paged_noalloc(const void *q, sap_dtype q_dtype, int64_t q_stride_t, int64_t q_stride_h,
                                  const void *win_pool, int64_t win_row_stride_bytes,
                                  const void *cmp_pool, int64_t cmp_row_stride_bytes,
                                  sap_dtype kv_dtype,
                                  const int32_t *idx, int64_t idx_stride, int n_win, int n_cmp,
                                  const float *win_scale, const float *cmp_scale,
                                  void *out, sap_dtype out_dtype, int64_t out_stride_t, int64_t out_stride_h,
                                  int T, int H, int D, float sm_scale, int num_splits, sap_stream_t stream)
{
    return attn_call(q, q_dtype, q_stride_t, q_stride_h, win_pool, win_row_stride_bytes, cmp_pool,
                     cmp_row_stride_bytes, kv_dtype, idx, idx_stride, n_win, n_cmp, win_scale, cmp_scale, out,
                     out_dtype, out_stride_t, out_stride_h, T, H, D, sm_scale, num_splits, nullptr, 0, true,
                     stream);
}

int sap_indexer_logits_packed(const void *q, int64_t q_stride_b,
                              const float *w, int64_t w_stride_b,
                              const int32_t *key_pool, int64_t key_row_words,
                              const int32_t *page_table, int64_t pt_stride_b, int page,
                              const int32_t *n_keys,
                              float *logits, int64_t logits_stride_b,
                              int B, int Hi, int D, int N, sap_stream_t stream)
{
    if (B < 0 || N < 0 || Hi < 1 || Hi > 32 || D != 128) return SAP_ERR_SHAPE;
    if (key_row_words < 17) return SAP_ERR_SHAPE;
    if (page_table && page < 1) return SAP_ERR_SHAPE;
    if (B == 0 || N == 0) return SAP_OK;
    if (!q || !w || !key_pool || !logits) return SAP_ERR_NULL;
    if (q_stride_b < 0 || w_stride_b < 0 || pt_stride_b < 0 || logits_stride_b < N) return SAP_ERR_SHAPE;
    if (!aligned(key_pool, 4)) return SAP_ERR_ALIGN;
    if (!aligned(q, 16) || (q_stride_b * 2) % 16) return SAP_ERR_ALIGN;
    if (!aligned(w, 4) || !aligned(logits, 4)) return SAP_ERR_ALIGN;
    sap::IndexerParams p{};
    p.q = (const uint16_t *)q;
    p.q_sb = q_stride_b;
    p.w = w;
    p.w_sb = w_stride_b;
    p.pool = key_pool;
    p.row_words = key_row_words;
    p.pt = page_table;
    p.pt_sb = pt_stride_b;
    p.page = page_table ? page : 1;
    p.n_keys = n_keys;
    p.logits = logits;
    p.logits_sb = logits_stride_b;
    p.B = B;
    p.Hi = Hi;
    p.N = N;
    // at most kIndexerWaves waves, each streaming its tiles with the next
    // tile's loads in flight
    const int64_t tiles = ((int64_t)N + 63) / 64 * B;
    p.tiles_per_wave = (int)((tiles + kIndexerWaves - 1) / kIndexerWaves);
    if (p.tiles_per_wave < 1) p.tiles_per_wave = 1;
    return launched(sap::launch_indexer(p, (hipStream_t)stream));
}

int sap_indexer_logits_candidates(const void *q, int64_t q_stride_t,
                                  const float *w, int64_t w_stride_t,
                                  const int32_t *key_pool, int64_t key_row_words,
                                  const int32_t *page_table, int64_t pt_stride_t, int page,
                                  const int32_t *cand, int64_t cand_stride_t,
                                  const int32_t *n_keys,
                                  float *logits, int64_t logits_stride_t,
                                  int T, int Hi, int D, int NC, sap_stream_t stream)
{
    if (T < 0 || NC < 0 || Hi < 1 || Hi > 32 || D != 128 || T > 65535) return SAP_ERR_SHAPE;
    if (key_row_words < 17) return SAP_ERR_SHAPE;
    if (page_table && page < 1) return SAP_ERR_SHAPE;
    if (T == 0 || NC == 0) return SAP_OK;
    if (!q || !w || !key_pool || !cand || !logits) return SAP_ERR_NULL;
    if (q_stride_t < 0 || w_stride_t < 0 || pt_stride_t < 0 || cand_stride_t < 0 ||
        logits_stride_t < NC)
        return SAP_ERR_SHAPE;
    if (!aligned(key_pool, 4)) return SAP_ERR_ALIGN;
    if (!aligned(q, 16) || (q_stride_t * 2) % 16) return SAP_ERR_ALIGN;
    if (!aligned(w, 4) || !aligned(cand, 4) || !aligned(logits, 4)) return SAP_ERR_ALIGN;
    sap::IndexerParams p{};
    p.q = (const uint16_t *)q;
    p.q_sb = q_stride_t;
    p.w = w;
    p.w_sb = w_stride_t;
    p.pool = key_pool;
    p.row_words = key_row_words;
    p.pt = page_table;
    p.pt_sb = pt_stride_t;
    p.page = page_table ? page : 1;
    p.n_keys = n_keys;
    p.logits = logits;
    p.logits_sb = logits_stride_t;
    p.B = T;
    p.Hi = Hi;
    p.N = NC;
    p.cand = cand;
    p.cand_sb = cand_stride_t;
    const int64_t tiles = ((int64_t)NC + 63) / 64 * T;
    p.tiles_per_wave = (int)((tiles + 2047) / 2048);
    if (p.tiles_per_wave < 1) p.tiles_per_wave = 1;
    return launched(sap::launch_indexer_candidates(p, (hipStream_t)stream));
}

int sap_indexer_logits_prefill(const void *q, int64_t q_stride_t,
                               const float *w, int64_t w_stride_t,
                               const int32_t *key_pool, int64_t key_row_words,
                               const int32_t *page_table, int64_t pt_stride_s, int page,
                               const int32_t *tok_start, int S, int max_tokens,
                               const int32_t *n_keys,
                               float *logits, int64_t logits_stride_t,
                               int Hi, int D, int N, sap_stream_t stream)
{
    if (S < 0 || max_tokens < 0 || N < 0 || Hi < 1 || Hi > 32 || D != 128 || S > 65535) return SAP_ERR_SHAPE;
    if (key_row_words < 17) return SAP_ERR_SHAPE;
    if (page_table && page < 1) return SAP_ERR_SHAPE;
    if (S == 0 || max_tokens == 0 || N == 0) return SAP_OK;
    if ((int64_t)max_tokens > (int64_t)65535 * 8) return SAP_ERR_SHAPE;
    if (!q || !w || !key_pool || !tok_start || !logits) return SAP_ERR_NULL;
    if (q_stride_t < 0 || w_stride_t < 0 || pt_stride_s < 0 || logits_stride_t < N) return SAP_ERR_SHAPE;
    if (!aligned(key_pool, 4)) return SAP_ERR_ALIGN;
    if (!aligned(q, 16) || (q_stride_t * 2) % 16) return SAP_ERR_ALIGN;
    if (!aligned(w, 4) || !aligned(logits, 4)) return SAP_ERR_ALIGN;
    sap::IndexerPrefillParams p{};
    p.q = (const uint16_t *)q;
    p.q_st = q_stride_t;
    p.w = w;
    p.w_st = w_stride_t;
    p.pool = key_pool;
    p.row_words = key_row_words;
    p.pt = page_table;
    p.pt_ss = pt_stride_s;
    p.page = page_table ? page : 1;
    p.tok_start = tok_start;
    p.n_keys = n_keys;
    p.logits = logits;
    p.logits_st = logits_stride_t;
    p.S = S;
    p.max_tokens = max_tokens;
    p.Hi = Hi;
    p.N = N;
    p.kc = sap::indexer_prefill_chunk(S, max_tokens, N);
    return launched(sap::launch_indexer_prefill(p, (hipStream_t)stream));
}

int sap_gated_pool(const void *x, sap_dtype x_dtype, int64_t x_stride_b, int64_t x_stride_r,
                   const void *gate, sap_dtype gate_dtype, int64_t gate_stride_b, int64_t gate_stride_r,
                   void *out, sap_dtype out_dtype, int64_t out_stride_b,
                   int B, int R, int D, sap_stream_t stream)
{
    if (B < 0 || R < 1 || D < 0 || B > 65535) return SAP_ERR_SHAPE;
    const bool dt_ok = (x_dtype == SAP_BF16 || x_dtype == SAP_F32) && (gate_dtype == SAP_BF16 || gate_dtype == SAP_F32) &&
                       (out_dtype == SAP_BF16 || out_dtype == SAP_F32);
    if (!dt_ok) return SAP_ERR_DTYPE;
    if (B == 0 || D == 0) return SAP_OK;
    if (!x || !gate || !out) return SAP_ERR_NULL;
    if (x_stride_b < 0 || x_stride_r < 0 || gate_stride_b < 0 || gate_stride_r < 0 || out_stride_b < 0)
        return SAP_ERR_SHAPE;
    if (!aligned(x, dtype_size(x_dtype)) || !aligned(gate, dtype_size(gate_dtype)) ||
        !aligned(out, dtype_size(out_dtype)))
        return SAP_ERR_ALIGN;
    sap::GatedPoolParams p{};
    p.x = x;
    p.x_sb = x_stride_b;
    p.x_sr = x_stride_r;
    p.g = gate;
    p.g_sb = gate_stride_b;
    p.g_sr = gate_stride_r;
    p.out = out;
    p.out_sb = out_stride_b;
    p.B = B;
    p.R = R;
    p.D = D;
    p.x_bf16 = x_dtype == SAP_BF16;
    p.g_bf16 = gate_dtype == SAP_BF16;
    p.out_bf16 = out_dtype == SAP_BF16;
    return launched(sap::launch_gated_pool(p, (hipStream_t)stream));
}

size_t sap_topk_workspace_bytes(int B, int N, int k)
{
    if (B <= 0 || N <= 0 || k < 1 || k > 4096) return 0;
    return sap::topk_workspace_bytes(B, N, k);
}

int sap_topk_select(const float *logits, int64_t stride_b, const int32_t *n_valid,
                    int B, int N, int k, int32_t *out_idx, int64_t out_stride_b,
                    void *workspace, size_t workspace_bytes, sap_stream_t stream)
{
    if (B < 0 || N < 0 || k < 1 || k > 4096) return SAP_ERR_SHAPE;
    if (B == 0) return SAP_OK;
    if (!out_idx || (N > 0 && !logits)) return SAP_ERR_NULL;
    if (out_stride_b < k || (N > 0 && stride_b < N)) return SAP_ERR_SHAPE;
    if (!aligned(out_idx, 4) || (logits && !aligned(logits, 4))) return SAP_ERR_ALIGN;
    const size_t need = sap_topk_workspace_bytes(B, N, k);
    if (need > 0 && (!workspace || workspace_bytes < need || !aligned(workspace, 256))) return SAP_ERR_WORKSPACE;
    sap::TopkParams p{};
    p.x = logits;
    p.x_sb = stride_b;
    p.n_valid = n_valid;
    p.B = B;
    p.N = N;
    p.k = k;
    p.out = out_idx;
    p.out_sb = out_stride_b;
    p.workspace = workspace;
    return launched(sap::launch_topk(p, (hipStream_t)stream));
}

int sap_topk_sparse_idx(const float *logits, int64_t stride_t, const int32_t *n_valid, int T, int N, int k,
                        const int32_t *pos, const int32_t *seq, int n_win,
                        const int32_t *win_pt, int64_t win_pt_stride, const int32_t *cmp_pt, int64_t cmp_pt_stride,
                        int page, int32_t *idx, int64_t idx_stride,
                        void *workspace, size_t workspace_bytes, sap_stream_t stream)
{
    if (T < 0 || N < 0 || k < 1 || k > 4096 || n_win < 0 || page <= 0) return SAP_ERR_SHAPE;
    if (T == 0) return SAP_OK;
    if (!idx || !pos || !seq || !cmp_pt || (N > 0 && !logits)) return SAP_ERR_NULL;
    if (n_win > 0 && !win_pt) return SAP_ERR_NULL;
    if (idx_stride < (int64_t)n_win + k || (N > 0 && stride_t < N) || win_pt_stride < 0 || cmp_pt_stride < 0)
        return SAP_ERR_SHAPE;
    if (!aligned(idx, 4) || (logits && !aligned(logits, 4))) return SAP_ERR_ALIGN;
    const size_t need = sap_topk_workspace_bytes(T, N, k);
    if (need > 0 && (!workspace || workspace_bytes < need || !aligned(workspace, 256))) return SAP_ERR_WORKSPACE;
    sap::TopkParams p{};
    p.x = logits;
    p.x_sb = stride_t;
    p.n_valid = n_valid;
    p.B = T;
    p.N = N;
    p.k = k;
    p.workspace = workspace;
    p.idx = idx;
    p.idx_st = idx_stride;
    p.pos = pos;
    p.seq = seq;
    p.n_win = n_win;
    p.page = page;
    p.win_pt = win_pt;
    p.win_pt_sb = win_pt_stride;
    p.cmp_pt = cmp_pt;
    p.cmp_pt_sb = cmp_pt_stride;
    return launched(sap::launch_topk(p, (hipStream_t)stream));
}

int sap_debug_e4m3_table(uint16_t *out, float *fold_factor, sap_stream_t stream)
{
    if (!out || !fold_factor) return SAP_ERR_NULL;
    return launched(sap::launch_debug_e4m3(out, fold_factor, (hipStream_t)stream));
}

int sap_debug_e4m3_f16_table(uint16_t *out, sap_stream_t stream)
{
    if (!out) return SAP_ERR_NULL;
    return launched(sap::launch_debug_e4m3_f16(out, (hipStream_t)stream));
}

int sap_debug_fp4_table(uint16_t *out, sap_stream_t stream)
{
    if (!out) return SAP_ERR_NULL;
    return launched(sap::launch_debug_fp4(out, (hipStream_t)stream));
}

}  // extern "C"
