/*
 * sap.h -- C ABI of the gfx950 (MI355X) library for top-k sparse attention
 * over a paged KV cache, its fp4 indexer and its exact top-k selection.
 *
 * Conventions shared by every entry point:
 *  - Array pointers are DEVICE pointers owned by the caller.  The library
 *    never allocates, frees or synchronises; it enqueues kernels on `stream`
 *    (a hipStream_t; NULL is the default stream) and returns.
 *  - The return value is a host-side validation status (sap_status).  Nothing
 *    is launched when it is negative.  Faults inside kernels surface at the
 *    caller's next synchronisation.
 *  - Element strides are in elements of the array's own type unless the name
 *    ends in _bytes or _words.  The innermost dimension is contiguous.
 *  - Index values are trusted: an index that is not -1 must address a row
 *    that exists in its pool.  -1 is the only "unused" sentinel.
 *  - Calls on one stream run in order; concurrent calls that share a
 *    workspace race.
 */
#ifndef SAP_H
#define SAP_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

struct ihipStream_t;
typedef struct ihipStream_t *sap_stream_t;   /* the same type as hipStream_t */

typedef enum {
    SAP_OK = 0,
    SAP_ERR_NULL = -1,       /* a required pointer is NULL */
    SAP_ERR_ALIGN = -2,      /* a base address or row stride breaks the alignment contract */
    SAP_ERR_SHAPE = -3,      /* a size, stride or count is out of range */
    SAP_ERR_DTYPE = -4,      /* an unsupported element type */
    SAP_ERR_WORKSPACE = -5,  /* workspace missing or smaller than required */
    SAP_ERR_LAUNCH = -6,     /* the HIP runtime refused a launch */
    SAP_ERR_SCRATCH = -7     /* the allocation-free entry point's fixed scratch is too small */
} sap_status;

typedef enum {
    SAP_BF16 = 0,
    SAP_F32 = 1,
    SAP_FP8_E4M3 = 2         /* OCP E4M3 ("fn": no infinities, S.1111.111 = NaN) */
} sap_dtype;

/* Library version (major * 10000 + minor * 100 + patch) and a text for a status. */
int sap_version(void);
const char *sap_status_string(int status);

/* -------------------------------------------------------------------------
 * Index build (helper on the path, before the attention kernel).
 *
 * The gathered column set of one query token is a sliding window of n_win
 * positions plus n_cmp entries of the compressed pool ("perf(kernel): keep
 * 16-byte kv loads in dsv4 sparse attention and unroll gated pool",
 * Call paths / Changes / Kernel time: 128-token window, index top-k 512,
 * compressed pool with one entry per r tokens).  This call turns logical
 * positions and entries into physical pool rows through page tables:
 *
 *   idx[t][j]         = row of position p = pos[t] - (n_win-1) + j  (j < n_win),
 *                       win_pt[seq[t]][p / page] * page + p % page, or -1 if p < 0
 *   idx[t][n_win + j] = row of compressed entry L = cmp_logical[t][j],
 *                       cmp_pt[seq[t]][L / page] * page + L % page, or -1 if L < 0
 *
 * pos, seq: [T] int32.  win_pt: [B, *] int32 with row stride win_pt_stride.
 * cmp_logical: [T, n_cmp] int32 (row stride cmp_logical_stride); cmp_pt as
 * win_pt.  Both may be NULL when n_cmp == 0.  idx: [T, >= n_win + n_cmp]
 * int32 output with row stride idx_stride.  Page-table entries are trusted.
 * Errors: SAP_ERR_NULL, SAP_ERR_SHAPE (negative counts, page <= 0,
 * idx_stride < n_win + n_cmp).
 * ------------------------------------------------------------------------- */
int sap_build_sparse_idx(const int32_t *pos, const int32_t *seq, int T, int n_win,
                         const int32_t *win_pt, int64_t win_pt_stride, int page,
                         const int32_t *cmp_logical, int64_t cmp_logical_stride, int n_cmp,
                         const int32_t *cmp_pt, int64_t cmp_pt_stride,
                         int32_t *idx, int64_t idx_stride, sap_stream_t stream);

/* -------------------------------------------------------------------------
 * Sparse attention over a paged KV cache (prefill and split-K decode).
 *
 * For every query token t and head h (the H query heads share one KV head,
 * and one pool row serves as both key and value):
 *
 *   column c in [0, n_win + n_cmp) reads row r = idx[t][c] (skipped if -1)
 *   from win_pool when c < n_win and from cmp_pool otherwise ("perf(kernel):
 *   keep 16-byte kv loads ...", Changes: the per-column pool base);
 *   x_c = sm_scale * s_c * (q[t,h,:] . row_c),   p_c = exp(x_c - max x),
 *   out[t,h,:] = sum_c p_c s_c row_c / sum_c p_c   (zero if no valid column).
 *
 * s_c is the row's fp32 dequant scale for SAP_FP8_E4M3 pools and 1 otherwise;
 * it is applied to the dot outputs and folded into the softmax weights for
 * PV, never to the K/V tiles, and the denominator sums unscaled p ("Perf/kv
 * fp8 read path", What this changes).
 *
 * q:        [T, H, D] bf16, strides q_stride_t, q_stride_h (elements).
 *           Base and row starts 16-byte aligned.
 * win_pool: [Nw, D] rows of kv_dtype (SAP_BF16 or SAP_FP8_E4M3), row r at
 *           win_pool + r * win_row_stride_bytes.
 * cmp_pool: [Nc, D] likewise; may be NULL or alias win_pool when n_cmp == 0.
 *           Pool bases and row strides must be multiples of 16 bytes (the
 *           16-byte vector gathers of "Changes"); pool views with a row
 *           offset are fine when they keep that alignment.
 * win_scale, cmp_scale: [Nw], [Nc] fp32 per-row scales; required for
 *           SAP_FP8_E4M3 (the pool that has columns), ignored otherwise.
 * idx:      [T, n_win + n_cmp] int32 physical rows (below 2^31 - 1), -1 =
 *           no column; row stride idx_stride.  Columns marked -1 cost no
 *           gather or MFMA work.
 * out:      [T, H, D] of out_dtype (SAP_F32 or SAP_BF16), strides
 *           out_stride_t, out_stride_h; 16-byte aligned like q.
 * D:        64, 128, 256 or 512.  H >= 1.  n_win + n_cmp <= 65536.
 * num_splits: 1 = one pass per token (prefill); k > 1 = split the columns
 *           into k ranges and merge the partial (max, sum, output) triples
 *           (decode); 0 = choose automatically (about two 32-column tiles
 *           per split while the launch has fewer than 128 workgroups).  The
 *           merge is exact algebra, but each split rounds its softmax weights
 *           to bf16 against its own running max, so split counts agree with
 *           the single pass to the same tolerance as with an exact result,
 *           not bit for bit.  (At head_dim 512 with bf16 rows a split's
 *           partial output is kept in f16, scaled per head by a power of two
 *           so that its largest value sits in [2^14, 2^15): a rounding of at
 *           most 2^-11 of that value, below the bf16 weights' 2^-9.)
 * workspace: device scratch of at least sap_sparse_attn_workspace_bytes(T,
 *           H, D, n_win + n_cmp, num_splits) bytes, 256-byte aligned; may be
 *           NULL when that size is 0.
 * Errors: SAP_ERR_NULL, SAP_ERR_ALIGN, SAP_ERR_SHAPE, SAP_ERR_DTYPE,
 * SAP_ERR_WORKSPACE, SAP_ERR_LAUNCH.
 * ------------------------------------------------------------------------- */
int sap_sparse_attn_num_splits(int T, int H, int D, int n_cols, int num_splits);
size_t sap_sparse_attn_workspace_bytes(int T, int H, int D, int n_cols, int num_splits);
int sap_sparse_attn_paged(const void *q, sap_dtype q_dtype, int64_t q_stride_t, int64_t q_stride_h,
                          const void *win_pool, int64_t win_row_stride_bytes,
                          const void *cmp_pool, int64_t cmp_row_stride_bytes,
                          sap_dtype kv_dtype,
                          const int32_t *idx, int64_t idx_stride, int n_win, int n_cmp,
                          const float *win_scale, const float *cmp_scale,
                          void *out, sap_dtype out_dtype, int64_t out_stride_t, int64_t out_stride_h,
                          int T, int H, int D, float sm_scale, int num_splits,
                          void *workspace, size_t workspace_bytes, sap_stream_t stream);

/* -------------------------------------------------------------------------
 * Allocation-free sparse attention, for callers that cannot allocate device
 * memory: code under HIP graph capture, tight serving loops and harnesses
 * that forbid hipMalloc.  Same arguments and result as sap_sparse_attn_paged
 * without the workspace: the split partials of a call live in a fixed
 * device array of sap_sparse_attn_noalloc_max_bytes() bytes (32 MiB) that
 * the library holds on every GPU it runs on until the process ends.  The
 * call itself allocates nothing (no hipMalloc, no allocating library call).
 *
 * A call whose split plan needs more than that (sap_sparse_attn_workspace_bytes
 * of the same arguments) returns SAP_ERR_SCRATCH and launches nothing.  The
 * automatic plan (num_splits = 0) always fits for D <= 512; an explicit
 * split count may not.  All calls on one
 * GPU share its array and the array keeps the last call's contents: calls
 * that overlap on one GPU (different streams, or graphs replayed
 * concurrently) race and must be ordered by the caller.  Calls on one stream
 * are ordered.  The array needs no clearing: every split writes its whole
 * partial before the merge reads it.
 * Errors: those of sap_sparse_attn_paged except SAP_ERR_WORKSPACE, plus
 * SAP_ERR_SCRATCH.
 * ------------------------------------------------------------------------- */
size_t sap_sparse_attn_noalloc_max_bytes(void);
int sap_sparse_attn_paged_noalloc(const void *q, sap_dtype q_dtype, int64_t q_stride_t, int64_t q_stride_h,
                                  const void *win_pool, int64_t win_row_stride_bytes,
                                  const void *cmp_pool, int64_t cmp_row_stride_bytes,
                                  sap_dtype kv_dtype,
                                  const int32_t *idx, int64_t idx_stride, int n_win, int n_cmp,
                                  const float *win_scale, const float *cmp_scale,
                                  void *out, sap_dtype out_dtype, int64_t out_stride_t, int64_t out_stride_h,
                                  int T, int H, int D, float sm_scale, int num_splits, sap_stream_t stream);

/* -------------------------------------------------------------------------
 * Indexer logits over fp4_e8m0_b32 packed key rows ("perf(kernel): read dsv41
 * indexer key rows as int32 words", Changes: 17 int32 words per row, 16
 * words of e2m1 codes and one word of four ue8m0 block-32 scales).
 *
 *   logits[b][n] = sum_{h < Hi} w[b][h] * max(0, sum_{d < 128} q[b][h][d] * k_n[d])
 *                  for n < n_keys[b];  -inf for n_keys[b] <= n < N,
 *   k_n[d] = e2m1(nibble d) * 2^(scale byte (d / 32) - 127), a bf16 value;
 *   element 2i is the low nibble of byte i of words 0..15; scale byte j is
 *   byte j of word 16.
 *
 * q: [B, Hi, 128] bf16, batch stride q_stride_b, head stride 128; 16-byte aligned.
 * w: [B, Hi] fp32, batch stride w_stride_b.
 * key_pool: int32 rows of key_row_words (>= 17) words; base 4-byte aligned.
 * page_table: [B, ceil(N / page)] int32 (row stride pt_stride_b); key n of
 *   batch row b is pool row page_table[b][n / page] * page + n % page.  NULL
 *   means pool row b * N + n.
 * n_keys: [B] int32 valid key counts (NULL = N everywhere).  Keys at or past
 *   n_keys[b] score -inf; their rows are read only where they share a
 *   64-key tile (inside one page) with a valid key, so every page that holds
 *   a valid key must be whole in the pool.
 * logits: [B, N] fp32, batch stride logits_stride_b.
 * Limits: Hi in [1, 32], D == 128, 0 <= N, page >= 1.
 * Errors: SAP_ERR_NULL, SAP_ERR_ALIGN, SAP_ERR_SHAPE, SAP_ERR_LAUNCH.
 * ------------------------------------------------------------------------- */
int sap_indexer_logits_packed(const void *q, int64_t q_stride_b,
                              const float *w, int64_t w_stride_b,
                              const int32_t *key_pool, int64_t key_row_words,
                              const int32_t *page_table, int64_t pt_stride_b, int page,
                              const int32_t *n_keys,
                              float *logits, int64_t logits_stride_b,
                              int B, int Hi, int D, int N, sap_stream_t stream);

/* -------------------------------------------------------------------------
 * Indexer logits, candidate mode ("perf(kernel): read dsv41 indexer key rows
 * as int32 words", Call path: the Reindex layers score a list of candidate
 * rows; Kernel time: NC = 16384 candidates per query).  Token t scores the
 * keys whose logical positions are listed in cand[t, 0 .. NC-1]:
 *
 *   logits[t, c] = sum_h w[t, h] * max(0, q[t, h, :] . k(cand[t, c]))
 *
 * and -inf where cand[t, c] < 0 (no candidate) or cand[t, c] >= n_keys[t].
 * Position n maps to pool row page_table[t * pt_stride_t + n / page] * page
 * + n % page (pt_stride_t = 0 when every token reads one sequence), or to
 * row n itself when page_table is NULL.  Keys decode as in full mode.
 *
 * q [T, Hi, 128] bf16 (16-byte aligned rows), w [T, Hi] fp32,
 * cand [T, NC] int32 (row stride cand_stride_t), n_keys [T] or NULL (no
 * bound), logits [T, NC] fp32.  1 <= Hi <= 32, D = 128, T <= 65535.
 * Candidate values below n_keys[t] must address rows inside the pool and
 * pages inside the page table (not checked on the device).  With a page
 * table and n_keys, the page-table row of token t must hold
 * ceil(n_keys[t] / page) entries (the pages of its visible keys): up to 4096
 * of them are staged on chip in one read.
 * Errors: SAP_ERR_NULL, SAP_ERR_ALIGN, SAP_ERR_SHAPE, SAP_ERR_LAUNCH.
 * ------------------------------------------------------------------------- */
int sap_indexer_logits_candidates(const void *q, int64_t q_stride_t,
                                  const float *w, int64_t w_stride_t,
                                  const int32_t *key_pool, int64_t key_row_words,
                                  const int32_t *page_table, int64_t pt_stride_t, int page,
                                  const int32_t *cand, int64_t cand_stride_t,
                                  const int32_t *n_keys,
                                  float *logits, int64_t logits_stride_t,
                                  int T, int Hi, int D, int NC, sap_stream_t stream);

/* -------------------------------------------------------------------------
 * Indexer logits, prefill mode with causal masking ("perf(kernel): read
 * dsv41 indexer key rows as int32 words", Call path: the indexer runs in
 * prefill and decode; Kernel time: full prefill of 2k / 8k prompts, 2k chunks
 * at 128k context, bounded decoder variants).  S sequences; the query tokens
 * of sequence s are rows tok_start[s] .. tok_start[s+1]-1 and score that
 * sequence's keys:
 *
 *   logits[t, n] = sum_h w[t, h] * max(0, q[t, h, :] . k_s(n))  for n < n_keys[t]
 *   logits[t, n] = -inf                                        for n_keys[t] <= n < N
 *
 * n_keys[t] is the number of keys token t may see (the caller's causal
 * bound, e.g. ceil((p+1)/r) for a token at position p over entries of
 * ratio r); NULL means N for every token.  Key n of sequence s is pool row
 * page_table[s * pt_stride_s + n / page] * page + n % page, or s * N + n when
 * page_table is NULL.
 *
 * tok_start [S + 1] int32 (device, non-decreasing); max_tokens >= every
 * sequence's token count (the launch covers that many tokens per sequence).
 * q [T, Hi, 128] bf16, w [T, Hi] fp32, logits [T, N] fp32 (row stride
 * logits_stride_t >= N).  1 <= Hi <= 32, D = 128, S <= 65535.
 * Errors: SAP_ERR_NULL, SAP_ERR_ALIGN, SAP_ERR_SHAPE, SAP_ERR_LAUNCH.
 * ------------------------------------------------------------------------- */
int sap_indexer_logits_prefill(const void *q, int64_t q_stride_t,
                               const float *w, int64_t w_stride_t,
                               const int32_t *key_pool, int64_t key_row_words,
                               const int32_t *page_table, int64_t pt_stride_s, int page,
                               const int32_t *tok_start, int S, int max_tokens,
                               const int32_t *n_keys,
                               float *logits, int64_t logits_stride_t,
                               int Hi, int D, int N, sap_stream_t stream);

/* -------------------------------------------------------------------------
 * Gated pool: the compressor step that turns R raw rows into one compressed
 * row ("perf(kernel): keep 16-byte kv loads in dsv4 sparse attention and
 * unroll gated pool", Call paths: Compressor.decode_step -> gated_pool;
 * Changes: a max loop and a second loop over R; Kernel time: B 1 / 8,
 * R 8 / 128, D 128 / 512).  The pages print no formula; the reading
 * implemented is a softmax over R of each channel's gate scores:
 *
 *   out[b, d] = sum_r exp(g[b,r,d] - m) x[b,r,d] / sum_r exp(g[b,r,d] - m),
 *   m = max_r g[b,r,d];  -inf gates add nothing; an all -inf column gives 0.
 *
 * x, gate: [B, R, D] of SAP_BF16 or SAP_F32 with element strides (b, r) and
 * unit stride along d; out: [B, D] of SAP_BF16 or SAP_F32 (row stride
 * out_stride_b).  Computed in fp32.  R >= 1, B <= 65535.
 * Errors: SAP_ERR_NULL, SAP_ERR_ALIGN (element alignment), SAP_ERR_SHAPE,
 * SAP_ERR_DTYPE, SAP_ERR_LAUNCH.
 * ------------------------------------------------------------------------- */
int sap_gated_pool(const void *x, sap_dtype x_dtype, int64_t x_stride_b, int64_t x_stride_r,
                   const void *gate, sap_dtype gate_dtype, int64_t gate_stride_b, int64_t gate_stride_r,
                   void *out, sap_dtype out_dtype, int64_t out_stride_b,
                   int B, int R, int D, sap_stream_t stream);

/* -------------------------------------------------------------------------
 * Exact top-k selection (the index top-k of "perf(kernel): keep 16-byte kv
 * loads ...", Kernel time).  For each row b the candidates are the n <
 * n_valid[b] (n < N when n_valid is NULL) whose value is neither NaN nor -inf.
 * The k largest are kept, equal values going to the lower index; their
 * indices are written in ascending order, padded with -1.
 *
 * logits: [B, N] fp32 (row stride stride_b).  out_idx: [B, k] int32 (row
 * stride out_stride_b).
 * workspace: device memory of sap_topk_workspace_bytes(B, N, k) bytes,
 *   256-byte aligned.  Rows of up to 16384 entries are selected by one
 *   workgroup entirely on chip and need none (size 0, NULL allowed).  Longer
 *   rows take two launches: a filter launch in which each 4096-entry chunk of
 *   a row compacts its keys above a sampled threshold into a slot of the
 *   workspace, then a select launch over the slots.  With nch =
 *   ceil(N / 4096) the size is then a(4 B nch) + a(4 B) + 2 a(8192 B nch)
 *   bytes, a() rounding up to a multiple of 256 (about 512 KiB per row at
 *   N = 131072).
 * Limits: 1 <= k <= 4096, 0 <= N < 2^31.
 * Errors: SAP_ERR_NULL, SAP_ERR_SHAPE, SAP_ERR_WORKSPACE, SAP_ERR_LAUNCH.
 * ------------------------------------------------------------------------- */
size_t sap_topk_workspace_bytes(int B, int N, int k);
int sap_topk_select(const float *logits, int64_t stride_b, const int32_t *n_valid,
                    int B, int N, int k, int32_t *out_idx, int64_t out_stride_b,
                    void *workspace, size_t workspace_bytes, sap_stream_t stream);

/* -------------------------------------------------------------------------
 * Top-k selection fused with the index build (the decode step's selection:
 * the indexer's logits -> the attention's column rows in one launch).  The
 * result is exactly that of sap_topk_select(logits, ..., k, sel) followed by
 * sap_build_sparse_idx(pos, seq, T, n_win, win_pt, ..., cmp_logical = sel,
 * n_cmp = k, cmp_pt, ..., idx): for token t,
 *
 *   idx[t][j]         = window row of position pos[t] - (n_win-1) + j, or -1,
 *   idx[t][n_win + j] = cmp_pt row of the j-th selected entry (ascending
 *                       entry order), or -1 past the selected count.
 *
 * logits: [T, N] fp32 (row stride stride_t), candidates as for
 * sap_topk_select (n_valid may be NULL); pos, seq: [T] int32; page tables as
 * for sap_build_sparse_idx (cmp_pt required, win_pt when n_win > 0).  Every
 * cmp_pt row holds ceil(N / page) entries (the pages of entries 0 .. N-1),
 * and every win_pt row the pages of positions 0 .. pos[t]: the kernel may read
 * any of them, not only those of selected entries.
 * idx: [T, >= n_win + k] int32.  workspace: sap_topk_workspace_bytes(T, N, k)
 * bytes, 256-byte aligned: zero for N <= 16384 (the decode step's 8192
 * compressed entries), else the two-launch filter/select slots described
 * for sap_topk_select.  Limits as sap_topk_select.
 * Errors: SAP_ERR_NULL, SAP_ERR_ALIGN, SAP_ERR_SHAPE, SAP_ERR_WORKSPACE,
 * SAP_ERR_LAUNCH.
 * ------------------------------------------------------------------------- */
int sap_topk_sparse_idx(const float *logits, int64_t stride_t, const int32_t *n_valid, int T, int N, int k,
                        const int32_t *pos, const int32_t *seq, int n_win,
                        const int32_t *win_pt, int64_t win_pt_stride, const int32_t *cmp_pt, int64_t cmp_pt_stride,
                        int page, int32_t *idx, int64_t idx_stride,
                        void *workspace, size_t workspace_bytes, sap_stream_t stream);

/* -------------------------------------------------------------------------
 * Format hooks: run the device decode functions of the hot path over every
 * code, so tests can compare them bit for bit with the format definitions.
 *
 * sap_debug_e4m3_table: out[c] = bf16 bits the attention row loader produces
 *   for e4m3 code c (c = 0..255); *fold_factor = the factor that multiplies
 *   that 16-bit value to give the code's value (folded into the row scale).
 * sap_debug_e4m3_f16_table: out[c] = f16 bits of e4m3 code c as the one-pass
 *   kernel at head_dim 512 widens its V^T operand (fold factor 1).
 * sap_debug_fp4_table: out[(c * 256 + s) * 2 + j] = bf16 bits of nibble j
 *   (0 = low, 1 = high) of code byte c times scale byte s, as the indexer's
 *   row loader dequantises them.
 * All pointers are device pointers.
 * ------------------------------------------------------------------------- */
int sap_debug_e4m3_table(uint16_t *out /* [256] */, float *fold_factor /* [1] */,
                         sap_stream_t stream);
int sap_debug_e4m3_f16_table(uint16_t *out /* [256] */, sap_stream_t stream);
int sap_debug_fp4_table(uint16_t *out /* [256 * 256 * 2] */, sap_stream_t stream);

#ifdef __cplusplus
}
#endif
#endif /* SAP_H */
