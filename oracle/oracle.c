/*
 * oracle.c -- the parity oracle for top-k sparse attention over a paged KV
 * cache, its fp8/fp4 row formats, the indexer logits and the top-k selection.
 *
 * TEST INFRASTRUCTURE ONLY.  This is plain, slow, obviously correct CPU code
 * in double precision.  It shares no code, header, table or helper with the
 * HIP library; only the test suite, the smoke check and the benchmark's CPU
 * baseline load it.  The product path never calls it.
 *
 * Sources (the pages are cited by title and section):
 *  - "perf(kernel): keep 16-byte kv loads in dsv4 sparse attention and unroll
 *    gated pool" (FreeToken PR #633), "Call paths" / "Changes": each query
 *    attends to a gathered set of KV rows; per column the row comes from the
 *    window pool or the compressed pool; DeepSeek-V4 shapes: 64 heads,
 *    head_dim 512, 128-token window, index top-k 512, r = compress ratio.
 *  - "Perf/kv fp8 read path" (FreeToken fork PR #3), "What this changes": the
 *    per-(token, kv_head) dequant scale is constant along the reduction, so
 *    scores[m,n] = (sum_d q k) s_k[n] and p (diag(s_v) v) = (p s_v) v, with the
 *    softmax denominator built from unscaled p.  The oracle dequantises first
 *    (v = s * decode(code)); the identity says the GPU's folding must agree.
 *  - "perf(kernel): read dsv41 indexer key rows as int32 words" (FreeToken PR
 *    #634), "Changes" / "Correctness and tests": fp4_e8m0_b32 key rows of 17
 *    int32 words (16 words of e2m1 codes, one word of four ue8m0 scales, one
 *    scale per 32 elements), dequantised to bf16; code 0x8 is -0.0.
 *  - The indexer score sum_h w_h * max(0, q_h . k) and the exact top-k with
 *    ties to the lower index are the plain definitions this build adopts
 *    where the pages print no formula.
 *
 * Every exported function returns 0 on success and a negative value on a
 * rejected argument.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* ------------------------------------------------------------------ */
/* Number formats                                                       */
/* ------------------------------------------------------------------ */

/* bf16 is the upper half of an IEEE binary32: widen by appending 16 zero bits. */
double orc_bf16_to_double(uint16_t bits)
{
    uint32_t u = (uint32_t)bits << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

/* OCP 8-bit floating point, E4M3 ("fn" variant): 1 sign bit, 4 exponent bits
 * with bias 7, 3 mantissa bits; exponent 0 encodes subnormals m/8 * 2^-6; the
 * all-ones pattern S.1111.111 is NaN; there is no infinity. */
double orc_e4m3_to_double(uint8_t code)
{
    int s = (code >> 7) & 1;
    int e = (code >> 3) & 0xF;
    int m = code & 0x7;
    double v;
    if (e == 0xF && m == 0x7)
        return NAN;
    if (e == 0)
        v = ldexp((double)m / 8.0, -6);
    else
        v = ldexp(1.0 + (double)m / 8.0, e - 7);
    return s ? -v : v;
}

/* OCP MX E2M1: 1 sign bit, 2 exponent bits with bias 1, 1 mantissa bit;
 * exponent 0 encodes the subnormal m * 2^-1.  Code 0x8 is negative zero. */
double orc_e2m1_to_double(unsigned nibble)
{
    int s = (nibble >> 3) & 1;
    int e = (nibble >> 1) & 0x3;
    int m = nibble & 0x1;
    double v = (e == 0) ? 0.5 * (double)m : ldexp(1.0 + 0.5 * (double)m, e - 1);
    return s ? -v : v;
}

/* UE8M0 scale byte: 2^(e-127); 0xFF is NaN. */
double orc_ue8m0_to_double(unsigned e)
{
    if ((e & 0xFF) == 0xFF)
        return NAN;
    return ldexp(1.0, (int)(e & 0xFF) - 127);
}

/* Round a double to the nearest bf16 (ties to even), with bf16 subnormals
 * (quantum 2^-133), overflow to infinity and a quiet NaN. */
uint16_t orc_double_to_bf16(double x)
{
    uint16_t sign;
    double a, n, r, v;
    int e, ub, qexp;
    if (isnan(x))
        return 0x7FC0;
    sign = signbit(x) ? 0x8000 : 0x0000;
    a = fabs(x);
    if (a == 0.0)
        return sign;
    if (isinf(a))
        return (uint16_t)(sign | 0x7F80);
    frexp(a, &e);                 /* a in [2^(e-1), 2^e) */
    ub = e - 1;                   /* exponent of the leading bit */
    qexp = (ub < -126) ? -133 : ub - 7;   /* spacing of bf16 values here */
    n = ldexp(a, -qexp);          /* exact: scaling by a power of two */
    r = nearbyint(n);             /* default rounding mode: ties to even */
    v = ldexp(r, qexp);
    if (v >= ldexp(1.0, 128))
        return (uint16_t)(sign | 0x7F80);
    if (v < ldexp(1.0, -126)) {
        /* subnormal: value = r * 2^-133 with r < 128 (r == 128 is 2^-126,
         * whose encoding 0x0080 is the same integer) */
        return (uint16_t)(sign | (uint16_t)r);
    }
    frexp(v, &e);
    {
        int biased = (e - 1) + 127;
        double frac = ldexp(v, -(e - 1)) - 1.0;          /* in [0, 1) */
        int mant = (int)ldexp(frac, 7);                  /* exact */
        return (uint16_t)(sign | (uint16_t)(biased << 7) | (uint16_t)mant);
    }
}

/* Value of element d (0..127) of an fp4_e8m0_b32 packed key row: the nibble
 * (d & 7) of word d >> 3 (element 2i is the low nibble of byte i), times the
 * scale byte d >> 5 of word 16, rounded once to bf16. */
double orc_fp4_row_element(const int32_t *row, int d)
{
    uint32_t word = (uint32_t)row[d >> 3];
    unsigned nib = (word >> (4 * (d & 7))) & 0xFu;
    unsigned sbyte = ((uint32_t)row[16] >> (8 * (d >> 5))) & 0xFFu;
    double v = orc_e2m1_to_double(nib) * orc_ue8m0_to_double(sbyte);
    return orc_bf16_to_double(orc_double_to_bf16(v));
}

/* Decode n packed rows (row_words words apart) into out[n][128]. */
void orc_fp4_decode_rows(const int32_t *rows, int64_t n, int64_t row_words, double *out)
{
    for (int64_t i = 0; i < n; ++i)
        for (int d = 0; d < 128; ++d)
            out[i * 128 + d] = orc_fp4_row_element(rows + i * row_words, d);
}

/* The 256 x 256 dequant table: entry [code_byte][scale_byte][j] for the two
 * nibbles j = 0 (low), 1 (high) of code_byte, as bf16 bits. */
void orc_fp4_table(uint16_t *out /* [256*256*2] */)
{
    for (int c = 0; c < 256; ++c)
        for (int s = 0; s < 256; ++s)
            for (int j = 0; j < 2; ++j) {
                unsigned nib = (j == 0) ? (unsigned)(c & 0xF) : (unsigned)(c >> 4);
                double v = orc_e2m1_to_double(nib) * orc_ue8m0_to_double((unsigned)s);
                out[((size_t)c * 256 + s) * 2 + j] = orc_double_to_bf16(v);
            }
}

void orc_e4m3_table(double *out /* [256] */)
{
    for (int c = 0; c < 256; ++c)
        out[c] = orc_e4m3_to_double((uint8_t)c);
}

/* ------------------------------------------------------------------ */
/* Index build: logical positions / entries -> physical pool rows       */
/* ------------------------------------------------------------------ */

/* For query token t at position pos[t] of sequence seq[t]:
 *   window column j (0 <= j < n_win) is position p = pos[t] - (n_win-1) + j,
 *     its physical row win_pt[seq][p / page] * page + p % page, or -1 if p < 0;
 *   compressed column n_win + j is logical entry L = cmp_logical[t][j], row
 *     cmp_pt[seq][L / page] * page + L % page, or -1 if L < 0. */
int orc_build_idx(int T, const int32_t *pos, const int32_t *seq, int n_win,
                  const int32_t *win_pt, int64_t win_pt_stride, int page,
                  const int32_t *cmp_logical, int64_t cmp_logical_stride, int n_cmp,
                  const int32_t *cmp_pt, int64_t cmp_pt_stride,
                  int32_t *idx, int64_t idx_stride)
{
    if (T < 0 || n_win < 0 || n_cmp < 0 || page <= 0)
        return -3;
    for (int t = 0; t < T; ++t) {
        int s = seq[t];
        for (int j = 0; j < n_win; ++j) {
            int64_t p = (int64_t)pos[t] - (n_win - 1) + j;
            int32_t r = -1;
            if (p >= 0)
                r = win_pt[(int64_t)s * win_pt_stride + p / page] * page + (int32_t)(p % page);
            idx[(int64_t)t * idx_stride + j] = r;
        }
        for (int j = 0; j < n_cmp; ++j) {
            int32_t L = cmp_logical[(int64_t)t * cmp_logical_stride + j];
            int32_t r = -1;
            if (L >= 0)
                r = cmp_pt[(int64_t)s * cmp_pt_stride + L / page] * page + L % page;
            idx[(int64_t)t * idx_stride + n_win + j] = r;
        }
    }
    return 0;
}

/* ------------------------------------------------------------------ */
/* Sparse attention                                                     */
/* ------------------------------------------------------------------ */

enum { ORC_BF16 = 0, ORC_F32 = 1, ORC_E4M3 = 2 };

static double load_elem(const void *base, int64_t byte_off, int dtype)
{
    const unsigned char *p = (const unsigned char *)base + byte_off;
    if (dtype == ORC_BF16) {
        uint16_t b;
        memcpy(&b, p, 2);
        return orc_bf16_to_double(b);
    }
    if (dtype == ORC_F32) {
        float f;
        memcpy(&f, p, 4);
        return (double)f;
    }
    return orc_e4m3_to_double(*p);
}

static int dtype_size(int dtype)
{
    return dtype == ORC_BF16 ? 2 : dtype == ORC_F32 ? 4 : 1;
}

/* out[t,h,:] = sum_c p_c v_c / sum_c p_c over the valid columns c of idx[t,:],
 *   v_c[d] = s_c * decode(pool_c[idx[t,c]][d])   (s_c = 1 unless e4m3),
 *   x_c    = sm_scale * sum_d q[t,h,d] v_c[d],   p_c = exp(x_c - max_c x_c),
 *   pool_c = win for c < n_win, cmp otherwise; idx < 0 marks an unused column.
 * A token with no valid column gets a zero output.
 * q: [T,H,D] with element strides q_st, q_sh (dtype bf16 or f32, d contiguous).
 * Pools: row r starts r * row_stride bytes after the base.
 * out: [T,H,D] doubles, contiguous. */
int orc_sparse_attn(int T, int H, int D,
                    const void *q, int q_dtype, int64_t q_st, int64_t q_sh,
                    const void *win, int64_t win_row_bytes,
                    const void *cmp, int64_t cmp_row_bytes, int kv_dtype,
                    const float *win_scale, const float *cmp_scale,
                    const int32_t *idx, int64_t idx_st, int n_win, int n_cmp,
                    double sm_scale, double *out)
{
    const int C = n_win + n_cmp;
    const int qsz = dtype_size(q_dtype);
    const int ksz = dtype_size(kv_dtype);
    if (T < 0 || H <= 0 || D <= 0 || n_win < 0 || n_cmp < 0)
        return -3;
    if (q_dtype == ORC_E4M3)
        return -4;
    if (kv_dtype == ORC_E4M3 && ((n_win > 0 && !win_scale) || (n_cmp > 0 && !cmp_scale)))
        return -1;

#pragma omp parallel for collapse(2) schedule(dynamic, 1)
    for (int t = 0; t < T; ++t) {
        for (int h = 0; h < H; ++h) {
            double *x = (double *)malloc(sizeof(double) * (size_t)(C > 0 ? C : 1));
            char *valid = (char *)malloc((size_t)(C > 0 ? C : 1));
            double *o = out + ((int64_t)t * H + h) * D;
            const unsigned char *qrow = (const unsigned char *)q + ((int64_t)t * q_st + (int64_t)h * q_sh) * qsz;
            double m = -INFINITY, l = 0.0;
            int any = 0;
            for (int c = 0; c < C; ++c) {
                int32_t r = idx[(int64_t)t * idx_st + c];
                valid[c] = (char)(r >= 0);
                if (r < 0)
                    continue;
                {
                    const void *pool = c < n_win ? win : cmp;
                    int64_t rb = c < n_win ? win_row_bytes : cmp_row_bytes;
                    double s = 1.0;
                    double dot = 0.0;
                    if (kv_dtype == ORC_E4M3)
                        s = (double)(c < n_win ? win_scale[r] : cmp_scale[r]);
                    for (int d = 0; d < D; ++d) {
                        double qd = load_elem(qrow, (int64_t)d * qsz, q_dtype);
                        double vd = s * load_elem(pool, (int64_t)r * rb + (int64_t)d * ksz, kv_dtype);
                        dot += qd * vd;
                    }
                    x[c] = sm_scale * dot;
                    if (x[c] > m)
                        m = x[c];
                    any = 1;
                }
            }
            for (int d = 0; d < D; ++d)
                o[d] = 0.0;
            if (any) {
                for (int c = 0; c < C; ++c) {
                    if (!valid[c])
                        continue;
                    {
                        int32_t r = idx[(int64_t)t * idx_st + c];
                        const void *pool = c < n_win ? win : cmp;
                        int64_t rb = c < n_win ? win_row_bytes : cmp_row_bytes;
                        double s = 1.0;
                        double p = exp(x[c] - m);
                        if (kv_dtype == ORC_E4M3)
                            s = (double)(c < n_win ? win_scale[r] : cmp_scale[r]);
                        l += p;
                        for (int d = 0; d < D; ++d)
                            o[d] += p * s * load_elem(pool, (int64_t)r * rb + (int64_t)d * ksz, kv_dtype);
                    }
                }
                for (int d = 0; d < D; ++d)
                    o[d] /= l;
            }
            free(x);
            free(valid);
        }
    }
    return 0;
}

/* ------------------------------------------------------------------ */
/* Indexer logits over fp4_e8m0_b32 packed key rows                     */
/* ------------------------------------------------------------------ */

/* logits[b, n] = sum_h w[b,h] * max(0, sum_d q[b,h,d] * k_n[d])  for n < n_keys[b],
 *              = -inf                                           for n_keys[b] <= n < N.
 * Key n of batch row b lives in pool row page_table[b][n / page] * page + n % page
 * (or b*N + n when page_table is NULL); each pool row has row_words int32 words.
 * q is bf16 [B, Hi, 128] with batch stride q_sb and head stride 128 elements. */
int orc_indexer_logits(int B, int Hi, int Dk, const uint16_t *q, int64_t q_sb,
                       const float *w, int64_t w_sb,
                       const int32_t *key_pool, int64_t row_words,
                       const int32_t *page_table, int64_t pt_sb, int page,
                       const int32_t *n_keys, int N, double *logits, int64_t logits_sb)
{
    if (Dk != 128 || row_words < 17 || B < 0 || Hi <= 0 || N < 0)
        return -3;
    if (page_table && page <= 0)
        return -3;
#pragma omp parallel for collapse(2) schedule(static)
    for (int b = 0; b < B; ++b) {
        for (int n = 0; n < N; ++n) {
            int nk = n_keys ? n_keys[b] : N;
            double acc = 0.0;
            double k[128];
            int64_t row;
            if (n >= nk) {
                logits[(int64_t)b * logits_sb + n] = -INFINITY;
                continue;
            }
            row = page_table ? (int64_t)page_table[(int64_t)b * pt_sb + n / page] * page + n % page
                             : (int64_t)b * N + n;
            for (int d = 0; d < 128; ++d)
                k[d] = orc_fp4_row_element(key_pool + row * row_words, d);
            for (int h = 0; h < Hi; ++h) {
                double dot = 0.0;
                for (int d = 0; d < 128; ++d)
                    dot += orc_bf16_to_double(q[(int64_t)b * q_sb + (int64_t)h * 128 + d]) * k[d];
                acc += (double)w[(int64_t)b * w_sb + h] * (dot > 0.0 ? dot : 0.0);
            }
            logits[(int64_t)b * logits_sb + n] = acc;
        }
    }
    return 0;
}

/*
 * Indexer logits, candidate mode ("perf(kernel): read dsv41 indexer key rows
 * as int32 words": the Reindex layers score a list of NC candidate rows per
 * query instead of every key).  Token t scores the keys whose logical
 * positions are listed in cand[t, 0 .. NC-1]:
 *   logits[t, c] = sum_h w[t, h] * max(0, q[t, h, :] . k_{cand[t, c]})
 * and -inf where cand[t, c] < 0 (no candidate) or cand[t, c] >= n_keys[t]
 * (not visible to the token).  A logical position n maps to pool row
 * page_table[t * pt_sb + n / page] * page + n % page, or to row n itself
 * when page_table is NULL.  Same key decode and score as full mode.
 */
int orc_indexer_candidates(int T, int Hi, int Dk, const uint16_t *q, int64_t q_sb,
                           const float *w, int64_t w_sb,
                           const int32_t *key_pool, int64_t row_words,
                           const int32_t *page_table, int64_t pt_sb, int page,
                           const int32_t *cand, int64_t cand_sb, const int32_t *n_keys,
                           int NC, double *logits, int64_t logits_sb)
{
    if (Dk != 128 || row_words < 17 || T < 0 || Hi <= 0 || NC < 0)
        return -3;
    if (page_table && page <= 0)
        return -3;
#pragma omp parallel for collapse(2) schedule(static)
    for (int t = 0; t < T; ++t) {
        for (int c = 0; c < NC; ++c) {
            const int32_t n = cand[(int64_t)t * cand_sb + c];
            double acc = 0.0;
            double k[128];
            int64_t row;
            if (n < 0 || (n_keys && n >= n_keys[t])) {
                logits[(int64_t)t * logits_sb + c] = -INFINITY;
                continue;
            }
            row = page_table ? (int64_t)page_table[(int64_t)t * pt_sb + n / page] * page + n % page
                             : (int64_t)n;
            for (int d = 0; d < 128; ++d)
                k[d] = orc_fp4_row_element(key_pool + row * row_words, d);
            for (int h = 0; h < Hi; ++h) {
                double dot = 0.0;
                for (int d = 0; d < 128; ++d)
                    dot += orc_bf16_to_double(q[(int64_t)t * q_sb + (int64_t)h * 128 + d]) * k[d];
                acc += (double)w[(int64_t)t * w_sb + h] * (dot > 0.0 ? dot : 0.0);
            }
            logits[(int64_t)t * logits_sb + c] = acc;
        }
    }
    return 0;
}

/* ------------------------------------------------------------------ */
/* Gated pool (the compressor step that produces compressed rows)      */
/* ------------------------------------------------------------------ */

/*
 * "perf(kernel): keep 16-byte kv loads in dsv4 sparse attention and unroll
 * gated pool" names gated_pool (Call paths: the compressor's decode step)
 * and says it runs a max loop and a second loop over R; it prints no
 * formula.  Reading taken: each of the D channels of R raw rows is pooled by
 * a softmax over R of its gate scores,
 *   out[b, d] = sum_r exp(g[b,r,d] - m) x[b,r,d] / sum_r exp(g[b,r,d] - m),
 *   m = max_r g[b,r,d]   (the max loop),
 * with -inf gates contributing nothing and an all -inf column giving 0.
 * x, g: [B, R, D] contiguous doubles (exact copies of the bf16 / fp32
 * inputs); out: [B, D].
 */
int orc_gated_pool(int B, int R, int D, const double *x, const double *g, double *out)
{
    if (B < 0 || R < 1 || D < 0)
        return -3;
#pragma omp parallel for collapse(2) schedule(static)
    for (int b = 0; b < B; ++b) {
        for (int d = 0; d < D; ++d) {
            double m = -INFINITY, s = 0.0, a = 0.0;
            for (int r = 0; r < R; ++r) {
                double v = g[((int64_t)b * R + r) * D + d];
                if (v > m)
                    m = v;
            }
            if (m == -INFINITY) {
                out[(int64_t)b * D + d] = 0.0;
                continue;
            }
            for (int r = 0; r < R; ++r) {
                int64_t i = ((int64_t)b * R + r) * D + d;
                double e = exp(g[i] - m);
                s += e;
                a += e * x[i];
            }
            out[(int64_t)b * D + d] = a / s;
        }
    }
    return 0;
}

/* ------------------------------------------------------------------ */
/* Exact top-k selection                                                */
/* ------------------------------------------------------------------ */

typedef struct {
    float v;
    int32_t i;
} orc_cand;

/* larger value first; equal values: lower index first */
static int cand_cmp(const void *a, const void *b)
{
    const orc_cand *x = (const orc_cand *)a, *y = (const orc_cand *)b;
    if (x->v > y->v)
        return -1;
    if (x->v < y->v)
        return 1;
    return (x->i > y->i) - (x->i < y->i);
}

static int int_cmp(const void *a, const void *b)
{
    int32_t x = *(const int32_t *)a, y = *(const int32_t *)b;
    return (x > y) - (x < y);
}

/* For each row b: the candidates are the n < n_valid[b] (all n < N when
 * n_valid is NULL) whose value is neither NaN nor -inf.  Keep the k largest,
 * equal values going to the lower index, and write their indices in ascending
 * order, padding with -1 when fewer than k candidates exist. */
int orc_topk(int B, int N, const float *x, int64_t x_sb, const int32_t *n_valid, int k,
             int32_t *out, int64_t out_sb)
{
    if (B < 0 || N < 0 || k < 0)
        return -3;
    for (int b = 0; b < B; ++b) {
        int nv = n_valid ? n_valid[b] : N;
        int cnt = 0, take;
        orc_cand *c;
        int32_t *sel;
        if (nv > N)
            nv = N;
        c = (orc_cand *)malloc(sizeof(orc_cand) * (size_t)(nv > 0 ? nv : 1));
        for (int n = 0; n < nv; ++n) {
            float v = x[(int64_t)b * x_sb + n];
            if (isnan(v) || (isinf(v) && v < 0))
                continue;
            c[cnt].v = v;
            c[cnt].i = n;
            ++cnt;
        }
        qsort(c, (size_t)cnt, sizeof(orc_cand), cand_cmp);
        take = cnt < k ? cnt : k;
        sel = (int32_t *)malloc(sizeof(int32_t) * (size_t)(take > 0 ? take : 1));
        for (int j = 0; j < take; ++j)
            sel[j] = c[j].i;
        qsort(sel, (size_t)take, sizeof(int32_t), int_cmp);
        for (int j = 0; j < k; ++j)
            out[(int64_t)b * out_sb + j] = j < take ? sel[j] : -1;
        free(sel);
        free(c);
    }
    return 0;
}

int orc_num_threads(void)
{
#ifdef _OPENMP
    extern int omp_get_max_threads(void);
    return omp_get_max_threads();
#else
    return 1;
#endif
}
