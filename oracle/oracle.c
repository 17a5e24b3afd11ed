/*
 * Oracle for paged MQA logits, one-head indexer scores and the block-max
 * proxy score: a plain, slow,
 * float64 CPU implementation of the definitions.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg may load or call this code.  The GPU library
 * never links it, and this file shares no code, header or table with it.
 *
 * Sources (FlashInfer documentation pages):
 *   [attn_scores]   "flashinfer.attn_scores": the introductory equation
 *                   logits[t,p] = sum_h w[t,h] * relu(q[t,h] . k_p), the two
 *                   bullets after it (rectifier per head before the sum; FP8
 *                   multiplies by the per-token FP32 scale s_p kept in the
 *                   trailing scale region of each kv_fused block; MXFP4 folds
 *                   its per-32 block scales into the dequantised values), and
 *                   the output-contract note (unconditional writes within a
 *                   row's scheduled extent; rows of requests with
 *                   seq_lens == 0 are never written).
 *   [proxy]         "flashinfer.msa_ops.msa_proxy_score_fp4": per-KV-block
 *                   max of the unscaled, causally masked Q K^T logits with
 *                   NVFP4 query and keys, global scales folded before the
 *                   max, output (heads, max_k_tiles, total_q) or (1, ...)
 *                   with reduce_heads.
 *   [indexer]       "flashinfer.sdsa.indexer_scores": one head, so a score is
 *                   the plain dot product of a query row and a key; pages of
 *                   64 keys; scores[q,k] is written for k below the group's
 *                   length and not beyond; BF16 inputs, or NVFP4 inputs
 *                   (packed e2m1 with an e4m3 scale per 16 values, the key
 *                   scales paged like the keys).
 *
 * Readings taken where the pages are silent (each is listed in the design notes):
 *   - the scheduled extent of every row of request b is the request's length
 *     rounded up to whole 64-token pages, E_b = ceil(L_b/64)*64, clamped to
 *     max_context; a non-positive length writes nothing;
 *   - the FP8 query is consumed as decoded e4m3 (the pages give no q scale);
 *   - e4m3 is OCP E4M3FN, e2m1/e8m0 are OCP MX; the even element of a packed
 *     FP4 byte is its low nibble;
 *   - FP8 page layout: 64 tokens x D bytes, then 64 little-endian fp32 scales;
 *     MXFP4 page layout: 64 tokens x D/2 bytes, then 64 x D/32 e8m0 codes;
 *   - MXFP4 with sf_vec_size = 16 (the attn_scores paragraph names
 *     sf_vec_size and is_kv_sf_interleaved without defining them): one e8m0
 *     code per 16 values instead of 32, for q_sf [B, N, H, D/16] and for the
 *     keys (D/16 codes per token); with is_kv_sf_interleaved = 1 a page holds
 *     64 token records, each the token's D/2 packed bytes followed by its
 *     D/sf_vec_size codes (same page size as the trailing layout);
 *   - the block table is int32 [B, bt_stride], page j of request b is
 *     block_table[b*bt_stride + j]; page i starts at kv + i*page_stride.
 *
 * Every arithmetic step is float64 on decoded values.  For each output the
 * oracle also returns A = s_p * sum_h |w[t,h]| * relu(q[t,h].k_p) (FP8/MXFP4)
 * or sum_d |q_d k_d| (indexer), the magnitude the parity tolerance scales with.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define TOK_PER_PAGE 64

/* ---------------------------------------------------------------- decoders */

/* OCP E4M3FN: sign, 4-bit exponent (bias 7), 3-bit mantissa; e=15,m=7 is NaN. */
double oracle_e4m3(uint8_t c)
{
    int s = c >> 7, e = (c >> 3) & 15, m = c & 7;
    double v;
    if (e == 15 && m == 7)
        return NAN;
    if (e == 0)
        v = ldexp((double)m, -9); /* m/8 * 2^-6 */
    else
        v = ldexp((double)(8 + m), e - 10); /* (1 + m/8) * 2^(e-7) */
    return s ? -v : v;
}

/* OCP E2M1: sign, 2-bit exponent (bias 1), 1-bit mantissa; no NaN/Inf. */
double oracle_e2m1(uint8_t nib)
{
    int s = (nib >> 3) & 1, e = (nib >> 1) & 3, m = nib & 1;
    double v;
    if (e == 0)
        v = 0.5 * m; /* subnormal: m/2 * 2^0 */
    else
        v = ldexp((double)(2 + m), e - 2); /* (1 + m/2) * 2^(e-1) */
    return s ? -v : v;
}

/* OCP E8M0 scale: 2^(c-127); 0xFF is NaN. */
double oracle_e8m0(uint8_t c)
{
    if (c == 0xFF)
        return NAN;
    return ldexp(1.0, (int)c - 127);
}

/* bfloat16: the upper half of an IEEE binary32. */
double oracle_bf16(uint16_t b)
{
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, 4);
    return (double)f;
}

static double f32_at(const uint8_t* p)
{
    float f;
    memcpy(&f, p, 4);
    return (double)f;
}

/* -------------------------------------------------------- extent (reading) */

static int64_t extent_of(int32_t L, int32_t max_context)
{
    int64_t E;
    if (L <= 0)
        return 0;
    E = ((int64_t)L + TOK_PER_PAGE - 1) / TOK_PER_PAGE * TOK_PER_PAGE;
    return E < max_context ? E : max_context;
}

/* ------------------------------------------------------------- MQA logits */

/*
 * Shapes (variant 0 = FP8, 1 = MXFP4):
 *   q        FP8  : e4m3 [B, N, H, D]
 *            MXFP4: packed e2m1 [B, N, H, D/2], q_sf e8m0 [B, N, H, D/32]
 *   kv       pages, page i at kv + i*page_stride (layouts above)
 *   w        fp32 [B*N, H]
 *   seq_lens int32 [B]; block_table int32 [B, bt_stride]
 */
typedef struct {
    int variant;
    const uint8_t* q;
    const uint8_t* q_sf;
    const uint8_t* kv;
    int64_t page_stride;
    const float* w;
    const int32_t* seq_lens;
    const int32_t* bt;
    int64_t bt_stride;
    int32_t B, N, H, D, max_context;
    int32_t sfv;         /* MXFP4: values per e8m0 code (32 or 16) */
    int32_t interleaved; /* MXFP4: 1 = each token's codes follow its packed bytes */
} mqa_args;

/* Decoded key vector of KV position p of request b (float64), and its s_p. */
static double decode_key(const mqa_args* a, int32_t b, int64_t p, double* k)
{
    int32_t page = a->bt[(int64_t)b * a->bt_stride + p / TOK_PER_PAGE];
    int64_t j = p % TOK_PER_PAGE;
    const uint8_t* pg = a->kv + (int64_t)page * a->page_stride;
    int D = a->D, d;
    if (a->variant == 0) {
        const uint8_t* row = pg + j * D;
        for (d = 0; d < D; ++d)
            k[d] = oracle_e4m3(row[d]);
        return f32_at(pg + (int64_t)TOK_PER_PAGE * D + j * 4); /* s_p */
    } else {
        int nsf = D / a->sfv; /* codes per token */
        const uint8_t* row;
        const uint8_t* sf;
        if (a->interleaved) {
            row = pg + j * (D / 2 + nsf);
            sf = row + D / 2;
        } else {
            row = pg + j * (D / 2);
            sf = pg + (int64_t)TOK_PER_PAGE * (D / 2) + j * nsf;
        }
        for (d = 0; d < D; ++d) {
            uint8_t byte = row[d / 2];
            uint8_t nib = (d & 1) ? (byte >> 4) : (byte & 15);
            k[d] = oracle_e2m1(nib) * oracle_e8m0(sf[d / a->sfv]);
        }
        return 1.0; /* MXFP4 has no per-position factor */
    }
}

/* Decoded query vector for (b, t, h). */
static void decode_query(const mqa_args* a, int32_t b, int32_t t, int32_t h, double* qv)
{
    int D = a->D, d;
    int64_t qi = (((int64_t)b * a->N + t) * a->H + h);
    if (a->variant == 0) {
        const uint8_t* row = a->q + qi * D;
        for (d = 0; d < D; ++d)
            qv[d] = oracle_e4m3(row[d]);
    } else {
        const uint8_t* row = a->q + qi * (D / 2);
        const uint8_t* sf = a->q_sf + qi * (D / a->sfv);
        for (d = 0; d < D; ++d) {
            uint8_t byte = row[d / 2];
            uint8_t nib = (d & 1) ? (byte >> 4) : (byte & 15);
            qv[d] = oracle_e2m1(nib) * oracle_e8m0(sf[d / a->sfv]);
        }
    }
}

/*
 * The logit of output row r = b*N + t at KV position p:
 *   s_p * sum_h w[r,h] * max(0, sum_d q[b,t,h,d] * k_p[d])
 * with the rectifier applied to each head's score before the weighted sum.
 * qdec holds the decoded query of (b, t): qdec[h*D + d].
 */
static double logit_at(const mqa_args* a, int32_t b, int32_t t, const double* k, double s_p,
                       const double* qdec, double* amag)
{
    int32_t r = b * a->N + t;
    double acc = 0.0, mag = 0.0;
    int h, d;
    for (h = 0; h < a->H; ++h) {
        double dot = 0.0, relu, wh = (double)a->w[(int64_t)r * a->H + h];
        for (d = 0; d < a->D; ++d)
            dot += qdec[(int64_t)h * a->D + d] * k[d];
        relu = dot > 0.0 ? dot : 0.0;
        acc += wh * relu;
        mag += fabs(wh) * relu;
    }
    *amag = s_p * mag;
    return s_p * acc;
}

/* Decoded query of (b, t) for all heads. */
static void decode_query_rows(const mqa_args* a, int32_t b, int32_t t, double* qdec)
{
    int32_t h;
    for (h = 0; h < a->H; ++h)
        decode_query(a, b, t, h, qdec + (int64_t)h * a->D);
}

/* Dense evaluation: ref/amag are [B*N, max_context] float64, written is u8 of
 * the same shape (1 where the operation writes the cell).  Cells outside the
 * written set are left as they are. */
static int mqa_dense(const mqa_args* a, double* ref, double* amag, uint8_t* written, int nthreads)
{
    int32_t b;
    (void)nthreads;
#pragma omp parallel for schedule(dynamic, 1) num_threads(nthreads > 0 ? nthreads : 1)
    for (b = 0; b < a->B; ++b) {
        int64_t E = extent_of(a->seq_lens[b], a->max_context), p;
        double* k = (double*)malloc(sizeof(double) * a->D);
        double* qdec = (double*)malloc(sizeof(double) * (size_t)a->N * a->H * a->D);
        int32_t t;
        for (t = 0; t < a->N; ++t)
            decode_query_rows(a, b, t, qdec + (int64_t)t * a->H * a->D);
        for (p = 0; p < E; ++p) {
            double s_p = decode_key(a, b, p, k);
            for (t = 0; t < a->N; ++t) {
                int64_t o = ((int64_t)b * a->N + t) * a->max_context + p;
                double m;
                ref[o] = logit_at(a, b, t, k, s_p, qdec + (int64_t)t * a->H * a->D, &m);
                amag[o] = m;
                written[o] = 1;
            }
        }
        free(k);
        free(qdec);
    }
    return 0;
}

/* Point evaluation at (rows[i], cols[i]); written[i] says whether the cell is
 * in the written set (ref/amag are NaN/0 where it is not). */
static int mqa_points(const mqa_args* a, int64_t npts, const int32_t* rows, const int32_t* cols,
                      double* ref, double* amag, uint8_t* written, int nthreads)
{
    int64_t i;
    (void)nthreads;
#pragma omp parallel for schedule(dynamic, 64) num_threads(nthreads > 0 ? nthreads : 1)
    for (i = 0; i < npts; ++i) {
        int32_t r = rows[i], b = r / a->N, t = r % a->N;
        int64_t p = cols[i], E = extent_of(a->seq_lens[b], a->max_context);
        if (p < 0 || p >= E) {
            ref[i] = NAN;
            amag[i] = 0.0;
            written[i] = 0;
        } else {
            double* k = (double*)malloc(sizeof(double) * a->D);
            double* qdec = (double*)malloc(sizeof(double) * (size_t)a->H * a->D);
            double s_p = decode_key(a, b, p, k), m;
            decode_query_rows(a, b, t, qdec);
            ref[i] = logit_at(a, b, t, k, s_p, qdec, &m);
            amag[i] = m;
            written[i] = 1;
            free(k);
            free(qdec);
        }
    }
    return 0;
}

static int mqa_check(const mqa_args* a)
{
    if (a->B < 0 || a->N < 1 || a->H < 1 || a->D < 1 || a->max_context < 0)
        return -2;
    if (a->variant == 1 && ((a->sfv != 32 && a->sfv != 16) || a->D % a->sfv != 0 ||
                            (a->interleaved != 0 && a->interleaved != 1)))
        return -2;
    return 0;
}

/* sfv / interleaved describe the MXFP4 scale layout (32 / 0 is the layout of
 * the variant's defaults); they are ignored for FP8. */
int oracle_mqa_logits(int variant, const uint8_t* q, const uint8_t* q_sf, const uint8_t* kv,
                      int64_t page_stride, const float* w, const int32_t* seq_lens,
                      const int32_t* bt, int64_t bt_stride, int32_t B, int32_t N, int32_t H,
                      int32_t D, int32_t max_context, int32_t sfv, int32_t interleaved,
                      double* ref, double* amag, uint8_t* written, int nthreads)
{
    mqa_args a = {variant, q, q_sf, kv, page_stride, w, seq_lens, bt, bt_stride,
                  B, N, H, D, max_context, sfv, interleaved};
    int rc = mqa_check(&a);
    if (rc)
        return rc;
    return mqa_dense(&a, ref, amag, written, nthreads);
}

int oracle_mqa_logits_points(int variant, const uint8_t* q, const uint8_t* q_sf,
                             const uint8_t* kv, int64_t page_stride, const float* w,
                             const int32_t* seq_lens, const int32_t* bt, int64_t bt_stride,
                             int32_t B, int32_t N, int32_t H, int32_t D, int32_t max_context,
                             int32_t sfv, int32_t interleaved, int64_t npts, const int32_t* rows,
                             const int32_t* cols, double* ref, double* amag, uint8_t* written,
                             int nthreads)
{
    mqa_args a = {variant, q, q_sf, kv, page_stride, w, seq_lens, bt, bt_stride,
                  B, N, H, D, max_context, sfv, interleaved};
    int rc = mqa_check(&a);
    if (rc)
        return rc;
    return mqa_points(&a, npts, rows, cols, ref, amag, written, nthreads);
}

/* The written set alone ([B*N, max_context] u8): cheap, for full-size checks. */
int oracle_mqa_written(const int32_t* seq_lens, int32_t B, int32_t N, int32_t max_context,
                       uint8_t* written)
{
    int32_t b, t;
    if (B < 0 || N < 1 || max_context < 0)
        return -2;
    for (b = 0; b < B; ++b) {
        int64_t E = extent_of(seq_lens[b], max_context);
        for (t = 0; t < N; ++t) {
            uint8_t* row = written + ((int64_t)b * N + t) * max_context;
            memset(row, 0, (size_t)max_context);
            memset(row, 1, (size_t)E);
        }
    }
    return 0;
}

/* ---------------------------------------------------------- indexer scores */

/*
 * query bf16 [rows, D]; key pages bf16 [64, D] at key_cache + i*page_stride;
 * block_table int32 [requests, bt_stride]; group g covers rows
 * row_offsets[g] .. row_offsets[g+1]-1, belongs to request requests[g] and has
 * context_lengths[g] keys.  scores/amag/written are [rows, max_context].
 * A group of non-positive length reads nothing (its request is not looked at).
 */
int oracle_indexer_scores(const uint16_t* query, int32_t rows, int32_t D, const uint8_t* key_cache,
                          int64_t page_stride, const int32_t* bt, int64_t bt_stride,
                          const int32_t* context_lengths, const int32_t* requests,
                          const int32_t* row_offsets, int32_t groups, int32_t max_context,
                          double* scores, double* amag, uint8_t* written, int nthreads)
{
    int32_t g;
    (void)nthreads;
    if (rows < 0 || groups < 0 || D < 1 || max_context < 0)
        return -2;
#pragma omp parallel for schedule(dynamic, 1) num_threads(nthreads > 0 ? nthreads : 1)
    for (g = 0; g < groups; ++g) {
        int32_t L = context_lengths[g], r;
        int64_t k;
        if (L > max_context)
            L = max_context;
        if (L <= 0)
            continue;
        for (r = row_offsets[g]; r < row_offsets[g + 1]; ++r) {
            for (k = 0; k < L; ++k) {
                int32_t page = bt[(int64_t)requests[g] * bt_stride + k / TOK_PER_PAGE];
                const uint16_t* key = (const uint16_t*)(key_cache + (int64_t)page * page_stride) +
                                      (k % TOK_PER_PAGE) * D;
                double dot = 0.0, mag = 0.0;
                int d;
                for (d = 0; d < D; ++d) {
                    double prod = oracle_bf16(query[(int64_t)r * D + d]) * oracle_bf16(key[d]);
                    dot += prod;
                    mag += fabs(prod);
                }
                scores[(int64_t)r * max_context + k] = dot;
                amag[(int64_t)r * max_context + k] = mag;
                written[(int64_t)r * max_context + k] = 1;
            }
        }
    }
    return 0;
}

/*
 * One-head indexer scores with NVFP4 inputs ([indexer], query / key_cache /
 * query_scales / key_scales parameters): the query is packed e2m1
 * [rows, D/2] with one e4m3 scale per 16 values in query_scales [rows, D/16];
 * each key page holds 64 keys of packed e2m1 [64, D/2] at its start, and the
 * page's e4m3 scales [64, D/16] sit at key_scales + page*scale_page_stride
 * ("paged like the keys").  A score is the dot product of the dequantised
 * vectors: sum_d (e2m1(q_d) * qs[d/16]) * (e2m1(k_d) * ks[d/16]).  Packed
 * bytes hold the even element in the low nibble.  amag = sum_d |q_d k_d| of
 * the dequantised values.  Same extent and group rules as the BF16 form.
 */
static double nvfp4_at(const uint8_t* packed, const uint8_t* scales, int d)
{
    uint8_t byte = packed[d / 2];
    uint8_t nib = (d & 1) ? (byte >> 4) : (byte & 15);
    return oracle_e2m1(nib) * oracle_e4m3(scales[d / 16]);
}

int oracle_indexer_scores_nvfp4(const uint8_t* query, const uint8_t* query_scales, int32_t rows,
                                int32_t D, const uint8_t* key_cache, int64_t page_stride,
                                const uint8_t* key_scales, int64_t scale_page_stride,
                                const int32_t* bt, int64_t bt_stride,
                                const int32_t* context_lengths, const int32_t* requests,
                                const int32_t* row_offsets, int32_t groups, int32_t max_context,
                                double* scores, double* amag, uint8_t* written, int nthreads)
{
    int32_t g;
    (void)nthreads;
    if (rows < 0 || groups < 0 || D < 16 || D % 16 != 0 || max_context < 0)
        return -2;
#pragma omp parallel for schedule(dynamic, 1) num_threads(nthreads > 0 ? nthreads : 1)
    for (g = 0; g < groups; ++g) {
        int32_t L = context_lengths[g], r;
        int64_t k;
        if (L > max_context)
            L = max_context;
        if (L <= 0)
            continue;
        for (r = row_offsets[g]; r < row_offsets[g + 1]; ++r) {
            const uint8_t* qrow = query + (int64_t)r * (D / 2);
            const uint8_t* qsc = query_scales + (int64_t)r * (D / 16);
            for (k = 0; k < L; ++k) {
                int32_t page = bt[(int64_t)requests[g] * bt_stride + k / TOK_PER_PAGE];
                int64_t j = k % TOK_PER_PAGE;
                const uint8_t* krow = key_cache + (int64_t)page * page_stride + j * (D / 2);
                const uint8_t* ksc = key_scales + (int64_t)page * scale_page_stride + j * (D / 16);
                double dot = 0.0, mag = 0.0;
                int d;
                for (d = 0; d < D; ++d) {
                    double prod = nvfp4_at(qrow, qsc, d) * nvfp4_at(krow, ksc, d);
                    dot += prod;
                    mag += fabs(prod);
                }
                scores[(int64_t)r * max_context + k] = dot;
                amag[(int64_t)r * max_context + k] = mag;
                written[(int64_t)r * max_context + k] = 1;
            }
        }
    }
    return 0;
}

/* ------------------------------------------------- block-max proxy score */

/*
 * Per-KV-block max of the unscaled, causally masked Q K^T logits with NVFP4
 * inputs ([proxy] "flashinfer.msa_ops.msa_proxy_score_fp4": description,
 * parameter list and "Returns").  The page defers most parameters to another
 * page that is not available; the readings taken here (each listed in the
 * design notes):
 *   - head_dim 128 (64 packed bytes per row); each row has 8 e4m3 scales, one
 *     per 16 values, stored row-major (8 bytes per row) with the page's row
 *     index: query row = token * Hq + head; flat key row = token * Hkv +
 *     kv_head; paged key row = (page * Hkv + kv_head) * 128 + token_in_page;
 *   - a dequantised value is e2m1(nibble) * e4m3(scale of its 16-block); the
 *     logit of (query token i, head h, key k) is
 *         (q_global_scale * k_global_scale) * sum_d q[i,h,d] * k[k,kvh,d],
 *     kvh = h / (Hq / Hkv) (consecutive heads share a KV head), with no other
 *     scale ("unscaled"); the global scales multiply before the max;
 *   - a KV block is 128 consecutive keys of a request (the paged K's page):
 *     block t covers keys 128t .. 128t+127;
 *   - query token i belongs to request r with cu_q[r] <= i < cu_q[r+1], at
 *     position p = i - cu_q[r]; Lq = cu_q[r+1] - cu_q[r]; the request's key
 *     count Lk is cu_k[r+1] - cu_k[r] (flat) or seqused_k[r] (paged, at most
 *     pt_width * 128); negative counts are 0;
 *   - causal: key k is visible to token p iff k <= q_offset[r] + p, with
 *     q_offset[r] defaulting to Lk - Lq (the last query token sees the last
 *     key); not causal: every key below Lk is visible;
 *   - out[h, t, i] = max over visible keys k of block t of the logit; -inf
 *     when block t holds no visible key (past the request's keys, fully
 *     masked, or token i in no request); a paged block whose page id is
 *     outside [0, num_pages) is never read, and every output of it that has
 *     a visible key is NaN;
 *   - reduce_heads: out[0, t, i] = max over heads of out[h, t, i] (NaN if
 *     any is NaN).
 * Output layout [H_out, max_k_tiles, total_q]; amag has the same layout:
 * the largest |q_global_scale * k_global_scale| * sum_d |q_d k_d| over the
 * visible keys of the block (0 where the output is -inf or NaN), the
 * magnitude the parity tolerance scales with.
 */
#define PROXY_BLOCK 128

typedef struct {
    const uint8_t *q, *q_scale, *k, *k_scale;
    const int32_t *cu_q, *cu_k, *page_table, *seqused_k, *q_offset;
    int64_t page_stride, pt_stride;
    int32_t total_q, Hq, Hkv, num_pages, pt_width, B, max_k_tiles;
    int paged, causal, reduce_heads;
    double g; /* q_global_scale * k_global_scale */
} proxy_args;

static double proxy_value(const uint8_t* row, const uint8_t* scales, int d)
{
    uint8_t byte = row[d / 2];
    uint8_t nib = (d & 1) ? (byte >> 4) : (byte & 15);
    return oracle_e2m1(nib) * oracle_e4m3(scales[d / 16]);
}

/* Key count of request r (reading: at most pt_width blocks when paged). */
static int64_t proxy_lk(const proxy_args* a, int32_t r)
{
    int64_t Lk = a->paged ? a->seqused_k[r] : (int64_t)a->cu_k[r + 1] - a->cu_k[r];
    if (Lk < 0)
        Lk = 0;
    if (a->paged && Lk > (int64_t)a->pt_width * PROXY_BLOCK)
        Lk = (int64_t)a->pt_width * PROXY_BLOCK;
    return Lk;
}

/* Block max of head h over block t for token p of request r: -inf if the
 * block holds no visible key, NaN if its page id is out of range. */
static void proxy_cell(const proxy_args* a, int32_t r, int32_t p, int32_t h, int32_t t,
                       double* val, double* mag)
{
    const int64_t Lq = (int64_t)a->cu_q[r + 1] - a->cu_q[r], Lk = proxy_lk(a, r);
    const int64_t off = a->q_offset ? (int64_t)a->q_offset[r] : Lk - Lq;
    const int64_t i = (int64_t)a->cu_q[r] + p;
    const int32_t kvh = h / (a->Hq / a->Hkv);
    const uint8_t* qrow = a->q + (i * a->Hq + h) * 64;
    const uint8_t* qsc = a->q_scale + (i * a->Hq + h) * 8;
    double best = -INFINITY, best_mag = 0.0;
    int32_t page = 0;
    int any = 0;
    int64_t kk;
    if (a->paged && (int64_t)t * PROXY_BLOCK < Lk)
        page = a->page_table[(int64_t)r * a->pt_stride + t];
    for (kk = (int64_t)t * PROXY_BLOCK; kk < (int64_t)(t + 1) * PROXY_BLOCK; ++kk) {
        const uint8_t *krow, *ksc;
        double dot = 0.0, m = 0.0;
        int d;
        if (kk >= Lk || (a->causal && kk > off + p))
            continue;
        any = 1;
        if (a->paged) {
            if (page < 0 || page >= a->num_pages)
                break;
            krow = a->k + (int64_t)page * a->page_stride +
                   ((int64_t)kvh * PROXY_BLOCK + kk % PROXY_BLOCK) * 64;
            ksc = a->k_scale + (((int64_t)page * a->Hkv + kvh) * PROXY_BLOCK + kk % PROXY_BLOCK) * 8;
        } else {
            const int64_t row = ((int64_t)a->cu_k[r] + kk) * a->Hkv + kvh;
            krow = a->k + row * 64;
            ksc = a->k_scale + row * 8;
        }
        for (d = 0; d < 128; ++d) {
            const double prod = proxy_value(qrow, qsc, d) * proxy_value(krow, ksc, d);
            dot += prod;
            m += fabs(prod);
        }
        if (a->g * dot > best)
            best = a->g * dot;
        if (fabs(a->g) * m > best_mag)
            best_mag = fabs(a->g) * m;
    }
    if (any && a->paged && (page < 0 || page >= a->num_pages)) {
        *val = NAN;
        *mag = 0.0;
        return;
    }
    *val = best;
    *mag = best_mag;
}

/* Output hout (a head, or 0 with reduce_heads: the max over heads). */
static void proxy_out(const proxy_args* a, int32_t r, int32_t p, int32_t hout, int32_t t,
                      double* val, double* mag)
{
    int32_t h;
    if (!a->reduce_heads) {
        proxy_cell(a, r, p, hout, t, val, mag);
        return;
    }
    *val = -INFINITY;
    *mag = 0.0;
    for (h = 0; h < a->Hq; ++h) {
        double v, m;
        proxy_cell(a, r, p, h, t, &v, &m);
        if (isnan(v) || isnan(*val)) {
            *val = NAN;
            *mag = 0.0;
            continue;
        }
        if (v > *val)
            *val = v;
        if (m > *mag)
            *mag = m;
    }
}

static int proxy_check(const proxy_args* a)
{
    int32_t r;
    if (a->total_q < 0 || a->Hq < 1 || a->Hkv < 1 || a->Hq % a->Hkv != 0 || a->B < 0 ||
        a->max_k_tiles < 0)
        return -2;
    if (a->paged && (a->pt_width < 0 || a->pt_stride < a->pt_width))
        return -2;
    for (r = 0; r < a->B; ++r)
        if (a->cu_q[r] < 0 || a->cu_q[r + 1] < a->cu_q[r] || a->cu_q[r + 1] > a->total_q)
            return -2;
    return 0;
}

static void proxy_fill(proxy_args* a, const uint8_t* q, const uint8_t* q_scale, int32_t total_q,
                       int32_t Hq, int32_t Hkv, const uint8_t* k, const uint8_t* k_scale,
                       int paged, int64_t page_stride, int32_t num_pages, const int32_t* cu_q,
                       const int32_t* cu_k, const int32_t* page_table, int64_t pt_stride,
                       int32_t pt_width, const int32_t* seqused_k, int32_t B, double qgs,
                       double kgs, int causal, const int32_t* q_offset, int32_t max_k_tiles,
                       int reduce_heads)
{
    a->q = q, a->q_scale = q_scale, a->k = k, a->k_scale = k_scale;
    a->cu_q = cu_q, a->cu_k = cu_k, a->page_table = page_table, a->seqused_k = seqused_k;
    a->q_offset = q_offset;
    a->page_stride = page_stride, a->pt_stride = pt_stride;
    a->total_q = total_q, a->Hq = Hq, a->Hkv = Hkv, a->num_pages = num_pages;
    a->pt_width = pt_width, a->B = B, a->max_k_tiles = max_k_tiles;
    a->paged = paged, a->causal = causal, a->reduce_heads = reduce_heads;
    a->g = qgs * kgs;
}

/* Dense: out and amag are [H_out, max_k_tiles, total_q]. */
int oracle_proxy_score_fp4(const uint8_t* q, const uint8_t* q_scale, int32_t total_q, int32_t Hq,
                           int32_t Hkv, const uint8_t* k, const uint8_t* k_scale, int paged,
                           int64_t page_stride, int32_t num_pages, const int32_t* cu_q,
                           const int32_t* cu_k, const int32_t* page_table, int64_t pt_stride,
                           int32_t pt_width, const int32_t* seqused_k, int32_t B, double qgs,
                           double kgs, int causal, const int32_t* q_offset, int32_t max_k_tiles,
                           int reduce_heads, double* out, double* amag, int nthreads)
{
    proxy_args a;
    int32_t Hout, r;
    int64_t idx, plane;
    proxy_fill(&a, q, q_scale, total_q, Hq, Hkv, k, k_scale, paged, page_stride, num_pages, cu_q,
               cu_k, page_table, pt_stride, pt_width, seqused_k, B, qgs, kgs, causal, q_offset,
               max_k_tiles, reduce_heads);
    if (proxy_check(&a) != 0)
        return -2;
    Hout = reduce_heads ? 1 : Hq;
    plane = (int64_t)max_k_tiles * total_q;
    for (idx = 0; idx < (int64_t)Hout * plane; ++idx) {
        out[idx] = -INFINITY; /* tokens in no request */
        amag[idx] = 0.0;
    }
    (void)nthreads;
#pragma omp parallel for schedule(dynamic, 1) num_threads(nthreads > 0 ? nthreads : 1)
    for (r = 0; r < B; ++r) {
        int32_t p, h, t;
        for (p = 0; p < cu_q[r + 1] - cu_q[r]; ++p)
            for (h = 0; h < Hout; ++h)
                for (t = 0; t < max_k_tiles; ++t) {
                    const int64_t o = ((int64_t)h * max_k_tiles + t) * total_q + cu_q[r] + p;
                    proxy_out(&a, r, p, h, t, &out[o], &amag[o]);
                }
    }
    return 0;
}

/* Points (hs[n], ts[n], is[n]): the same values one by one. */
int oracle_proxy_score_fp4_points(const uint8_t* q, const uint8_t* q_scale, int32_t total_q,
                                  int32_t Hq, int32_t Hkv, const uint8_t* k,
                                  const uint8_t* k_scale, int paged, int64_t page_stride,
                                  int32_t num_pages, const int32_t* cu_q, const int32_t* cu_k,
                                  const int32_t* page_table, int64_t pt_stride, int32_t pt_width,
                                  const int32_t* seqused_k, int32_t B, double qgs, double kgs,
                                  int causal, const int32_t* q_offset, int32_t max_k_tiles,
                                  int reduce_heads, int64_t npts, const int32_t* hs,
                                  const int32_t* ts, const int32_t* is, double* out,
                                  double* amag, int nthreads)
{
    proxy_args a;
    int64_t n;
    proxy_fill(&a, q, q_scale, total_q, Hq, Hkv, k, k_scale, paged, page_stride, num_pages, cu_q,
               cu_k, page_table, pt_stride, pt_width, seqused_k, B, qgs, kgs, causal, q_offset,
               max_k_tiles, reduce_heads);
    if (proxy_check(&a) != 0)
        return -2;
    for (n = 0; n < npts; ++n)
        if (hs[n] < 0 || hs[n] >= (reduce_heads ? 1 : Hq) || ts[n] < 0 || ts[n] >= max_k_tiles ||
            is[n] < 0 || is[n] >= total_q)
            return -2;
    (void)nthreads;
#pragma omp parallel for schedule(dynamic, 16) num_threads(nthreads > 0 ? nthreads : 1)
    for (n = 0; n < npts; ++n) {
        int32_t r, found = -1;
        for (r = 0; r < B; ++r)
            if (cu_q[r] <= is[n] && is[n] < cu_q[r + 1]) {
                found = r;
                break;
            }
        if (found < 0) {
            out[n] = -INFINITY;
            amag[n] = 0.0;
        } else {
            proxy_out(&a, found, is[n] - cu_q[found], hs[n], ts[n], &out[n], &amag[n]);
        }
    }
    return 0;
}

int oracle_max_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
