/*
 * pmqa.h - paged MQA logits for AMD Instinct MI355X (gfx950).
 *
 * C ABI of libpmqa.so.  Operations (FlashInfer documentation pages):
 *
 *   "flashinfer.attn_scores", introductory equation:
 *       logits[t, p] = s_p * sum_h w[t, h] * relu(q[t, h] . k_p)
 *   with the rectifier applied per head before the weighted sum (so a negative
 *   weight can make a logit negative).  The FP8 variant multiplies by the
 *   per-token fp32 scale s_p held in the trailing scale region of each KV page;
 *   the MXFP4 variant has no s_p (its per-32-element block scales are part of
 *   the dequantised q and k values).
 *
 *   "flashinfer.sdsa.indexer_scores": the one-head case, a plain dot product of
 *   each query row with each key of its request, for groups of 1..8 query rows.
 *
 *   "flashinfer.msa_ops.msa_proxy_score_fp4": the per-KV-block max of the
 *   causally masked Q K^T logits with NVFP4 query and keys.
 *
 * Conventions shared by every entry point:
 *   - Every tensor pointer is a DEVICE pointer owned by the caller.  The
 *     library never reads device memory on the host, never allocates per call,
 *     never synchronises, and never prints.  Work is enqueued on `stream`
 *     (a hipStream_t; NULL = the legacy default stream), so a whole call can be
 *     captured in a HIP graph.
 *   - Return value: PMQA_OK (0) or a negative pmqa_status.  Invalid arguments
 *     are rejected on the host before anything is enqueued.  A failed launch
 *     returns PMQA_ERR_HIP.
 *   - Device-data preconditions (not checkable without reading the device):
 *     seq_lens / context_lengths in [0, max_context] (larger values are clamped
 *     to max_context, negative ones count as 0), page ids below num_pages, and
 *     request ids below num_requests.  A page id or request id out of range is
 *     never dereferenced: the outputs that would depend on it are written as
 *     NaN instead.
 *   - Pages hold 64 tokens.
 */
#ifndef PMQA_H
#define PMQA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    PMQA_OK = 0,
    PMQA_ERR_NULL = -1,        /* a required pointer is NULL                    */
    PMQA_ERR_SHAPE = -2,       /* a size or stride is out of range              */
    PMQA_ERR_UNSUPPORTED = -3, /* a valid but unimplemented option              */
    PMQA_ERR_ALIGN = -4,       /* a pointer or stride is not aligned as needed  */
    PMQA_ERR_WORKSPACE = -5,   /* workspace smaller than mqa_logits_workspace_bytes() */
    PMQA_ERR_HIP = -6          /* the HIP runtime reported an error             */
} pmqa_status;

enum { PMQA_F32 = 0, PMQA_BF16 = 1 };               /* output / accumulator dtypes */
enum { PMQA_VARIANT_FP8 = 0, PMQA_VARIANT_MXFP4 = 1 };

#define PMQA_PAGE_TOKENS 64
#define PMQA_MAX_BATCH 8192  /* requests per call                       */
#define PMQA_MAX_NEXT_N 8    /* query tokens per request (next_n)       */

/*
 * mqa_logits_fp8 - FP8 paged MQA logits.
 * ("flashinfer.attn_scores": equation, the s_p bullet, the output-contract note.)
 *
 *   q            e4m3fn [batch, next_n, num_heads, head_dim], contiguous, 16-B aligned.
 *                Consumed as decoded e4m3 (no separate query scale).
 *   kv_fused     num_pages pages; page i starts at kv_fused + i*page_stride bytes
 *                and holds 64 x head_dim e4m3 key bytes (token-major) followed
 *                by 64 little-endian fp32 scales s_p.  page_stride >= 64*(head_dim+4),
 *                a multiple of 16; kv_fused 16-B aligned.
 *   weights      fp32 [batch*next_n, num_heads], contiguous, 16-B aligned.
 *   seq_lens     int32 [batch].
 *   block_table  int32 [batch, bt_stride]; entry j of row b is the page holding
 *                tokens 64j..64j+63 of request b.  bt_width = usable entries per
 *                row; bt_width*64 >= max_context.  Entries at or beyond
 *                ceil(seq_lens[b]/64) are never read.
 *   out          [batch*next_n, out_row_stride] of out_dtype (PMQA_F32 or PMQA_BF16).
 *                Row b*next_n+t is written at columns 0 .. E_b-1, where
 *                E_b = min(ceil(seq_lens[b]/64)*64, max_context) (whole pages,
 *                unconditionally, no causal or length mask); later columns and
 *                every row of a request with seq_lens[b] <= 0 are not touched.
 *                Only columns 0 .. seq_lens[b]-next_n+t of row b*next_n+t are
 *                meaningful; masking beyond that is the caller's job.
 *                max_context % 64 == 0, out_row_stride >= max_context.
 *                The rectifier and the weighted head sum run in fp32 for both
 *                output types; PMQA_BF16 rounds the result to nearest even.
 *   acc_dtype    PMQA_F32 (the only accumulator; anything else -> UNSUPPORTED).
 *                Every product is exact and the sums keep fp32 precision: the
 *                e4m3 values are widened exactly to f16 and multiplied on the
 *                matrix unit's f16 path.  (The unit's FP8 path truncates each
 *                run of 8 products below 2^-13 of the run's largest, which can
 *                lose the whole value of a cancelling dot product, so it is not
 *                used.)
 *   schedule     NULL (the kernel splits the work itself, on the GPU) or a buffer
 *                filled by mqa_logits_schedule() with the same next_n, variant
 *                and max_context, valid only while seq_lens is unchanged
 *                ("flashinfer.attn_scores", Scheduling and Setup, and its warning).
 *                A schedule built for other arguments is detected on the device
 *                and ignored.
 *   workspace, workspace_bytes
 *                NULL, or caller-owned device memory of at least
 *                mqa_logits_workspace_bytes() bytes, 16-B aligned (smaller ->
 *                PMQA_ERR_WORKSPACE), zero-filled before its first use.  Used
 *                only when schedule is NULL, by the 64-head x 128 kernels: it
 *                holds a work counter with which the workgroups that finish
 *                their share first take the last items of the call in small
 *                chunks (the per-call work assignment on the GPU of
 *                "flashinfer.attn_scores", Scheduling and Setup).  Every
 *                completed call leaves it zero-filled again, so calls and graph
 *                replays need no clearing; two calls that may run at the same
 *                time must not share one.  NULL: the kernel's static split.
 *                The logits do not depend on the split.
 *   Supported (the FP8 variant's shapes are parametric: "flashinfer.attn_scores",
 *   paragraph on how the variants differ): 1 <= num_heads <= 128,
 *   head_dim a multiple of 16 in 16..256, 1 <= next_n <= 8; other values ->
 *   UNSUPPORTED.  A call is one or more kernel launches on `stream`, each over
 *   a group of query slots (up to 4 with 64 heads x 128; otherwise as many as
 *   fit a 32 KB query slice of the padded heads).  q and weights are read
 *   once per launch; the pages once per launch.
 */
int mqa_logits_fp8(const void* q, const void* kv_fused, int64_t page_stride, int32_t num_pages,
                   const float* weights, const int32_t* seq_lens, const int32_t* block_table,
                   int64_t bt_stride, int32_t bt_width, int32_t batch, int32_t next_n,
                   int32_t num_heads, int32_t head_dim, void* out, int64_t out_row_stride,
                   int32_t max_context, int32_t out_dtype, int32_t acc_dtype,
                   const int32_t* schedule, void* workspace, size_t workspace_bytes,
                   void* stream);

/*
 * mqa_logits_fp8_no_alloc - mqa_logits_fp8 for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses
 * that forbid allocation): the same arguments and results, without the
 * workspace.  The work counters (1 KiB) live in a device array of the library,
 * one per GPU, zero when the library is loaded and left zero by every
 * completed call; the call allocates nothing and clears nothing.  Every call
 * on one GPU shares that array: calls that may overlap on one GPU (different
 * streams) race on it, so such callers use mqa_logits_fp8 with a workspace
 * each.  Errors as mqa_logits_fp8 (the first call on a device also
 * initialises it, as mqa_logits_init).
 */
int mqa_logits_fp8_no_alloc(const void* q, const void* kv_fused, int64_t page_stride,
                            int32_t num_pages, const float* weights, const int32_t* seq_lens,
                            const int32_t* block_table, int64_t bt_stride, int32_t bt_width,
                            int32_t batch, int32_t next_n, int32_t num_heads, int32_t head_dim,
                            void* out, int64_t out_row_stride, int32_t max_context,
                            int32_t out_dtype, int32_t acc_dtype, const int32_t* schedule,
                            void* stream);

/*
 * mqa_logits_mxfp4 - MXFP4 paged MQA logits (no s_p; block scales folded).
 * ("flashinfer.attn_scores": equation, the MXFP4 bullet, and the paragraph on
 * q_sf / sf_vec_size / is_kv_sf_interleaved, two FP4 values per byte, exactly
 * 64 heads and head_dim 128.)
 *
 *   q            packed e2m1 [batch, next_n, 64, 64] (two values per byte, the
 *                even element in the low nibble), 16-B aligned.
 *   sf_vec_size  32 or 16: values per e8m0 scale code, along head_dim, for
 *                query and keys alike (other values -> UNSUPPORTED).  The
 *                pages leave 16 open; this library reads it as one code per
 *                16 consecutive values, the codes of a row in order.
 *   q_sf         e8m0 [batch, next_n, 64, 128/sf_vec_size], contiguous.
 *   is_kv_sf_interleaved  0: each page holds 64 x 64 packed key bytes, then
 *                64 x 128/sf_vec_size codes (token-major).  1: each page
 *                holds 64 token records, a token's 64 packed bytes followed
 *                by its 128/sf_vec_size codes (records of 68 or 72 bytes; the
 *                pages name the flag without its layout, this is the reading
 *                taken).  Other values -> UNSUPPORTED.
 *   kv_fused     page i at kv_fused + i*page_stride; page_stride >=
 *                64 * (64 + 128/sf_vec_size) (4352 or 4608), a multiple of 16.
 *   out_dtype    PMQA_BF16 (the default of this variant, round to nearest even)
 *                or PMQA_F32.  The e2m1 products and their block scales are
 *                exact on the matrix unit and blocks add at fp32 precision.
 *                PMQA_F32 sums the heads in fp32.  PMQA_BF16 sums them on the
 *                matrix unit in bf16 products: each rectified score and each
 *                weight is rounded to bf16 once, with fp32 accumulation.  That
 *                adds at most 2^-8 * sum_h |w_h| relu(q_h . k) of error before
 *                the output's own bf16 rounding.
 *   Supported: num_heads == 64, head_dim == 128 (other values -> UNSUPPORTED),
 *   1 <= next_n <= 8 (next_n above 4 runs as two launches over the slots).
 *   Everything else as in mqa_logits_fp8.
 */
int mqa_logits_mxfp4(const void* q, const void* q_sf, int32_t sf_vec_size,
                     int32_t is_kv_sf_interleaved, const void* kv_fused, int64_t page_stride,
                     int32_t num_pages, const float* weights, const int32_t* seq_lens,
                     const int32_t* block_table, int64_t bt_stride, int32_t bt_width,
                     int32_t batch, int32_t next_n, int32_t num_heads, int32_t head_dim,
                     void* out, int64_t out_row_stride, int32_t max_context, int32_t out_dtype,
                     const int32_t* schedule, void* workspace, size_t workspace_bytes,
                     void* stream);

/*
 * indexer_scores - one-head BF16 indexer scores.
 * ("flashinfer.sdsa.indexer_scores": description and parameter list.)
 *
 *   query            bf16 [rows, 128], contiguous, 16-B aligned.
 *   key_cache        bf16 key pages [64, 128]; page i at key_cache + i*page_stride
 *                    bytes, page_stride >= 16384 and a multiple of 16 (views into
 *                    a cache that also holds other data per page are fine).
 *   block_table      int32 [num_requests, bt_stride], bt_width usable entries per
 *                    row, bt_width*64 >= max_context.
 *   context_lengths  int32 [groups]: keys of each group.
 *   requests         int32 [groups]: the block-table row of each group; its value
 *                    is not used for a group of length <= 0, so any value is
 *                    allowed there (nothing is looked up with it).
 *   group_row_offsets  NULL: every group has rows/groups consecutive rows (an
 *                    integer in 1..8).  Otherwise int32 [groups+1], nondecreasing
 *                    from 0 to rows, each group 1..8 rows (device data: the host
 *                    cannot check it; a group outside 1..8 rows is skipped).
 *   scores           fp32 [rows, scores_row_stride]: scores[r, k] for k below the
 *                    group's length (clamped to max_context) is the dot product
 *                    of query row r with key k; later entries are not written.
 *                    max_context % 64 == 0 and at most 65535 pages (4194240
 *                    keys), scores_row_stride >= max_context; groups <= 65535.
 */
int indexer_scores(const void* query, int32_t rows, int32_t head_dim, const void* key_cache,
                   int64_t page_stride, int32_t num_pages, const int32_t* block_table,
                   int64_t bt_stride, int32_t bt_width, int32_t num_requests,
                   const int32_t* context_lengths, const int32_t* requests, int32_t groups,
                   const int32_t* group_row_offsets, float* scores, int64_t scores_row_stride,
                   int32_t max_context, void* stream);

/*
 * indexer_scores_nvfp4 - one-head indexer scores with NVFP4 query and keys.
 * ("flashinfer.sdsa.indexer_scores": the NVFP4 forms of query and key_cache
 * and the query_scales / key_scales parameters.)
 *
 * A score is the dot product of the dequantised query row and key, where an
 * NVFP4 value is an e2m1 code (two per byte, the even element in the low
 * nibble) times the e4m3 scale of its block of 16 values.
 *
 *   query            packed e2m1 [rows, 64] (head_dim 128), contiguous, 16-B aligned.
 *   query_scales     e4m3 [rows, 8], contiguous, 2-B aligned.
 *   key_cache        packed e2m1 key pages [64, 64]; page i at key_cache +
 *                    i*page_stride bytes, page_stride >= 4096 and a multiple of 16.
 *   key_scales       e4m3 [64, 8] per page, paged like the keys: page i's scales at
 *                    key_scales + i*scale_page_stride bytes, scale_page_stride >= 512
 *                    and a multiple of 8 (the pages allow any multiple of 8).
 *   Everything else (block table, lengths, groups, scores, errors) as in
 *   indexer_scores; head_dim must be 128.
 */
int indexer_scores_nvfp4(const void* query, const void* query_scales, int32_t rows,
                         int32_t head_dim, const void* key_cache, int64_t page_stride,
                         const void* key_scales, int64_t scale_page_stride, int32_t num_pages,
                         const int32_t* block_table, int64_t bt_stride, int32_t bt_width,
                         int32_t num_requests, const int32_t* context_lengths,
                         const int32_t* requests, int32_t groups,
                         const int32_t* group_row_offsets, float* scores,
                         int64_t scores_row_stride, int32_t max_context, void* stream);

/*
 * msa_proxy_score_fp4 - per-KV-block max of the unscaled, causally masked
 * Q K^T logits with NVFP4 query and keys.
 * ("flashinfer.msa_ops.msa_proxy_score_fp4": description, parameter list and
 * "Returns".  The page defers most parameters to a page that is not
 * available; the readings taken are stated below.)
 *
 *   out[h, t, i] = max over the keys k of block t visible to query token i of
 *                  g * sum_d q[i, h, d] * k[k, kvh, d],
 *   g = q_global_scale * k_global_scale (multiplied before the max, as the
 *   page states), kvh = h / (num_qo_heads / num_kv_heads), block t = keys
 *   128t .. 128t+127 of token i's request; -inf where block t holds no
 *   visible key (past the request's keys, fully masked, t at or beyond the
 *   blocks that exist, or token i in no request).  With reduce_heads != 0
 *   out[0, t, i] = max over heads.  A dequantised value is e2m1 times the
 *   e4m3 scale of its 16-value block; products are exact and sums fp32.
 *
 *   q_fp4        packed e2m1 [total_q, num_qo_heads, 64] (head_dim 128, even
 *                element in the low nibble), 16-B aligned.
 *   q_scale      e4m3 [total_q * num_qo_heads, 8], row token*Hq + head,
 *                2-B aligned.  (The page's cuBLAS 128x4 tiled scale layout is
 *                not used: each row's 8 scales are contiguous.)
 *   k_fp4        paged (page_table != NULL): page i at k_fp4 + i*page_stride
 *                holds [num_kv_heads, 128, 64] packed bytes; page_stride >=
 *                num_kv_heads * 8192, a multiple of 16.  Flat (page_table ==
 *                NULL): [total_k, num_kv_heads, 64].  16-B aligned.
 *   k_scale      e4m3 rows of 8: paged row (page*Hkv + kv_head)*128 + token
 *                (num_pages*Hkv*128 rows); flat row token*Hkv + kv_head
 *                (total_k*Hkv rows).  2-B aligned.
 *   cu_seqlens_q [batch+1] int32, nondecreasing, cu_seqlens_q[batch] <=
 *                total_q: request r owns query tokens cu[r] .. cu[r+1]-1.
 *   cu_seqlens_k flat: [batch+1] int32 key offsets (ignored when paged).
 *   page_table   paged: [batch, pt_stride] int32, block t of request r is
 *                page page_table[r*pt_stride + t] (t < pt_width).
 *   seqused_k    paged: [batch] int32 key counts (at most pt_width*128 are
 *                used).
 *   causal       nonzero: key k is visible to the p-th token of its request
 *                iff k <= q_offset[r] + p; zero: every key is visible.
 *   q_offset     NULL (default Lk - Lq per request: the last query token sees
 *                the last key) or [batch] int32.
 *   max_seqlen_q the longest request's token count, or 0 (unknown: total_q);
 *                used to choose the kernel instance, never to clamp.
 *   max_k_tiles  blocks per output row (>= 0).
 *   out          float32 [reduce_heads ? 1 : num_qo_heads, max_k_tiles,
 *                total_q], contiguous, 4-B aligned; every element is written.
 *   Supported: num_qo_heads a multiple of num_kv_heads with at most 64 query
 *   heads per KV head, batch <= 4096, num_kv_heads * total_q * max_k_tiles
 *   < 2^31 (otherwise UNSUPPORTED).  A page id outside [0, num_pages) or a
 *   flat request whose keys lie outside [0, total_k) is never read: its
 *   blocks' outputs are NaN where a key would be visible.
 */
int msa_proxy_score_fp4(const void* q_fp4, const void* q_scale, int32_t total_q,
                        int32_t num_qo_heads, const void* k_fp4, const void* k_scale,
                        int32_t num_kv_heads, int64_t page_stride, int32_t num_pages,
                        int64_t total_k, float q_global_scale, float k_global_scale,
                        const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k,
                        const int32_t* page_table, int64_t pt_stride, int32_t pt_width,
                        const int32_t* seqused_k, int32_t batch, int32_t causal,
                        const int32_t* q_offset, int32_t max_seqlen_q, int32_t max_k_tiles,
                        int32_t reduce_heads, float* out, void* stream);

/*
 * mqa_logits_schedule - the per-call work split, computed on the GPU.
 * ("flashinfer.attn_scores", Scheduling and Setup: a per-call work assignment
 * computed on the device, which a caller may build once and pass back.)
 *
 * Splits the (request, 64-token page) work items of one call, in request-major
 * order, into num_units contiguous ranges and writes the opaque int32 buffer
 * `schedule` of mqa_logits_schedule_ints(num_units) entries.  The ranges are
 * of near-equal length, except that with FP8, next_n >= 4 and the default
 * unit count the units of workgroups dispatched earlier on a compute unit get
 * proportionally more items (the split the kernel makes by itself).
 * num_units in 1 .. 1<<20; 0 means mqa_logits_num_units(current device,
 * next_n, variant).  The result depends only on seq_lens, batch, next_n,
 * variant and max_context; it must be rebuilt whenever seq_lens changes
 * (including on every graph replay).  Any schedule gives the same logits.
 */
int mqa_logits_schedule(const int32_t* seq_lens, int32_t batch, int32_t next_n, int32_t variant,
                        int32_t max_context, int32_t num_units, int32_t* schedule, void* stream);

/* Number of int32 entries of a schedule buffer for num_units units. */
int64_t mqa_logits_schedule_ints(int32_t num_units);

/*
 * mqa_logits_workspace_bytes - bytes of the optional workspace of
 * mqa_logits_fp8 / mqa_logits_mxfp4 (a work counter; the same for every call
 * and device).  See the workspace argument of mqa_logits_fp8.
 */
size_t mqa_logits_workspace_bytes(void);

/* The unit count a NULL-schedule call with 64 heads and head_dim 128 uses on
 * `device` for this next_n and variant: the workgroups of the call's first
 * launch resident on the whole GPU, one contiguous range each; < 0 on error.
 * A schedule built with this count gives each of them one range, like the
 * in-call split (other shapes run another grid, which strides over the
 * units). */
int32_t mqa_logits_num_units(int device, int32_t next_n, int32_t variant);

/* Columns written per row for a request of seq_len tokens: ceil(seq_len/64)*64
 * (0 for seq_len <= 0).  ("flashinfer.attn_scores": padded_seq_len.) */
int32_t mqa_logits_padded_seq_len(int32_t seq_len, int32_t next_n, int32_t variant);

/* Block-table entries a request of max_seq_len tokens needs: ceil(max_seq_len/64).
 * ("flashinfer.attn_scores": min_block_table_width.) */
int32_t mqa_logits_min_block_table_width(int32_t max_seq_len, int32_t next_n, int32_t variant);

/* Loads the code objects on `device` and caches its compute-unit count.  Call
 * it once per device before capturing a call in a HIP graph.  Idempotent. */
int mqa_logits_init(int device);

/* A static, human-readable name for a status code. */
const char* mqa_logits_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* PMQA_H */
