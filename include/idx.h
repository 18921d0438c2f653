/*
 * idx.h - C ABI of libidx, the sparse-attention indexer for MI355X (gfx950).
 *
 * The indexer scores every cached key s for every query row t,
 *
 *     I[t, s] = sum_h w[t, h] * ReLU( dequant(q[t, h, :]) . dequant(k[s, :]) ),
 *
 * writes -inf outside each row's valid range [start_t, end_t), and picks each
 * row's top-k keys. The operation is the one the vLLM API pages state:
 *   - page "vllm.v1.attention.ops.rocm_aiter_mla_sparse", functions
 *     fp8_mqa_logits_torch / rocm_fp8_mqa_logits (contiguous fp8 chunk) and
 *     rocm_fp8_paged_mqa_logits (paged fp8 decode and MTP);
 *   - page "vllm.v1.attention.ops.rocm_paged_mxfp4_indexer", functions
 *     rocm_mxfp4_sparse_attn_indexer (MXFP4 query and K cache) and _topk;
 *   - page "vllm.models.deepseek_v41.amd.rocm", functions
 *     rocm_mxfp4_indexer_k_store and rocm_mxfp4_indexer_q_quant (the K store and
 *     the query quantiser that feed the cache and the query).
 *
 * Conventions shared by every call
 *   - Every pointer argument that names tensor data is DEVICE memory owned by the
 *     caller; descriptors (idx_paged_cache) are host structs. The library
 *     allocates nothing and keeps no state besides a per-device cache of the
 *     device's properties.
 *   - Each call enqueues its kernels on `stream` (NULL = the null stream) and
 *     returns without synchronising the host. No call allocates, copies to the
 *     host or waits, so every call may be captured in a HIP graph; grids depend
 *     only on the arguments, never on device-resident values.
 *   - Arguments the host can see (pointers, sizes, strides, alignments, enums,
 *     workspace sizes) are checked before anything is launched; a failed check
 *     returns an error and launches nothing. Values that live on the device
 *     (lengths, block-table entries, slots) are trusted to be in range; the
 *     kernels clamp every address they form so an out-of-range value yields
 *     unspecified results for the rows it touches, never an out-of-bounds access.
 *   - A call whose work is empty (no rows, no keys) returns IDX_OK and launches
 *     nothing.
 *   - The only device supported is gfx950; IDX_ERR_DEVICE otherwise.
 */
#ifndef IDX_H
#define IDX_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define IDX_ABI_VERSION 1

typedef enum {
  IDX_OK = 0,
  IDX_ERR_NULL = 1,      /* a required pointer is NULL */
  IDX_ERR_SHAPE = 2,     /* a size is negative or outside what the kernels support */
  IDX_ERR_STRIDE = 3,    /* a stride or an alignment requirement is not met */
  IDX_ERR_FORMAT = 4,    /* an enum argument holds an unknown value */
  IDX_ERR_WORKSPACE = 5, /* the workspace is smaller than the matching *_workspace() query */
  IDX_ERR_LAUNCH = 6,    /* a kernel launch failed (hipGetLastError after the launch) */
  IDX_ERR_DEVICE = 7     /* no current HIP device, or it is not a gfx950 */
} idx_status;

/* Format of a paged K cache. */
typedef enum {
  /* e4m3 (OCP float8_e4m3fn) values plus one fp32 scale per key. A page of P keys
   * holds P*D value bytes (key u at u*D) followed by P little-endian fp32 scales
   * (key u at P*D + 4u): page "vllm.v1.attention.ops.rocm_aiter_mla_sparse",
   * rocm_fp8_paged_mqa_logits and rocm_fp8_paged_mqa_logits_triton. */
  IDX_KV_FP8_E4M3 = 0,
  /* MXFP4: D/2 bytes of packed e2m1 (element 2i in the low nibble of byte i) and
   * D/32 e8m0 scales (bias 127) per key. The page is cut into runs of 16 keys; in a
   * run the packed bytes are stored [16-byte chunk, key, byte] and the scale bytes
   * [scale % 4, key, scale / 4]. The value bytes of all runs come first, the scale
   * bytes of all runs follow them: page
   * "vllm.v1.attention.ops.rocm_paged_mxfp4_indexer", RocmPagedMxfp4CacheLayout and
   * rocm_paged_mxfp4_cache_layout. */
  IDX_KV_MXFP4_E2M1 = 1
} idx_kv_format;

/* Element type of full-precision rows handed to the quantisers. */
typedef enum { IDX_IN_F32 = 0, IDX_IN_BF16 = 1 } idx_in_dtype;

/* A paged K cache (host struct; `base` is device memory). Logical page p of
 * sequence b is physical page block_table[b * block_table_stride + p]; key slot
 * `slot` is entry slot % page_size of page slot / page_size. Page n starts at
 * base + n * page_stride_bytes: the stride is the pool's and may exceed the page
 * size (page "vllm.v1.attention.ops.rocm_paged_mxfp4_indexer", _kv_view). */
typedef struct {
  int32_t fmt;               /* idx_kv_format */
  int32_t page_size;         /* keys per page P: a multiple of 16 in [16, 1024] */
  int32_t num_pages;         /* pages in the pool, >= 1 */
  int32_t head_dim;          /* D: must be 128 */
  int64_t page_stride_bytes; /* >= bytes of one page, a multiple of 16 */
  void *base;                /* device address of page 0, 16-byte aligned */
} idx_paged_cache;

/* Bytes one page of `fmt` needs: P*(D+4) for fp8, P*(D/2+D/32) for MXFP4; 0 for an
 * unknown format. */
size_t idx_page_bytes(int32_t fmt, int32_t page_size, int32_t head_dim);

/*
 * idx_mqa_logits - logits of a contiguous fp8 chunk (prefill).
 * Page "vllm.v1.attention.ops.rocm_aiter_mla_sparse", fp8_mqa_logits_torch and
 * rocm_fp8_mqa_logits.
 *
 *   q          [M, H, D] e4m3 bytes; row t starts at q + t*q_row_stride, head h of
 *              it at + h*D. q_row_stride >= H*D and a multiple of 16 bytes.
 *   k          [N, D] e4m3 bytes; key s at k + s*k_row_stride (multiple of 16, >= D).
 *   k_scale    [N] fp32 per-key scales (> 0).
 *   w          [M, H] fp32 head weights, row t at w + t*w_row_stride (elements,
 *              >= H).
 *   row_start  [M] int32, first valid key of row t (inclusive).
 *   row_end    [M] int32, end of row t's valid keys (exclusive).
 *   logits     [M, N] fp32 out, row t at logits + t*logits_row_stride (elements,
 *              >= N, a multiple of 4; logits 16-byte aligned). Every column
 *              0..N-1 of every row is written: I[t, s] on [row_start_t,
 *              min(row_end_t, N)), -inf elsewhere.
 *   Limits: D == 128, 1 <= H <= 128, M, N >= 0.
 */
idx_status idx_mqa_logits(const uint8_t *q, int64_t q_row_stride, const uint8_t *k, int64_t k_row_stride,
                          const float *k_scale, const float *w, int64_t w_row_stride,
                          const int32_t *row_start, const int32_t *row_end, int32_t M, int32_t N, int32_t H,
                          int32_t D, float *logits, int64_t logits_row_stride, hipStream_t stream);

/*
 * idx_paged_mqa_logits - logits of a decode / MTP step over a paged K cache.
 * Page "vllm.v1.attention.ops.rocm_aiter_mla_sparse", rocm_fp8_paged_mqa_logits
 * (fp8); page "vllm.v1.attention.ops.rocm_paged_mxfp4_indexer",
 * rocm_mxfp4_sparse_attn_indexer (MXFP4).
 *
 *   cache         the paged K cache (format, geometry, base).
 *   q             fp8:   [B, next_n, H, D] e4m3 bytes, contiguous.
 *                 MXFP4: [B, next_n, H, D/2] packed e2m1 bytes, contiguous.
 *   q_scale       MXFP4: [B, next_n, H] int32, one per head holding its D/32 = 4
 *                 e8m0 bytes, byte j (little-endian) for elements 32j..32j+31.
 *                 Must be NULL for fp8 (the fp8 query carries no scale).
 *   w             [B*next_n, H] fp32, contiguous; the softmax and head scales are
 *                 already folded in.
 *   context_lens  ctx_per_row == 0: [B] keys each sequence holds; row
 *                 r = b*next_n + j is valid on [0, ctx_b - next_n + j + 1) (row j
 *                 of a next_n-token verify sees its own token and those before it:
 *                 page "vllm.v1.attention.backends.mla.rocm_aiter_mla",
 *                 dcp_local_verify_row_lens).
 *                 ctx_per_row != 0: [B*next_n], row r is valid on
 *                 [0, context_lens[r]).
 *                 Every end is clamped to [0, min(width, max_blocks*page_size)].
 *   block_table   [B, max_blocks] int32, row b at block_table + b*block_table_stride.
 *   logits        [B*next_n, width] fp32 out, row r at logits + r*logits_row_stride
 *                 (elements, >= width, a multiple of 4; 16-byte aligned). Every
 *                 column 0..width-1 is written (-inf past the row's end).
 *   row_end_out   [B*next_n] int32 out, or NULL: each row's clamped end, ready to
 *                 pass to idx_topk.
 *   workspace     device scratch of at least idx_paged_mqa_logits_workspace()
 *                 bytes (NULL when that is 0).
 *   Limits: D == 128, 1 <= H <= 128, 1 <= next_n <= 4, 0 <= B <= 8192,
 *   width >= 0.
 */
idx_status idx_paged_mqa_logits(const idx_paged_cache *cache, const void *q, const int32_t *q_scale,
                                const float *w, const int32_t *context_lens, int32_t ctx_per_row,
                                const int32_t *block_table, int64_t block_table_stride, int32_t max_blocks,
                                int32_t B, int32_t next_n, int32_t H, float *logits, int64_t logits_row_stride,
                                int32_t width, int32_t *row_end_out, void *workspace, size_t workspace_bytes,
                                hipStream_t stream);
size_t idx_paged_mqa_logits_workspace(int32_t B, int32_t next_n, int32_t H, const idx_paged_cache *cache);

/*
 * idx_topk - per-row top-k over [row_start, row_end).
 * Page "vllm.v1.attention.ops.rocm_paged_mxfp4_indexer", _topk.
 *
 *   logits     [rows, width] fp32, row r at logits + r*logits_row_stride (elements).
 *   row_start  [rows] int32 or NULL (all 0); row_end [rows] int32. Both are clamped
 *              to [0, width].
 *   out        [rows, k] int32, row r at out + r*out_row_stride (elements, >= k).
 *              Row r receives the columns of its min(k, end - start) largest
 *              logits, as column - start, in ascending column order, then -1 up to
 *              k entries. Ties at the k-th value go to the lowest column; -0.0 and
 *              +0.0 compare equal. NaN logits are not supported.
 *   workspace  at least idx_topk_workspace(rows, width, k) bytes of device memory,
 *              ZERO-FILLED before its first use; every call leaves it zero-filled
 *              again, so one buffer serves any number of calls. Calls that share a
 *              workspace must not overlap (issue them on one stream). NULL is allowed
 *              when the query returns 0 (more than 256 rows).
 *              With up to 256 rows of more than 65536 columns, 16-byte aligned rows
 *              (logits and a row stride that is a multiple of 4) and rows * width
 *              below 2^30, several workgroups share each row: the page treats few rows
 *              and many rows as different regimes, and one workgroup per long row
 *              would leave most of the device idle while it walks its row. The workgroups of a row meet at counters in the
 *              workspace; all of them are resident at once (the grid is sized from the
 *              device's occupancy), and every wait is bounded: should another kernel
 *              keep them from being resident for about a second, the call still
 *              returns but its output is unspecified. Otherwise one workgroup per row.
 *              The workspace is laid out as 2048 records of 16 bytes (one per
 *              workgroup) followed by one 36928-byte record per row.
 *   Limits: 1 <= k <= 65536, rows >= 0, width >= 0.
 */
idx_status idx_topk(const float *logits, int64_t logits_row_stride, int32_t rows, int32_t width,
                    const int32_t *row_start, const int32_t *row_end, int32_t k, int32_t *out,
                    int64_t out_row_stride, void *workspace, size_t workspace_bytes, hipStream_t stream);
/* Bytes of workspace idx_topk needs: 2048 * 16 + rows * 36928 for 1 <= rows <= 256,
 * else 0. */
size_t idx_topk_workspace(int32_t rows, int32_t width, int32_t k);

/*
 * idx_topk_noalloc - idx_topk for callers that cannot allocate device memory: code
 * under HIP graph capture, tight serving loops, harnesses that forbid hipMalloc. Same
 * arguments and output as idx_topk, without the workspace.
 *   The several-workgroups-per-row path keeps its records in an array the library
 *   owns instead: 2048 * 16 + 256 * 36928 bytes (about 9 MiB) of device memory per
 *   GPU, enough for the 256 rows that path takes at most, held until the process
 *   ends. The array is zero when the library loads and every call leaves it zero.
 *   All calls on one GPU share it: calls that overlap on one GPU (several streams,
 *   several host threads) race, and their outputs are unspecified.
 *   The call allocates nothing and calls no allocating routine. Errors as idx_topk;
 *   IDX_ERR_DEVICE also when the array's address cannot be looked up.
 */
idx_status idx_topk_noalloc(const float *logits, int64_t logits_row_stride, int32_t rows, int32_t width,
                            const int32_t *row_start, const int32_t *row_end, int32_t k, int32_t *out,
                            int64_t out_row_stride, hipStream_t stream);

/*
 * idx_k_store - quantise key rows and write them into their cache slots.
 * Page "vllm.models.deepseek_v41.amd.rocm", rocm_mxfp4_indexer_k_store (the
 * quantise-and-write part; the RMSNorm and RoPE before it are not applied here).
 *
 *   k             [N, D] fp32 or bf16 (k_dtype), row i at k + i*k_row_stride
 *                 (elements, >= D).
 *   slot_mapping  [N] int64: key i goes to slot slot_mapping[i]; a negative slot
 *                 skips the key (padding).
 *   fp8:   scale = amax / 448 in fp32 (1.0 when the row is all zero); each value
 *          becomes e4m3(k / scale) with an IEEE fp32 division, rounded to nearest
 *          even and saturated at +-448.
 *   MXFP4: per 32-value block, the e8m0 byte b is the smallest in [0, 254] with
 *          amax <= 6 * 2^(b - 127); each value becomes e2m1(k * 2^(127 - b)),
 *          rounded to nearest even (the e8m0 rule of _mxfp8_scale_bits on page
 *          "vllm.v1.attention.ops.rocm_aiter_mla_sparse" with 6, the e2m1 maximum,
 *          in place of 448).
 *   Limits: D == 128, N >= 0.
 */
idx_status idx_k_store(const idx_paged_cache *cache, const void *k, int32_t k_dtype, int64_t k_row_stride,
                       const int64_t *slot_mapping, int32_t N, hipStream_t stream);

/*
 * idx_q_quant - quantise query rows into the format the logits calls read.
 * Page "vllm.models.deepseek_v41.amd.rocm", rocm_mxfp4_indexer_q_quant (the
 * quantisation part: packed [T, H, D/2] plus one int32 of e8m0 bytes per head;
 * RoPE and the weight scaling are not applied here).
 *
 *   q        [T, H, D] fp32 or bf16 (q_dtype), row t at q + t*q_row_stride
 *            (elements, >= H*D), head h at + h*D.
 *   fmt      IDX_KV_FP8_E4M3: q_out is [T, H, D] e4m3 (no scale: each value rounded
 *            to nearest even, saturated at +-448); q_scale_out must be NULL.
 *            IDX_KV_MXFP4_E2M1: q_out is [T, H, D/2] packed e2m1 and q_scale_out is
 *            [T, H] int32 with the same block rule as idx_k_store.
 *   Limits: D == 128, T, H >= 0.
 */
idx_status idx_q_quant(const void *q, int32_t q_dtype, int64_t q_row_stride, int32_t T, int32_t H, int32_t D,
                       int32_t fmt, void *q_out, int32_t *q_scale_out, hipStream_t stream);

/*
 * idx_k_norm_rope_store - the key side of a step in one pass: RMSNorm, RoPE, then
 * the K store. Page "vllm.models.deepseek_v41.amd.rocm", rocm_mxfp4_indexer_k_store
 * (the pre-norm key, its position, the rotary cos/sin table, the norm weight and
 * epsilon, the cache and the slot mapping go to one cache op).
 *
 *   k, k_dtype, k_row_stride, slot_mapping, N   as idx_k_store (pre-norm keys).
 *   norm_weight   [D] fp32, 16-byte aligned; eps > 0.
 *   positions     [N] int64: the rotary position of key i, clamped to
 *                 [0, max_position - 1] (a compressed cache passes the position
 *                 of the stored key).
 *   cos_sin       [max_position, rope_dim] fp32: row p holds cos of the rope_dim/2
 *                 pair angles at position p, then their sin.
 *   rope_dim      even, 0..D (0: no rotation; positions and cos_sin may be NULL).
 *   Each key becomes y = x / sqrt(mean(x^2) + eps) * norm_weight (fp32, correctly
 *   rounded square root and division); the trailing rope_dim channels of y are
 *   rotated in pairs (D - rope_dim + 2i, D - rope_dim + 2i + 1) by
 *   (a, b) -> (a cos_i - b sin_i, b cos_i + a sin_i), the GPT-J form whose inverse
 *   page "vllm.v1.attention.ops.rocm_aiter_mla_sparse" gives (_inverse_rope_gptj_kernel);
 *   the result is quantised and written exactly as idx_k_store does.
 *   Limits: D == 128, N >= 0.
 */
idx_status idx_k_norm_rope_store(const idx_paged_cache *cache, const void *k, int32_t k_dtype, int64_t k_row_stride,
                                 const int64_t *positions, const float *cos_sin, int32_t max_position,
                                 int32_t rope_dim, const float *norm_weight, float eps,
                                 const int64_t *slot_mapping, int32_t N, hipStream_t stream);

/*
 * idx_q_rope_quant - the query side of a step in one pass: RoPE, quantisation and
 * the weights scaled for scoring. Page "vllm.models.deepseek_v41.amd.rocm",
 * rocm_mxfp4_indexer_q_quant (queries, positions, the rotary table and the indexer
 * weights in; quantised queries and weights times softmax_scale * n_head^-0.5 out).
 *
 *   q, q_dtype, q_row_stride, T, H, D, fmt, q_out, q_scale_out   as idx_q_quant,
 *                 the quantisation applying to the rotated query.
 *   positions     [T] int64: token t's rotary position (all heads), clamped as in
 *                 idx_k_norm_rope_store; cos_sin, max_position, rope_dim likewise.
 *   weights       [T, H] fp32, row t at weights + t*weights_row_stride (>= H).
 *   weight_scale  multiplies every weight (softmax_scale * n_head^-0.5 on the page).
 *   weights_out   [T, H] fp32 dense: weights * weight_scale, one fp32 rounding.
 *   Limits: D == 128, T, H >= 0; q_out 8-byte (fp8) or 4-byte (MXFP4) aligned.
 */
idx_status idx_q_rope_quant(const void *q, int32_t q_dtype, int64_t q_row_stride, const int64_t *positions,
                            const float *cos_sin, int32_t max_position, int32_t rope_dim, const float *weights,
                            int64_t weights_row_stride, float weight_scale, int32_t T, int32_t H, int32_t D,
                            int32_t fmt, void *q_out, int32_t *q_scale_out, float *weights_out,
                            hipStream_t stream);

/*
 * idx_topk_to_slots - top-k rows of local key positions to a ragged stream of
 * physical cache slots, the form the sparse-attention step consumes. Page
 * "vllm.v1.attention.ops.rocm_aiter_mla_sparse", build_prefill_topk_ragged_indices
 * (positions local to each sequence mapped through its block table and packed row
 * after row); page "vllm.models.deepseek_v41.amd.rocm", _decode_topk_ragged (the same
 * for decode rows, with each row's request and validity flag).
 *
 *   topk          [rows, k] int32 (idx_topk's output), row r at topk + r*topk_row_stride.
 *                 Entries < 0 (pads) and positions >= max_blocks*page_size are dropped.
 *   row_seq       [rows] int32 or NULL: the sequence of row r (NULL: r / next_n);
 *                 clamped to [0, B - 1].
 *   row_valid     [rows] uint8 or NULL: a row whose flag is 0 contributes nothing.
 *   block_table   [B, max_blocks] int32 with block_table_stride (>= max_blocks);
 *                 position p of sequence b is slot
 *                 block_table[b][p / page_size] * page_size + p % page_size.
 *   slots_out     ragged slots (capacity rows*k int32); row r's slots, in the order
 *                 of its entries, at slots_out[indptr_out[r] .. indptr_out[r+1]).
 *   indptr_out    [rows + 1] int32 (indptr_out[0] = 0); lens_out [rows] int32 or NULL.
 *   Limits: rows, k >= 0; B, max_blocks, page_size >= 1.
 */
idx_status idx_topk_to_slots(const int32_t *topk, int64_t topk_row_stride, int32_t rows, int32_t k,
                             const int32_t *row_seq, int32_t next_n, int32_t B, const uint8_t *row_valid,
                             const int32_t *block_table, int64_t block_table_stride, int32_t max_blocks,
                             int32_t page_size, int32_t *slots_out, int32_t *indptr_out, int32_t *lens_out,
                             hipStream_t stream);

/*
 * idx_paged_prefill_logits - a prefill chunk straight off the paged cache: M query rows
 * of one sequence, row r scoring keys [0, row_end[r]) of that sequence through its
 * block-table row, with no gather of K. Page "vllm.v1.attention.ops.rocm_paged_mxfp4_indexer",
 * module description (the kernel reads the paged K cache in place, prefill included)
 * and rocm_mxfp4_sparse_attn_indexer (prefill chunks walk the same cache as decode).
 * Every row's logit of key s is the one idx_paged_mqa_logits defines; up to 64 heads
 * (MXFP4) or 128 (fp8) the rows are scored eight at a time with each key chunk shared
 * through LDS and the ReLU split as (x + |x|) / 2, so values agree with the decode
 * walk up to float32 rounding (bit for bit for MXFP4 with more than 64 heads, which
 * walks rows in pairs).
 *
 *   cache         the paged K cache (fp8 or MXFP4), as idx_paged_mqa_logits.
 *   q             [M, H, D] e4m3 (fp8) or [M, H, D/2] packed e2m1 (MXFP4), 16-byte aligned.
 *   q_scale       MXFP4: [M, H] int32 (4 e8m0 bytes, as idx_q_quant); fp8: NULL.
 *   w             [M, H] fp32.
 *   row_end       [M] int32: row r's causal end (e.g. position + 1, or the compressed
 *                 count), clamped to [0, min(width, max_blocks * page_size)].
 *   block_table   [max_blocks] int32: the sequence's pages.
 *   logits        [M, width] fp32 with logits_row_stride (multiple of 4, 16-byte
 *                 aligned); -inf at and past each row's end.
 *   Limits: 0 <= M <= 16384; M * ceil(width / 64) < 2^31; 1 <= H <= 128.
 */
idx_status idx_paged_prefill_logits(const idx_paged_cache *cache, const void *q, const int32_t *q_scale,
                                    const float *w, const int32_t *row_end, const int32_t *block_table,
                                    int32_t max_blocks, int32_t M, int32_t H, float *logits,
                                    int64_t logits_row_stride, int32_t width, hipStream_t stream);

/*
 * Two-level indexer. Page "vllm.v1.attention.ops.rocm_paged_mxfp4_indexer": a candidate
 * source layer takes block maxima from the same walk that writes its logits
 * (rocm_mxfp4_sparse_attn_indexer with candidate_write; block scores sized
 * [rows, ceil(width / block)] fp32 by reserve_rocm_mxfp4_indexer_workspace); the
 * candidate pool is resolved from them once per step; consumer layers either run the
 * dense walk masked to the pool or score only the pool (rocm_mxfp4_sparse_mqa_indexer),
 * and a top-k over a pool is turned back into positions (_remap_compact_topk). Page
 * "vllm.v1.attention.ops.rocm_aiter_mla_sparse", _apply_candidate_mask_strided: the
 * mask over [0, end) with row_repeat query rows per candidate row. The pages show the
 * interfaces, not how the pool is chosen; here it is each row's n_cand best blocks.
 *
 * A candidate list is int32 [rows / row_repeat, n_cand] (row c at cand + c*cand_row_stride,
 * 4-byte aligned): block indices, block b covering positions [b*block_size,
 * (b+1)*block_size). Query row r uses candidate row r / row_repeat.
 */

/*
 * idx_paged_mqa_logits_block_max - idx_paged_mqa_logits that also writes each row's
 * block maxima from the same walk (the candidate source).
 *
 *   All arguments up to row_end_out and the workspace are as idx_paged_mqa_logits.
 *   block_max     [B*next_n, ceil(width / block_size)] fp32, row r at
 *                 block_max + r*block_max_row_stride (>= ceil(width / block_size)):
 *                 entry j is the largest logit of columns [j*block_size,
 *                 (j+1)*block_size) below the row's end, -inf when there is none.
 *   block_size    16, 32 or 64 (0: no block maxima, block_max ignored).
 */
idx_status idx_paged_mqa_logits_block_max(const idx_paged_cache *cache, const void *q, const int32_t *q_scale,
                                          const float *w, const int32_t *context_lens, int32_t ctx_per_row,
                                          const int32_t *block_table, int64_t block_table_stride,
                                          int32_t max_blocks, int32_t B, int32_t next_n, int32_t H, float *logits,
                                          int64_t logits_row_stride, int32_t width, int32_t *row_end_out,
                                          float *block_max, int64_t block_max_row_stride, int32_t block_size,
                                          void *workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * idx_candidate_blocks - the candidate pool: per row, the n_cand blocks with the
 * largest block maxima, ties to the lower block, listed in ascending block order and
 * padded with -1. It is idx_topk over the block maxima with each row's end rounded up
 * to blocks.
 *
 *   block_max     [rows, num_blocks] fp32 with block_max_row_stride (>= num_blocks).
 *   row_end       [rows] int32: the rows' logits ends (columns, e.g. the row_end_out of
 *                 the source call); row r considers blocks [0, ceil(row_end[r] / block_size)).
 *   block_size    a power of two.
 *   cand_out      [rows, n_cand] int32 with cand_row_stride (>= n_cand). A row whose end
 *                 covers b blocks gets min(n_cand, b) entries, then -1.
 *   workspace     as idx_topk (idx_topk_workspace(rows, num_blocks, n_cand) bytes).
 */
idx_status idx_candidate_blocks(const float *block_max, int64_t block_max_row_stride, int32_t rows,
                                int32_t num_blocks, const int32_t *row_end, int32_t block_size, int32_t n_cand,
                                int32_t *cand_out, int64_t cand_row_stride, void *workspace,
                                size_t workspace_bytes, hipStream_t stream);

/*
 * idx_apply_candidate_mask - a dense logits row restricted to its pool, in place:
 * every column c < row_end[r] whose block c / block_size is not in the row's candidate
 * list becomes -inf (columns at or past the end are left alone).
 *
 *   logits        [rows, width] fp32, 16-byte aligned, logits_row_stride a multiple of 4.
 *   row_end       [rows] int32, clamped to [0, width].
 *   cand ...      a candidate list (see above); entries < 0 or past the end are ignored.
 *   block_size    a power of two with ceil(width / block_size) < 65536.
 */
idx_status idx_apply_candidate_mask(float *logits, int64_t logits_row_stride, int32_t rows, int32_t width,
                                    const int32_t *row_end, const int32_t *cand, int64_t cand_row_stride,
                                    int32_t n_cand, int32_t block_size, int32_t row_repeat, hipStream_t stream);

/*
 * idx_paged_mqa_logits_gather - the candidate consumer that scores only its pool: pool
 * slot j of row r holds the logit of position p = cand[j / block_size]*block_size +
 * j % block_size of row r's sequence (computed exactly as idx_paged_mqa_logits computes
 * that position's logit), or -inf when the entry is < 0 or p is at or past the row's
 * end. Any list works; the walk covers each row's slots up to the last one that names a
 * position, which for a list as idx_candidate_blocks writes it (ascending, then -1) is
 * nearly the whole list for long rows and little of it for short ones.
 *
 *   cache ... H   as idx_paged_mqa_logits (rows r = b*next_n + j, same row ends).
 *   cand ...      a candidate list (see above); block_size a power of two, >= 16.
 *   pool_logits   [B*next_n, n_cand*block_size] fp32, 16-byte aligned,
 *                 pool_row_stride a multiple of 4; every slot is written.
 *   pool_end_out  [B*next_n] int32, required: one past the row's last slot that names a
 *                 position (the row end for idx_topk over the pool). A first small
 *                 kernel writes it and the walk reads it back.
 *   Limits: B*next_n <= 8192.
 */
idx_status idx_paged_mqa_logits_gather(const idx_paged_cache *cache, const void *q, const int32_t *q_scale,
                                       const float *w, const int32_t *context_lens, int32_t ctx_per_row,
                                       const int32_t *block_table, int64_t block_table_stride, int32_t max_blocks,
                                       int32_t B, int32_t next_n, int32_t H, const int32_t *cand,
                                       int64_t cand_row_stride, int32_t n_cand, int32_t block_size,
                                       int32_t row_repeat, float *pool_logits, int64_t pool_row_stride,
                                       int32_t *pool_end_out, hipStream_t stream);

/*
 * idx_remap_compact_topk - a top-k over pool slots to positions, in place: an entry
 * j >= 0 becomes cand[j / block_size]*block_size + j % block_size of its row's
 * candidate row; -1 stays -1, and so does an entry whose candidate is -1 or lies past
 * the list.
 *
 *   topk          [rows, k] int32 with topk_row_stride (>= k).
 *   cand ...      the candidate list the pool was gathered with; block_size a power of two.
 */
idx_status idx_remap_compact_topk(int32_t *topk, int64_t topk_row_stride, int32_t rows, int32_t k,
                                  const int32_t *cand, int64_t cand_row_stride, int32_t n_cand, int32_t block_size,
                                  int32_t row_repeat, hipStream_t stream);

/*
 * Debug build. The library can be built a second time with -DIDX_DEBUG (the build
 * script links it as libidx_debug.so next to libidx.so). Its kernels compute exactly
 * what the release kernels compute and also record, in a device word, every
 * device-resident value that had to be clamped or dropped, one bit per kind:
 */
#define IDX_DBG_LENGTH 1u   /* a sequence length or row bound outside its range: a
                               context length < 0, or a row end past
                               min(width, max_blocks*page_size) (the table's reach
                               alone for the gathered walk); a row_start < 0, a
                               row_end < 0, or a row_end past the row's columns
                               (idx_mqa_logits, idx_topk, idx_candidate_blocks,
                               idx_apply_candidate_mask); for idx_topk also a
                               row_start past the width */
#define IDX_DBG_PAGE 2u     /* a block-table entry outside [0, num_pages) read for a
                               key below its row's end */
#define IDX_DBG_SLOT 4u     /* a slot >= 0 whose page is outside the pool (the key is
                               dropped as padding would be) */
#define IDX_DBG_POSITION 8u /* a rotary position outside [0, max_position) */
#define IDX_DBG_SEQ 16u     /* a row_seq entry outside [0, B) (idx_topk_to_slots) */
/*
 * idx_debug_flags - waits for the current device to finish its work (like
 * hipDeviceSynchronize), then stores the OR of the recorded bits in *flags and, when
 * clear != 0, resets them. The bits persist across calls until cleared. The release
 * library records nothing: *flags is always 0. Not for use under graph capture.
 * IDX_ERR_NULL for a NULL flags; IDX_ERR_LAUNCH when a HIP call fails.
 * idx_debug_build - 1 for the debug build, 0 for the release build.
 */
idx_status idx_debug_flags(uint32_t *flags, int32_t clear);
int32_t idx_debug_build(void);

/* Static text naming a status; never NULL. */
const char *idx_status_str(idx_status s);
/* IDX_ABI_VERSION of the built library. */
int32_t idx_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* IDX_H */
