// Host-side argument checks of the indexer ABI (no HIP calls; see validate.h).
#include "validate.h"

#include <climits>

namespace idx {
namespace {

bool aligned(const void *p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

}  // namespace

size_t page_bytes(int32_t fmt, int32_t page_size, int32_t head_dim) {
  if (page_size <= 0 || head_dim <= 0) return 0;
  if (fmt == IDX_KV_FP8_E4M3) return size_t(page_size) * size_t(head_dim + 4);
  if (fmt == IDX_KV_MXFP4_E2M1) return size_t(page_size) * size_t(head_dim / 2 + head_dim / 32);
  return 0;
}

idx_status check_cache(const idx_paged_cache *cache) {
  if (!cache) return IDX_ERR_NULL;
  if (cache->fmt != IDX_KV_FP8_E4M3 && cache->fmt != IDX_KV_MXFP4_E2M1) return IDX_ERR_FORMAT;
  if (cache->head_dim != kHeadDim) return IDX_ERR_SHAPE;
  if (cache->page_size < 16 || cache->page_size > 1024 || cache->page_size % 16) return IDX_ERR_SHAPE;
  if (cache->num_pages < 1) return IDX_ERR_SHAPE;
  if (!cache->base) return IDX_ERR_NULL;
  const size_t pb = page_bytes(cache->fmt, cache->page_size, cache->head_dim);
  if (cache->page_stride_bytes < int64_t(pb) || cache->page_stride_bytes % 16) return IDX_ERR_STRIDE;
  if (!aligned(cache->base, 16)) return IDX_ERR_STRIDE;
  return IDX_OK;
}

idx_status check_mqa_logits(const void *q, int64_t q_row_stride, const void *k, int64_t k_row_stride,
                            const void *k_scale, const void *w, int64_t w_row_stride, const void *row_start,
                            const void *row_end, int32_t M, int32_t N, int32_t H, int32_t D, const void *logits,
                            int64_t logits_row_stride, bool *empty) {
  *empty = false;
  if (M < 0 || N < 0) return IDX_ERR_SHAPE;
  if (D != kHeadDim || H < 1 || H > kMaxHeads) return IDX_ERR_SHAPE;
  if (M == 0 || N == 0) {
    *empty = true;
    return IDX_OK;
  }
  if (!q || !k || !k_scale || !w || !row_start || !row_end || !logits) return IDX_ERR_NULL;
  if (q_row_stride < int64_t(H) * D || q_row_stride % 16 || !aligned(q, 16)) return IDX_ERR_STRIDE;
  if (k_row_stride < D || k_row_stride % 16 || !aligned(k, 16)) return IDX_ERR_STRIDE;
  if (w_row_stride < H || !aligned(w, 4) || !aligned(k_scale, 4)) return IDX_ERR_STRIDE;
  if (!aligned(row_start, 4) || !aligned(row_end, 4)) return IDX_ERR_STRIDE;
  if (logits_row_stride < N || logits_row_stride % 4 || !aligned(logits, 16)) return IDX_ERR_STRIDE;
  return IDX_OK;
}

size_t paged_workspace_bytes(int32_t, int32_t, int32_t, const idx_paged_cache *) { return 0; }

idx_status check_paged_mqa_logits(const idx_paged_cache *cache, const void *q, const void *q_scale, const void *w,
                                  const void *context_lens, const void *block_table, int64_t block_table_stride,
                                  int32_t max_blocks, int32_t B, int32_t next_n, int32_t H, const void *logits,
                                  int64_t logits_row_stride, int32_t width, const void *workspace,
                                  size_t workspace_bytes, bool *empty) {
  *empty = false;
  idx_status s = check_cache(cache);
  if (s != IDX_OK) return s;
  if (B < 0 || B > kMaxBatch || next_n < 1 || next_n > kMaxNextN || H < 1 || H > kMaxHeads) return IDX_ERR_SHAPE;
  if (width < 0 || max_blocks < 0) return IDX_ERR_SHAPE;
  // chunk offsets of 64 keys are kept in int32
  if (int64_t(B) * ((int64_t(width) + 63) / 64) > INT32_MAX) return IDX_ERR_SHAPE;
  if (B == 0) {
    *empty = true;
    return IDX_OK;
  }
  if (!q || !w || !context_lens) return IDX_ERR_NULL;
  if (max_blocks > 0 && !block_table) return IDX_ERR_NULL;
  if (width > 0 && !logits) return IDX_ERR_NULL;
  if (cache->fmt == IDX_KV_MXFP4_E2M1 && !q_scale) return IDX_ERR_NULL;
  if (cache->fmt == IDX_KV_FP8_E4M3 && q_scale) return IDX_ERR_FORMAT;
  if (!aligned(q, 16) || !aligned(w, 4) || !aligned(context_lens, 4)) return IDX_ERR_STRIDE;
  if (q_scale && !aligned(q_scale, 4)) return IDX_ERR_STRIDE;
  if (max_blocks > 0 && (block_table_stride < max_blocks || !aligned(block_table, 4))) return IDX_ERR_STRIDE;
  if (width > 0 && (logits_row_stride < width || logits_row_stride % 4 || !aligned(logits, 16)))
    return IDX_ERR_STRIDE;
  const size_t need = paged_workspace_bytes(B, next_n, H, cache);
  if (workspace_bytes < need) return IDX_ERR_WORKSPACE;
  if (need > 0 && !workspace) return IDX_ERR_NULL;
  return IDX_OK;
}

size_t topk_workspace_bytes(int32_t rows, int32_t, int32_t) { return topk_scratch_bytes(rows); }

idx_status check_topk_args(const void *logits, int64_t logits_row_stride, int32_t rows, int32_t width,
                           const void *row_end, int32_t k, const void *out, int64_t out_row_stride, bool *empty) {
  *empty = false;
  if (rows < 0 || width < 0 || k < 1 || k > kMaxTopK) return IDX_ERR_SHAPE;
  if (rows == 0) {
    *empty = true;
    return IDX_OK;
  }
  if (!row_end || !out) return IDX_ERR_NULL;
  if (width > 0 && !logits) return IDX_ERR_NULL;
  if (width > 0 && (logits_row_stride < width || !aligned(logits, 4))) return IDX_ERR_STRIDE;
  if (out_row_stride < k || !aligned(out, 4) || !aligned(row_end, 4)) return IDX_ERR_STRIDE;
  return IDX_OK;
}

idx_status check_topk(const void *logits, int64_t logits_row_stride, int32_t rows, int32_t width,
                      const void *row_end, int32_t k, const void *out, int64_t out_row_stride,
                      const void *workspace, size_t workspace_bytes, bool *empty) {
  const idx_status s = check_topk_args(logits, logits_row_stride, rows, width, row_end, k, out, out_row_stride, empty);
  if (s != IDX_OK || *empty) return s;
  const size_t need = topk_workspace_bytes(rows, width, k);
  if (workspace_bytes < need) return IDX_ERR_WORKSPACE;
  if (need > 0 && !workspace) return IDX_ERR_NULL;
  return IDX_OK;
}

idx_status check_k_store(const idx_paged_cache *cache, const void *k, int32_t k_dtype, int64_t k_row_stride,
                         const void *slot_mapping, int32_t N, bool *empty) {
  *empty = false;
  idx_status s = check_cache(cache);
  if (s != IDX_OK) return s;
  if (k_dtype != IDX_IN_F32 && k_dtype != IDX_IN_BF16) return IDX_ERR_FORMAT;
  if (N < 0) return IDX_ERR_SHAPE;
  if (N == 0) {
    *empty = true;
    return IDX_OK;
  }
  if (!k || !slot_mapping) return IDX_ERR_NULL;
  if (k_row_stride < cache->head_dim) return IDX_ERR_STRIDE;
  if (!aligned(k, k_dtype == IDX_IN_F32 ? 4 : 2) || !aligned(slot_mapping, 8)) return IDX_ERR_STRIDE;
  return IDX_OK;
}

idx_status check_q_quant(const void *q, int32_t q_dtype, int64_t q_row_stride, int32_t T, int32_t H, int32_t D,
                         int32_t fmt, const void *q_out, const void *q_scale_out, bool *empty) {
  *empty = false;
  if (fmt != IDX_KV_FP8_E4M3 && fmt != IDX_KV_MXFP4_E2M1) return IDX_ERR_FORMAT;
  if (q_dtype != IDX_IN_F32 && q_dtype != IDX_IN_BF16) return IDX_ERR_FORMAT;
  if (T < 0 || H < 0 || D != kHeadDim) return IDX_ERR_SHAPE;
  if (T == 0 || H == 0) {
    *empty = true;
    return IDX_OK;
  }
  if (!q || !q_out) return IDX_ERR_NULL;
  if (fmt == IDX_KV_MXFP4_E2M1 && !q_scale_out) return IDX_ERR_NULL;
  if (fmt == IDX_KV_FP8_E4M3 && q_scale_out) return IDX_ERR_FORMAT;
  if (q_row_stride < int64_t(H) * D) return IDX_ERR_STRIDE;
  if (!aligned(q, q_dtype == IDX_IN_F32 ? 4 : 2)) return IDX_ERR_STRIDE;
  if (q_scale_out && !aligned(q_scale_out, 4)) return IDX_ERR_STRIDE;
  return IDX_OK;
}

idx_status check_norm_rope(const void *positions, const void *cos_sin, int32_t max_position, int32_t rope_dim,
                           const void *norm_weight, float eps) {
  if (rope_dim < 0 || rope_dim > kHeadDim || rope_dim % 2) return IDX_ERR_SHAPE;
  if (rope_dim > 0) {
    if (!positions || !cos_sin) return IDX_ERR_NULL;
    if (max_position < 1) return IDX_ERR_SHAPE;
    if (!aligned(positions, 8) || !aligned(cos_sin, 4)) return IDX_ERR_STRIDE;
  }
  if (norm_weight) {
    if (!(eps > 0.f) || eps != eps) return IDX_ERR_SHAPE;
    if (!aligned(norm_weight, 16)) return IDX_ERR_STRIDE;
  }
  return IDX_OK;
}

idx_status check_q_rope_quant(const void *q, int32_t q_dtype, int64_t q_row_stride, const void *positions,
                              const void *cos_sin, int32_t max_position, int32_t rope_dim, const void *weights,
                              int64_t weights_row_stride, int32_t T, int32_t H, int32_t D, int32_t fmt,
                              const void *q_out, const void *q_scale_out, const void *weights_out, bool *empty) {
  idx_status s = check_q_quant(q, q_dtype, q_row_stride, T, H, D, fmt, q_out, q_scale_out, empty);
  if (s != IDX_OK || *empty) return s;
  if ((s = check_norm_rope(positions, cos_sin, max_position, rope_dim, nullptr, 0.f)) != IDX_OK) return s;
  if (!weights || !weights_out) return IDX_ERR_NULL;
  if (weights_row_stride < H || !aligned(weights, 4) || !aligned(weights_out, 4)) return IDX_ERR_STRIDE;
  if (!aligned(q_out, fmt == IDX_KV_FP8_E4M3 ? 8 : 4)) return IDX_ERR_STRIDE;
  return IDX_OK;
}

idx_status check_topk_to_slots(const void *topk, int64_t topk_row_stride, int32_t rows, int32_t k,
                               const void *row_seq, int32_t next_n, int32_t B, const void *block_table,
                               int64_t block_table_stride, int32_t max_blocks, int32_t page_size,
                               const void *slots_out, const void *indptr_out, bool *empty) {
  *empty = false;
  if (rows < 0 || k < 0 || B < 1 || max_blocks < 1 || page_size < 1) return IDX_ERR_SHAPE;
  if (!row_seq && next_n < 1) return IDX_ERR_SHAPE;
  if (!indptr_out) return IDX_ERR_NULL;
  if (int64_t(max_blocks) * page_size > INT32_MAX) return IDX_ERR_SHAPE;
  if (rows == 0) {
    *empty = true;  // indptr is the single 0, written by the launch of the scan
    return IDX_OK;
  }
  if (!topk || !block_table || (k > 0 && !slots_out)) return IDX_ERR_NULL;
  if (topk_row_stride < k || block_table_stride < max_blocks) return IDX_ERR_STRIDE;
  if (!aligned(topk, 4) || !aligned(block_table, 4) || !aligned(indptr_out, 4)) return IDX_ERR_STRIDE;
  if (row_seq && !aligned(row_seq, 4)) return IDX_ERR_STRIDE;
  if (slots_out && !aligned(slots_out, 4)) return IDX_ERR_STRIDE;
  return IDX_OK;
}

namespace {
bool pow2(int64_t x) { return x > 0 && (x & (x - 1)) == 0; }
}  // namespace

idx_status check_block_max(const void *block_max, int64_t block_max_row_stride, int32_t block_size, int32_t width) {
  if (block_size != 16 && block_size != 32 && block_size != 64) return IDX_ERR_SHAPE;
  if (!block_max) return IDX_ERR_NULL;
  if (block_max_row_stride < (int64_t(width) + block_size - 1) / block_size || !aligned(block_max, 4))
    return IDX_ERR_STRIDE;
  return IDX_OK;
}

idx_status check_candidate_list(const void *cand, int64_t cand_row_stride, int32_t n_cand, int32_t block_size,
                                int32_t row_repeat) {
  if (n_cand < 1 || !pow2(block_size) || row_repeat < 1) return IDX_ERR_SHAPE;
  if (int64_t(n_cand) * block_size > INT32_MAX) return IDX_ERR_SHAPE;
  if (!cand) return IDX_ERR_NULL;
  if (cand_row_stride < n_cand || !aligned(cand, 4)) return IDX_ERR_STRIDE;
  return IDX_OK;
}

idx_status check_gather(int32_t B, int32_t next_n, int32_t block_size, const void *pool_logits,
                        int64_t pool_row_stride, int32_t n_cand, const void *pool_end_out) {
  // the per-row walk keeps three ints per row in LDS; chunk offsets stay in int32
  if (B < 0 || next_n < 1 || int64_t(B) * next_n > kMaxBatch) return IDX_ERR_SHAPE;
  if (int64_t(B) * next_n * ((int64_t(n_cand) * block_size + 63) / 64) > INT32_MAX) return IDX_ERR_SHAPE;
  // a 16-key group of the walk lies inside one pool block and one page
  if (block_size < 16 || block_size > (1 << 20)) return IDX_ERR_SHAPE;
  if (B > 0 && (!pool_logits || !pool_end_out)) return IDX_ERR_NULL;
  if (B > 0 && !aligned(pool_end_out, 4)) return IDX_ERR_STRIDE;
  const int64_t width = int64_t(n_cand) * block_size;
  if (B > 0 && (pool_row_stride < width || pool_row_stride % 4 || !aligned(pool_logits, 16))) return IDX_ERR_STRIDE;
  return IDX_OK;
}

idx_status check_candidate_mask(const void *logits, int64_t logits_row_stride, int32_t rows, int32_t width,
                                const void *row_end, int32_t block_size, bool *empty) {
  *empty = false;
  if (rows < 0 || width < 0 || !pow2(block_size)) return IDX_ERR_SHAPE;
  // one LDS byte per block of the row
  if ((int64_t(width) + block_size - 1) / block_size >= 65536) return IDX_ERR_SHAPE;
  if (rows == 0 || width == 0) {
    *empty = true;
    return IDX_OK;
  }
  if (!logits || !row_end) return IDX_ERR_NULL;
  if (logits_row_stride < width || logits_row_stride % 4 || !aligned(logits, 16) || !aligned(row_end, 4))
    return IDX_ERR_STRIDE;
  return IDX_OK;
}

idx_status check_remap(const void *topk, int64_t topk_row_stride, int32_t rows, int32_t k, bool *empty) {
  *empty = false;
  if (rows < 0 || k < 0) return IDX_ERR_SHAPE;
  if (rows == 0 || k == 0) {
    *empty = true;
    return IDX_OK;
  }
  if (!topk) return IDX_ERR_NULL;
  if (topk_row_stride < k || !aligned(topk, 4)) return IDX_ERR_STRIDE;
  return IDX_OK;
}

}  // namespace idx
