// Host-side argument checks of the indexer ABI. Plain C++ (no HIP), so the checks
// can be exercised on a machine without a GPU. Each check returns IDX_OK, an
// error, or IDX_OK with *empty set when the call has no work to launch.
#pragma once

#include <cstddef>
#include <cstdint>

#include "../../include/idx.h"

namespace idx {

constexpr int32_t kHeadDim = 128;
constexpr int32_t kMaxHeads = 128;
constexpr int32_t kMaxNextN = 4;
constexpr int32_t kMaxBatch = 8192;
constexpr int32_t kMaxTopK = 65536;

// The several-workgroups-per-row top-k: up to kCoopMaxRows rows, at most kCoopMaxUnits
// workgroups. Its scratch holds one 16-byte record per workgroup, then one
// kCoopRowBytes record per row.
constexpr int kCoopMaxRows = 256;
constexpr int kCoopMaxUnits = 2048;
constexpr size_t kCoopUnitBytes = 16;
constexpr size_t kCoopRowBytes = 36928;
constexpr size_t topk_scratch_bytes(int rows) {
  return rows < 1 || rows > kCoopMaxRows ? 0 : size_t(kCoopMaxUnits) * kCoopUnitBytes + size_t(rows) * kCoopRowBytes;
}

size_t page_bytes(int32_t fmt, int32_t page_size, int32_t head_dim);

idx_status check_cache(const idx_paged_cache *cache);

idx_status check_mqa_logits(const void *q, int64_t q_row_stride, const void *k, int64_t k_row_stride,
                            const void *k_scale, const void *w, int64_t w_row_stride, const void *row_start,
                            const void *row_end, int32_t M, int32_t N, int32_t H, int32_t D, const void *logits,
                            int64_t logits_row_stride, bool *empty);

size_t paged_workspace_bytes(int32_t B, int32_t next_n, int32_t H, const idx_paged_cache *cache);

idx_status check_paged_mqa_logits(const idx_paged_cache *cache, const void *q, const void *q_scale, const void *w,
                                  const void *context_lens, const void *block_table, int64_t block_table_stride,
                                  int32_t max_blocks, int32_t B, int32_t next_n, int32_t H, const void *logits,
                                  int64_t logits_row_stride, int32_t width, const void *workspace,
                                  size_t workspace_bytes, bool *empty);

size_t topk_workspace_bytes(int32_t rows, int32_t width, int32_t k);

// idx_topk's checks of everything but the workspace
idx_status check_topk_args(const void *logits, int64_t logits_row_stride, int32_t rows, int32_t width,
                           const void *row_end, int32_t k, const void *out, int64_t out_row_stride, bool *empty);

idx_status check_topk(const void *logits, int64_t logits_row_stride, int32_t rows, int32_t width,
                      const void *row_end, int32_t k, const void *out, int64_t out_row_stride,
                      const void *workspace, size_t workspace_bytes, bool *empty);

idx_status check_k_store(const idx_paged_cache *cache, const void *k, int32_t k_dtype, int64_t k_row_stride,
                         const void *slot_mapping, int32_t N, bool *empty);

idx_status check_q_quant(const void *q, int32_t q_dtype, int64_t q_row_stride, int32_t T, int32_t H, int32_t D,
                         int32_t fmt, const void *q_out, const void *q_scale_out, bool *empty);

// The RoPE table and RMSNorm arguments of the fused producers (norm_weight may be
// NULL when no norm is applied, as in the query op).
idx_status check_norm_rope(const void *positions, const void *cos_sin, int32_t max_position, int32_t rope_dim,
                           const void *norm_weight, float eps);

idx_status check_q_rope_quant(const void *q, int32_t q_dtype, int64_t q_row_stride, const void *positions,
                              const void *cos_sin, int32_t max_position, int32_t rope_dim, const void *weights,
                              int64_t weights_row_stride, int32_t T, int32_t H, int32_t D, int32_t fmt,
                              const void *q_out, const void *q_scale_out, const void *weights_out, bool *empty);

idx_status check_topk_to_slots(const void *topk, int64_t topk_row_stride, int32_t rows, int32_t k,
                               const void *row_seq, int32_t next_n, int32_t B, const void *block_table,
                               int64_t block_table_stride, int32_t max_blocks, int32_t page_size,
                               const void *slots_out, const void *indptr_out, bool *empty);

// two-level indexer
idx_status check_block_max(const void *block_max, int64_t block_max_row_stride, int32_t block_size, int32_t width);
idx_status check_candidate_list(const void *cand, int64_t cand_row_stride, int32_t n_cand, int32_t block_size,
                                int32_t row_repeat);
idx_status check_gather(int32_t B, int32_t next_n, int32_t block_size, const void *pool_logits,
                        int64_t pool_row_stride, int32_t n_cand, const void *pool_end_out);
idx_status check_candidate_mask(const void *logits, int64_t logits_row_stride, int32_t rows, int32_t width,
                                const void *row_end, int32_t block_size, bool *empty);
idx_status check_remap(const void *topk, int64_t topk_row_stride, int32_t rows, int32_t k, bool *empty);

}  // namespace idx
