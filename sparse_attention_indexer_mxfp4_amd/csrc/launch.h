// Kernel launchers behind the C ABI. Arguments reaching these have passed the host
// checks of validate.h; each launcher only shapes the grid and enqueues.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "validate.h"

namespace idx {

struct MqaArgs {
  const uint8_t *q;
  int64_t q_row_stride;  // bytes
  const uint8_t *k;
  int64_t k_row_stride;  // bytes
  const float *k_scale;
  const float *w;
  int64_t w_row_stride;  // elements
  const int32_t *row_start;
  const int32_t *row_end;
  int32_t M, N, H;
  float *logits;
  int64_t logits_row_stride;  // elements
  // keys straight off an fp8 paged cache (paged != 0; k and k_scale unused): key s
  // lives in page block_table[s / page_size], keys at or past key_limit are not read
  // (with key_limit == 0 neither the table nor a page is touched and every column
  // is -inf); columns still run over [0, N)
  int32_t paged;
  const uint8_t *kbase;
  int64_t page_stride;  // bytes
  const int32_t *block_table;
  int32_t page_size, page_shift, num_pages, key_limit;
};

struct PagedArgs {
  const uint8_t *base;
  int64_t page_stride;  // bytes
  int32_t page_size;
  int32_t page_shift;  // log2(page_size) when it is a power of two, else -1
  int32_t num_pages;
  int32_t fmt;
  const uint8_t *q;
  const int32_t *q_scale;
  const float *w;
  const int32_t *context_lens;
  int32_t ctx_per_row;
  const int32_t *block_table;
  int64_t block_table_stride;
  int32_t max_blocks;
  int32_t B, next_n, H;
  float *logits;
  int64_t logits_row_stride;
  int32_t width;
  int32_t *row_end_out;
  // dense walk: block maxima of every row (block_max != nullptr), block_size 16, 32 or 64
  float *block_max;
  int64_t block_max_row_stride;
  int32_t block_size;  // also the pool block of the gather walk
  // gather walk (cand != nullptr): row r scores only its candidate pool, slot j being
  // position cand[r / row_repeat][j / block_size] * block_size + j % block_size
  const int32_t *cand;
  int64_t cand_row_stride;
  int32_t n_cand;
  int32_t row_repeat;
};

struct TopkArgs {
  const float *logits;
  int64_t logits_row_stride;
  int32_t rows, width;
  const int32_t *row_start;
  const int32_t *row_end;
  int32_t k;
  int32_t *out;
  int64_t out_row_stride;
  int32_t end_div;  // the row end used is ceil(row_end[r] / end_div) (1: row_end itself)
};

struct MaskArgs {
  float *logits;
  int64_t logits_row_stride;
  int32_t rows, width;
  const int32_t *row_end;
  const int32_t *cand;
  int64_t cand_row_stride;
  int32_t n_cand, block_size, row_repeat;
};

struct RemapArgs {
  int32_t *topk;
  int64_t topk_row_stride;
  int32_t rows, k;
  const int32_t *cand;
  int64_t cand_row_stride;
  int32_t n_cand, block_size, row_repeat;
};

struct KStoreArgs {
  uint8_t *base;
  int64_t page_stride;
  int32_t page_size;
  int32_t num_pages;
  int32_t fmt;
  const void *k;
  int32_t k_dtype;
  int64_t k_row_stride;  // elements
  const int64_t *slots;
  int32_t N;
  // RMSNorm + RoPE before the store (norm_weight != NULL)
  const float *norm_weight;
  float eps;
  const int64_t *positions;
  const float *cos_sin;
  int32_t max_position, rope_dim;
};

struct QRopeArgs {
  const void *q;
  int32_t q_dtype;
  int64_t q_row_stride;  // elements
  const int64_t *positions;
  const float *cos_sin;
  int32_t max_position, rope_dim;
  const float *weights;
  int64_t weights_row_stride;  // elements
  float weight_scale;
  int32_t T, H;
  int32_t fmt;
  uint8_t *q_out;
  int32_t *q_scale_out;
  float *weights_out;
};

struct QQuantArgs {
  const void *q;
  int32_t q_dtype;
  int64_t q_row_stride;  // elements
  int32_t T, H;
  int32_t fmt;
  uint8_t *q_out;
  int32_t *q_scale_out;
};

struct SlotsArgs {
  const int32_t *topk;
  int64_t topk_row_stride;
  int32_t rows, k;
  const int32_t *row_seq;
  int32_t next_n, B;
  const uint8_t *row_valid;
  const int32_t *block_table;
  int64_t block_table_stride;
  int32_t max_blocks, page_size;
  int32_t *slots;
  int32_t *indptr;
  int32_t *lens;
};

hipError_t launch_mqa_logits(const MqaArgs &a, int num_cus, hipStream_t stream);
hipError_t launch_paged_logits(const PagedArgs &a, int num_cus, hipStream_t stream);
// a prefill chunk of one sequence off its MXFP4 pages: rows a.B, row ends in
// a.context_lens, the sequence's pages in a.block_table; H <= 64
hipError_t launch_paged_prefill_fp4(const PagedArgs &a, int num_cus, hipStream_t stream);
// Per-row top-k. With a scratch buffer of at least topk_scratch_bytes(rows) bytes (zero
// before the first call; every call leaves it zero) and few rows, several workgroups
// share each row (topk_coop.hip); otherwise one workgroup per row (topk.hip).
hipError_t launch_topk(const TopkArgs &a, int num_cus, void *scratch, size_t scratch_bytes, hipStream_t stream);

int topk_coop_grid(int num_cus, int rows, int width);  // its grid for these rows (0: cannot run)
hipError_t launch_topk_coop(const TopkArgs &a, void *scratch, int grid, hipStream_t stream);
// One 256-thread workgroup per row with the row's keys in registers (no scratch), for
// rows of at most topk_solo_cap() columns (the width bounds them).
int topk_solo_cap();
hipError_t launch_topk_solo(const TopkArgs &a, hipStream_t stream);
// The current device's address of the library-owned top-k scratch (topk_scratch_bytes(
// kCoopMaxRows) bytes, in *bytes), looked up once per device; nullptr on failure.
void *topk_static_scratch(size_t *bytes);
hipError_t launch_k_store(const KStoreArgs &a, hipStream_t stream);
hipError_t launch_q_quant(const QQuantArgs &a, hipStream_t stream);
hipError_t launch_q_rope_quant(const QRopeArgs &a, hipStream_t stream);
hipError_t launch_topk_to_slots(const SlotsArgs &a, hipStream_t stream);
hipError_t launch_candidate_mask(const MaskArgs &a, hipStream_t stream);
hipError_t launch_remap_compact_topk(const RemapArgs &a, hipStream_t stream);

#ifdef IDX_DEBUG
// The debug build's device word of each kernel source (current device): copied to
// *out, reset with `clear`.
hipError_t debug_word_mqa_logits(uint32_t *out, bool clear);
hipError_t debug_word_paged_logits(uint32_t *out, bool clear);
hipError_t debug_word_paged_prefill(uint32_t *out, bool clear);
hipError_t debug_word_topk(uint32_t *out, bool clear);
hipError_t debug_word_topk_coop(uint32_t *out, bool clear);
hipError_t debug_word_candidates(uint32_t *out, bool clear);
hipError_t debug_word_quant(uint32_t *out, bool clear);
hipError_t debug_word_slots(uint32_t *out, bool clear);
#endif

}  // namespace idx
