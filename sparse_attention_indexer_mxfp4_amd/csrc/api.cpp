// The C ABI of libidx (declared in include/idx.h): argument checks, the device
// check, and the launch of each call's kernels on the caller's stream.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstring>
#include <mutex>

#include "../../include/idx.h"
#include "launch.h"
#include "validate.h"

namespace {

struct DeviceInfo {
  bool known = false;
  bool gfx950 = false;
  int num_cus = 0;
};

constexpr int kMaxDevices = 64;
std::mutex g_mu;
DeviceInfo g_dev[kMaxDevices];

// Current device's properties, looked up once per device.
idx_status current_device(int *num_cus) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return IDX_ERR_DEVICE;
  std::lock_guard<std::mutex> lock(g_mu);
  DeviceInfo &d = g_dev[dev];
  if (!d.known) {
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return IDX_ERR_DEVICE;
    d.gfx950 = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0;
    d.num_cus = prop.multiProcessorCount;
    d.known = true;
  }
  if (!d.gfx950 || d.num_cus <= 0) return IDX_ERR_DEVICE;
  *num_cus = d.num_cus;
  return IDX_OK;
}

idx_status launched(hipError_t e) { return e == hipSuccess ? IDX_OK : IDX_ERR_LAUNCH; }

}  // namespace

extern "C" {

size_t idx_page_bytes(int32_t fmt, int32_t page_size, int32_t head_dim) {
  return idx::page_bytes(fmt, page_size, head_dim);
}

idx_status idx_mqa_logits(const uint8_t *q, int64_t q_row_stride, const uint8_t *k, int64_t k_row_stride,
                          const float *k_scale, const float *w, int64_t w_row_stride,
                          const int32_t *row_start, const int32_t *row_end, int32_t M, int32_t N, int32_t H,
                          int32_t D, float *logits, int64_t logits_row_stride, hipStream_t stream) {
  bool empty = false;
  idx_status s = idx::check_mqa_logits(q, q_row_stride, k, k_row_stride, k_scale, w, w_row_stride, row_start,
                                       row_end, M, N, H, D, logits, logits_row_stride, &empty);
  if (s != IDX_OK || empty) return s;
  int cus = 0;
  if ((s = current_device(&cus)) != IDX_OK) return s;
  idx::MqaArgs a{q, q_row_stride, k, k_row_stride, k_scale, w, w_row_stride, row_start, row_end,
                 M, N, H, logits, logits_row_stride};
  return launched(idx::launch_mqa_logits(a, cus, stream));
}

size_t idx_paged_mqa_logits_workspace(int32_t B, int32_t next_n, int32_t H, const idx_paged_cache *cache) {
  return idx::paged_workspace_bytes(B, next_n, H, cache);
}

namespace {
idx::PagedArgs paged_args(const idx_paged_cache *cache, const void *q, const int32_t *q_scale, const float *w,
                          const int32_t *context_lens, int32_t ctx_per_row, const int32_t *block_table,
                          int64_t block_table_stride, int32_t max_blocks, int32_t B, int32_t next_n, int32_t H,
                          float *logits, int64_t logits_row_stride, int32_t width, int32_t *row_end_out) {
  int shift = -1;
  for (int sh = 4; sh <= 10; ++sh)
    if (cache->page_size == (1 << sh)) shift = sh;
  idx::PagedArgs a{};
  a.base = static_cast<const uint8_t *>(cache->base);
  a.page_stride = cache->page_stride_bytes;
  a.page_size = cache->page_size;
  a.page_shift = shift;
  a.num_pages = cache->num_pages;
  a.fmt = cache->fmt;
  a.q = static_cast<const uint8_t *>(q);
  a.q_scale = q_scale;
  a.w = w;
  a.context_lens = context_lens;
  a.ctx_per_row = ctx_per_row != 0;
  a.block_table = block_table;
  a.block_table_stride = block_table_stride;
  a.max_blocks = max_blocks;
  a.B = B;
  a.next_n = next_n;
  a.H = H;
  a.logits = logits;
  a.logits_row_stride = logits_row_stride;
  a.width = width;
  a.row_end_out = row_end_out;
  return a;
}
}  // namespace

idx_status idx_paged_mqa_logits(const idx_paged_cache *cache, const void *q, const int32_t *q_scale,
                                const float *w, const int32_t *context_lens, int32_t ctx_per_row,
                                const int32_t *block_table, int64_t block_table_stride, int32_t max_blocks,
                                int32_t B, int32_t next_n, int32_t H, float *logits, int64_t logits_row_stride,
                                int32_t width, int32_t *row_end_out, void *workspace, size_t workspace_bytes,
                                hipStream_t stream) {
  return idx_paged_mqa_logits_block_max(cache, q, q_scale, w, context_lens, ctx_per_row, block_table,
                                        block_table_stride, max_blocks, B, next_n, H, logits, logits_row_stride,
                                        width, row_end_out, nullptr, 0, 0, workspace, workspace_bytes, stream);
}

idx_status idx_paged_mqa_logits_block_max(const idx_paged_cache *cache, const void *q, const int32_t *q_scale,
                                          const float *w, const int32_t *context_lens, int32_t ctx_per_row,
                                          const int32_t *block_table, int64_t block_table_stride,
                                          int32_t max_blocks, int32_t B, int32_t next_n, int32_t H, float *logits,
                                          int64_t logits_row_stride, int32_t width, int32_t *row_end_out,
                                          float *block_max, int64_t block_max_row_stride, int32_t block_size,
                                          void *workspace, size_t workspace_bytes, hipStream_t stream) {
  bool empty = false;
  idx_status s = idx::check_paged_mqa_logits(cache, q, q_scale, w, context_lens, block_table, block_table_stride,
                                             max_blocks, B, next_n, H, logits, logits_row_stride, width,
                                             workspace, workspace_bytes, &empty);
  if (s != IDX_OK) return s;
  if (block_size != 0 && (s = idx::check_block_max(block_max, block_max_row_stride, block_size, width)) != IDX_OK)
    return s;
  if (empty) return IDX_OK;
  int cus = 0;
  if ((s = current_device(&cus)) != IDX_OK) return s;
  idx::PagedArgs a = paged_args(cache, q, q_scale, w, context_lens, ctx_per_row, block_table, block_table_stride,
                                max_blocks, B, next_n, H, logits, logits_row_stride, width, row_end_out);
  if (block_size != 0) {
    a.block_max = block_max;
    a.block_max_row_stride = block_max_row_stride;
    a.block_size = block_size;
  }
  return launched(idx::launch_paged_logits(a, cus, stream));
}

idx_status idx_paged_mqa_logits_gather(const idx_paged_cache *cache, const void *q, const int32_t *q_scale,
                                       const float *w, const int32_t *context_lens, int32_t ctx_per_row,
                                       const int32_t *block_table, int64_t block_table_stride, int32_t max_blocks,
                                       int32_t B, int32_t next_n, int32_t H, const int32_t *cand,
                                       int64_t cand_row_stride, int32_t n_cand, int32_t block_size,
                                       int32_t row_repeat, float *pool_logits, int64_t pool_row_stride,
                                       int32_t *pool_end_out, hipStream_t stream) {
  idx_status s = idx::check_candidate_list(cand, cand_row_stride, n_cand, block_size, row_repeat);
  if (s != IDX_OK) return s;
  if ((s = idx::check_gather(B, next_n, block_size, pool_logits, pool_row_stride, n_cand, pool_end_out)) != IDX_OK)
    return s;
  const int32_t width = n_cand * block_size;
  bool empty = false;
  s = idx::check_paged_mqa_logits(cache, q, q_scale, w, context_lens, block_table, block_table_stride, max_blocks,
                                  B, next_n, H, pool_logits, pool_row_stride, width, nullptr, 0, &empty);
  if (s != IDX_OK || empty) return s;
  int cus = 0;
  if ((s = current_device(&cus)) != IDX_OK) return s;
  idx::PagedArgs a = paged_args(cache, q, q_scale, w, context_lens, ctx_per_row, block_table, block_table_stride,
                                max_blocks, B, next_n, H, pool_logits, pool_row_stride, width, pool_end_out);
  a.block_size = block_size;
  a.cand = cand;
  a.cand_row_stride = cand_row_stride;
  a.n_cand = n_cand;
  a.row_repeat = row_repeat;
  return launched(idx::launch_paged_logits(a, cus, stream));
}

idx_status idx_paged_prefill_logits(const idx_paged_cache *cache, const void *q, const int32_t *q_scale,
                                    const float *w, const int32_t *row_end, const int32_t *block_table,
                                    int32_t max_blocks, int32_t M, int32_t H, float *logits,
                                    int64_t logits_row_stride, int32_t width, hipStream_t stream) {
  // MXFP4 pages with more than 64 heads: pairs of consecutive rows share one walk over
  // the sequence's pages (two rows per walk keep two waves per SIMD; measured on the
  // 8192 x 8192 MXFP4 chunk: 524 us against 650 us for one row and 783 us for four);
  // an odd last row walks alone
  constexpr int32_t kWalkRows = 2;
  if (M < 0) return IDX_ERR_SHAPE;
  const int32_t groups = M / kWalkRows, tail = M % kWalkRows;
  bool empty = false;
  idx_status s = idx::check_paged_mqa_logits(cache, q, q_scale, w, row_end, block_table, max_blocks, max_blocks,
                                             groups + tail, 1, H, logits, logits_row_stride, width, nullptr, 0,
                                             &empty);
  if (s != IDX_OK || empty) return s;
  if (int64_t(M) * ((int64_t(width) + 63) / 64) > INT32_MAX) return IDX_ERR_SHAPE;
  if (width == 0) return IDX_OK;  // no column to write
  int cus = 0;
  if ((s = current_device(&cus)) != IDX_OK) return s;
  if (cache->fmt == IDX_KV_MXFP4_E2M1 && H <= 64) {
    // MXFP4 pages: eight rows per workgroup share each key chunk through LDS
    const idx::PagedArgs a = paged_args(cache, q, q_scale, w, row_end, 1, block_table, 0, max_blocks, M, 1, H,
                                        logits, logits_row_stride, width, nullptr);
    return launched(idx::launch_paged_prefill_fp4(a, cus, stream));
  }
  if (cache->fmt == IDX_KV_FP8_E4M3) {
    // fp8 pages: the contiguous prefill kernel with its keys read through the block table
    idx::MqaArgs a{};
    a.q = static_cast<const uint8_t *>(q);
    a.q_row_stride = int64_t(H) * cache->head_dim;
    a.k_row_stride = cache->head_dim;
    a.w = w;
    a.w_row_stride = H;
    a.row_end = row_end;  // row_start stays NULL: every row starts at key 0
    a.M = M;
    a.N = width;
    a.H = H;
    a.logits = logits;
    a.logits_row_stride = logits_row_stride;
    a.paged = 1;  // the paged kernel even for an empty table: it then reads nothing
    a.kbase = static_cast<const uint8_t *>(cache->base);
    a.page_stride = cache->page_stride_bytes;
    a.block_table = block_table;
    a.page_size = cache->page_size;
    a.page_shift = -1;
    for (int sh = 4; sh <= 10; ++sh)
      if (cache->page_size == (1 << sh)) a.page_shift = sh;
    a.num_pages = cache->num_pages;
    a.key_limit = int32_t(std::min<int64_t>(width, int64_t(max_blocks) * cache->page_size));
    return launched(idx::launch_mqa_logits(a, cus, stream));
  }
  const int64_t qrow = int64_t(H) * (cache->fmt == IDX_KV_FP8_E4M3 ? cache->head_dim : cache->head_dim / 2);
  if (groups > 0) {
    idx::PagedArgs a = paged_args(cache, q, q_scale, w, row_end, 1, block_table, 0, max_blocks, groups, kWalkRows,
                                  H, logits, logits_row_stride, width, nullptr);
    if ((s = launched(idx::launch_paged_logits(a, cus, stream))) != IDX_OK) return s;
  }
  if (tail > 0) {
    const int64_t r0 = int64_t(groups) * kWalkRows;
    idx::PagedArgs a = paged_args(cache, static_cast<const uint8_t *>(q) + r0 * qrow,
                                  q_scale ? q_scale + r0 * H : nullptr, w + r0 * H, row_end + r0, 1, block_table, 0,
                                  max_blocks, tail, 1, H, logits + r0 * logits_row_stride, logits_row_stride, width,
                                  nullptr);
    if ((s = launched(idx::launch_paged_logits(a, cus, stream))) != IDX_OK) return s;
  }
  return IDX_OK;
}

idx_status idx_candidate_blocks(const float *block_max, int64_t block_max_row_stride, int32_t rows,
                                int32_t num_blocks, const int32_t *row_end, int32_t block_size, int32_t n_cand,
                                int32_t *cand_out, int64_t cand_row_stride, void *workspace,
                                size_t workspace_bytes, hipStream_t stream) {
  if (block_size < 1 || (block_size & (block_size - 1))) return IDX_ERR_SHAPE;
  bool empty = false;
  idx_status s = idx::check_topk(block_max, block_max_row_stride, rows, num_blocks, row_end, n_cand, cand_out,
                                 cand_row_stride, workspace, workspace_bytes, &empty);
  if (s != IDX_OK || empty) return s;
  int cus = 0;
  if ((s = current_device(&cus)) != IDX_OK) return s;
  idx::TopkArgs a{block_max, block_max_row_stride, rows, num_blocks, nullptr, row_end, n_cand, cand_out,
                  cand_row_stride, block_size};
  return launched(idx::launch_topk(a, cus, workspace, workspace_bytes, stream));
}

idx_status idx_apply_candidate_mask(float *logits, int64_t logits_row_stride, int32_t rows, int32_t width,
                                    const int32_t *row_end, const int32_t *cand, int64_t cand_row_stride,
                                    int32_t n_cand, int32_t block_size, int32_t row_repeat, hipStream_t stream) {
  bool empty = false;
  idx_status s = idx::check_candidate_mask(logits, logits_row_stride, rows, width, row_end, block_size, &empty);
  if (s != IDX_OK) return s;
  if ((s = idx::check_candidate_list(cand, cand_row_stride, n_cand, block_size, row_repeat)) != IDX_OK) return s;
  if (empty) return IDX_OK;
  int cus = 0;
  if ((s = current_device(&cus)) != IDX_OK) return s;
  idx::MaskArgs a{logits, logits_row_stride, rows, width, row_end, cand, cand_row_stride, n_cand, block_size,
                  row_repeat};
  return launched(idx::launch_candidate_mask(a, stream));
}

idx_status idx_remap_compact_topk(int32_t *topk, int64_t topk_row_stride, int32_t rows, int32_t k,
                                  const int32_t *cand, int64_t cand_row_stride, int32_t n_cand, int32_t block_size,
                                  int32_t row_repeat, hipStream_t stream) {
  bool empty = false;
  idx_status s = idx::check_remap(topk, topk_row_stride, rows, k, &empty);
  if (s != IDX_OK) return s;
  if ((s = idx::check_candidate_list(cand, cand_row_stride, n_cand, block_size, row_repeat)) != IDX_OK) return s;
  if (empty) return IDX_OK;
  int cus = 0;
  if ((s = current_device(&cus)) != IDX_OK) return s;
  idx::RemapArgs a{topk, topk_row_stride, rows, k, cand, cand_row_stride, n_cand, block_size, row_repeat};
  return launched(idx::launch_remap_compact_topk(a, stream));
}

size_t idx_topk_workspace(int32_t rows, int32_t width, int32_t k) { return idx::topk_workspace_bytes(rows, width, k); }

idx_status idx_topk(const float *logits, int64_t logits_row_stride, int32_t rows, int32_t width,
                    const int32_t *row_start, const int32_t *row_end, int32_t k, int32_t *out,
                    int64_t out_row_stride, void *workspace, size_t workspace_bytes, hipStream_t stream) {
  bool empty = false;
  idx_status s = idx::check_topk(logits, logits_row_stride, rows, width, row_end, k, out, out_row_stride, workspace,
                                 workspace_bytes, &empty);
  if (s != IDX_OK || empty) return s;
  int cus = 0;
  if ((s = current_device(&cus)) != IDX_OK) return s;
  idx::TopkArgs a{logits, logits_row_stride, rows, width, row_start, row_end, k, out, out_row_stride, 1};
  return launched(idx::launch_topk(a, cus, workspace, workspace_bytes, stream));
}

idx_status idx_topk_noalloc(const float *logits, int64_t logits_row_stride, int32_t rows, int32_t width,
                            const int32_t *row_start, const int32_t *row_end, int32_t k, int32_t *out,
                            int64_t out_row_stride, hipStream_t stream) {
  bool empty = false;
  idx_status s = idx::check_topk_args(logits, logits_row_stride, rows, width, row_end, k, out, out_row_stride,
                                      &empty);
  if (s != IDX_OK || empty) return s;
  int cus = 0;
  if ((s = current_device(&cus)) != IDX_OK) return s;
  size_t bytes = 0;
  void *ws = idx::topk_static_scratch(&bytes);
  if (!ws) return IDX_ERR_DEVICE;
  // more rows than the array has records for never take the path that uses it
  if (idx::topk_scratch_bytes(rows) > bytes) return IDX_ERR_WORKSPACE;
  idx::TopkArgs a{logits, logits_row_stride, rows, width, row_start, row_end, k, out, out_row_stride, 1};
  return launched(idx::launch_topk(a, cus, ws, bytes, stream));
}

idx_status idx_k_store(const idx_paged_cache *cache, const void *k, int32_t k_dtype, int64_t k_row_stride,
                       const int64_t *slot_mapping, int32_t N, hipStream_t stream) {
  bool empty = false;
  idx_status s = idx::check_k_store(cache, k, k_dtype, k_row_stride, slot_mapping, N, &empty);
  if (s != IDX_OK || empty) return s;
  int cus = 0;
  if ((s = current_device(&cus)) != IDX_OK) return s;
  idx::KStoreArgs a{static_cast<uint8_t *>(cache->base), cache->page_stride_bytes, cache->page_size,
                    cache->num_pages, cache->fmt, k, k_dtype, k_row_stride, slot_mapping, N,
                    nullptr, 0.f, nullptr, nullptr, 0, 0};
  return launched(idx::launch_k_store(a, stream));
}

idx_status idx_k_norm_rope_store(const idx_paged_cache *cache, const void *k, int32_t k_dtype, int64_t k_row_stride,
                                 const int64_t *positions, const float *cos_sin, int32_t max_position,
                                 int32_t rope_dim, const float *norm_weight, float eps,
                                 const int64_t *slot_mapping, int32_t N, hipStream_t stream) {
  bool empty = false;
  idx_status s = idx::check_k_store(cache, k, k_dtype, k_row_stride, slot_mapping, N, &empty);
  if (s != IDX_OK || empty) return s;
  if ((s = idx::check_norm_rope(positions, cos_sin, max_position, rope_dim, norm_weight, eps)) != IDX_OK) return s;
  int cus = 0;
  if ((s = current_device(&cus)) != IDX_OK) return s;
  idx::KStoreArgs a{static_cast<uint8_t *>(cache->base), cache->page_stride_bytes, cache->page_size,
                    cache->num_pages, cache->fmt, k, k_dtype, k_row_stride, slot_mapping, N,
                    norm_weight, eps, positions, cos_sin, max_position, rope_dim};
  return launched(idx::launch_k_store(a, stream));
}

idx_status idx_q_quant(const void *q, int32_t q_dtype, int64_t q_row_stride, int32_t T, int32_t H, int32_t D,
                       int32_t fmt, void *q_out, int32_t *q_scale_out, hipStream_t stream) {
  bool empty = false;
  idx_status s = idx::check_q_quant(q, q_dtype, q_row_stride, T, H, D, fmt, q_out, q_scale_out, &empty);
  if (s != IDX_OK || empty) return s;
  int cus = 0;
  if ((s = current_device(&cus)) != IDX_OK) return s;
  idx::QQuantArgs a{q, q_dtype, q_row_stride, T, H, fmt, static_cast<uint8_t *>(q_out), q_scale_out};
  return launched(idx::launch_q_quant(a, stream));
}

idx_status idx_q_rope_quant(const void *q, int32_t q_dtype, int64_t q_row_stride, const int64_t *positions,
                            const float *cos_sin, int32_t max_position, int32_t rope_dim, const float *weights,
                            int64_t weights_row_stride, float weight_scale, int32_t T, int32_t H, int32_t D,
                            int32_t fmt, void *q_out, int32_t *q_scale_out, float *weights_out,
                            hipStream_t stream) {
  bool empty = false;
  idx_status s = idx::check_q_rope_quant(q, q_dtype, q_row_stride, positions, cos_sin, max_position, rope_dim,
                                         weights, weights_row_stride, T, H, D, fmt, q_out, q_scale_out, weights_out,
                                         &empty);
  if (s != IDX_OK || empty) return s;
  int cus = 0;
  if ((s = current_device(&cus)) != IDX_OK) return s;
  idx::QRopeArgs a{q, q_dtype, q_row_stride, positions, cos_sin, max_position, rope_dim, weights,
                   weights_row_stride, weight_scale, T, H, fmt, static_cast<uint8_t *>(q_out), q_scale_out,
                   weights_out};
  return launched(idx::launch_q_rope_quant(a, stream));
}

idx_status idx_topk_to_slots(const int32_t *topk, int64_t topk_row_stride, int32_t rows, int32_t k,
                             const int32_t *row_seq, int32_t next_n, int32_t B, const uint8_t *row_valid,
                             const int32_t *block_table, int64_t block_table_stride, int32_t max_blocks,
                             int32_t page_size, int32_t *slots_out, int32_t *indptr_out, int32_t *lens_out,
                             hipStream_t stream) {
  bool empty = false;  // no rows: only indptr[0] = 0 is written
  idx_status s = idx::check_topk_to_slots(topk, topk_row_stride, rows, k, row_seq, next_n, B, block_table,
                                          block_table_stride, max_blocks, page_size, slots_out, indptr_out, &empty);
  if (s != IDX_OK) return s;
  int cus = 0;
  if ((s = current_device(&cus)) != IDX_OK) return s;
  idx::SlotsArgs a{topk, topk_row_stride, rows, k, row_seq, next_n, B, row_valid, block_table, block_table_stride,
                   max_blocks, page_size, slots_out, indptr_out, lens_out};
  return launched(idx::launch_topk_to_slots(a, stream));
}

idx_status idx_debug_flags(uint32_t *flags, int32_t clear) {
  if (!flags) return IDX_ERR_NULL;
  *flags = 0;
#ifdef IDX_DEBUG
  if (hipDeviceSynchronize() != hipSuccess) return IDX_ERR_LAUNCH;
  hipError_t (*const words[])(uint32_t *, bool) = {
      idx::debug_word_mqa_logits, idx::debug_word_paged_logits, idx::debug_word_paged_prefill,
      idx::debug_word_topk,       idx::debug_word_topk_coop,    idx::debug_word_candidates,
      idx::debug_word_quant,      idx::debug_word_slots};
  for (auto word : words) {
    uint32_t v = 0;
    if (word(&v, clear != 0) != hipSuccess) return IDX_ERR_LAUNCH;
    *flags |= v;
  }
#else
  (void)clear;
#endif
  return IDX_OK;
}

int32_t idx_debug_build(void) {
#ifdef IDX_DEBUG
  return 1;
#else
  return 0;
#endif
}

const char *idx_status_str(idx_status s) {
  switch (s) {
    case IDX_OK: return "IDX_OK";
    case IDX_ERR_NULL: return "IDX_ERR_NULL: a required pointer is NULL";
    case IDX_ERR_SHAPE: return "IDX_ERR_SHAPE: a size is negative or outside the supported range";
    case IDX_ERR_STRIDE: return "IDX_ERR_STRIDE: a stride or alignment requirement is not met";
    case IDX_ERR_FORMAT: return "IDX_ERR_FORMAT: unknown format or dtype";
    case IDX_ERR_WORKSPACE: return "IDX_ERR_WORKSPACE: workspace too small";
    case IDX_ERR_LAUNCH: return "IDX_ERR_LAUNCH: kernel launch failed";
    case IDX_ERR_DEVICE: return "IDX_ERR_DEVICE: no current gfx950 device";
  }
  return "unknown idx_status";
}

int32_t idx_abi_version(void) { return IDX_ABI_VERSION; }

}  // extern "C"
