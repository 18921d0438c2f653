// The consumer side of the two-level indexer: masking a dense logits row to its
// candidate pool, and turning a top-k over a gathered pool back into context positions.
//
// Page "vllm.v1.attention.ops.rocm_aiter_mla_sparse", _apply_candidate_mask_strided:
// over each row's [0, end), columns outside the row's candidate blocks become -inf,
// with row_repeat query rows sharing one candidate row. Page
// "vllm.v1.attention.ops.rocm_paged_mxfp4_indexer", _remap_compact_topk: pool slot j
// lies in pool block j / block, which starts at that block's first position.
//
// Both are a few bytes per column or entry: the mask only writes (-inf over the
// non-candidate part of [0, end), from a per-row block bitmap in LDS), the remap reads
// one candidate entry per top-k entry.
#include "debug.h"
#include "device.h"
#include "launch.h"

namespace idx {
namespace {

constexpr int kMaskThreads = 256;

__global__ __launch_bounds__(kMaskThreads) void candidate_mask_kernel(MaskArgs a) {
  extern __shared__ uint8_t s_flag[];  // 1 for a candidate block of [0, end)
  const int r = blockIdx.x;
  const int tid = threadIdx.x;
  const int end = min(max(a.row_end[r], 0), a.width);
  IDX_DEBUG_NOTE(a.row_end[r] < 0 || a.row_end[r] > a.width, IDX_DBG_LENGTH);
  const int bsh = 31 - __builtin_clz(a.block_size);
  const int nb = (end >> bsh) + ((end & (a.block_size - 1)) != 0);
  for (int i = tid; i < nb; i += kMaskThreads) s_flag[i] = 0;
  __syncthreads();
  const int32_t *cr = a.cand + int64_t(r / a.row_repeat) * a.cand_row_stride;
  for (int i = tid; i < a.n_cand; i += kMaskThreads) {
    const int b = cr[i];
    if (b >= 0 && b < nb) s_flag[b] = 1;
  }
  __syncthreads();
  float *row = a.logits + int64_t(r) * a.logits_row_stride;
  const float ninf = neg_inf();
  if (a.block_size >= 4) {
    // four columns at a time, all in one block (the row is 16-byte aligned)
    const int end4 = end & ~3;
    for (int c = 4 * tid; c < end4; c += 4 * kMaskThreads)
      if (!s_flag[c >> bsh]) *reinterpret_cast<v4f *>(row + c) = v4f{ninf, ninf, ninf, ninf};
    for (int c = end4 + tid; c < end; c += kMaskThreads)
      if (!s_flag[c >> bsh]) row[c] = ninf;
  } else {
    for (int c = tid; c < end; c += kMaskThreads)
      if (!s_flag[c >> bsh]) row[c] = ninf;
  }
}

__global__ __launch_bounds__(256) void remap_kernel(RemapArgs a) {
  const int64_t i = int64_t(blockIdx.x) * 256 + threadIdx.x;
  if (i >= int64_t(a.rows) * a.k) return;
  const int r = int(i / a.k), e = int(i % a.k);
  int32_t *p = a.topk + int64_t(r) * a.topk_row_stride + e;
  const int j = *p;
  if (j < 0) return;
  const int bsh = 31 - __builtin_clz(a.block_size);
  int out = -1;
  if ((j >> bsh) < a.n_cand) {
    const int blk = a.cand[int64_t(r / a.row_repeat) * a.cand_row_stride + (j >> bsh)];
    if (blk >= 0) out = int(min(int64_t(blk) * a.block_size + (j & (a.block_size - 1)), int64_t(INT32_MAX)));
  }
  *p = out;
}

}  // namespace

hipError_t launch_candidate_mask(const MaskArgs &a, hipStream_t stream) {
  const int bsh = 31 - __builtin_clz(a.block_size);
  const size_t lds = size_t((a.width >> bsh) + 1);
  candidate_mask_kernel<<<dim3(a.rows), kMaskThreads, lds, stream>>>(a);
  return hipGetLastError();
}

hipError_t launch_remap_compact_topk(const RemapArgs &a, hipStream_t stream) {
  const int64_t n = int64_t(a.rows) * a.k;
  remap_kernel<<<dim3(unsigned((n + 255) / 256)), 256, 0, stream>>>(a);
  return hipGetLastError();
}

IDX_DEBUG_READER(debug_word_candidates)

}  // namespace idx
