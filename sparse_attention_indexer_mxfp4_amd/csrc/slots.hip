// Top-k rows of local key positions -> a ragged stream of physical cache slots for
// the sparse-attention consumer: page "vllm.v1.attention.ops.rocm_aiter_mla_sparse",
// build_prefill_topk_ragged_indices (local positions mapped through each sequence's
// block table and packed row after row); page "vllm.models.deepseek_v41.amd.rocm",
// _decode_topk_ragged (the same for decode rows, with a validity flag per row).
//
// Three short launches: per-row counts (into lens and indptr[r + 1]), one workgroup's
// running scan of the counts into indptr, and the per-row ordered write, where each
// wave places its 64 entries with a ballot and the waves of a step take consecutive
// ranges through a scan of their counts.
#include "debug.h"
#include "device.h"
#include "launch.h"

namespace idx {
namespace {

constexpr int kThreads = 256;

__device__ __forceinline__ int lane_prefix(uint64_t mask) {
  return __builtin_amdgcn_mbcnt_hi(uint32_t(mask >> 32), __builtin_amdgcn_mbcnt_lo(uint32_t(mask), 0u));
}

__device__ __forceinline__ int row_seq(const SlotsArgs &a, int r) {
  const int b = a.row_seq ? a.row_seq[r] : r / a.next_n;
  IDX_DEBUG_NOTE(b < 0 || b >= a.B, IDX_DBG_SEQ);
  return min(max(b, 0), a.B - 1);
}

__device__ __forceinline__ bool row_live(const SlotsArgs &a, int r) { return !a.row_valid || a.row_valid[r] != 0; }

// entry i of row r as a slot, or -1 when it is a pad or past the block table
__device__ __forceinline__ int entry_slot(const SlotsArgs &a, int b, int p) {
  if (p < 0 || p >= a.max_blocks * a.page_size) return -1;
  const int page = a.block_table[int64_t(b) * a.block_table_stride + p / a.page_size];
  return page * a.page_size + p % a.page_size;
}

__global__ __launch_bounds__(kThreads) void count_kernel(SlotsArgs a) {
  __shared__ int s_part[kThreads / 64];
  const int r = blockIdx.x, tid = threadIdx.x;
  int c = 0;
  if (row_live(a, r)) {
    const int32_t *row = a.topk + int64_t(r) * a.topk_row_stride;
    const int lim = a.max_blocks * a.page_size;
    for (int i = tid; i < a.k; i += kThreads) {
      const int p = row[i];
      c += int(p >= 0 && p < lim);
    }
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) c += __shfl_xor(c, off);
  if ((tid & 63) == 0) s_part[tid >> 6] = c;
  __syncthreads();
  if (tid == 0) {
    int t = 0;
    for (int w = 0; w < kThreads / 64; ++w) t += s_part[w];
    a.indptr[r + 1] = t;
    if (a.lens) a.lens[r] = t;
  }
}

// indptr[0] = 0 and indptr[1..rows] becomes the running sum of the counts it holds
__global__ __launch_bounds__(1024) void scan_kernel(SlotsArgs a) {
  __shared__ int s_wave[16];
  __shared__ int s_carry;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  if (tid == 0) {
    s_carry = 0;
    a.indptr[0] = 0;
  }
  __syncthreads();
  for (int base = 0; base < a.rows; base += 1024) {
    const int i = base + tid;
    const int v = i < a.rows ? a.indptr[i + 1] : 0;
    int x = v;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int y = __shfl_up(x, off);
      if (lane >= off) x += y;
    }
    if (lane == 63) s_wave[wave] = x;
    __syncthreads();
    int before = s_carry;
    for (int w = 0; w < wave; ++w) before += s_wave[w];
    if (i < a.rows) a.indptr[i + 1] = before + x;
    __syncthreads();
    if (tid == 1023) s_carry = before + x;
    __syncthreads();
  }
}

__global__ __launch_bounds__(kThreads) void write_kernel(SlotsArgs a) {
  __shared__ int s_cnt[kThreads / 64];
  const int r = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  if (!row_live(a, r)) return;  // uniform per workgroup
  const int b = row_seq(a, r);
  const int32_t *row = a.topk + int64_t(r) * a.topk_row_stride;
  int32_t *dst = a.slots + a.indptr[r];
  int run = 0;
  for (int base = 0; base < a.k; base += kThreads) {
    const int i = base + tid;
    const int s = i < a.k ? entry_slot(a, b, row[i]) : -1;
    const uint64_t m = __ballot(s >= 0);
    if (lane == 0) s_cnt[wave] = int(__popcll(m));
    __syncthreads();
    int before = run, total = 0;
#pragma unroll
    for (int w = 0; w < kThreads / 64; ++w) {
      const int c = s_cnt[w];
      if (w < wave) before += c;
      total += c;
    }
    if (s >= 0) dst[before + lane_prefix(m)] = s;
    run += total;
    __syncthreads();
  }
}

}  // namespace

hipError_t launch_topk_to_slots(const SlotsArgs &a, hipStream_t stream) {
  if (a.rows > 0) count_kernel<<<dim3(a.rows), kThreads, 0, stream>>>(a);
  scan_kernel<<<dim3(1), 1024, 0, stream>>>(a);  // with no rows: just indptr[0] = 0
  if (a.rows > 0) write_kernel<<<dim3(a.rows), kThreads, 0, stream>>>(a);
  return hipGetLastError();
}

IDX_DEBUG_READER(debug_word_slots)

}  // namespace idx
