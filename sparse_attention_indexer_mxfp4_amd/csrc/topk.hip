// Per-row top-k over [row_start, row_end): page
// "vllm.v1.attention.ops.rocm_paged_mxfp4_indexer", _topk (-1 pads rows shorter than k).
//
// One workgroup of 1024 threads per row. Logits become order-preserving 32-bit keys
// (-0.0 folded onto +0.0). A most-significant-digit-first radix select, 8 bits per
// pass with per-wave LDS histograms, finds the k-th largest key T and how many
// keys equal to T belong to the answer. A final pass in column order emits every
// key above T and the lowest-column ties, so the k indices come out in ascending
// column order and equal values resolve to the lowest columns. Rows whose valid
// range fits the LDS budget are read from global memory once and kept in LDS for
// the remaining passes.
#include "device.h"
#include "launch.h"

namespace idx {
namespace {

constexpr int kThreads = 1024;
constexpr int kWaves = kThreads / 64;
constexpr int kMaxCache = 32768;  // keys kept in LDS (128 KiB)

__device__ __forceinline__ uint32_t order_key(float x) {
  uint32_t u = __float_as_uint(x);
  if (u == 0x80000000u) u = 0u;  // -0.0 ranks with +0.0
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ uint64_t lanes_below() {
  const int lane = threadIdx.x & 63;
  return lane == 0 ? 0ull : (~0ull >> (64 - lane));
}

__global__ __launch_bounds__(kThreads) void topk_kernel(TopkArgs a, int cache_cap) {
  extern __shared__ uint32_t s_keys[];  // cache_cap keys
  __shared__ uint32_t hist[kWaves][256];
  __shared__ int s_digit, s_above;
  __shared__ int s_cnt[kWaves][2];

  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int row = blockIdx.x;
  const int start = a.row_start ? min(max(a.row_start[row], 0), a.width) : 0;
  const int end = min(max(a.row_end[row], 0), a.width);
  const int n = max(end - start, 0);
  const int k = a.k;
  int32_t *out = a.out + int64_t(row) * a.out_row_stride;

  if (n <= k) {
    for (int i = tid; i < k; i += kThreads) out[i] = i < n ? i : -1;
    return;
  }
  const float *lr = a.logits + int64_t(row) * a.logits_row_stride + start;
  const bool cached = n <= cache_cap;

  uint32_t prefix = 0, pmask = 0;
  int kr = k;
  for (int pass = 0; pass < 4; ++pass) {
    const int shift = 24 - 8 * pass;
    for (int i = tid; i < kWaves * 256; i += kThreads) (&hist[0][0])[i] = 0u;
    __syncthreads();
    for (int i = tid; i < n; i += kThreads) {
      uint32_t key;
      if (cached) {
        if (pass == 0) {
          key = order_key(lr[i]);
          s_keys[i] = key;
        } else {
          key = s_keys[i];
        }
      } else {
        key = order_key(lr[i]);
      }
      if ((key & pmask) == prefix) atomicAdd(&hist[wave][(key >> shift) & 255u], 1u);
    }
    __syncthreads();
    if (wave == 0) {
      // lane L owns digits 255-4L .. 252-4L (descending); find the digit d with
      // (# keys above d) < kr <= (# keys at or above d)
      int cnt[4];
      int local = 0;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int d = 255 - 4 * lane - i;
        int t = 0;
#pragma unroll
        for (int w = 0; w < kWaves; ++w) t += int(hist[w][d]);
        cnt[i] = t;
        local += t;
      }
      int incl = local;
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        const int y = __shfl_up(incl, off);
        if (lane >= off) incl += y;
      }
      int running = incl - local;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        if (running < kr && running + cnt[i] >= kr) {
          s_digit = 255 - 4 * lane - i;
          s_above = running;
        }
        running += cnt[i];
      }
    }
    __syncthreads();
    prefix |= uint32_t(s_digit) << shift;
    pmask |= 255u << shift;
    kr -= s_above;
    __syncthreads();
  }

  // prefix is the k-th largest key; kr keys equal to it complete the answer
  const uint32_t T = prefix;
  int run_eq = 0, run_sel = 0;
  for (int base = 0; base < n && run_sel < k; base += kThreads) {
    const int i = base + tid;
    const bool in = i < n;
    const uint32_t key = in ? (cached ? s_keys[i] : order_key(lr[i])) : 0u;
    const bool gt = in && key > T;
    const bool eq = in && key == T;
    const uint64_t beq = __ballot(eq);
    if (lane == 0) s_cnt[wave][0] = __popcll(beq);
    __syncthreads();
    int eq_before = run_eq, eq_all = run_eq;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      const int t = s_cnt[w][0];
      if (w < wave) eq_before += t;
      eq_all += t;
    }
    const int tie_rank = eq_before + __popcll(beq & lanes_below());
    const bool sel = gt || (eq && tie_rank < kr);
    const uint64_t bsel = __ballot(sel);
    if (lane == 0) s_cnt[wave][1] = __popcll(bsel);
    __syncthreads();
    int sel_before = run_sel, sel_all = run_sel;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      const int t = s_cnt[w][1];
      if (w < wave) sel_before += t;
      sel_all += t;
    }
    const int pos = sel_before + __popcll(bsel & lanes_below());
    if (sel && pos < k) out[pos] = i;
    run_eq = eq_all;
    run_sel = sel_all;
    __syncthreads();
  }
}

}  // namespace

hipError_t launch_topk(const TopkArgs &a, int, hipStream_t stream) {
  const int cap = min(a.width, kMaxCache);
  const size_t lds = size_t(cap) * sizeof(uint32_t);
  static bool lds_raised = false;
  if (!lds_raised) {
    const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(&topk_kernel),
                                             hipFuncAttributeMaxDynamicSharedMemorySize,
                                             int(kMaxCache * sizeof(uint32_t)));
    if (e != hipSuccess) return e;
    lds_raised = true;
  }
  topk_kernel<<<dim3(a.rows), kThreads, lds, stream>>>(a, cap);
  return hipGetLastError();
}

}  // namespace idx
