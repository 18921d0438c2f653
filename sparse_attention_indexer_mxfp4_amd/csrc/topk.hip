// Per-row top-k over [row_start, row_end): page
// "vllm.v1.attention.ops.rocm_paged_mxfp4_indexer", _topk (-1 pads rows shorter than k).
//
// One workgroup per row. Logits become order-preserving 32-bit keys (-0.0 folded onto
// +0.0). The row is read from global memory once: that pass keeps the keys in LDS
// (when the row fits) and builds a histogram of their top 11 bits. The bin holding
// the k-th largest key is found by a suffix scan over the 2048 bins; its keys - a
// small set for any continuous distribution - are compacted into an LDS candidate
// list, and two more radix digits (11 and 10 bits) over that list give the exact
// k-th largest key T and how many keys equal to T complete the answer. When the
// bin holds too many keys for the list (heavy ties), the two digits run over the
// whole row instead. A last pass in column order, several consecutive keys per thread
// and one workgroup scan per 4096 keys, emits every key above T and the lowest-column
// ties, so the k indices come out in ascending column order.
#include "device.h"
#include "launch.h"

namespace idx {
namespace {

constexpr int kMaxCache = 32768;  // keys kept in LDS (128 KiB)
constexpr int kBins = 2048;       // first digit: 11 bits
constexpr int kMaxCand = 2048;    // candidate list
constexpr int kUnroll = 16;       // loads in flight per thread in the first pass

__device__ __forceinline__ uint32_t order_key(float x) {
  uint32_t u = __float_as_uint(x);
  if (u == 0x80000000u) u = 0u;  // -0.0 ranks with +0.0
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ uint64_t lanes_below() {
  const int lane = threadIdx.x & 63;
  return lane == 0 ? 0ull : (~0ull >> (64 - lane));
}

template <int NT>
struct Smem {
  uint32_t hist[kBins];
  uint32_t cand[kMaxCand];
  int wsum[NT / 64];
  int sel_digit, sel_above, ncand;
};

// Exclusive prefix sum of v over the workgroup (thread order); *total gets the sum.
template <int NT>
__device__ int block_scan(int v, int *wsum, int *total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int x = v;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int y = __shfl_up(x, off);
    if (lane >= off) x += y;
  }
  __syncthreads();
  if (lane == 63) wsum[wave] = x;
  __syncthreads();
  int before = 0, all = 0;
#pragma unroll
  for (int w = 0; w < NT / 64; ++w) {
    const int t = wsum[w];
    if (w < wave) before += t;
    all += t;
  }
  *total = all;
  return before + x - v;
}

// Given counts per digit value in hist[0..nbins) (larger digit = larger key), find the
// digit d with (# above d) < kr <= (# at or above d); writes sel_digit / sel_above.
template <int NT>
__device__ void select_digit(Smem<NT> &sm, int nbins, int kr) {
  const int per = (nbins + NT - 1) / NT;  // bins per thread, walked from the top
  const int top = nbins - 1 - threadIdx.x * per;
  int local = 0;
  for (int i = 0; i < per; ++i) {
    const int d = top - i;
    if (d >= 0) local += int(sm.hist[d]);
  }
  int total;
  int run = block_scan<NT>(local, sm.wsum, &total);
  for (int i = 0; i < per; ++i) {
    const int d = top - i;
    if (d < 0) break;
    const int c = int(sm.hist[d]);
    if (run < kr && run + c >= kr) {
      sm.sel_digit = d;
      sm.sel_above = run;
    }
    run += c;
  }
  __syncthreads();
}

// Ordered emission: KPT consecutive keys per thread per round. Writes every key above
// T and the first kr keys equal to T, in column order, as out[pos] = column.
template <int NT, int KPT, typename KeyAt>
__device__ void emit(Smem<NT> &sm, KeyAt key_at, int n, int k, uint32_t T, int kr, int32_t *out) {
  int run_eq = 0, run_sel = 0;
  for (int base = 0; base < n && run_sel < k; base += KPT * NT) {
    const int i0 = base + KPT * threadIdx.x;
    uint32_t key[KPT];
    int gt = 0, eq = 0;
#pragma unroll
    for (int j = 0; j < KPT; ++j) {
      const bool in = i0 + j < n;
      key[j] = in ? key_at(i0 + j) : 0u;
      gt += int(in && key[j] > T);
      eq += int(in && key[j] == T);
    }
    // exclusive prefixes of (gt, eq) in thread order; a round counts at most
    // KPT * NT = 4096 keys, so each fits 16 bits
    int tot;
    const int pre = block_scan<NT>(gt | (eq << 16), sm.wsum, &tot);
    int eq_before = run_eq + (pre >> 16);
    int pos = run_sel + (pre & 0xFFFF) + min(max(kr - run_eq, 0), pre >> 16);
#pragma unroll
    for (int j = 0; j < KPT; ++j) {
      if (i0 + j < n) {
        bool sel = key[j] > T;
        if (key[j] == T) {
          sel = eq_before < kr;
          ++eq_before;
        }
        if (sel) {
          if (pos < k) out[pos] = i0 + j;
          ++pos;
        }
      }
    }
    const int tot_gt = tot & 0xFFFF, tot_eq = tot >> 16;
    run_sel += tot_gt + min(max(kr - run_eq, 0), tot_eq);
    run_eq += tot_eq;
  }
}

template <int NT>
__global__ __launch_bounds__(NT) void topk_kernel(TopkArgs a, int cache_cap) {
  extern __shared__ uint32_t s_keys[];  // cache_cap keys
  __shared__ Smem<NT> sm;

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
    for (int i = tid; i < k; i += NT) out[i] = i < n ? i : -1;
    return;
  }
  const float *lr = a.logits + int64_t(row) * a.logits_row_stride + start;
  const bool cached = n <= cache_cap;
  auto key_at = [&](int i) -> uint32_t { return cached ? s_keys[i] : order_key(lr[i]); };

  // ---- pass 1: read the row, cache it, histogram of the top 11 bits ------------------
  // kUnroll independent loads per thread are issued before any of them is used, so a
  // batch costs one memory round trip
  for (int i = tid; i < kBins; i += NT) sm.hist[i] = 0u;
  if (tid == 0) sm.ncand = 0;
  __syncthreads();
  for (int base = 0; base < n; base += kUnroll * NT) {
    float x[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int i = base + u * NT + tid;
      x[u] = i < n ? lr[i] : 0.f;
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int i = base + u * NT + tid;
      if (i < n) {
        const uint32_t key = order_key(x[u]);
        if (cached) s_keys[i] = key;
        atomicAdd(&sm.hist[key >> 21], 1u);
      }
    }
  }
  __syncthreads();
  select_digit<NT>(sm, kBins, k);
  const uint32_t d1 = uint32_t(sm.sel_digit);
  int kr = k - sm.sel_above;
  const int c1 = int(sm.hist[d1]);

  uint32_t T;  // the k-th largest key
  if (c1 == kr) {
    // the whole bin is selected: any key of the bin works as the cut, with all its
    // keys taken; use the bin's lowest key so "above T or tie" selects exactly it
    T = d1 << 21;
    kr = n;  // every key equal to T is taken (there are at most c1 of them)
    __syncthreads();
    // keys of bin d1 are >= T; "key > T" plus all ties == the whole bin
  } else {
    __syncthreads();
    const bool use_cand = c1 <= kMaxCand;
    if (use_cand) {
      for (int i = tid; i < n; i += NT) {
        const uint32_t key = key_at(i);
        if ((key >> 21) == d1) sm.cand[atomicAdd(&sm.ncand, 1)] = key;
      }
    }
    // digits 2 (bits 20..10) and 3 (bits 9..0)
    uint32_t prefix = d1 << 21, pmask = 0xFFE00000u;
#pragma unroll
    for (int dg = 0; dg < 2; ++dg) {
      const int shift = dg == 0 ? 10 : 0;
      const int nb = dg == 0 ? 2048 : 1024;
      for (int i = tid; i < kBins; i += NT) sm.hist[i] = 0u;
      __syncthreads();
      if (use_cand) {
        const int nc = sm.ncand;
        for (int i = tid; i < nc; i += NT) {
          const uint32_t key = sm.cand[i];
          if ((key & pmask) == prefix) atomicAdd(&sm.hist[(key >> shift) & uint32_t(nb - 1)], 1u);
        }
      } else {
        for (int i = tid; i < n; i += NT) {
          const uint32_t key = key_at(i);
          if ((key & pmask) == prefix) atomicAdd(&sm.hist[(key >> shift) & uint32_t(nb - 1)], 1u);
        }
      }
      __syncthreads();
      select_digit<NT>(sm, nb, kr);
      prefix |= uint32_t(sm.sel_digit) << shift;
      pmask |= uint32_t(nb - 1) << shift;
      kr -= sm.sel_above;
      __syncthreads();
    }
    T = prefix;
  }

  // ---- ordered emission ---------------------------------------------------------------
  if (cached)
    emit<NT, 4096 / NT>(sm, [&](int i) { return s_keys[i]; }, n, k, T, kr, out);
  else
    emit<NT, 4>(sm, [&](int i) { return order_key(lr[i]); }, n, k, T, kr, out);
}

}  // namespace

hipError_t launch_topk(const TopkArgs &a, int, hipStream_t stream) {
  const int cap = min(a.width, kMaxCache);
  const size_t lds = size_t(cap) * sizeof(uint32_t);
  static bool lds_raised = false;
  if (!lds_raised) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(&topk_kernel<1024>),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, int(kMaxCache * sizeof(uint32_t)));
    if (e != hipSuccess) return e;
    e = hipFuncSetAttribute(reinterpret_cast<const void *>(&topk_kernel<256>),
                            hipFuncAttributeMaxDynamicSharedMemorySize, int(kMaxCache * sizeof(uint32_t)));
    if (e != hipSuccess) return e;
    lds_raised = true;
  }
  // few rows: the widest workgroup per row; many rows: narrower ones, more per CU
  if (a.rows >= 1024)
    topk_kernel<256><<<dim3(a.rows), 256, lds, stream>>>(a, cap);
  else
    topk_kernel<1024><<<dim3(a.rows), 1024, lds, stream>>>(a, cap);
  return hipGetLastError();
}

}  // namespace idx
