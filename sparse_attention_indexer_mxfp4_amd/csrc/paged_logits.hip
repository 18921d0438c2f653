// Paged indexer logits for a decode / MTP step, over an fp8 or an MXFP4 K cache.
//
// Row r = b * next_n + j scores keys [0, end_r) of sequence b, where
// end_r = ctx_b - next_n + j + 1 (or context_lens[r] with per-row lengths), clamped
// to [0, min(width, max_blocks * page_size)]: page "vllm.v1.attention.ops.rocm_aiter_mla_sparse",
// rocm_fp8_paged_mqa_logits; page "vllm.v1.attention.ops.rocm_paged_mxfp4_indexer",
// rocm_mxfp4_sparse_attn_indexer. Every column of [0, width) is written.
//
// The step is HBM-bound: each key's bytes are read once for all next_n rows of its
// sequence and all heads. Work unit = one 64-key chunk of one sequence. Every
// workgroup first computes the prefix sum of chunks per sequence in LDS (from
// context_lens, on the device, so the grid never depends on lengths), then each
// wave takes an equal contiguous share of the concatenated chunk list, whatever
// the mix of lengths. Waves of workgroups on the same XCD get neighbouring shares,
// so a sequence's queries and block-table row stay in one L2. A wave holds its
// sequence's queries as MFMA A operands (16 heads x 128 channels per tile) and
// reads each 16-key group of a page straight into B operands:
//   fp8   lane L loads key L%16's bytes [16g, 16g+16) and [64+16g, 64+16g+16),
//         g = L/16, from the block-flat page (the query uses the same byte order);
//   MXFP4 lane L loads 16 bytes at run base + 16L - the run stores [chunk, key,
//         byte], so one wavefront load covers the run's kilobyte exactly and lands
//         in the scaled MFMA's operand order - plus the e8m0 byte at
//         scale base + 64 * run + L, which is that lane's own block scale.
// After the compute share, every wave writes an equal share of the -inf tail
// (columns past the last chunk of each row's sequence) with 16-byte stores.
#include "device.h"
#include "launch.h"

namespace idx {
namespace {

constexpr int kThreads = 256;
constexpr int kChunk = 64;

struct SeqRows {
  int end[4];
  int len;
};

template <int NR>
__device__ __forceinline__ SeqRows seq_rows(const PagedArgs &a, int b, int cap) {
  SeqRows s;
  s.len = 0;
#pragma unroll
  for (int j = 0; j < NR; ++j) {
    int e = a.ctx_per_row ? a.context_lens[b * NR + j] : a.context_lens[b] - NR + j + 1;
    e = min(max(e, 0), cap);
    s.end[j] = e;
    s.len = max(s.len, e);
  }
  return s;
}

// Exclusive prefix sum of per-thread values over the workgroup; returns the
// thread's offset and stores the total in *total.
__device__ int block_exclusive_scan(int v, int *scratch, int *total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int x = v;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int y = __shfl_up(x, off);
    if (lane >= off) x += y;
  }
  if (lane == 63) scratch[wave] = x;
  __syncthreads();
  int before = 0, all = 0;
#pragma unroll
  for (int w = 0; w < kThreads / 64; ++w) {
    const int t = scratch[w];
    if (w < wave) before += t;
    all += t;
  }
  *total = all;
  return before + x - v;
}

template <int FMT, int HT, int NR>
__global__ __launch_bounds__(kThreads) void paged_logits_kernel(PagedArgs a) {
  extern __shared__ int s_pref[];  // B + 1 chunk offsets
  __shared__ int s_scan[kThreads / 64];

  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int g = lane >> 4;
  const int n = lane & 15;
  const int P = a.page_size;
  const int cap = int(min(int64_t(a.width), int64_t(a.max_blocks) * P));

  // ---- chunk counts per sequence and their prefix sum (LDS) -------------------
  const int per = (a.B + kThreads - 1) / kThreads;
  const int b_lo = min(a.B, tid * per), b_hi = min(a.B, b_lo + per);
  int mine = 0;
  for (int b = b_lo; b < b_hi; ++b) mine += (seq_rows<NR>(a, b, cap).len + kChunk - 1) / kChunk;
  int total = 0;
  int run = block_exclusive_scan(mine, s_scan, &total);
  for (int b = b_lo; b < b_hi; ++b) {
    s_pref[b] = run;
    run += (seq_rows<NR>(a, b, cap).len + kChunk - 1) / kChunk;
  }
  if (tid == 0) s_pref[a.B] = total;
  if (blockIdx.x == 0 && a.row_end_out) {
    for (int r = tid; r < a.B * NR; r += kThreads) a.row_end_out[r] = seq_rows<NR>(a, r / NR, cap).end[r % NR];
  }
  __syncthreads();

  // ---- this wave's share of the chunk list -------------------------------------
  const int nwg = gridDim.x;  // a multiple of 8 (one slice per XCD)
  const int logical = (blockIdx.x % 8) * (nwg / 8) + blockIdx.x / 8;
  const int64_t V = int64_t(nwg) * (kThreads / 64);
  const int64_t v = int64_t(logical) * (kThreads / 64) + wave;
  const int64_t U = total;
  const int u0 = int(U * v / V), u1 = int(U * (v + 1) / V);

  int b = -1, b_next = 0;
  SeqRows rows;
  v8i qa[NR][HT];
  float wv[NR][HT][4];
  int qs[NR][HT];
  const int32_t *bt_row = a.block_table;

  for (int u = u0; u < u1; ++u) {
    if (u >= b_next) {
      // largest b with s_pref[b] <= u; s_pref[B] = total > u bounds it to [0, B)
      int lo = 0, hi = a.B;
      while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (s_pref[mid] <= u) lo = mid; else hi = mid;
      }
      b = lo;
      b_next = s_pref[b + 1];
      rows = seq_rows<NR>(a, b, cap);
      bt_row = a.block_table + int64_t(b) * a.block_table_stride;
#pragma unroll
      for (int j = 0; j < NR; ++j) {
        const int64_t r = int64_t(b) * NR + j;
#pragma unroll
        for (int ht = 0; ht < HT; ++ht) {
          const int h = ht * 16 + n;
          if (h < a.H) {
            if (FMT == 0) {
              const uint8_t *p = a.q + (r * a.H + h) * 128 + g * 16;
              qa[j][ht] = cat(load16(p), load16(p + 64));
              qs[j][ht] = 0;
            } else {
              const uint8_t *p = a.q + (r * a.H + h) * 64 + g * 16;
              const v4i z = {0, 0, 0, 0};
              qa[j][ht] = cat(load16(p), z);
              qs[j][ht] = (a.q_scale[r * a.H + h] >> (8 * g)) & 0xFF;
            }
          } else {
            qa[j][ht] = zero8();
            qs[j][ht] = 127;
          }
#pragma unroll
          for (int jj = 0; jj < 4; ++jj) {
            const int hh = ht * 16 + 4 * g + jj;
            wv[j][ht][jj] = hh < a.H ? a.w[r * a.H + hh] : 0.f;
          }
        }
      }
    }

    const int key0 = (u - s_pref[b]) * kChunk;
    v8i kb[4];
    int ksb[4];
    float ksc = 0.f;
    const uint8_t *scale_ptr = nullptr;
#pragma unroll
    for (int kg = 0; kg < 4; ++kg) {
      const int s = key0 + kg * 16;  // first key of the group; 16 | P keeps the group in one page
      kb[kg] = zero8();
      ksb[kg] = 127;
      if (s < rows.len) {
        int page = bt_row[s / P];
        page = min(max(page, 0), a.num_pages - 1);
        const uint8_t *pb = a.base + int64_t(page) * a.page_stride;
        const int e0 = s % P;
        if (FMT == 0) {
          const uint8_t *p = pb + (e0 + n) * 128 + g * 16;
          kb[kg] = cat(load16(p), load16(p + 64));
          if (g == kg) scale_ptr = pb + P * 128 + 4 * (e0 + n);
        } else {
          const int run_i = e0 >> 4;
          const v4i z = {0, 0, 0, 0};
          kb[kg] = cat(load16(pb + run_i * 1024 + lane * 16), z);
          ksb[kg] = pb[P * 64 + run_i * 64 + lane];
        }
      }
    }
    if (FMT == 0 && scale_ptr) ksc = *reinterpret_cast<const float *>(scale_ptr);

    float res[NR];
#pragma unroll
    for (int j = 0; j < NR; ++j) res[j] = 0.f;
#pragma unroll
    for (int kg = 0; kg < 4; ++kg) {
#pragma unroll
      for (int j = 0; j < NR; ++j) {
        float acc = 0.f;
#pragma unroll
        for (int ht = 0; ht < HT; ++ht) {
          const v4f s = FMT == 0 ? mfma_fp8(qa[j][ht], kb[kg]) : mfma_fp4(qa[j][ht], kb[kg], qs[j][ht], ksb[kg]);
#pragma unroll
          for (int jj = 0; jj < 4; ++jj) acc = fmaf(wv[j][ht][jj], fmaxf(s[jj], 0.f), acc);
        }
        acc = sum_row_groups(acc);
        if (g == kg) res[j] = acc;
      }
    }
    const int col = key0 + lane;
    if (col < a.width) {
#pragma unroll
      for (int j = 0; j < NR; ++j) {
        const int64_t r = int64_t(b) * NR + j;
        const float val = FMT == 0 ? res[j] * ksc : res[j];
        a.logits[r * a.logits_row_stride + col] = col < rows.end[j] ? val : neg_inf();
      }
    }
  }

  // ---- -inf past each sequence's last chunk -------------------------------------
  const int NU = (a.width + 255) / 256;
  const int64_t R = int64_t(a.B) * NR;
  const float ninf = neg_inf();
  for (int64_t f = v; f < R * NU; f += V) {
    const int64_t r = f / NU;
    const int col = int(f % NU) * 256 + lane * 4;
    const int bb = int(r / NR);
    const int tail = (s_pref[bb + 1] - s_pref[bb]) * kChunk;
    if (col >= tail && col < a.width) {
      float *p = a.logits + r * a.logits_row_stride + col;
      if (col + 4 <= a.width) {
        *reinterpret_cast<v4f *>(p) = v4f{ninf, ninf, ninf, ninf};
      } else {
        for (int i = 0; col + i < a.width; ++i) p[i] = ninf;
      }
    }
  }
}

template <int FMT, int HT>
hipError_t launch_nr(const PagedArgs &a, dim3 grid, size_t lds, hipStream_t stream) {
  switch (a.next_n) {
    case 1: paged_logits_kernel<FMT, HT, 1><<<grid, kThreads, lds, stream>>>(a); break;
    case 2: paged_logits_kernel<FMT, HT, 2><<<grid, kThreads, lds, stream>>>(a); break;
    case 3: paged_logits_kernel<FMT, HT, 3><<<grid, kThreads, lds, stream>>>(a); break;
    default: paged_logits_kernel<FMT, HT, 4><<<grid, kThreads, lds, stream>>>(a); break;
  }
  return hipGetLastError();
}

template <int FMT>
hipError_t launch_fmt(const PagedArgs &a, dim3 grid, size_t lds, hipStream_t stream) {
  const int ht = (a.H + 15) / 16;
  if (ht <= 1) return launch_nr<FMT, 1>(a, grid, lds, stream);
  if (ht <= 2) return launch_nr<FMT, 2>(a, grid, lds, stream);
  if (ht <= 4) return launch_nr<FMT, 4>(a, grid, lds, stream);
  return launch_nr<FMT, 8>(a, grid, lds, stream);
}

}  // namespace

hipError_t launch_paged_logits(const PagedArgs &a, int num_cus, hipStream_t stream) {
  const int nwg = ((2 * num_cus + 7) / 8) * 8;
  const size_t lds = size_t(a.B + 1) * sizeof(int);
  const dim3 grid(nwg);
  return a.fmt == 0 ? launch_fmt<0>(a, grid, lds, stream) : launch_fmt<1>(a, grid, lds, stream);
}

}  // namespace idx
