// Contiguous fp8 indexer logits (a prefill chunk).
//
// I[t, s] = k_scale[s] * sum_h w[t, h] * max(q[t, h, :] . k[s, :], 0) on each row's
// [row_start, row_end), -inf elsewhere: page "vllm.v1.attention.ops.rocm_aiter_mla_sparse",
// fp8_mqa_logits_torch. k_scale > 0, so it is applied once per (t, s) after the head
// sum instead of once per head.
//
// Work split: a workgroup owns 8 query rows (two per wave) and one key split. Each
// wave keeps its rows' queries in registers as MFMA A operands (16 heads per tile,
// all 128 channels in one 16x16x128 fp8 MFMA), and the workgroup streams 64-key
// chunks of K through LDS, shared by its four waves. The epilogue turns each
// 16x16 (head, key) tile into ReLU * w partial sums, adds the four lane groups, and
// stores one coalesced 256-byte row segment per chunk. Columns of the split outside
// the rows' key range are filled with -inf without touching K. Row tiles are
// launched longest-first so a causal chunk's long rows do not trail the grid.
#include <climits>

#include "device.h"
#include "launch.h"

namespace idx {
namespace {

constexpr int kWaves = 4;
constexpr int kRowsPerWave = 2;
constexpr int kRowsPerWG = kWaves * kRowsPerWave;
constexpr int kChunk = 64;
constexpr int kKeyStride = 144;  // LDS bytes per key: 128 + 16 of padding against bank conflicts

// -inf into row[from, to); `from` is a multiple of 4 and the row is 16-byte aligned.
__device__ void fill_neg_inf(float *row, int from, int to, int lane) {
  const float ninf = neg_inf();
  for (int c = from + 4 * lane; c < to; c += 256) {
    if (c + 4 <= to) {
      *reinterpret_cast<v4f *>(row + c) = v4f{ninf, ninf, ninf, ninf};
    } else {
      for (int i = 0; i < 4 && c + i < to; ++i) row[c + i] = ninf;
    }
  }
}

template <int HT>
__global__ __launch_bounds__(256, 2) void mqa_logits_fp8_kernel(MqaArgs a, int split_keys) {
  __shared__ __attribute__((aligned(16))) uint8_t sk[kChunk * kKeyStride];
  __shared__ float ss[kChunk];
  __shared__ int s_range[2];

  const int tid = threadIdx.x;
  const int wave = uniform(tid >> 6);
  const int lane = tid & 63;
  const int g = lane >> 4;
  const int n = lane & 15;
  const int tile = int(gridDim.x) - 1 - int(blockIdx.x);
  const int row0 = tile * kRowsPerWG;
  const int s0 = int(blockIdx.y) * split_keys;
  const int s1 = min(a.N, s0 + split_keys);

  if (tid < 64) {
    int lo = INT_MAX, hi = INT_MIN;
    if (lane < kRowsPerWG && row0 + lane < a.M) {
      const int rl = max(a.row_start[row0 + lane], 0);
      const int rh = min(a.row_end[row0 + lane], a.N);
      if (rl < rh) {
        lo = rl;
        hi = rh;
      }
    }
    for (int off = 4; off > 0; off >>= 1) {
      lo = min(lo, __shfl_xor(lo, off));
      hi = max(hi, __shfl_xor(hi, off));
    }
    if (lane == 0) {
      s_range[0] = lo;
      s_range[1] = hi;
    }
  }
  __syncthreads();
  const int lo = max(s_range[0], s0);
  const int hi = min(s_range[1], s1);
  int c0 = s0, c_end = s0;
  if (lo < hi) {
    c0 = (lo / kChunk) * kChunk;
    c_end = min(((hi + kChunk - 1) / kChunk) * kChunk, s1);
  }

  // this wave's rows: queries as A operands, weights in the C-layout head order
  const int r_base = row0 + wave * kRowsPerWave;
  v8i qa[kRowsPerWave][HT];
  float wv[kRowsPerWave][HT][4];
  int rlo[kRowsPerWave], rhi[kRowsPerWave];
  bool active[kRowsPerWave];
#pragma unroll
  for (int rr = 0; rr < kRowsPerWave; ++rr) {
    const int r = r_base + rr;
    active[rr] = r < a.M;
    rlo[rr] = active[rr] ? a.row_start[r] : 0;
    rhi[rr] = active[rr] ? min(a.row_end[r], a.N) : 0;
#pragma unroll
    for (int ht = 0; ht < HT; ++ht) {
      const int h = ht * 16 + n;
      if (active[rr] && h < a.H) {
        const uint8_t *p = a.q + int64_t(r) * a.q_row_stride + h * 128 + g * 16;
        qa[rr][ht] = cat(load16(p), load16(p + 64));
      } else {
        qa[rr][ht] = zero8();
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int hh = ht * 16 + 4 * g + j;
        wv[rr][ht][j] = (active[rr] && hh < a.H) ? a.w[int64_t(r) * a.w_row_stride + hh] : 0.f;
      }
    }
    if (active[rr]) {
      float *orow = a.logits + int64_t(r) * a.logits_row_stride;
      fill_neg_inf(orow, s0, c0, lane);
      fill_neg_inf(orow, c_end, s1, lane);
    }
  }

  for (int c = c0; c < c_end; c += kChunk) {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int idx = tid + 256 * i;
      const int key = idx >> 3;
      const int part = idx & 7;
      v4i v = {0, 0, 0, 0};
      if (c + key < a.N) v = load16(a.k + int64_t(c + key) * a.k_row_stride + part * 16);
      *reinterpret_cast<v4i *>(sk + key * kKeyStride + part * 16) = v;
    }
    if (tid < kChunk) ss[tid] = (c + tid < a.N) ? a.k_scale[c + tid] : 0.f;
    __syncthreads();

    float part[kRowsPerWave][4];
#pragma unroll
    for (int kg = 0; kg < 4; ++kg) {
      const uint8_t *kp = sk + (kg * 16 + n) * kKeyStride + g * 16;
      const v8i kb = cat(*reinterpret_cast<const v4i *>(kp), *reinterpret_cast<const v4i *>(kp + 64));
#pragma unroll
      for (int rr = 0; rr < kRowsPerWave; ++rr) {
        float acc = 0.f;
#pragma unroll
        for (int ht = 0; ht < HT; ++ht) {
          const v4f s = mfma_fp8(qa[rr][ht], kb);
#pragma unroll
          for (int j = 0; j < 4; ++j) acc = fmaf(wv[rr][ht][j], relu(s[j]), acc);
        }
        part[rr][kg] = acc;
      }
    }
    float res[kRowsPerWave];
#pragma unroll
    for (int rr = 0; rr < kRowsPerWave; ++rr) res[rr] = transpose_reduce4(part[rr]);
    const int col = c + lane;
    const float sc = ss[lane];
#pragma unroll
    for (int rr = 0; rr < kRowsPerWave; ++rr) {
      if (active[rr] && col < c_end) {
        const int r = r_base + rr;
        a.logits[int64_t(r) * a.logits_row_stride + col] =
            (col >= rlo[rr] && col < rhi[rr]) ? res[rr] * sc : neg_inf();
      }
    }
    __syncthreads();
  }
}

}  // namespace

hipError_t launch_mqa_logits(const MqaArgs &a, int num_cus, hipStream_t stream) {
  const int tiles = (a.M + kRowsPerWG - 1) / kRowsPerWG;
  const int nchunks = (a.N + kChunk - 1) / kChunk;
  int splits = (4 * num_cus + tiles - 1) / tiles;
  splits = max(1, min(splits, nchunks));
  const int split_keys = ((nchunks + splits - 1) / splits) * kChunk;
  splits = (a.N + split_keys - 1) / split_keys;
  const dim3 grid(tiles, splits);
  const int ht = (a.H + 15) / 16;
  if (ht <= 1)
    mqa_logits_fp8_kernel<1><<<grid, 256, 0, stream>>>(a, split_keys);
  else if (ht <= 2)
    mqa_logits_fp8_kernel<2><<<grid, 256, 0, stream>>>(a, split_keys);
  else if (ht <= 4)
    mqa_logits_fp8_kernel<4><<<grid, 256, 0, stream>>>(a, split_keys);
  else
    mqa_logits_fp8_kernel<8><<<grid, 256, 0, stream>>>(a, split_keys);
  return hipGetLastError();
}

}  // namespace idx
