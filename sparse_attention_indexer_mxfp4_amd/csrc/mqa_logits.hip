// Contiguous fp8 indexer logits (a prefill chunk).
//
// I[t, s] = k_scale[s] * sum_h w[t, h] * max(q[t, h, :] . k[s, :], 0) on each row's
// [row_start, row_end), -inf elsewhere: page "vllm.v1.attention.ops.rocm_aiter_mla_sparse",
// fp8_mqa_logits_torch. k_scale > 0, so it is applied once per (t, s) after the head
// sum instead of once per head.
//
// The contraction runs on the fp8 matrix cores; what limits it on gfx950 is the
// per-element epilogue, because the VALU and the matrix core barely overlap: a ReLU
// plus a multiply-add per (t, h, s) costs as much time as the MFMA that produced it.
// The kernel therefore uses max(x, 0) = (x + |x|) / 2:
//
//   sum_h w_h max(S_h, 0) = 1/2 * ( sum_h w_h |S_h|  +  sum_h w_h S_h ).
//
// The first sum is one fused multiply-add per element (|x| is a free source
// modifier). The second is linear in the query: sum_h w_h S_h = qt . k with
// qt[t, :] = sum_h w[t, h] q[t, h, :], a single extra "head" per row. qt is computed
// once per row in fp32 and split into four e4m3 parts with a power-of-two row scale
// (qt ~= 2^-e (p1 + p2 + p3 + p4), each part the e4m3 rounding of what the previous
// ones left, about 16 significant bits together), so it too runs on the fp8 matrix
// cores: one MFMA per 16-key group covers the 2 rows x 4 parts of a wave.
//
// Work split: a workgroup owns 8 query rows (two per wave) and one key split. Each
// wave keeps its rows' queries in registers as MFMA A operands (16 heads per tile,
// all 128 channels in one 16x16x128 fp8 MFMA), and the workgroup streams 64-key
// chunks of K through two LDS buffers shared by its four waves (each chunk's
// global loads are issued two chunks ahead of its scoring). Within a chunk the MFMAs of
// 16-key group kg+1 are interleaved with the epilogue of group kg. Head sums go
// through a transposed permlane reduction that leaves key L of the chunk in lane L,
// and one coalesced 256-byte row segment per chunk is stored. Columns of the split
// outside the rows' key range are filled with -inf without touching K. Row tiles are
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
constexpr int kKeyStride = 144;  // LDS bytes per key / query row: 128 + 16 of padding against bank conflicts

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
  __shared__ __attribute__((aligned(16))) uint8_t sk[2][kChunk * kKeyStride];
  __shared__ float ss[2][kChunk];
  __shared__ __attribute__((aligned(16))) uint8_t sl[kWaves][16 * kKeyStride];  // qt parts, A-operand rows
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

  // ---- this wave's rows: queries as A operands, weights in the C-layout head order --
  const int r_base = row0 + wave * kRowsPerWave;
  v8i qa[kRowsPerWave][HT];
  float wv[kRowsPerWave][HT][4];
  int rlo[kRowsPerWave], rhi[kRowsPerWave];
  bool active[kRowsPerWave];
  float lscale[kRowsPerWave];  // 2^e of each row's qt split
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

    // qt[d] = sum_h w[h] q[h, d], from the query bytes already in registers: lane
    // (g, n) holds heads ht*16 + n of K-group g; sum its HT heads, then the 16 lanes of
    // its row with DPP rotations, and keep the two of group g's 32 channels this lane
    // writes out: i = 2n, 2n+1.
    float pq[32];
#pragma unroll
    for (int i = 0; i < 32; ++i) pq[i] = 0.f;
#pragma unroll
    for (int ht = 0; ht < HT; ++ht) {
      const int h = ht * 16 + n;
      const float wh = (active[rr] && h < a.H) ? a.w[int64_t(r) * a.w_row_stride + h] : 0.f;
#pragma unroll
      for (int i = 0; i < 32; ++i) pq[i] = fmaf(wh, dec_e4m3((uint32_t(qa[rr][ht][i >> 2]) >> (8 * (i & 3))) & 0xFFu), pq[i]);
    }
#pragma unroll
    for (int i = 0; i < 32; ++i) {
      float x = pq[i];
      x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x128, 0xF, 0xF, false));  // row_ror:8
      x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x124, 0xF, 0xF, false));  // row_ror:4
      x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x122, 0xF, 0xF, false));  // row_ror:2
      x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x121, 0xF, 0xF, false));  // row_ror:1
      pq[i] = x;
    }
    float q0 = pq[0], q1 = pq[1];
#pragma unroll
    for (int i = 2; i < 32; i += 2) {
      if (n == i / 2) {
        q0 = pq[i];
        q1 = pq[i + 1];
      }
    }
    // byte offset of channels 2n, 2n+1 of K-group g
    const int qoff = n < 8 ? 16 * g + 2 * n : 64 + 16 * g + 2 * (n - 8);
    float m = fmaxf(fabsf(q0), fabsf(q1));
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) m = fmaxf(m, __shfl_xor(m, off));
    // power-of-two scale putting the row maximum in [128, 256)
    const int ex = m > 0.f ? max(int((__float_as_uint(m) >> 23) & 0xFFu) - 127, -119) : 0;
    const float inv = __uint_as_float(uint32_t(max(min(7 - ex + 127, 254), 1)) << 23);
    lscale[rr] = __uint_as_float(uint32_t(max(min(ex - 7 + 127, 254), 1)) << 23);
    float x0 = q0 * inv, x1 = q1 * inv;
#pragma unroll
    for (int part = 0; part < 4; ++part) {
      const uint32_t e0 = enc_e4m3(x0), e1 = enc_e4m3(x1);
      x0 -= dec_e4m3(e0);
      x1 -= dec_e4m3(e1);
      *reinterpret_cast<uint16_t *>(&sl[wave][(rr * 4 + part) * kKeyStride + qoff]) = uint16_t(e0 | (e1 << 8));
    }
  }
  // rows 8..15 of the qt operand tile stay zero
  for (int i = lane; i < 8 * kKeyStride / 16; i += 64)
    *reinterpret_cast<v4i *>(&sl[wave][8 * kKeyStride + 16 * i]) = v4i{0, 0, 0, 0};
  __syncthreads();
  v8i la;  // A operand of the qt MFMA: row m = 4 * (row in wave) + part
  {
    const uint8_t *p = &sl[wave][n * kKeyStride + g * 16];
    la = cat(*reinterpret_cast<const v4i *>(p), *reinterpret_cast<const v4i *>(p + 64));
  }

  const int lo = max(s_range[0], s0);
  const int hi = min(s_range[1], s1);
  int c0 = s0, c_end = s0;
  if (lo < hi) {
    c0 = (lo / kChunk) * kChunk;
    c_end = min(((hi + kChunk - 1) / kChunk) * kChunk, s1);
  }
#pragma unroll
  for (int rr = 0; rr < kRowsPerWave; ++rr) {
    if (active[rr]) {
      float *orow = a.logits + int64_t(r_base + rr) * a.logits_row_stride;
      fill_neg_inf(orow, s0, c0, lane);
      fill_neg_inf(orow, c_end, s1, lane);
    }
  }

  // K chunks stream through two LDS buffers. The global loads of chunk i+2 are issued
  // while chunk i is scored and staged into LDS a whole iteration later, so a load has
  // two chunks of scoring to arrive in; one barrier per chunk hands a buffer over.
  struct Fetch {
    v4i kv[2];
    float ks;
  };
  auto fetch = [&](Fetch &f, int c) {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int idx = tid + 256 * i;
      const int key = idx >> 3, part = idx & 7;
      f.kv[i] = v4i{0, 0, 0, 0};
      if (c + key < a.N) f.kv[i] = load16(a.k + int64_t(c + key) * a.k_row_stride + part * 16);
    }
    f.ks = (tid < kChunk && c + tid < a.N) ? a.k_scale[c + tid] : 0.f;
  };
  auto stage = [&](const Fetch &f, int buf) {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int idx = tid + 256 * i;
      const int key = idx >> 3, part = idx & 7;
      *reinterpret_cast<v4i *>(&sk[buf][key * kKeyStride + part * 16]) = f.kv[i];
    }
    if (tid < kChunk) ss[buf][tid] = f.ks;
  };

  auto score = [&](int c, int buf) {
    v8i kb[4];
#pragma unroll
    for (int kg = 0; kg < 4; ++kg) {
      const uint8_t *kp = &sk[buf][(kg * 16 + n) * kKeyStride + g * 16];
      kb[kg] = cat(*reinterpret_cast<const v4i *>(kp), *reinterpret_cast<const v4i *>(kp + 64));
    }
    float part[kRowsPerWave][4];  // sum over this lane's 16 heads of w * |S|
    float lin[4];                 // qt . k for row g of the wave (g < 2), before the 2^e scale
    v4f sv[2][kRowsPerWave][HT];
    v4f lv[2];
#pragma unroll
    for (int rr = 0; rr < kRowsPerWave; ++rr)
#pragma unroll
      for (int ht = 0; ht < HT; ++ht) sv[0][rr][ht] = mfma_fp8(qa[rr][ht], kb[0]);
    lv[0] = mfma_fp8(la, kb[0]);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int kg = 0; kg < 4; ++kg) {
      if (kg < 3) {
#pragma unroll
        for (int rr = 0; rr < kRowsPerWave; ++rr)
#pragma unroll
          for (int ht = 0; ht < HT; ++ht) sv[(kg + 1) & 1][rr][ht] = mfma_fp8(qa[rr][ht], kb[kg + 1]);
        lv[(kg + 1) & 1] = mfma_fp8(la, kb[kg + 1]);
      }
#pragma unroll
      for (int rr = 0; rr < kRowsPerWave; ++rr) {
        float acc = 0.f;
#pragma unroll
        for (int ht = 0; ht < HT; ++ht)
#pragma unroll
          for (int j = 0; j < 4; ++j) acc = fmaf(wv[rr][ht][j], fabsf(sv[kg & 1][rr][ht][j]), acc);
        part[rr][kg] = acc;
      }
      const v4f l4 = lv[kg & 1];
      lin[kg] = (l4[0] + l4[1]) + (l4[2] + l4[3]);
      // within this fenced region no VALU op reads an MFMA issued in it: one MFMA,
      // then a run of VALU ops, repeated, keeps both units fed
      if (kg < 3) {
#pragma unroll
        for (int i = 0; i < kRowsPerWave * HT + 1; ++i) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x002, 4, 0);
        }
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    // lane L: |S| sums for key L of each row; qt . k for key L of rows 0 and 1
    transpose4(lin);
    const int col = c + lane;
    const float sc = 0.5f * ss[buf][lane];
#pragma unroll
    for (int rr = 0; rr < kRowsPerWave; ++rr) {
      const float val = (transpose_reduce4(part[rr]) + lin[rr] * lscale[rr]) * sc;
      if (active[rr] && col < c_end) {
        const int r = r_base + rr;
        a.logits[int64_t(r) * a.logits_row_stride + col] = (col >= rlo[rr] && col < rhi[rr]) ? val : neg_inf();
      }
    }
  };

  Fetch fa, fb;
  if (c0 < c_end) {
    fetch(fa, c0);
    stage(fa, 0);
    if (c0 + kChunk < c_end) fetch(fa, c0 + kChunk);
  }
  __syncthreads();
  // invariant at the top of a step: buffer `buf` holds chunk c, the loads of chunk
  // c + 64 are in flight in one Fetch set
  int buf = 0;
  for (int c = c0; c < c_end; c += 2 * kChunk) {
    // chunk c (in flight: c + 64 in fa)
    if (c + 2 * kChunk < c_end) fetch(fb, c + 2 * kChunk);
    score(c, buf);
    if (c + kChunk < c_end) stage(fa, buf ^ 1);
    __syncthreads();
    buf ^= 1;
    if (c + kChunk >= c_end) break;
    // chunk c + 64 (in flight: c + 128 in fb)
    if (c + 3 * kChunk < c_end) fetch(fa, c + 3 * kChunk);
    score(c + kChunk, buf);
    if (c + 2 * kChunk < c_end) stage(fb, buf ^ 1);
    __syncthreads();
    buf ^= 1;
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
