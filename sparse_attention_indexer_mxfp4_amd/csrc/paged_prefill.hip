// A prefill chunk of one sequence scored straight off its MXFP4 pages: M query rows,
// row r scoring keys [0, end_r) of the sequence through its block-table row, with no
// gather of K (page "vllm.v1.attention.ops.rocm_paged_mxfp4_indexer", module
// description and rocm_mxfp4_sparse_attn_indexer: prefill chunks read the paged cache
// in place). Every logit is the one the paged decode walk computes:
// I[r, s] = sum_h w[r, h] * max(sum_j 2^(eq - 127) 2^(ek - 127) q_hj . k_sj, 0).
//
// Unlike decode, many rows share each key, so the work is a dense contraction with a
// causal mask. A workgroup owns 8 query rows (two per wave, queries and their block
// scales held as MFMA A operands) and one key split, and streams the sequence's keys
// through two LDS buffers in 64-key chunks shared by its four waves. A chunk is four
// 16-key runs: wave w fetches run w of the chunk - its page from the block table
// (one scalar load: the run lies inside one page), then the run's kilobyte (lane L's
// 16 bytes at 16L, already in the scaled MFMA's B-operand order) and its 64 e8m0
// bytes (lane L's own block scale) - two chunks ahead of their scoring. Scoring runs
// the scaled fp4 MFMA (16 heads x 16 keys x 128 channels) with the MFMAs of key group
// kg+1 interleaved with the head sums of group kg, then the transposed permlane
// reduction that leaves key L of the chunk in lane L and one 256-byte store per row.
//
// The head sums use max(x, 0) = (x + |x|) / 2, as the contiguous fp8 kernel does:
// sum_h w_h |S_h| is one multiply-add per score (|x| is a source modifier, where the
// ReLU costs a second instruction), and sum_h w_h S_h = qt . k with
// qt[r, d] = sum_h w[r, h] 2^(eq[r, h, d/32] - 127) e2m1(q[r, h, d]). qt is built once
// per row in fp32, scaled by a power of two and split into four e4m3 parts (about 16
// significant bits together), and scored against the fp4 keys by one mixed-format
// MFMA per 16-key group (e4m3 A, e2m1 B with the keys' block scales) covering the
// 2 rows x 4 parts of a wave.
//
// Columns of the split past the rows' longest end are filled with -inf without
// touching K. Row tiles are launched longest-first (the causal chunk's last rows see
// the most keys).
#include <climits>

#include "debug.h"
#include "device.h"
#include "launch.h"

namespace idx {
namespace {

constexpr int kWaves = 4;
constexpr int kRowsPerWave = 2;
constexpr int kRowsPerWG = kWaves * kRowsPerWave;
constexpr int kChunk = 64;
constexpr int kDepth = 2;  // chunks requested ahead of the one being scored
constexpr int kQtStride = 144;  // LDS bytes per qt A-operand row (128 + 16 against bank conflicts)

// e4m3 A operand (rows: qt parts) times e2m1 B operand (keys) with the keys' block scales
__device__ __forceinline__ v4f mfma_qt_fp4(const v8i &a, const v8i &b, int scale_b) {
  const v4f zero = {0.f, 0.f, 0.f, 0.f};
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, zero, 0, 4, 0, 127, 0, scale_b);
}

template <int HT>
__global__ __launch_bounds__(256, 2) void paged_prefill_fp4_kernel(PagedArgs a, int split_keys) {
  __shared__ __attribute__((aligned(16))) uint8_t sk[2][kChunk * 64];  // run kg at kg * 1024, lane L at 16 L
  __shared__ uint8_t ss[2][kChunk * 4];                                // run kg's scale bytes at kg * 64 + L
  __shared__ __attribute__((aligned(16))) uint8_t sl[kWaves][16 * kQtStride];  // qt parts, A-operand rows
  __shared__ int s_hi;

  const int tid = threadIdx.x;
  const int wave = uniform(tid >> 6);
  const int lane = tid & 63;
  const int g = lane >> 4;
  const int n = lane & 15;
  const int M = a.B;
  const int P = a.page_size;
  const int cap = int(min(int64_t(a.width), int64_t(a.max_blocks) * P));
  const int tile = int(gridDim.x) - 1 - int(blockIdx.x);
  const int row0 = tile * kRowsPerWG;
  const int s0 = int(blockIdx.y) * split_keys;
  const int s1 = min(a.width, s0 + split_keys);

  if (tid < 64) {
    int hi = 0;
    if (lane < kRowsPerWG && row0 + lane < M) hi = min(max(a.context_lens[row0 + lane], 0), cap);
    IDX_DEBUG_NOTE(lane < kRowsPerWG && row0 + lane < M && hi != a.context_lens[row0 + lane], IDX_DBG_LENGTH);
    for (int off = 4; off > 0; off >>= 1) hi = max(hi, __shfl_xor(hi, off));
    if (lane == 0) s_hi = hi;
  }

  // ---- this wave's rows: queries and block scales as A operands, weights in the
  // C-layout head order (lane (g, n) holds heads 16 ht + 4 g + j of its C rows) --------
  const int r_base = row0 + wave * kRowsPerWave;
  v8i qa[kRowsPerWave][HT];
  int qs[kRowsPerWave][HT];
  float wv[kRowsPerWave][HT][4];
  int rend[kRowsPerWave];
  bool active[kRowsPerWave];
  float lscale[kRowsPerWave];  // 2^e of each row's qt split
#pragma unroll
  for (int rr = 0; rr < kRowsPerWave; ++rr) {
    const int r = r_base + rr;
    active[rr] = r < M;
    rend[rr] = active[rr] ? min(max(a.context_lens[r], 0), cap) : 0;
#pragma unroll
    for (int ht = 0; ht < HT; ++ht) {
      const int h = ht * 16 + n;
      if (active[rr] && h < a.H) {
        const v4i z = {0, 0, 0, 0};
        qa[rr][ht] = cat(load16(a.q + (int64_t(r) * a.H + h) * 64 + g * 16), z);
        qs[rr][ht] = (a.q_scale[int64_t(r) * a.H + h] >> (8 * g)) & 0xFF;
      } else {
        qa[rr][ht] = zero8();
        qs[rr][ht] = 127;
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int hh = ht * 16 + 4 * g + j;
        wv[rr][ht][j] = (active[rr] && hh < a.H) ? a.w[int64_t(r) * a.H + hh] : 0.f;
      }
    }

    // qt over channels [32 g, 32 g + 32): lane (g, n) holds head ht*16 + n's 32 values
    // of block g for every ht (byte b: values 2b and 2b + 1 in its low and high
    // nibble). Weight times block scale, values converted two per instruction, summed
    // over ht, then over the 16 head lanes by a reduce-scatter that leaves channels
    // 32 g + 2 n and 32 g + 2 n + 1 in lane n.
    float pq[32];
#pragma unroll
    for (int i = 0; i < 32; ++i) pq[i] = 0.f;
#pragma unroll
    for (int ht = 0; ht < HT; ++ht) {
      const int h = ht * 16 + n;
      const float wh = (active[rr] && h < a.H) ? a.w[int64_t(r) * a.H + h] : 0.f;
      // 2^(e - 127) for the e8m0 byte e (e = 0 is the subnormal 2^-127)
      const uint32_t e = uint32_t(qs[rr][ht]);
      const float ws = wh * (e > 0 ? __uint_as_float(e << 23) : __uint_as_float(0x00400000u));
#pragma unroll
      for (int wd = 0; wd < 4; ++wd) {
        const uint32_t word = uint32_t(qa[rr][ht][wd]);
        const v2f b0 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(word, 1.0f, 0);
        const v2f b1 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(word, 1.0f, 1);
        const v2f b2 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(word, 1.0f, 2);
        const v2f b3 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(word, 1.0f, 3);
        pq[8 * wd + 0] = fmaf(ws, b0[0], pq[8 * wd + 0]);
        pq[8 * wd + 1] = fmaf(ws, b0[1], pq[8 * wd + 1]);
        pq[8 * wd + 2] = fmaf(ws, b1[0], pq[8 * wd + 2]);
        pq[8 * wd + 3] = fmaf(ws, b1[1], pq[8 * wd + 3]);
        pq[8 * wd + 4] = fmaf(ws, b2[0], pq[8 * wd + 4]);
        pq[8 * wd + 5] = fmaf(ws, b2[1], pq[8 * wd + 5]);
        pq[8 * wd + 6] = fmaf(ws, b3[0], pq[8 * wd + 6]);
        pq[8 * wd + 7] = fmaf(ws, b3[1], pq[8 * wd + 7]);
      }
    }
    reduce_scatter_step<0x140, 16>(pq, n & 8);  // row_mirror: partner differs in bit 3
    reduce_scatter_step<0x141, 8>(pq, n & 4);   // row_half_mirror: bits 0..2
    reduce_scatter_step<0x1B, 4>(pq, n & 2);    // quad_perm [3,2,1,0]: bits 0, 1
    reduce_scatter_step<0xB1, 2>(pq, n & 1);    // quad_perm [1,0,3,2]: bit 0
    const float q0 = pq[0], q1 = pq[1];
    float m = fmaxf(fabsf(q0), fabsf(q1));
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) m = fmaxf(m, __shfl_xor(m, off));
    // power-of-two scale putting the row maximum in [128, 256)
    const int ex = m > 0.f ? max(int((__float_as_uint(m) >> 23) & 0xFFu) - 127, -119) : 0;
    const float inv = __uint_as_float(uint32_t(max(min(7 - ex + 127, 254), 1)) << 23);
    lscale[rr] = __uint_as_float(uint32_t(max(min(ex - 7 + 127, 254), 1)) << 23);
    float x0 = q0 * inv, x1 = q1 * inv;
    // each part is the round-to-nearest-even e4m3 value of what the previous parts
    // left; the remainder after subtracting it is exact in fp32
#pragma unroll
    for (int part = 0; part < 4; ++part) {
      const int ec = __builtin_amdgcn_cvt_pk_fp8_f32(x0, x1, 0, false);
      const v2f d = __builtin_amdgcn_cvt_pk_f32_fp8(ec, false);
      x0 -= d[0];
      x1 -= d[1];
      *reinterpret_cast<uint16_t *>(&sl[wave][(rr * 4 + part) * kQtStride + 32 * g + 2 * n]) = uint16_t(ec);
    }
  }
  // rows 8..15 of the qt operand tile stay zero
  for (int i = lane; i < 8 * kQtStride / 16; i += 64)
    *reinterpret_cast<v4i *>(&sl[wave][8 * kQtStride + 16 * i]) = v4i{0, 0, 0, 0};
  __syncthreads();
  // A operand of the qt MFMA: row m = 4 * (row in wave) + part. An e4m3 operand's lane
  // group g holds channels [16 g, 16 g + 16) and [64 + 16 g, 64 + 16 g + 16), paired in
  // that order with the e2m1 operand's channels [32 g, 32 g + 32) (measured on gfx950)
  v8i la;
  {
    const uint8_t *p = &sl[wave][n * kQtStride + 16 * g];
    la = cat(*reinterpret_cast<const v4i *>(p), *reinterpret_cast<const v4i *>(p + 64));
  }

  // chunks [s0, c_end) of the split reach some row of the tile; the rest is -inf
  const int hi = min(s_hi, s1);
  const int c_end = hi > s0 ? min(((hi + kChunk - 1) / kChunk) * kChunk, s1) : s0;
#pragma unroll
  for (int rr = 0; rr < kRowsPerWave; ++rr)
    if (active[rr]) fill_neg_inf(a.logits + int64_t(r_base + rr) * a.logits_row_stride, c_end, s1, lane);

  // wave w fetches run w of a chunk: the page of keys [c + 16 w, c + 16 w + 16) (inside
  // one page, since 16 divides the page size), then the run's values and scales; runs
  // at or past the tile's longest end are not read (zero values, unit scales)
  struct Fetch {
    v4i kv;
    int ks;
  };
  auto fetch = [&](Fetch &f, int c) {
    const int pos = c + 16 * wave;
    f.kv = v4i{0, 0, 0, 0};
    f.ks = 127;
    if (pos < hi) {
      const int pi = a.page_shift >= 0 ? pos >> a.page_shift : pos / P;
      const int e0 = a.page_shift >= 0 ? pos & (P - 1) : pos % P;
      const int page = min(max(a.block_table[pi], 0), a.num_pages - 1);
      IDX_DEBUG_NOTE(a.block_table[pi] != page, IDX_DBG_PAGE);
      const uint8_t *pb = a.base + int64_t(page) * a.page_stride;
      const int run = e0 >> 4;
      f.kv = load16(pb + run * 1024 + lane * 16);
      f.ks = pb[P * 64 + run * 64 + lane];
    }
  };
  auto stage = [&](const Fetch &f, int buf) {
    *reinterpret_cast<v4i *>(&sk[buf][wave * 1024 + lane * 16]) = f.kv;
    ss[buf][wave * 64 + lane] = uint8_t(f.ks);
  };

  // Scoring of one chunk as a fixed schedule: the MFMAs of key group kg+1 are issued
  // one at a time, each followed by the |S| multiply-adds of one (row, head tile) of
  // group kg; scheduling fences keep the compiler from regrouping them.
  auto score = [&](int c, int buf) {
    v8i kb[4];
    int ksb[4];
#pragma unroll
    for (int kg = 0; kg < 4; ++kg) {
      const v4i z = {0, 0, 0, 0};
      kb[kg] = cat(*reinterpret_cast<const v4i *>(&sk[buf][kg * 1024 + lane * 16]), z);
      ksb[kg] = ss[buf][kg * 64 + lane];
    }
    float part[kRowsPerWave][4];  // sum over this lane's heads of w * |S|, per key group
    float lin[4];                 // qt . k for row g of the wave (g < 2), before the 2^e scale
    v4f sv[2][kRowsPerWave][HT];
    v4f lv[2];
#pragma unroll
    for (int rr = 0; rr < kRowsPerWave; ++rr)
#pragma unroll
      for (int ht = 0; ht < HT; ++ht) sv[0][rr][ht] = mfma_fp4(qa[rr][ht], kb[0], qs[rr][ht], ksb[0]);
    lv[0] = mfma_qt_fp4(la, kb[0], ksb[0]);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int kg = 0; kg < 4; ++kg) {
      const int cur = kg & 1, nxt = cur ^ 1;
      float acc[kRowsPerWave];
#pragma unroll
      for (int rr = 0; rr < kRowsPerWave; ++rr) acc[rr] = 0.f;
#pragma unroll
      for (int u = 0; u < kRowsPerWave * HT; ++u) {
        const int rr = u % kRowsPerWave, ht = u / kRowsPerWave;
        if (kg < 3) sv[nxt][rr][ht] = mfma_fp4(qa[rr][ht], kb[kg + 1], qs[rr][ht], ksb[kg + 1]);
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[rr] = fmaf(wv[rr][ht][j], fabsf(sv[cur][rr][ht][j]), acc[rr]);
        pin(acc[rr]);  // computed here, not sunk towards its use
        __builtin_amdgcn_sched_barrier(0);
      }
      if (kg < 3) lv[nxt] = mfma_qt_fp4(la, kb[kg + 1], ksb[kg + 1]);
      const v4f l4 = lv[cur];
      lin[kg] = (l4[0] + l4[1]) + (l4[2] + l4[3]);
#pragma unroll
      for (int rr = 0; rr < kRowsPerWave; ++rr) part[rr][kg] = acc[rr];
      __builtin_amdgcn_sched_barrier(0);
    }
    // lane L: |S| sums for key L of each row; qt . k for key L of rows 0 and 1
    transpose4(lin);
    const int col = c + lane;
#pragma unroll
    for (int rr = 0; rr < kRowsPerWave; ++rr) {
      float val = (transpose_reduce4(part[rr]) + lin[rr] * lscale[rr]) * 0.5f;
      pin(val);  // a select below, not a branch around the arithmetic
      if (active[rr] && col < c_end)
        a.logits[int64_t(r_base + rr) * a.logits_row_stride + col] = col < rend[rr] ? val : neg_inf();
    }
  };

  Fetch f[kDepth];
  if (s0 < c_end) {
    fetch(f[0], s0);
    stage(f[0], 0);
#pragma unroll
    for (int u = 1; u < kDepth; ++u) fetch(f[u], s0 + u * kChunk);
  }
  __syncthreads();
  int buf = 0;
  for (int c = s0; c < c_end; c += kDepth * kChunk) {
#pragma unroll
    for (int u = 0; u < kDepth; ++u) {
      // buffer `buf` holds chunk cc; set u is free, set (u + 1) % kDepth holds cc + 64
      const int cc = c + u * kChunk;
      if (cc >= c_end) break;
      fetch(f[u], cc + kDepth * kChunk);
      score(cc, buf);
      stage(f[(u + 1) % kDepth], buf ^ 1);
      __syncthreads();
      buf ^= 1;
    }
  }
}

}  // namespace

hipError_t launch_paged_prefill_fp4(const PagedArgs &a, int num_cus, hipStream_t stream) {
  const int tiles = (a.B + kRowsPerWG - 1) / kRowsPerWG;
  const int nchunks = (a.width + kChunk - 1) / kChunk;
  int splits = (4 * num_cus + tiles - 1) / tiles;
  splits = max(1, min(splits, nchunks));
  const int split_keys = ((nchunks + splits - 1) / splits) * kChunk;
  splits = (a.width + split_keys - 1) / split_keys;
  const dim3 grid(tiles, splits);
  const int ht = (a.H + 15) / 16;
  if (ht <= 1)
    paged_prefill_fp4_kernel<1><<<grid, 256, 0, stream>>>(a, split_keys);
  else if (ht <= 2)
    paged_prefill_fp4_kernel<2><<<grid, 256, 0, stream>>>(a, split_keys);
  else
    paged_prefill_fp4_kernel<4><<<grid, 256, 0, stream>>>(a, split_keys);
  return hipGetLastError();
}

IDX_DEBUG_READER(debug_word_paged_prefill)

}  // namespace idx
