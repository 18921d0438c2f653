// Contiguous fp8 indexer logits (a prefill chunk).
//
// I[t, s] = k_scale[s] * sum_h w[t, h] * max(q[t, h, :] . k[s, :], 0) on each row's
// [row_start, row_end), -inf elsewhere: page "vllm.v1.attention.ops.rocm_aiter_mla_sparse",
// fp8_mqa_logits_torch. k_scale > 0, so it is applied once per (t, s) after the head
// sum instead of once per head.
//
// The contraction runs on the fp8 matrix cores; the per-element epilogue competes
// with them for instruction issue: about four vector multiply-adds fit beside each
// 16x16x128 MFMA (which occupies the issue port for roughly half of its 32 cycles),
// while a ReLU plus a multiply-add per (t, h, s) would need eight.
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
// Work split: a workgroup owns 8 query rows (two per wave; 4 rows, one per wave, with
// more than 64 heads) and one key split. Each
// wave keeps its rows' queries in registers as MFMA A operands (16 heads per tile,
// all 128 channels in one 16x16x128 fp8 MFMA), and the workgroup streams K through
// two LDS buffers shared by its four waves in stages of two 64-key chunks (a stage's
// global loads are issued two stages ahead of its scoring; one barrier per stage,
// which measured 2% faster than a stage per chunk). Within a chunk the MFMAs of
// 16-key group kg+1 are interleaved with the epilogue of group kg. Head sums go
// through a transposed permlane reduction that leaves key L of the chunk in lane L,
// and one coalesced 256-byte row segment per chunk is stored. Columns of the split
// outside the rows' key range are filled with -inf without touching K. Row tiles are
// launched longest-first so a causal chunk's long rows do not trail the grid.
//
// The same kernel scores a prefill chunk straight off an fp8 paged cache (PAGED): a
// chunk's keys are then read from the pages the sequence's block table names, with
// the same LDS staging and epilogue.
#include <climits>

#include "debug.h"
#include "device.h"
#include "launch.h"

namespace idx {
namespace {

constexpr int kWaves = 4;
// query rows per wave: two, or one with 128 heads (eight head tiles of queries,
// weights and scores for two rows do not fit a wave's 256 registers)
constexpr int rows_per_wave(int ht) { return ht > 4 ? 1 : 2; }
constexpr int kChunk = 64;   // keys scored at once: key L of a chunk ends in lane L
constexpr int kSub = 2;      // chunks per LDS stage (one barrier per stage)
constexpr int kStage = kChunk * kSub;
constexpr int kDepth = 2;  // K stages requested ahead of the one being scored
constexpr int kKeyStride = 160;  // LDS bytes per key / query row: 128 + 32 of padding (rocprofv3
                                  // counts no LDS bank conflicts at 160, 8.5 M cycles at 144, 176
                                  // or 208 and 25 M at 128 per 8192x8192 chunk)

template <int HT, bool PAGED>
__global__ __launch_bounds__(256, 2) void mqa_logits_fp8_kernel(MqaArgs a, int split_keys) {
  constexpr int kRowsPerWave = rows_per_wave(HT);
  constexpr int kRowsPerWG = kWaves * kRowsPerWave;
  __shared__ __attribute__((aligned(16))) uint8_t sk[2][kStage * kKeyStride];
  __shared__ float ss[2][kStage];
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
  const int klim = PAGED ? a.key_limit : a.N;  // keys that exist

  if (tid < 64) {
    int lo = INT_MAX, hi = INT_MIN;
    if (lane < kRowsPerWG && row0 + lane < a.M) {
      const int rl = a.row_start ? max(a.row_start[row0 + lane], 0) : 0;
      const int rh = min(a.row_end[row0 + lane], klim);
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
    rlo[rr] = active[rr] && a.row_start ? a.row_start[r] : 0;
    rhi[rr] = active[rr] ? min(a.row_end[r], klim) : 0;
    IDX_DEBUG_NOTE(active[rr] && (rlo[rr] < 0 || a.row_end[r] < 0 || a.row_end[r] > klim), IDX_DBG_LENGTH);
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
    // (g, n) holds head ht*16 + n's 32 channels of K-group g for every ht. Convert them
    // two per instruction, accumulate over ht, then sum over the 16 head lanes with a
    // reduce-scatter that leaves channels 2n, 2n+1 of the group in lane n.
    float pq[32];
#pragma unroll
    for (int i = 0; i < 32; ++i) pq[i] = 0.f;
#pragma unroll
    for (int ht = 0; ht < HT; ++ht) {
      const int h = ht * 16 + n;
      const float wh = (active[rr] && h < a.H) ? a.w[int64_t(r) * a.w_row_stride + h] : 0.f;
#pragma unroll
      for (int wd = 0; wd < 8; ++wd) {
        const v2f lo = __builtin_amdgcn_cvt_pk_f32_fp8(qa[rr][ht][wd], false);
        const v2f hi = __builtin_amdgcn_cvt_pk_f32_fp8(qa[rr][ht][wd], true);
        pq[4 * wd + 0] = fmaf(wh, lo[0], pq[4 * wd + 0]);
        pq[4 * wd + 1] = fmaf(wh, lo[1], pq[4 * wd + 1]);
        pq[4 * wd + 2] = fmaf(wh, hi[0], pq[4 * wd + 2]);
        pq[4 * wd + 3] = fmaf(wh, hi[1], pq[4 * wd + 3]);
      }
    }
    reduce_scatter_step<0x140, 16>(pq, n & 8);  // row_mirror: partner differs in bit 3
    reduce_scatter_step<0x141, 8>(pq, n & 4);   // row_half_mirror: bits 0..2
    reduce_scatter_step<0x1B, 4>(pq, n & 2);    // quad_perm [3,2,1,0]: bits 0, 1
    reduce_scatter_step<0xB1, 2>(pq, n & 1);    // quad_perm [1,0,3,2]: bit 0
    const float q0 = pq[0], q1 = pq[1];
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
    // |x| < 256 after the scaling, inside the e4m3 range: each part is the
    // round-to-nearest-even e4m3 value of what the previous parts left, and the
    // remainder after subtracting it is exact in fp32
#pragma unroll
    for (int part = 0; part < 4; ++part) {
      const int e = __builtin_amdgcn_cvt_pk_fp8_f32(x0, x1, 0, false);
      const v2f d = __builtin_amdgcn_cvt_pk_f32_fp8(e, false);
      x0 -= d[0];
      x1 -= d[1];
      *reinterpret_cast<uint16_t *>(&sl[wave][(rr * 4 + part) * kKeyStride + qoff]) = uint16_t(e);
    }
  }
  // the qt operand tile's rows past the wave's row parts stay zero
  for (int i = lane; i < (16 - 4 * kRowsPerWave) * kKeyStride / 16; i += 64)
    *reinterpret_cast<v4i *>(&sl[wave][4 * kRowsPerWave * kKeyStride + 16 * i]) = v4i{0, 0, 0, 0};
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

  // K stages stream through two LDS buffers, fed from kDepth sets of registers: the
  // global loads of stage i+kDepth are issued while stage i is scored and staged after
  // stage i+kDepth-1 is scored, so a load has kDepth stages of scoring to arrive in;
  // one barrier per stage hands a buffer over.
  // Loads and stores are buffer operations with hardware range checks (keys past N
  // read as zero, columns past the WG's range or rows past M are dropped), so the
  // loop has no data-dependent branches and the memory counter waits at the staging
  // step cover only the chunk being staged.
  constexpr int kLoads = kStage * 128 / (256 * 16);  // 16-byte loads per thread and stage
  struct Fetch {
    v4i kv[kLoads];
    float ks;
  };
  // Paged keys: the pages of the four 16-key groups of a chunk (each group inside one
  // page) are read one fetch ahead with one vector load (lane j: group j % 4) and
  // picked out with readlane, so a fetch never waits on its own block-table lookup;
  // the load sits ahead of the chunk's K loads in the memory counter's order.
  // The entry is kept raw (clamped to the pool where it is used) so that nothing waits
  // on it here; positions past the keys read the last valid entry, which is not used.
  int pg_next = 0;
  auto load_pages = [&](int c) {
    const int pos = min(c + 16 * (lane & (kStage / 16 - 1)), klim - 1);
    pg_next = a.block_table[a.page_shift >= 0 ? pos >> a.page_shift : pos / a.page_size];
  };
  auto fetch = [&](Fetch &f, int c) {
    if constexpr (PAGED) {
      // lane j: the page of group j (a select chain over per-group copies was turned
      // into a private array in scratch memory, read back for every load)
      const int pgv = min(max(pg_next, 0), a.num_pages - 1);
      IDX_DEBUG_NOTE(c + 16 * (lane & (kStage / 16 - 1)) < hi && pgv != pg_next, IDX_DBG_PAGE);
      load_pages(c + kStage);
      auto within = [&](int pos) { return a.page_shift >= 0 ? pos & (a.page_size - 1) : pos % a.page_size; };
      // a wave's 16-byte pieces of load i all lie in one 16-key group, so one page: a
      // range-checked buffer load over that page's values, keys past the end out of range
#pragma unroll
      for (int i = 0; i < kLoads; ++i) {
        const int idx = tid + 256 * i;
        const int key = idx >> 3, part = idx & 7;
        const int pos = c + key;
        const int grp = uniform(key >> 4);
        const int page = __builtin_amdgcn_readlane(pgv, grp);
        const buffer_rsrc pr = make_rsrc(a.kbase + int64_t(page) * a.page_stride, uint32_t(a.page_size) * 128u);
        f.kv[i] = buffer_load16(pr, pos < klim ? uint32_t(within(pos) * 128 + part * 16) : 0xFFFFFFF0u);
      }
      const int key = tid & (kStage - 1), pos = c + key;
      const int kpage = __builtin_amdgcn_ds_bpermute((key >> 4) << 2, pgv);  // lane key/16's page
      f.ks = 0.f;
      if (pos < klim)
        f.ks = *reinterpret_cast<const float *>(a.kbase + int64_t(kpage) * a.page_stride + a.page_size * 128 +
                                                within(pos) * 4);
    } else {
      const int64_t left = max(int64_t(a.N) - c, int64_t(0));
      const buffer_rsrc kr = make_rsrc(a.k + int64_t(c) * a.k_row_stride, range_bytes(left * a.k_row_stride));
      const buffer_rsrc sr = make_rsrc(a.k_scale + c, range_bytes(left * 4));
#pragma unroll
      for (int i = 0; i < kLoads; ++i) {
        const int idx = tid + 256 * i;
        const int key = idx >> 3, part = idx & 7;
        f.kv[i] = buffer_load16(kr, uint32_t(key * a.k_row_stride + part * 16));
      }
      f.ks = buffer_load_f32(sr, uint32_t((tid & (kStage - 1)) * 4));
    }
  };
  auto stage = [&](const Fetch &f, int buf) {
#pragma unroll
    for (int i = 0; i < kLoads; ++i) {
      const int idx = tid + 256 * i;
      const int key = idx >> 3, part = idx & 7;
      *reinterpret_cast<v4i *>(&sk[buf][key * kKeyStride + part * 16]) = f.kv[i];
    }
    if (tid < kStage) ss[buf][tid] = f.ks;
  };

  // one store range per row: [0, c_end) of the row for rows that exist, nothing else
  buffer_rsrc orow[kRowsPerWave];
#pragma unroll
  for (int rr = 0; rr < kRowsPerWave; ++rr)
    orow[rr] = make_rsrc(a.logits + int64_t(active[rr] ? r_base + rr : 0) * a.logits_row_stride,
                         active[rr] ? uint32_t(c_end) * 4u : 0u);

  // Scoring of one chunk as a fixed schedule: the MFMAs of key group kg+1 are issued
  // one at a time, each followed by the |S| multiply-adds of one (row, head tile) of
  // group kg, whose MFMA was issued a whole group earlier. Scheduling fences keep the
  // compiler from regrouping them, so the matrix core always has work queued while the
  // VALU runs.
  auto score = [&](int c, int buf, int sub) {
    v8i kb[4];
#pragma unroll
    for (int kg = 0; kg < 4; ++kg) {
      const uint8_t *kp = &sk[buf][(sub * kChunk + kg * 16 + n) * kKeyStride + g * 16];
      kb[kg] = cat(*reinterpret_cast<const v4i *>(kp), *reinterpret_cast<const v4i *>(kp + 64));
    }
    float part[kRowsPerWave][4];  // sum over this lane's heads of w * |S|, per key group
    float lin[4];                 // qt . k for row g of the wave (g < rows per wave), before the 2^e scale
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
      const int cur = kg & 1, nxt = cur ^ 1;
      float acc[kRowsPerWave];
#pragma unroll
      for (int rr = 0; rr < kRowsPerWave; ++rr) acc[rr] = 0.f;
#pragma unroll
      for (int u = 0; u < kRowsPerWave * HT; ++u) {
        const int rr = u % kRowsPerWave, ht = u / kRowsPerWave;
        if (kg < 3) sv[nxt][rr][ht] = mfma_fp8(qa[rr][ht], kb[(kg + 1) & 3]);
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[rr] = fmaf(wv[rr][ht][j], fabsf(sv[cur][rr][ht][j]), acc[rr]);
        pin(acc[rr]);  // computed here, not sunk towards its use
        __builtin_amdgcn_sched_barrier(0);
      }
      if (kg < 3) lv[nxt] = mfma_fp8(la, kb[(kg + 1) & 3]);
      const v4f l4 = lv[cur];
      lin[kg] = (l4[0] + l4[1]) + (l4[2] + l4[3]);
#pragma unroll
      for (int rr = 0; rr < kRowsPerWave; ++rr) part[rr][kg] = acc[rr];
      __builtin_amdgcn_sched_barrier(0);
    }
    // lane L: |S| sums for key L of each row; qt . k for key L of each row
    transpose4(lin);
    const int col = c + lane;
    const float sc = 0.5f * ss[buf][sub * kChunk + lane];
#pragma unroll
    for (int rr = 0; rr < kRowsPerWave; ++rr) {
      float val = (transpose_reduce4(part[rr]) + lin[rr] * lscale[rr]) * sc;
      pin(val);  // a select below, not a branch around the arithmetic
      const float out = (col >= rlo[rr] && col < rhi[rr]) ? val : neg_inf();
      buffer_store_f32_nt(out, orow[rr], uint32_t(col) * 4u);
    }
  };

  Fetch f[kDepth];
  if (c0 < c_end) {
    if constexpr (PAGED) load_pages(c0);
    fetch(f[0], c0);
    stage(f[0], 0);
#pragma unroll
    for (int u = 1; u < kDepth; ++u) fetch(f[u], c0 + u * kStage);
  }
  __syncthreads();
  int buf = 0;
  for (int c = c0; c < c_end; c += kDepth * kStage) {
#pragma unroll
    for (int u = 0; u < kDepth; ++u) {
      // buffer `buf` holds stage cc; set u is free, set (u + 1) % kDepth holds the next
      const int cc = c + u * kStage;
      if (cc >= c_end) break;
      fetch(f[u], cc + kDepth * kStage);
#pragma unroll
      for (int sub = 0; sub < kSub; ++sub)
        if (cc + sub * kChunk < c_end) score(cc + sub * kChunk, buf, sub);
      stage(f[(u + 1) % kDepth], buf ^ 1);
      __syncthreads();
      buf ^= 1;
    }
  }
}

}  // namespace

hipError_t launch_mqa_logits(const MqaArgs &a, int num_cus, hipStream_t stream) {
  const int ht = (a.H + 15) / 16;
  const int rows_wg = kWaves * rows_per_wave(ht <= 4 ? 4 : 8);
  const int tiles = (a.M + rows_wg - 1) / rows_wg;
  const int nchunks = (a.N + kChunk - 1) / kChunk;
  int splits = (4 * num_cus + tiles - 1) / tiles;
  splits = max(1, min(splits, nchunks));
  const int split_keys = ((nchunks + splits - 1) / splits) * kChunk;
  splits = (a.N + split_keys - 1) / split_keys;
  const dim3 grid(tiles, splits);
  if (a.paged) {
    if (ht <= 1)
      mqa_logits_fp8_kernel<1, true><<<grid, 256, 0, stream>>>(a, split_keys);
    else if (ht <= 2)
      mqa_logits_fp8_kernel<2, true><<<grid, 256, 0, stream>>>(a, split_keys);
    else if (ht <= 4)
      mqa_logits_fp8_kernel<4, true><<<grid, 256, 0, stream>>>(a, split_keys);
    else
      mqa_logits_fp8_kernel<8, true><<<grid, 256, 0, stream>>>(a, split_keys);
  } else {
    if (ht <= 1)
      mqa_logits_fp8_kernel<1, false><<<grid, 256, 0, stream>>>(a, split_keys);
    else if (ht <= 2)
      mqa_logits_fp8_kernel<2, false><<<grid, 256, 0, stream>>>(a, split_keys);
    else if (ht <= 4)
      mqa_logits_fp8_kernel<4, false><<<grid, 256, 0, stream>>>(a, split_keys);
    else
      mqa_logits_fp8_kernel<8, false><<<grid, 256, 0, stream>>>(a, split_keys);
  }
  return hipGetLastError();
}

IDX_DEBUG_READER(debug_word_mqa_logits)

}  // namespace idx
