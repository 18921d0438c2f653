// Paged indexer logits for a decode / MTP step, over an fp8 or an MXFP4 K cache.
//
// Row r = b * next_n + j scores keys [0, end_r) of sequence b, where
// end_r = ctx_b - next_n + j + 1 (or context_lens[r] with per-row lengths), clamped
// to [0, min(width, max_blocks * page_size)]: page "vllm.v1.attention.ops.rocm_aiter_mla_sparse",
// rocm_fp8_paged_mqa_logits; page "vllm.v1.attention.ops.rocm_paged_mxfp4_indexer",
// rocm_mxfp4_sparse_attn_indexer. Every column of [0, width) is written.
//
// The step streams the K cache once (HBM-bound). The work unit is a 64-key chunk of
// one sequence; all next_n rows of the sequence are scored from the same bytes.
// Every workgroup of a persistent grid first builds, in LDS, the prefix sum of chunk
// counts over the sequences (from context_lens on the device, so the grid never
// depends on lengths), and each wave takes an equal contiguous share of the
// concatenated chunk list, whatever the mix of lengths (at least a few chunks, so a
// wave's query reloads stay small next to its K bytes). Waves of one XCD get
// neighbouring shares, so a sequence's queries stay in one L2. A wave
//   - fetches the block-table entries of its next 16 chunks with one vector load
//     (lane l: chunk l/4, 16-key group l%4) and reads them back with readlane;
//   - keeps kRing chunks in registers: the loads of chunks i+1 .. i+kRing-1 are in
//     flight while chunk i is scored;
//   - holds its sequence's queries as MFMA A operands (16 heads x 128 channels per
//     tile), reloading them when its share crosses into the next sequence.
// K bytes go straight into MFMA B operands:
//   fp8   lane L loads bytes [16g, 16g+16) and [64+16g, 64+16g+16) of key L%16 of
//         each 16-key group, g = L/16 (the query uses the same byte order): the MFMA
//         B operand itself. A wavefront load reads 64 of the 128 bytes of 16
//         consecutive key rows; its partner load reads the other halves right after.
//         (Whole key rows per load, passed through an LDS tile to form the operands,
//         measured slower on an MI355X: MTP logits 99.6 against 96.4 us, B = 32
//         decode 15.3 against 15.0 us; only the fp8 gathered walk lost, 31.5 against
//         32.2 us);
//   MXFP4 lane L loads 16 bytes at run base + 16L - the run stores [chunk, key,
//         byte], so one wavefront load covers the run's kilobyte exactly and lands
//         in the scaled MFMA's operand order - plus the e8m0 byte at
//         scale base + 64 * run + L, which is that lane's own block scale.
// The epilogue sums ReLU(score) * w over the 16 heads of each lane (4 per tile), then
// over the four lane groups with a transposed permlane reduction that leaves key L of
// the chunk in lane L, scales by the key's fp32 scale (fp8; k_scale > 0 so it factors
// out of the ReLU) and stores one 256-byte segment per row and chunk. Every wave also
// writes an equal share of the -inf tail (columns past the last chunk of each row's
// sequence) with 16-byte streaming stores, a few units after each chunk's K loads are
// issued (and the rest after its last chunk).
//
// Two-level indexer (page "vllm.v1.attention.ops.rocm_paged_mxfp4_indexer", module
// description and rocm_mxfp4_sparse_mqa_indexer):
//   - block maxima: the candidate source's walk also reduces each chunk's stored
//     logits to the maxima of its 16-, 32- or 64-key blocks (DPP and permlane swaps) and
//     stores one value per block; blocks past a sequence's chunks get -inf with the
//     tail;
//   - gather walk: a consumer row scores only its candidate pool. Each query row is
//     its own walk (NR = 1) over pool slots; a 16-key group of slots lies inside one
//     pool block and so at 16 consecutive positions of one page, found through the
//     candidate entry and then the block table. Keys of a group whose candidate is
//     -1 or past the row's end are not loaded and score -inf. A first one-wave-per-row
//     kernel finds each row's pool length, which the walk uses as its sequence length.
#include <climits>
#include <mutex>

#include "debug.h"
#include "device.h"
#include "launch.h"

namespace idx {
namespace {

// Threads per workgroup: 512 for single-row walks, which then hold one workgroup of
// eight waves per CU, 256 for multi-row steps (two per CU). Measured on an MI355X
// against 256 for everything: B = 32 decode 15.1 -> 14.9 us, MXFP4 decode 28.4 ->
// 27.7 us, MXFP4 gathered walk 14.0 -> 12.8 us (fp8 gathered walk unchanged); the MTP
// step lost 0.7 us with 512. Capping 256-thread workgroups at two per CU instead
// helped the fp8 decode as much but cost the MXFP4 decode 1.4 us.
template <int NR>
constexpr int wg_threads() { return NR == 1 ? 512 : 256; }
constexpr int kChunk = 64;
constexpr int kMinChunksPerWave = 2;
// Chunk buffers a wave holds in registers; a chunk is scored from its buffer while
// the others are in flight. Two buffers for single rows, where a third would cost a
// wave per SIMD, and for fp8 (a third measured slower on the MTP step: 98.5 against
// 96.4 us); three for multi-row MXFP4 steps.
template <int FMT, int NR>
constexpr int ring_depth() { return FMT == 0 || NR == 1 ? 2 : 3; }

// largest b in [0, B) with pref[b] <= u (pref[B] > u)
__device__ __forceinline__ int find_seq(const int *pref, int B, int u) {
  int lo = 0, hi = B;
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (pref[mid] <= u) lo = mid; else hi = mid;
  }
  return lo;
}

template <int NR>
__device__ __forceinline__ void row_ends(const PagedArgs &a, int b, int cap, int (&end)[NR]) {
#pragma unroll
  for (int j = 0; j < NR; ++j) {
    const int e = a.ctx_per_row ? a.context_lens[b * NR + j] : a.context_lens[b] - NR + j + 1;
    end[j] = min(max(e, 0), cap);
    IDX_DEBUG_NOTE((a.ctx_per_row ? e : a.context_lens[b]) < 0 || e > cap, IDX_DBG_LENGTH);
  }
}

// One 64-key chunk in registers: the MFMA B operand of each 16-key group kg, for fp8
// the two halves raw[2 kg] and raw[2 kg + 1], for MXFP4 kb[kg].
template <int FMT>
struct Chunk;
// The gather walk also keeps, in lane L, the position of the first key of L's own
// 16-key group (group L / 16; -1 for a group that names no key of the row). A per-lane
// value rather than four per-group ones picked by lane: a pick indexed by lane would
// leave the ring in scratch memory.
template <>
struct Chunk<0> {
  v4i raw[8];
  float ksc;
  int lpos;
};
template <>
struct Chunk<1> {
  v8i kb[4];
  int ksb[4];
  int lpos;
};

// Gather walk: the row's own end (exclusive), as for the dense walk
__device__ __forceinline__ int gather_row_end(const PagedArgs &a, int r, int cap) {
  const int nn = a.next_n;
  const int e = a.ctx_per_row ? a.context_lens[r] : a.context_lens[r / nn] - nn + r % nn + 1;
  IDX_DEBUG_NOTE((a.ctx_per_row ? e : a.context_lens[r / nn]) < 0 || e > cap, IDX_DBG_LENGTH);
  return min(max(e, 0), cap);
}

// Gather walk, first pass (one wave per row): the pool length, one past the last slot
// that names a position below the row's end. Entry i of the candidate list names one
// iff 0 <= cand[i] < ceil(end / block); the last such entry i holds slots
// [i * block, i * block + min(block, end - cand[i] * block)). Written to row_end_out,
// from which the walk reads it back.
__global__ __launch_bounds__(64) void pool_length_kernel(PagedArgs a) {
  const int r = blockIdx.x;
  const int lane = threadIdx.x;
  const int bs = a.block_size;
  const int bsh = 31 - __builtin_clz(bs);
  const int e = gather_row_end(a, r, int(min(int64_t(INT_MAX), int64_t(a.max_blocks) * a.page_size)));
  const int nbe = (e >> bsh) + ((e & (bs - 1)) != 0);
  const int32_t *cr = a.cand + int64_t(r / a.row_repeat) * a.cand_row_stride;
  int last = -1, blk = 0;
  for (int i = lane; i < a.n_cand; i += 64) {
    const int b = cr[i];
    if (b >= 0 && b < nbe) {
      last = i;
      blk = b;
    }
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    const int ol = __shfl_xor(last, o), ob = __shfl_xor(blk, o);
    if (ol > last) {
      last = ol;
      blk = ob;
    }
  }
  if (lane == 0) a.row_end_out[r] = last < 0 ? 0 : last * bs + min(bs, e - (blk << bsh));
}

// Three waves per SIMD where one row's registers fit a third of the register file
// (168): one row with at most 64 heads, except the fp8 gathered walk (it fits, at 162
// registers, but ran no faster: 32.2 us either way). Two where the kernel fits half of it (256), or nearly: asked for one wave per
// SIMD, the compiler put each MFMA result in accumulation registers and copied it back
// one register per score (128 extra vector instructions per MTP chunk; MTP logits
// 102.0 -> 100.5 us with the request for two), and at three rows per sequence and 64
// heads it spilled to them (next_n = 3, B = 64: fp8 90 -> 69 us, MXFP4 79 -> 54 us;
// MXFP4 at four rows 96 -> 74 us). fp8 at four rows and 64 heads spills to scratch
// memory at two waves (110 against 141 us) and keeps one, as do 128 heads.
template <int FMT, int HT, int NR, bool GATHER>
constexpr int waves_per_simd() {
  return NR == 1 && (HT <= 2 || (HT == 4 && !(FMT == 0 && GATHER))) ? 3
         : ((NR <= 2 && (HT <= 4 || NR == 1)) || HT <= 2 || (HT == 4 && (NR == 3 || FMT == 1))) ? 2
                                                                                              : 1;
}

// GATHER: each query row walks its own candidate pool (NR = 1, one "sequence" per
// row); otherwise the dense walk over whole sequences, NR = next_n rows each.
template <int FMT, int HT, int NR, bool GATHER>
__global__ __launch_bounds__(wg_threads<NR>()) __attribute__((amdgpu_waves_per_eu(waves_per_simd<FMT, HT, NR, GATHER>())))
void paged_logits_kernel(PagedArgs a) {
  extern __shared__ int s_lds[];  // pref[S + 1], len[S] (+ end[S] for the gather walk)
  constexpr int kThreads = wg_threads<NR>();
  __shared__ int s_scan[kThreads / 64];
  const int S = GATHER ? a.B * a.next_n : a.B;  // walks: sequences, or rows for the gather walk
  int *s_pref = s_lds;
  int *s_len = s_lds + S + 1;
  int *s_end = s_lds + 2 * S + 1;

  const int tid = threadIdx.x;
  const int wave = uniform(tid >> 6);
  const int lane = tid & 63;
  const int g = lane >> 4;
  const int n = lane & 15;
  const int P = a.page_size;
  // dense: columns the row may reach; gather: positions the block table addresses
  const int cap = GATHER ? int(min(int64_t(INT_MAX), int64_t(a.max_blocks) * P))
                         : int(min(int64_t(a.width), int64_t(a.max_blocks) * P));
  const int bsh = GATHER || a.block_max ? 31 - __builtin_clz(a.block_size) : 0;

  // ---- chunks per sequence, their prefix sum, sequence lengths (LDS) -------------
  const int per = (S + kThreads - 1) / kThreads;
  const int b_lo = min(S, tid * per), b_hi = min(S, b_lo + per);
  int mine = 0;
  for (int b = b_lo; b < b_hi; ++b) {
    int len = 0;
    if constexpr (GATHER) {
      s_end[b] = gather_row_end(a, b, cap);
      len = min(max(a.row_end_out[b], 0), a.width);  // pool length from the first pass
    } else {
      int end[NR];
      row_ends<NR>(a, b, cap, end);
#pragma unroll
      for (int j = 0; j < NR; ++j) len = max(len, end[j]);
    }
    s_len[b] = len;
    mine += (len + kChunk - 1) / kChunk;
  }
  int total = 0;
  int run = block_excl_scan<kThreads>(mine, s_scan, &total);
  for (int b = b_lo; b < b_hi; ++b) {
    s_pref[b] = run;
    run += (s_len[b] + kChunk - 1) / kChunk;
  }
  if (tid == 0) s_pref[S] = total;
  if (!GATHER && blockIdx.x == 0 && a.row_end_out) {
    for (int r = tid; r < a.B * NR; r += kThreads) {
      int end[NR];
      row_ends<NR>(a, r / NR, cap, end);
      int e = end[0];
#pragma unroll
      for (int j = 1; j < NR; ++j)
        if (r % NR == j) e = end[j];
      a.row_end_out[r] = e;
    }
  }
  __syncthreads();

  // ---- this wave's share of the chunk list ---------------------------------------
  // Shares go to waves spread evenly over the whole grid (and so over every XCD)
  // when there are fewer shares than waves; neighbouring shares land on waves of
  // the same XCD.
  const int nwg = gridDim.x;  // a multiple of 8: one slice of workgroups per XCD
  const int logical = (blockIdx.x % 8) * (nwg / 8) + blockIdx.x / 8;
  const int V = nwg * (kThreads / 64);
  const int v = logical * (kThreads / 64) + wave;
  const int U = total;
  const int used = min(V, max(1, (U + kMinChunksPerWave - 1) / kMinChunksPerWave));
  const int k = int(int64_t(v) * used / V);
  const bool owner = v == 0 || int(int64_t(v - 1) * used / V) != k;
  const int u0 = owner ? int(int64_t(U) * k / used) : U;
  const int u1 = owner ? int(int64_t(U) * (k + 1) / used) : U;
  const float ninf = neg_inf();

  // ---- -inf past each sequence's last chunk ------------------------------------------
  // The wave's share of 256-column units is written a few units at a time, each batch
  // after a chunk's K loads are issued: memory operations complete in issue order, so
  // stores issued ahead of the block-table and K loads would delay them.
  // Unit u of the S * NR * fill_nu units is row u / fill_nu, columns from
  // 256 * (u % fill_nu); a wave takes units v, v + V, ..., its row and unit stepped by
  // V without a division per unit.
  const int fill_nu = max((a.width + 255) / 256, 1);
  const int fill_rows = a.width > 0 ? S * NR : 0;
  const int fill_dr = V / fill_nu, fill_dc = V % fill_nu;
  int fill_r = v / fill_nu, fill_c = v % fill_nu;  // this wave's next unit
  auto fill_some = [&](int units) {
    for (int i = 0; i < units && fill_r < fill_rows; ++i) {
      const int r = fill_r;
      const int col = fill_c * 256 + lane * 4;
      fill_c += fill_dc;
      fill_r += fill_dr;
      if (fill_c >= fill_nu) {
        fill_c -= fill_nu;
        ++fill_r;
      }
      const int bb = r / NR;
      const int tail = (s_pref[bb + 1] - s_pref[bb]) * kChunk;
      if (col >= tail && col < a.width) {
        float *p = a.logits + r * a.logits_row_stride + col;
        if (col + 4 <= a.width) {
          __builtin_nontemporal_store(v4f{ninf, ninf, ninf, ninf}, reinterpret_cast<v4f *>(p));
        } else {
          for (int e = 0; col + e < a.width; ++e) __builtin_nontemporal_store(ninf, p + e);
        }
      }
    }
  };

  // block-table entries of chunks [base, base + 16): lane l holds chunk base + l/4,
  // 16-key group l%4 (0 past the wave's share or the sequence's end). The gather walk
  // first reads the group's candidate block, and returns in `pos` the position of the
  // group's first key (-1 when the group names no key below the row's end).
  auto load_pages = [&](int base, int &pos) -> int {
    const int u = base + (lane >> 2);
    int pg = 0;
    pos = -1;
    if (u < u1) {
      const int bb = find_seq(s_pref, S, u);
      const int s = (u - s_pref[bb]) * kChunk + (lane & 3) * 16;
      if (s < s_len[bb]) {
        if constexpr (GATHER) {
          const int e = s_end[bb];
          const int blk = a.cand[int64_t(bb / a.row_repeat) * a.cand_row_stride + (s >> bsh)];
          if (blk >= 0 && blk < (e >> bsh) + ((e & (a.block_size - 1)) != 0)) {
            const int p = (blk << bsh) + (s & (a.block_size - 1));
            if (p < e) {
              pos = p;
              const int pi = a.page_shift >= 0 ? p >> a.page_shift : p / P;
              pg = min(max(a.block_table[int64_t(bb / a.next_n) * a.block_table_stride + pi], 0), a.num_pages - 1);
              IDX_DEBUG_NOTE(a.block_table[int64_t(bb / a.next_n) * a.block_table_stride + pi] != pg, IDX_DBG_PAGE);
            }
          }
        } else {
          const int pi = a.page_shift >= 0 ? s >> a.page_shift : s / P;
          pg = min(max(a.block_table[int64_t(bb) * a.block_table_stride + pi], 0), a.num_pages - 1);
          IDX_DEBUG_NOTE(a.block_table[int64_t(bb) * a.block_table_stride + pi] != pg, IDX_DBG_PAGE);
        }
      }
    }
    return pg;
  };

  // issue the loads of chunk `c` (index within sequence `b`) whose pages sit in lanes
  // 4*slot .. 4*slot+3 of `pg`
  auto issue = [&](Chunk<FMT> &ch, int pg, int pp, int slot, int b, int c) {
    const int key0 = c * kChunk;
    const int len = s_len[b];
    if constexpr (FMT == 0) ch.ksc = 0.f;
    if constexpr (GATHER) ch.lpos = -1;
#pragma unroll
    for (int kg = 0; kg < 4; ++kg) {
      const int s = key0 + kg * 16;  // 16 | P keeps a group inside one page
      if constexpr (FMT == 0) {
        ch.raw[2 * kg] = v4i{0, 0, 0, 0};
        ch.raw[2 * kg + 1] = v4i{0, 0, 0, 0};
      } else {
        ch.kb[kg] = zero8();
        ch.ksb[kg] = 127;
      }
      int kpos = s;  // position of the group's first key
      if constexpr (GATHER) {
        kpos = s < len ? __builtin_amdgcn_readlane(pp, 4 * slot + kg) : -1;
        if (g == kg) ch.lpos = kpos;
      }
      if (GATHER ? kpos >= 0 : s < len) {
        const int page = __builtin_amdgcn_readlane(pg, 4 * slot + kg);
        const uint8_t *pb = a.base + int64_t(page) * a.page_stride;
        const int e0 = a.page_shift >= 0 ? kpos & (P - 1) : kpos % P;
        if constexpr (FMT == 0) {
          const uint8_t *p = pb + (e0 + n) * 128 + g * 16;
          ch.raw[2 * kg] = load16(p);
          ch.raw[2 * kg + 1] = load16(p + 64);
          if (g == kg) ch.ksc = *reinterpret_cast<const float *>(pb + P * 128 + 4 * (e0 + n));
        } else {
          const int run_i = e0 >> 4;
          const v4i z = {0, 0, 0, 0};
          ch.kb[kg] = cat(load16(pb + run_i * 1024 + lane * 16), z);
          ch.ksb[kg] = pb[P * 64 + run_i * 64 + lane];
        }
      }
    }
  };

  v8i qa[NR][HT];
  float wv[NR][HT][4];
  int qs[NR][HT];
  int end[NR];
  // inlined by force: a call would need the kernel arguments it captures in scratch
  // memory (the compiler outlined it in the largest instantiations)
  auto load_queries = [&](int b) __attribute__((always_inline)) {
    if constexpr (GATHER)
      end[0] = s_end[b];
    else
      row_ends<NR>(a, b, cap, end);
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
  };

  // scores chunk c of sequence b
  auto score = [&](const Chunk<FMT> &ch, int b, int c) {
    const int col = c * kChunk + lane;
    float part[NR][4];
#pragma unroll
    for (int kg = 0; kg < 4; ++kg) {
      v8i kb;
      if constexpr (FMT == 0) {
        kb = cat(ch.raw[2 * kg], ch.raw[2 * kg + 1]);
      } else {
        kb = ch.kb[kg];
      }
#pragma unroll
      for (int j = 0; j < NR; ++j) {
        float acc = 0.f;
#pragma unroll
        for (int ht = 0; ht < HT; ++ht) {
          v4f sc;
          if constexpr (FMT == 0)
            sc = mfma_fp8(qa[j][ht], kb);
          else
            sc = mfma_fp4(qa[j][ht], kb, qs[j][ht], ch.ksb[kg]);
#pragma unroll
          for (int jj = 0; jj < 4; ++jj) acc = fmaf(wv[j][ht][jj], relu(sc[jj]), acc);
        }
        part[j][kg] = acc;
      }
    }
    float res[NR];
#pragma unroll
    for (int j = 0; j < NR; ++j) {
      float val = transpose_reduce4(part[j]);
      if constexpr (FMT == 0) val *= ch.ksc;
      if constexpr (GATHER) {
        // lane L holds key L = 16 g + n of the chunk, at position lpos + n
        res[j] = ch.lpos >= 0 && ch.lpos + n < end[j] ? val : ninf;
      } else {
        res[j] = col < end[j] ? val : ninf;
      }
    }
    if (col < a.width) {
#pragma unroll
      for (int j = 0; j < NR; ++j) a.logits[(int64_t(b) * NR + j) * a.logits_row_stride + col] = res[j];
    }
    if constexpr (!GATHER) {
      if (a.block_max) {
        // the chunk holds whole blocks (block_size divides 64): one store per block
#pragma unroll
        for (int j = 0; j < NR; ++j) {
          const float m = group_max(res[j], a.block_size);
          if ((lane & (a.block_size - 1)) == 0 && col < a.width)
            a.block_max[(int64_t(b) * NR + j) * a.block_max_row_stride + (col >> bsh)] = m;
        }
      }
    }
  };

  // ---- stream the share through a ring of kRing chunk buffers: while chunk i is
  // scored, chunks i+1 .. i+kRing-1 are in flight -----------------------------------------
  int qb = -1;  // sequence whose queries are loaded
  auto stream = [&](const int u0, const int u1) {
    if (u0 >= u1) return;
    int ib = find_seq(s_pref, S, u0);  // coordinates of the next chunk to issue
    // The first sequence's queries go out right behind the block-table load and
    // ahead of the K loads: the table's wait does not cover them (a burst of query
    // loads issued first held the table back by over a microsecond), and scoring the
    // first chunk waits on its K loads only (a query load issued behind the K loads
    // would hold that wait until every chunk in flight and the tail stores issued
    // before it had landed).
    int pg_base = u0;
    int pp = -1;
    int pg = load_pages(pg_base, pp);
    load_queries(ib);
    qb = ib;
    int ic = u0 - s_pref[ib];
    int iu = u0;
    constexpr int kRing = ring_depth<FMT, NR>();
    Chunk<FMT> ring[kRing];
    int rb[kRing], rc[kRing];  // sequence and chunk index held by each ring slot
    auto issue_next = [&](Chunk<FMT> &slot_buf, int &slot_b, int &slot_c) {
      if (iu - pg_base >= 16) {
        pg_base = iu;
        pg = load_pages(pg_base, pp);
      }
      issue(slot_buf, pg, pp, iu - pg_base, ib, ic);
      slot_b = ib;
      slot_c = ic;
      if (++iu < u1 && ++ic >= s_pref[ib + 1] - s_pref[ib]) {
        ib = find_seq(s_pref, S, s_pref[ib + 1]);
        ic = 0;
      }
    };
#pragma unroll
    for (int s = 0; s < kRing - 1; ++s)
      if (iu < u1) issue_next(ring[s], rb[s], rc[s]);
    for (int u = u0; u < u1; u += kRing) {
#pragma unroll
      for (int s = 0; s < kRing; ++s) {
        if (u + s >= u1) break;
        const int nxt = (s + kRing - 1) % kRing;  // slot of chunk u + s + kRing - 1
        if (iu < u1) issue_next(ring[nxt], rb[nxt], rc[nxt]);
        fill_some(2);
        if (rb[s] != qb) {
          load_queries(rb[s]);
          qb = rb[s];
        }
        score(ring[s], rb[s], rc[s]);
      }
    }
  };
  stream(u0, u1);
  fill_some(INT_MAX);
  if constexpr (!GATHER) {
    if (a.block_max) {
      // blocks past each sequence's last chunk
      const int nbm = (a.width + a.block_size - 1) >> bsh;
      for (int r = v; r < S * NR; r += V) {
        const int bb = r / NR;
        const int j0 = ((s_pref[bb + 1] - s_pref[bb]) * kChunk) >> bsh;
        for (int jb = j0 + lane; jb < nbm; jb += 64) a.block_max[int64_t(r) * a.block_max_row_stride + jb] = ninf;
      }
    }
  }
}

// Persistent grid: as many workgroups as can be resident at once (a multiple of 8,
// one equal slice per XCD), so every share starts immediately.
template <int FMT, int HT, int NR, bool GATHER>
hipError_t launch_one(const PagedArgs &a, int num_cus, size_t lds, hipStream_t stream) {
  // resident workgroups per CU for this kernel and LDS size, looked up once per size
  static std::mutex mu;
  static size_t cached_lds = ~size_t(0);
  static int cached = 0;
  int per_cu = 0;
  {
    std::lock_guard<std::mutex> lock(mu);
    if (cached_lds != lds) {
      const hipError_t e =
          hipOccupancyMaxActiveBlocksPerMultiprocessor(&cached, paged_logits_kernel<FMT, HT, NR, GATHER>, wg_threads<NR>(), lds);
      if (e != hipSuccess) return e;
      cached_lds = lds;
    }
    per_cu = cached;
  }
  const int nwg = max(8, (max(per_cu, 1) * num_cus) / 8 * 8);
  paged_logits_kernel<FMT, HT, NR, GATHER><<<dim3(nwg), wg_threads<NR>(), lds, stream>>>(a);
  return hipGetLastError();
}

template <int FMT, int HT>
hipError_t launch_nr(const PagedArgs &a, int num_cus, size_t lds, hipStream_t stream) {
  if (a.cand) return launch_one<FMT, HT, 1, true>(a, num_cus, lds, stream);
  switch (a.next_n) {
    case 1: return launch_one<FMT, HT, 1, false>(a, num_cus, lds, stream);
    case 2: return launch_one<FMT, HT, 2, false>(a, num_cus, lds, stream);
    case 3: return launch_one<FMT, HT, 3, false>(a, num_cus, lds, stream);
    default: return launch_one<FMT, HT, 4, false>(a, num_cus, lds, stream);
  }
}

template <int FMT>
hipError_t launch_fmt(const PagedArgs &a, int num_cus, size_t lds, hipStream_t stream) {
  const int ht = (a.H + 15) / 16;
  if (ht <= 1) return launch_nr<FMT, 1>(a, num_cus, lds, stream);
  if (ht <= 2) return launch_nr<FMT, 2>(a, num_cus, lds, stream);
  if (ht <= 4) return launch_nr<FMT, 4>(a, num_cus, lds, stream);
  return launch_nr<FMT, 8>(a, num_cus, lds, stream);
}

}  // namespace

hipError_t launch_paged_logits(const PagedArgs &a, int num_cus, hipStream_t stream) {
  if (a.cand) {
    // the gather walk reads each row's pool length from row_end_out
    pool_length_kernel<<<dim3(a.B * a.next_n), 64, 0, stream>>>(a);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  const size_t lds = a.cand ? size_t(3 * a.B * a.next_n + 1) * sizeof(int) : size_t(2 * a.B + 1) * sizeof(int);
  return a.fmt == 0 ? launch_fmt<0>(a, num_cus, lds, stream) : launch_fmt<1>(a, num_cus, lds, stream);
}

IDX_DEBUG_READER(debug_word_paged_logits)

}  // namespace idx
