// Per-row top-k over [row_start, row_end) with several workgroups per row, for steps
// with few rows (decode, MTP): page "vllm.v1.attention.ops.rocm_paged_mxfp4_indexer",
// _topk (-1 pads rows shorter than k). The page treats few rows and many rows as
// different regimes; with one workgroup per row a decode step keeps a few dozen of
// the 256 compute units busy and its time is the longest row's chain of phases.
//
// The answer is the one the single-workgroup kernel gives: keys become order-preserving
// 32-bit values, T is the k-th largest (radix select on digits of 11, 11 and 10 bits)
// and the output is every key above T plus the lowest-column keys equal to T, in
// ascending column order.
//
// Work split. Every workgroup reads the rows' [start, end) and computes the same
// table: a row with at most k keys is one unit (written as 0..n-1 and -1 pads); a
// longer row is cut into units of SEG consecutive columns, SEG chosen from the total
// so that every unit fits the grid (which is no larger than what the device holds at
// once) and its columns fit the registers. Workgroup g takes unit g.
//
// A row of one unit is selected inside its workgroup: digit histograms in LDS over the
// keys held in registers. The units of a longer row meet twice at counters in a
// per-row scratch record:
//   1. each unit histograms the top 11 bits of its keys and adds the non-zero bins to
//      the row's histogram; after the first meeting every unit reads it and finds the
//      bin d1 of the k-th key, and publishes how many of its keys lie above d1. Unless
//      bin d1 is taken whole, each unit appends its keys of bin d1 (its unit number and
//      the keys' low 21 bits, one word each) to the row's list;
//   2. after the second meeting every unit reads the list - the bin's keys of the whole
//      row, a few hundred to a few thousand - and finishes the selection in LDS: T, the
//      ties still to take, and how many selected keys the units before it hold, which is
//      where its first selected key goes. It writes its selected keys in column order.
// When bin d1 holds more keys than the list (heavy ties), the units meet once or twice
// more instead: a second row histogram over bin d1, then the keys of T's 22-bit
// prefix in the list, or a third histogram when even those overflow it.
// The last unit of a row to finish clears the row's record, so the scratch is all zero
// between calls (it must be zero before the first one).
//
// Every access to the shared scratch is a device-scope operation: atomic
// read-modify-writes (histograms, counters, list slots) and loads and stores with the
// device-coherence cache bit (lists, unit records), so values are coherent across the
// device's chiplets without writing back or invalidating L2. A meeting needs order
// only: each thread waits until all its memory operations have completed (s_waitcnt
// with every counter at zero), the workgroup synchronises, and one lane counts the unit
// in; a unit that has seen the count reach its target issues its reads of the records
// after that load returned. (Release/acquire fences at device scope would write back and
// invalidate the whole L2 at every meeting.) Every wait is a bounded poll: all units of
// a call are resident together (the grid is sized from the occupancy query), so a wait
// ends as soon as the row's other units arrive; should the bound ever be reached
// (another kernel holding the device's slots for very long), the wait gives up and the
// call's output is unspecified, but the kernel always exits.
#include <algorithm>
#include <climits>
#include <mutex>

#include "debug.h"
#include "device.h"
#include "launch.h"

namespace idx {
namespace {

constexpr int kNT = 256;                    // threads of a shared-row unit
constexpr int kKPL = 16;                    // keys per lane a shared-row unit holds in registers
constexpr int kMinSeg = 1024;               // smallest unit of a multi-unit row, in columns
constexpr int kBins = 2048;
constexpr int kList = 4096;                 // list entries per row
constexpr uint32_t kSpinLimit = 1u << 20;   // polls of one wait (about a second)
constexpr int kCohere = 16;                 // cache-policy bit of device-coherent loads / stores

struct RowState {
  uint32_t h1[kBins];   // digit 1 (top 11 bits) over the row
  uint32_t h2[kBins];   // digit 2 over the keys of bin d1 (list overflow only)
  uint32_t h3[1024];    // digit 3 over the keys of T's 22-bit prefix (second overflow)
  uint32_t arrive[4];   // meeting counters
  uint32_t depart;
  uint32_t nlist;
  uint32_t pad[10];
  uint32_t list[kList];  // (unit << 21) | low 21 bits of a key
};

struct UnitInfo {
  int32_t above1, above2, gt3, eq3;
};

static_assert(sizeof(RowState) == kCoopRowBytes && sizeof(UnitInfo) == kCoopUnitBytes, "scratch layout");
static_assert(kCoopMaxUnits <= 2048, "unit numbers fit the list entries' 11 bits");

__device__ __forceinline__ uint32_t ld(const uint32_t *p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st(uint32_t *p, uint32_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint32_t add(uint32_t *p, uint32_t v) {
  return __hip_atomic_fetch_add(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// 16 device-coherent bytes at byte `off` of a record of `bytes` bytes (zeros past it);
// unlike atomic loads these pipeline (no wait after each)
__device__ __forceinline__ v4i ld16(const void *base, uint32_t bytes, uint32_t off) {
  return __builtin_bit_cast(v4i, __builtin_amdgcn_raw_buffer_load_b128(make_rsrc(base, bytes), off, 0, kCohere));
}

__device__ __forceinline__ void drain() {
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_waitcnt(0);
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

// every thread's memory operations are complete; one lane counts the unit in
__device__ __forceinline__ void arrive(uint32_t *ctr) {
  drain();
  __syncthreads();
  if (threadIdx.x == 0) add(ctr, 1u);
}

// one lane polls until `target` units have arrived (or the poll bound is reached)
__device__ __forceinline__ void wait_for(const uint32_t *ctr, uint32_t target) {
  if (threadIdx.x == 0) {
    for (uint32_t spin = 0; spin < kSpinLimit; ++spin) {
      if (ld(ctr) >= target) break;
      __builtin_amdgcn_s_sleep(1);
    }
  }
  drain();
  __syncthreads();
}

// sum of one value per thread over a workgroup of NT threads (every thread gets it)
template <int NT>
__device__ __forceinline__ int block_sum(int v, int *scratch) {
  const int s = wave_sum(v);
  if ((threadIdx.x & 63) == 0) scratch[threadIdx.x >> 6] = s;
  __syncthreads();
  int t = 0;
#pragma unroll
  for (int w = 0; w < NT / 64; ++w) t += scratch[w];
  __syncthreads();
  return t;
}

// largest i in [0, n) with pref[i] <= g
__device__ __forceinline__ int find_unit_row(const int *pref, int n, int g) {
  int lo = 0, hi = n;
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (pref[mid] <= g) lo = mid; else hi = mid;
  }
  return lo;
}

template <int NT>
__device__ __forceinline__ void zero_lds(uint32_t *p, int n) {
  for (int i = threadIdx.x; i < n; i += NT) p[i] = 0u;
}

// NT threads, KPL keys per lane in registers. SOLO: workgroup r selects row r alone,
// the caller guarantees width <= NT * KPL (every row fits the registers at once) and no
// scratch is used; otherwise the shared-row kernel described above.
template <int NT, int KPL, bool SOLO>
__global__ __launch_bounds__(NT) void topk_reg_kernel(TopkArgs a, uint8_t *ws) {
  constexpr int kWaves = NT / 64;
  constexpr int kSteps = KPL / 4;          // 256-key steps of a wave (4 consecutive keys per lane)
  constexpr int kWaveCap = 64 * KPL;       // keys a wave holds per pass
  __shared__ int s_pref[SOLO ? 1 : kCoopMaxRows + 1];
  __shared__ int s_st[SOLO ? 1 : kCoopMaxRows], s_en[SOLO ? 1 : kCoopMaxRows];
  // [0, kList): the row's list (or a copy of a row histogram); then this unit's
  // histograms (a solo row needs only those)
  __shared__ __attribute__((aligned(16))) uint32_t s_big[(SOLO ? 0 : kList) + kBins];
  __shared__ int s_red[kWaves];
  __shared__ int s_sel[2];
  __shared__ int s_wcnt[2][kWaves];
  __shared__ int s_slot[kWaves];
  __shared__ int s_last;
  uint32_t *const s_list = s_big;
  uint32_t *const s_h = s_big + (SOLO ? 0 : kList);

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int rows = a.rows, k = a.k;
  UnitInfo *const info = reinterpret_cast<UnitInfo *>(ws);
  RowState *const state = reinterpret_cast<RowState *>(ws + size_t(kCoopMaxUnits) * sizeof(UnitInfo));

  auto clamp_row = [&](int row, int &st0, int &en) {
    st0 = a.row_start ? min(max(a.row_start[row], 0), a.width) : 0;
    const int e_in = max(a.row_end[row], 0);
    const int en0 = min(a.end_div == 1 ? e_in : e_in / a.end_div + (e_in % a.end_div != 0), a.width);
    IDX_DEBUG_NOTE((a.row_start && (a.row_start[row] < 0 || a.row_start[row] > a.width)) || a.row_end[row] < 0 ||
                   (a.end_div == 1 ? e_in : e_in / a.end_div + (e_in % a.end_div != 0)) > a.width,
               IDX_DBG_LENGTH);
    en = max(en0, st0);
  };
  int r, g0 = 0, u = 0, nu = 1, seg = 0, st0, en;
  if constexpr (SOLO) {
    r = blockIdx.x;
    clamp_row(r, st0, en);
    seg = en - (st0 & ~3);
  } else {
    // ---- the unit table (identical in every workgroup) -------------------------------
    int units = 0, span = 0;
    if (tid < rows) {
      int s0, e0;
      clamp_row(tid, s0, e0);
      s_st[tid] = s0;
      s_en[tid] = e0;
      if (e0 - s0 > k) span = e0 - (s0 & ~3);  // columns from the aligned start
    }
    const int total_span = block_sum<NT>(span, s_red);
    const int free_units = max(1, int(gridDim.x) - rows);
    seg = max(kMinSeg, ((total_span + free_units - 1) / free_units + 255) & ~255);
    if (tid < rows) units = span > 0 ? (span + seg - 1) / seg : 1;
    int n_units = 0;
    const int first = block_excl_scan<NT>(units, s_red, &n_units);
    if (tid < rows) s_pref[tid] = first;
    if (tid == 0) s_pref[rows] = n_units;
    __syncthreads();
    const int g = blockIdx.x;
    if (g >= n_units) return;
    r = find_unit_row(s_pref, rows, g);
    g0 = s_pref[r];
    u = g - g0;
    nu = s_pref[r + 1] - g0;
    st0 = s_st[r];
    en = s_en[r];
  }
  const int n = en - st0;
  int32_t *out = a.out + int64_t(r) * a.out_row_stride;
  if (n <= k) {
    for (int i = tid; i < k; i += NT) out[i] = i < n ? i : -1;
    return;
  }
  const bool solo = SOLO || nu == 1;
  RowState &rs = state[SOLO ? 0 : r];
  UnitInfo *const ui = info + (SOLO ? 0 : g0 + u);

  // ---- this unit's columns, wave segments of whole 256-key steps ----------------------
  const int a0 = st0 & ~3;
  const int lo = a0 + u * seg, hi = min(en, lo + seg);
  const int wseg = ((hi - lo + kWaves - 1) / kWaves + 255) & ~255;
  const int wlo = min(hi, lo + wave * wseg), whi = min(hi, wlo + wseg);
  const bool single = SOLO || wseg <= kWaveCap;  // the segment fits the registers: one load
  const float *lr = a.logits + int64_t(r) * a.logits_row_stride;
  const buffer_rsrc rsrc = make_rsrc(lr, uint32_t(en) * 4u);

  uint32_t kr4[kSteps][4];
  // keys of the pass starting at column cb: 0 (no key) outside [st0, whi)
  // (the raw bits land in kr4 and are converted in place, so a pass needs no second
  // set of registers)
  auto load_pass = [&](int cb) {
    // steps at or past the segment's end are neither loaded nor converted: the walks
    // stop before them
#pragma unroll
    for (int s = 0; s < kSteps; ++s) {
      if (uniform(int(cb + s * 256 < whi))) {
        const v4i x = buffer_load16(rsrc, uint32_t(cb + s * 256 + 4 * lane) * 4u);  // zero past the row
#pragma unroll
        for (int e = 0; e < 4; ++e) kr4[s][e] = uint32_t(x[e]);
      }
    }
#pragma unroll
    for (int s = 0; s < kSteps; ++s) {
      const int cs = cb + s * 256;
      if (uniform(int(cs >= whi))) break;
      if (uniform(int(cs >= st0 && cs + 256 <= whi))) {
        // every column of the step is in the row (all but a row's first and last steps)
#pragma unroll
        for (int e = 0; e < 4; ++e) kr4[s][e] = order_key(__uint_as_float(kr4[s][e]));
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int c = cs + 4 * lane + e;
          kr4[s][e] = (c >= st0 && c < whi) ? order_key(__uint_as_float(kr4[s][e])) : 0u;
        }
      }
    }
  };
  // fn(keys of 4 consecutive columns, first column) over the wave's segment in column
  // order, each lane holding 4 consecutive columns of a step; loads again only when the
  // segment does not fit the registers. Steps past the segment's end hold no key and
  // are skipped (a short causal row fills a few of its steps).
  auto walk = [&](auto &&fn, bool load_first) {
    for (int cb = wlo; cb < whi; cb += kWaveCap) {
      if (load_first || !single) load_pass(cb);
      // one step at a time: the scheduler would otherwise hoist every step's comparisons
      // ahead of the first and hold them all in registers
#pragma unroll
      for (int s = 0; s < kSteps; ++s) {
        if (cb + s * 256 >= whi) break;
        fn(kr4[s], cb + s * 256 + 4 * lane);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  };
  auto flush = [&](uint32_t *dst, int nbins) {
    for (int b = tid; b < nbins; b += NT) {
      const uint32_t c = s_h[b];
      if (c) add(dst + b, c);
    }
  };
  // a row histogram of nbins words into s_list (copy)
  auto read_hist = [&](const uint32_t *src, int nbins) {
    for (int i = 4 * tid; i < nbins; i += 4 * NT)
      *reinterpret_cast<v4i *>(s_list + i) = ld16(src, uint32_t(nbins) * 4u, uint32_t(i) * 4u);
  };
  // local histogram of the keys `pick` accepts, bin(key) in [0, nbins)
  auto local_hist = [&](int nbins, auto &&pick, auto &&bin) {
    zero_lds<NT>(s_h, nbins);
    __syncthreads();
    walk([&](const uint32_t (&key)[4], int) {
#pragma unroll
      for (int e = 0; e < 4; ++e)
        if (pick(key[e])) atomicAdd(&s_h[bin(key[e])], 1u);
    }, false);
    __syncthreads();
  };
  auto select = [&](const uint32_t *hist, int nbins, int kr) {
    if (nbins == kBins)
      select_bin<kBins>(hist, kr, s_sel);
    else
      select_bin<1024>(hist, kr, s_sel);
    __syncthreads();
  };
  // appends this unit's keys that `pick` accepts to the row's list: each wave reserves
  // room for all of its keys at once, then writes them
  auto append = [&](auto &&pick) {
    int m = 0;
    walk([&](const uint32_t (&key)[4], int) {
#pragma unroll
      for (int e = 0; e < 4; ++e) m += int(pick(key[e]));
    }, false);
    m = wave_sum(m);
    if (lane == 0) s_slot[wave] = m ? int(add(&rs.nlist, uint32_t(m))) : 0;
    __syncthreads();
    int slot = s_slot[wave];
    const buffer_rsrc lst = make_rsrc(rs.list, uint32_t(kList) * 4u);
    const uint32_t tag = uint32_t(u) << 21;
    walk([&](const uint32_t (&key)[4], int) {
      int c = 0;
#pragma unroll
      for (int e = 0; e < 4; ++e) c += int(pick(key[e]));
      const int incl = wave_incl_scan(c);
      int p = slot + incl - c;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        if (pick(key[e])) {
          __builtin_amdgcn_raw_buffer_store_b32(tag | (key[e] & 0x1FFFFFu), lst, uint32_t(p) * 4u, 0, kCohere);
          ++p;
        }
      }
      slot += __builtin_amdgcn_readlane(incl, 63);
    }, false);
  };
  // the row's list of c entries into s_list
  auto read_list = [&](int c) {
    for (int i = 4 * tid; i < c; i += 4 * NT)
      *reinterpret_cast<v4i *>(s_list + i) = ld16(rs.list, uint32_t(c) * 4u, uint32_t(i) * 4u);
  };
  // sum of field f of the records of the row's units before this one
  auto units_before = [&](int f) {
    int x = 0;
    for (int v = tid; v < u; v += NT) x += ld16(info + g0 + v, 16u, 0u)[f];
    return block_sum<NT>(x, s_red);
  };

  // ---- 1. digit-1 histogram ----------------------------------------------------------
  zero_lds<NT>(s_h, kBins);
  __syncthreads();
  walk([&](const uint32_t (&key)[4], int) {
#pragma unroll
    for (int e = 0; e < 4; ++e)
      if (key[e]) atomicAdd(&s_h[key[e] >> 21], 1u);
  }, true);
  __syncthreads();

  uint32_t T;
  int kr3 = 0;   // ties (keys equal to T) to take
  int tie0 = 0;  // ties in the row's columns before this unit
  int base = 0;  // output slots the row's units before this one fill
  if (solo) {
    // ---- the whole row in this workgroup ---------------------------------------------
    select(s_h, kBins, k);
    const uint32_t d1 = uint32_t(s_sel[0]);
    const int kr1 = k - s_sel[1];
    const bool whole1 = int(s_h[d1]) == kr1;
    __syncthreads();
    if (whole1) {
      T = (d1 << 21) - 1u;  // d1 >= 1: a whole bottom bin would mean n == k
    } else {
      local_hist(kBins, [&](uint32_t key) { return (key >> 21) == d1; },
                 [&](uint32_t key) { return (key >> 10) & uint32_t(kBins - 1); });
      select(s_h, kBins, kr1);
      const uint32_t p2 = (d1 << 11) | uint32_t(s_sel[0]);
      const int kr2 = kr1 - s_sel[1];
      const bool whole2 = int(s_h[s_sel[0]]) == kr2;
      __syncthreads();
      if (whole2) {
        T = (p2 << 10) - 1u;
      } else {
        local_hist(1024, [&](uint32_t key) { return (key >> 10) == p2; }, [&](uint32_t key) { return key & 1023u; });
        select(s_h, 1024, kr2);
        T = (p2 << 10) | uint32_t(s_sel[0]);
        kr3 = kr2 - s_sel[1];
        if (int(s_h[s_sel[0]]) == kr3) {
          T -= 1u;  // every key equal to T is taken: keys > T - 1, no ties to rank
          kr3 = 0;
        }
      }
    }
  } else if constexpr (!SOLO) {
    // ---- 1 (cont). the row histogram; bin d1 -----------------------------------------
    flush(rs.h1, kBins);
    arrive(&rs.arrive[0]);
    wait_for(&rs.arrive[0], nu);
    read_hist(rs.h1, kBins);
    __syncthreads();
    select(s_list, kBins, k);
    const uint32_t d1 = uint32_t(s_sel[0]);
    const int kr1 = k - s_sel[1];
    const int c1 = int(s_list[d1]);
    const bool whole1 = c1 == kr1;
    int mine = 0;
    for (int b = tid; b < kBins; b += NT) mine += int(b > int(d1) || (whole1 && b == int(d1))) * int(s_h[b]);
    const int above1 = block_sum<NT>(mine, s_red);
    if (tid == 0) st(reinterpret_cast<uint32_t *>(&ui->above1), uint32_t(above1));
    // mode 0: bin d1 whole; 1: its keys in the list; 2: overflow (more meetings)
    const int mode = whole1 ? 0 : (c1 <= kList ? 1 : 2);
    if (mode == 1)
      append([&](uint32_t key) { return (key >> 21) == d1; });
    else if (mode == 2) {
      local_hist(kBins, [&](uint32_t key) { return (key >> 21) == d1; },
                 [&](uint32_t key) { return (key >> 10) & uint32_t(kBins - 1); });
      flush(rs.h2, kBins);
    }
    arrive(&rs.arrive[1]);
    wait_for(&rs.arrive[1], nu);

    // ---- 2. T and the selected keys of the units before this one ----------------------
    base = units_before(0);
    if (mode == 0) {
      T = (d1 << 21) - 1u;
    } else if (mode == 1) {
      // the row's keys of bin d1, finished here: digit 2, then digit 3, over the list
      read_list(c1);
      zero_lds<NT>(s_h, kBins);
      __syncthreads();
      for (int i = tid; i < c1; i += NT) atomicAdd(&s_h[(s_list[i] >> 10) & uint32_t(kBins - 1)], 1u);
      __syncthreads();
      select(s_h, kBins, kr1);
      const uint32_t d2 = uint32_t(s_sel[0]);
      const int kr2 = kr1 - s_sel[1];
      const bool whole2 = int(s_h[d2]) == kr2;
      __syncthreads();
      const uint32_t p2 = (d1 << 11) | d2;
      if (whole2) {
        T = (p2 << 10) - 1u;
      } else {
        zero_lds<NT>(s_h, 1024);
        __syncthreads();
        for (int i = tid; i < c1; i += NT)
          if (((s_list[i] >> 10) & uint32_t(kBins - 1)) == d2) atomicAdd(&s_h[s_list[i] & 1023u], 1u);
        __syncthreads();
        select(s_h, 1024, kr2);
        T = (p2 << 10) | uint32_t(s_sel[0]);
        kr3 = kr2 - s_sel[1];
      }
      // list keys of earlier units above T and equal to T (all in bin d1, so their low
      // 21 bits order them)
      const uint32_t tl = T & 0x1FFFFFu;
      int gt = 0, eq = 0;
      for (int i = tid; i < c1; i += NT) {
        const bool earlier = int(s_list[i] >> 21) < u;
        const uint32_t low = s_list[i] & 0x1FFFFFu;
        gt += int(earlier && low > tl);
        eq += int(earlier && low == tl);
      }
      base += block_sum<NT>(gt, s_red);
      tie0 = kr3 > 0 ? block_sum<NT>(eq, s_red) : 0;
      base += min(tie0, kr3);
    } else {
      // ---- overflow: digit 2 from a second row histogram ------------------------------
      read_hist(rs.h2, kBins);
      __syncthreads();
      select(s_list, kBins, kr1);
      const uint32_t p2 = (d1 << 11) | uint32_t(s_sel[0]);
      const int kr2 = kr1 - s_sel[1];
      const int c2 = int(s_list[s_sel[0]]);
      const int mode2 = c2 == kr2 ? 0 : (c2 <= kList ? 1 : 2);
      int gt = 0, eq = 0;
      walk([&](const uint32_t (&key)[4], int) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          gt += int((key[e] >> 21) == d1 && (key[e] >> 10) > p2);
          eq += int((key[e] >> 10) == p2);
        }
      }, false);
      const int above2 = block_sum<NT>(mode2 == 0 ? gt + eq : gt, s_red);
      if (tid == 0) st(reinterpret_cast<uint32_t *>(&ui->above2), uint32_t(above2));
      if (mode2 == 1)
        append([&](uint32_t key) { return (key >> 10) == p2; });
      else if (mode2 == 2) {
        local_hist(1024, [&](uint32_t key) { return (key >> 10) == p2; }, [&](uint32_t key) { return key & 1023u; });
        flush(rs.h3, 1024);
      }
      arrive(&rs.arrive[2]);
      wait_for(&rs.arrive[2], nu);
      base += units_before(1);
      if (mode2 == 0) {
        T = (p2 << 10) - 1u;
      } else if (mode2 == 1) {
        read_list(c2);
        zero_lds<NT>(s_h, 1024);
        __syncthreads();
        for (int i = tid; i < c2; i += NT) atomicAdd(&s_h[s_list[i] & 1023u], 1u);
        __syncthreads();
        select(s_h, 1024, kr2);
        T = (p2 << 10) | uint32_t(s_sel[0]);
        kr3 = kr2 - s_sel[1];
        const uint32_t tl = T & 0x1FFFFFu;
        int g3 = 0, e3 = 0;
        for (int i = tid; i < c2; i += NT) {
          const bool earlier = int(s_list[i] >> 21) < u;
          const uint32_t low = s_list[i] & 0x1FFFFFu;
          g3 += int(earlier && low > tl);
          e3 += int(earlier && low == tl);
        }
        base += block_sum<NT>(g3, s_red);
        tie0 = block_sum<NT>(e3, s_red);
        base += min(tie0, kr3);
      } else {
        read_hist(rs.h3, 1024);
        __syncthreads();
        select(s_list, 1024, kr2);
        T = (p2 << 10) | uint32_t(s_sel[0]);
        kr3 = kr2 - s_sel[1];
        int g3 = 0, e3 = 0;
        walk([&](const uint32_t (&key)[4], int) {
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            g3 += int((key[e] >> 10) == p2 && key[e] > T);
            e3 += int(key[e] == T);
          }
        }, false);
        g3 = block_sum<NT>(g3, s_red);
        e3 = block_sum<NT>(e3, s_red);
        if (tid == 0) {
          st(reinterpret_cast<uint32_t *>(&ui->gt3), uint32_t(g3));
          st(reinterpret_cast<uint32_t *>(&ui->eq3), uint32_t(e3));
        }
        arrive(&rs.arrive[3]);
        wait_for(&rs.arrive[3], nu);
        base += units_before(2);
        tie0 = units_before(3);
        base += min(tie0, kr3);
      }
    }
  }

  // ---- emission in column order -------------------------------------------------------
  // Each walk compares against its own copy of T that the optimiser cannot see
  // through: with one shared T the compiler keeps the counting walk's comparisons
  // alive for the emitting walk (all 32 per lane, packed into bytes and unpacked per
  // step), which costs several times more than comparing again. Rows with no ties to
  // place (kr3 == 0, the usual case) take walks that never look at keys equal to T.
  {
    const bool ties = kr3 > 0;
    uint32_t Tc = uint32_t(uniform(int(T)));
    asm volatile("" : "+s"(Tc));
    int gt = 0, eq = 0;
    if (!ties) {
      walk([&](const uint32_t (&key)[4], int) {
#pragma unroll
        for (int e = 0; e < 4; ++e) gt += int(key[e] > Tc);
      }, false);
    } else {
      walk([&](const uint32_t (&key)[4], int) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          gt += int(key[e] > Tc);
          eq += int(key[e] == Tc);
        }
      }, false);
    }
    gt = wave_sum(gt);
    eq = ties ? wave_sum(eq) : 0;
    if (lane == 0) {
      s_wcnt[0][wave] = gt;
      s_wcnt[1][wave] = eq;
    }
    __syncthreads();
    int gtb = 0, eqb = 0;
    for (int w = 0; w < wave; ++w) {
      gtb += s_wcnt[0][w];
      eqb += s_wcnt[1][w];
    }
    int tie_run = tie0 + eqb;  // row tie rank of the next tie met in this wave
    int pos = base + gtb + max(0, min(eqb, kr3 - tie0));
    const buffer_rsrc orsrc = make_rsrc(out, uint32_t(k) * 4u);  // slots past k are dropped
    uint32_t Te = uint32_t(uniform(int(T)));
    asm volatile("" : "+s"(Te));
    if (!ties) {
      walk([&](const uint32_t (&key)[4], int c0) {
        int ns = 0;
#pragma unroll
        for (int e = 0; e < 4; ++e) ns += int(key[e] > Te);
        const int incl = wave_incl_scan(ns);
        int p = pos + incl - ns;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          if (key[e] > Te) {
            __builtin_amdgcn_raw_buffer_store_b32(uint32_t(c0 + e - st0), orsrc, uint32_t(p) * 4u, 0, 0);
            ++p;
          }
        }
        pos += __builtin_amdgcn_readlane(incl, 63);
      }, false);
    } else {
      walk([&](const uint32_t (&key)[4], int c0) {
        // bit e: key e is selected (above T, or a tie whose row rank is below kr3)
        uint32_t sel = 0;
        int neq = 0;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          sel |= uint32_t(key[e] > Te) << e;
          neq += int(key[e] == Te);
        }
        if (__ballot(neq != 0) != 0ull) {
          const int incl = wave_incl_scan(neq);
          int rk = tie_run + incl - neq;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            if (key[e] == Te) {
              sel |= uint32_t(rk < kr3) << e;
              ++rk;
            }
          }
          tie_run += __builtin_amdgcn_readlane(incl, 63);
        }
        const int ns = __builtin_popcount(sel);
        const int incl = wave_incl_scan(ns);
        int p = pos + incl - ns;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          if ((sel >> e) & 1u) {
            __builtin_amdgcn_raw_buffer_store_b32(uint32_t(c0 + e - st0), orsrc, uint32_t(p) * 4u, 0, 0);
            ++p;
          }
        }
        pos += __builtin_amdgcn_readlane(incl, 63);
      }, false);
    }
  }
  if (solo) return;

  // ---- the row's last unit clears its record ------------------------------------------
  if constexpr (SOLO) return;
  __syncthreads();
  if (tid == 0) s_last = add(&rs.depart, 1u) == uint32_t(nu - 1);
  __syncthreads();
  if (s_last) {
    for (int b = tid; b < kBins; b += NT) {
      st(&rs.h1[b], 0u);
      st(&rs.h2[b], 0u);
    }
    for (int b = tid; b < 1024; b += NT) st(&rs.h3[b], 0u);
    if (tid < 4) st(&rs.arrive[tid], 0u);
    if (tid == 4) st(&rs.nlist, 0u);
    if (tid == 5) st(&rs.depart, 0u);
  }
}

// The records of the cooperative kernel for up to kCoopMaxRows rows, owned by the
// library for callers that cannot allocate (idx_topk_noalloc). Zero when the code object
// loads, and every call leaves it zero. Host code never passes this name to a kernel:
// it is a host-side stand-in; the device address comes from hipGetSymbolAddress.
static __device__ __align__(256) uint8_t scratch[topk_scratch_bytes(kCoopMaxRows)];

}  // namespace

void *topk_static_scratch(size_t *bytes) {
  constexpr int kDevices = 64;
  static std::mutex mu;
  static void *addr[kDevices] = {};
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kDevices) return nullptr;
  std::lock_guard<std::mutex> lock(mu);
  if (!addr[dev]) {
    // this device is current: its own copy of the array
    void *p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return nullptr;
    addr[dev] = p;
  }
  *bytes = sizeof(scratch);
  return addr[dev];
}

constexpr int kCap = kNT * kKPL;  // keys a shared-row unit holds at once

// Workgroups of the cooperative kernel for these rows: enough units of at most kCap
// columns for rows of `width`, no more than the device holds at once (0: it cannot
// run). Fewer workgroups also start sooner.
int topk_coop_grid(int num_cus, int rows, int width) {
  static std::mutex mu;
  static int per_cu = -1;
  int resident = 0;
  {
    std::lock_guard<std::mutex> lock(mu);
    if (per_cu < 0) {
      int n = 0;
      if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, topk_reg_kernel<kNT, kKPL, false>, kNT, 0) != hipSuccess) n = 0;
      per_cu = n;
    }
    resident = per_cu * num_cus;
  }
  const int64_t want = int64_t(rows) + (int64_t(rows) * (int64_t(width) + 3) + kCap - 1) / kCap;
  return int(std::min<int64_t>({want, int64_t(resident), int64_t(kCoopMaxUnits)}));
}

hipError_t launch_topk_coop(const TopkArgs &a, void *scratch, int grid, hipStream_t stream) {
  topk_reg_kernel<kNT, kKPL, false><<<dim3(grid), kNT, 0, stream>>>(a, static_cast<uint8_t *>(scratch));
  return hipGetLastError();
}

int topk_solo_cap() { return 256 * 32; }

hipError_t launch_topk_solo(const TopkArgs &a, hipStream_t stream) {
  topk_reg_kernel<256, 32, true><<<dim3(a.rows), 256, 0, stream>>>(a, nullptr);
  return hipGetLastError();
}

IDX_DEBUG_READER(debug_word_topk_coop)

}  // namespace idx
