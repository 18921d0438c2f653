// Per-row top-k over [row_start, row_end): page
// "vllm.v1.attention.ops.rocm_paged_mxfp4_indexer", _topk (-1 pads rows shorter than k).
//
// One workgroup per row; logits become order-preserving 32-bit keys (-0.0 folded onto
// +0.0). The k-th largest key T is found by a three-digit radix select (11, 11 and 10
// bits) and the answer is every key above T plus the lowest-column keys equal to T,
// written in ascending column order. The kernel is a short chain of phases, each
// cheap in latency:
//   1. one read of the row from global memory: keys into LDS (rows up to kMaxCache)
//      and a histogram of the top 11 bits;
//   2. wave 0 alone finds the bin of the k-th key (lane sums of 32 bins, a DPP lane
//      scan and a ballot name a lane; its 32 bins, one per lane, a second scan and
//      ballot name the bin), then one barrier;
//   3. each wave walks its own contiguous segment of the row: it counts the keys in
//      higher bins, compacts the keys of the selected bin into a candidate list (one
//      LDS atomic per wave and step) tagged with the wave's number, and histograms
//      their next 11 bits;
//   4. digits 2 and 3 are selected over the candidates, and each candidate above or
//      equal to T is counted against its wave;
//   5. every wave then knows how many selected keys precede its segment and walks it
//      once more, placing the selected keys with ballots and lane-prefix counts.
// Rows too long for the key cache use the cache's LDS as their candidate list. If the
// selected bin holds more keys than the list (heavy ties), digit 3 and the per-wave
// counts come from extra passes over the row instead.
#include <cstddef>
#include <mutex>
#include <type_traits>

#include "debug.h"
#include "device.h"
#include "launch.h"

namespace idx {
namespace {

constexpr int kMaxCache = 32768;  // keys kept in LDS (128 KiB)
constexpr int kBins = 2048;       // digits 1 and 2: 11 bits; digit 3: 10 bits
constexpr int kUnroll = 16;       // loads in flight per thread in the first pass

// Candidate list size: long rows (few rows, 1024 threads) get more room, up to what
// LDS holds beside a full key cache (160 KiB per workgroup).
template <int NT>
struct Cfg {
  static constexpr int kCand = NT >= 1024 ? 3840 : 1024;
  static constexpr int kWaves = NT / 64;
};

template <int NT>
struct __attribute__((aligned(16))) Smem {
  uint32_t hist[kBins];           // digit 1, then digit 3
  uint32_t hist2[kBins];          // digit 2
  uint32_t cand[Cfg<NT>::kCand];  // (wave << 21) | low 21 bits of a key of the selected bin
  int wgt[Cfg<NT>::kWaves];       // per wave segment: keys above T
  int weq[Cfg<NT>::kWaves];       // per wave segment: keys equal to T
  int sel[2];  // selected digit, keys above it
  int ncand;
};

// select_bin over hist[0..NBINS), published to the workgroup in sm.sel
template <int NT, int NBINS>
__device__ __forceinline__ void select_digit(Smem<NT> &sm, const uint32_t *hist, int kr) {
  select_bin<NBINS>(hist, kr, sm.sel);
  __syncthreads();
}

// This wave's contiguous segment [lo, hi) of the row: equal shares, whole steps.
template <int NT, int KPL>
__device__ __forceinline__ void segment(int n, int wave, int &lo, int &hi) {
  constexpr int kStep = 64 * KPL;
  const int seg = (n + Cfg<NT>::kWaves * kStep - 1) / (Cfg<NT>::kWaves * kStep) * kStep;
  lo = min(n, wave * seg);
  hi = min(n, lo + seg);
}

// Selected keys (above T) and ties counted in the segments of waves before `wave`:
// lane w reads wave w's counts, and a lane scan sums them.
template <int NT>
__device__ __forceinline__ void before_wave(const Smem<NT> &sm, int wave, int lane, int &gt, int &eq) {
  const int g = wave_incl_scan(lane < Cfg<NT>::kWaves ? sm.wgt[lane] : 0);
  const int e = wave_incl_scan(lane < Cfg<NT>::kWaves ? sm.weq[lane] : 0);
  gt = wave > 0 ? __builtin_amdgcn_readlane(g, wave - 1) : 0;
  eq = wave > 0 ? __builtin_amdgcn_readlane(e, wave - 1) : 0;
}

// Phases 3 to 5 for one row, with the keys read through key_at (LDS or global) and
// KPL keys per lane in flight per step. The candidate list `cand` holds up to
// cand_cap entries: the small list in Smem for rows whose keys sit in LDS, the unused
// key cache for longer rows.
template <int NT, int KPL, typename KeyAt>
__device__ __forceinline__ void finish_row(Smem<NT> &sm, KeyAt key_at, int n, int k, int32_t *out, uint32_t *cand,
                           int cand_cap) {
  constexpr int kStep = 64 * KPL;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  int lo, hi;
  segment<NT, KPL>(n, wave, lo, hi);

  const uint32_t d1 = uint32_t(sm.sel[0]);
  int kr = k - sm.sel[1];  // keys still needed from bin d1
  const int c1 = int(sm.hist[d1]);
  const bool whole_bin = c1 == kr;
  const bool use_cand = !whole_bin && c1 <= cand_cap;
  __syncthreads();  // every thread has read hist before it is cleared below

  // ---- phase 3: per-segment counts, candidates, digit-2 histogram --------------------
  for (int i = tid; i < kBins; i += NT) sm.hist[i] = 0u;
  int above = 0, match = 0;
  for (int base = lo; base < hi; base += kStep) {
    uint32_t key[KPL];
#pragma unroll
    for (int j = 0; j < KPL; ++j) {
      const int i = base + lane + 64 * j;
      key[j] = i < hi ? key_at(i) : 0u;
    }
    uint64_t bm[KPL];
    int cnt = 0;
#pragma unroll
    for (int j = 0; j < KPL; ++j) {
      const bool in = base + lane + 64 * j < hi;
      above += int(in && (key[j] >> 21) > d1);
      bm[j] = __ballot(in && (key[j] >> 21) == d1);
      cnt += int(__popcll(bm[j]));
    }
    match += cnt;
    if (!whole_bin && cnt != 0) {
      int slot = 0;
      if (use_cand) {
        if (lane == 0) slot = atomicAdd(&sm.ncand, cnt);
        slot = __builtin_amdgcn_readfirstlane(slot);
      }
#pragma unroll
      for (int j = 0; j < KPL; ++j) {
        if ((bm[j] >> lane) & 1ull) {
          atomicAdd(&sm.hist2[(key[j] >> 10) & uint32_t(kBins - 1)], 1u);
          if (use_cand) cand[slot + lane_prefix(bm[j])] = (uint32_t(wave) << 21) | (key[j] & 0x1FFFFFu);
        }
        slot += int(__popcll(bm[j]));
      }
    }
  }
  above = wave_sum(above);
  if (lane == 0) {
    sm.wgt[wave] = whole_bin ? above + match : above;
    sm.weq[wave] = 0;
  }
  __syncthreads();

  // ---- phase 4: T, the k-th largest key, and the per-segment counts -----------------
  uint32_t T;
  if (whole_bin) {
    // all keys of bin d1 are taken: T sits just below the bin (d1 >= 1 here, since
    // a whole bottom bin would mean n == k), and no tie is taken
    T = (d1 << 21) - 1u;
    kr = 0;
  } else {
    select_digit<NT, kBins>(sm, sm.hist2, kr);
    const uint32_t p2 = (d1 << 11) | uint32_t(sm.sel[0]);  // top 22 bits of T
    kr -= sm.sel[1];
    if (use_cand) {
      const int nc = sm.ncand;
      for (int i = tid; i < nc; i += NT) {
        const uint32_t key = (d1 << 21) | (cand[i] & 0x1FFFFFu);
        if ((key >> 10) == p2) atomicAdd(&sm.hist[key & 1023u], 1u);
      }
    } else {
      for (int base = lo; base < hi; base += kStep) {
        uint32_t key[KPL];
#pragma unroll
        for (int j = 0; j < KPL; ++j) {
          const int i = base + lane + 64 * j;
          key[j] = i < hi ? key_at(i) : 0u;
        }
#pragma unroll
        for (int j = 0; j < KPL; ++j)
          if (base + lane + 64 * j < hi && (key[j] >> 10) == p2) atomicAdd(&sm.hist[key[j] & 1023u], 1u);
      }
    }
    __syncthreads();
    select_digit<NT, 1024>(sm, sm.hist, kr);
    T = (p2 << 10) | uint32_t(sm.sel[0]);
    kr -= sm.sel[1];  // ties (keys equal to T) still to take, >= 1
    if (use_cand) {
      const int nc = sm.ncand;
      for (int i = tid; i < nc; i += NT) {
        const uint32_t c = cand[i];
        const uint32_t key = (d1 << 21) | (c & 0x1FFFFFu);
        if (key > T)
          atomicAdd(&sm.wgt[c >> 21], 1);
        else if (key == T)
          atomicAdd(&sm.weq[c >> 21], 1);
      }
    } else {
      int gt = 0, eq = 0;
      for (int base = lo; base < hi; base += kStep) {
        uint32_t key[KPL];
#pragma unroll
        for (int j = 0; j < KPL; ++j) {
          const int i = base + lane + 64 * j;
          key[j] = i < hi ? key_at(i) : 0u;
        }
#pragma unroll
        for (int j = 0; j < KPL; ++j) {
          const bool in = base + lane + 64 * j < hi && (key[j] >> 21) == d1;
          gt += int(in && key[j] > T);
          eq += int(in && key[j] == T);
        }
      }
      gt = wave_sum(gt);
      eq = wave_sum(eq);
      if (lane == 0) {
        sm.wgt[wave] += gt;
        sm.weq[wave] = eq;
      }
    }
    __syncthreads();
  }

  // ---- phase 5: ordered emission ------------------------------------------------------
  int gt_before, eq_before;
  before_wave(sm, wave, lane, gt_before, eq_before);
  int pos = gt_before + min(eq_before, kr);  // output slots taken by earlier segments
  int eq_run = eq_before;                    // ties met before this point
  for (int base = lo; base < hi; base += kStep) {
    uint32_t key[KPL];
#pragma unroll
    for (int j = 0; j < KPL; ++j) {
      const int i = base + lane + 64 * j;
      key[j] = i < hi ? key_at(i) : 0u;
    }
#pragma unroll
    for (int j = 0; j < KPL; ++j) {
      // most steps hold no tie and few selected keys: wave-uniform branches skip the
      // lane-prefix work for them
      const int i = base + lane + 64 * j;
      const bool in = i < hi;
      bool sel = in && key[j] > T;
      const uint64_t beq = __ballot(in && key[j] == T);
      if (beq != 0ull) {
        sel = sel || ((beq >> lane) & 1ull && eq_run + lane_prefix(beq) < kr);
        eq_run += int(__popcll(beq));
      }
      const uint64_t bsel = __ballot(sel);
      if (bsel != 0ull) {
        const int p = pos + lane_prefix(bsel);
        if (sel && p < k) out[p] = i;
        pos += int(__popcll(bsel));
      }
    }
  }
}

// The cached walks take KS sub-steps of 64 * B keys per wave step: in sub-step j lane L
// holds the B consecutive columns base + 64 B j + B L + e, e < B, and a per-lane bit
// mask marks keys (bit B j + e), so a step of 64 B KS keys costs two lane scans instead
// of KS, and stores loop over set bits only (few keys of a row are selected).
constexpr int kSubSteps = 4;

// Output slots of the keys whose bits are set in `sel`, in column order (sub-step,
// then lane, then column): each lane's first slot per sub-step comes from lane scans
// of packed per-sub-step counts (16-bit fields: a sub-step holds at most 64 B keys).
// Writes the columns (relative to the row start) below k; returns pos advanced by the
// wave's selected keys.
template <int B, int KS>
__device__ __forceinline__ int emit_bits(uint32_t sel, int base, int lane, int pos, int k, int32_t *out) {
  static_assert(B * KS <= 32 && KS % 2 == 0, "bit layout");
  constexpr uint32_t kMask = (1u << B) - 1u;
  if (__ballot(sel != 0u) == 0ull) return pos;
  int first[KS], total[KS];
#pragma unroll
  for (int j = 0; j < KS; j += 2) {
    const uint32_t c0 = uint32_t(__builtin_popcount((sel >> (B * j)) & kMask));
    const uint32_t c1 = uint32_t(__builtin_popcount((sel >> (B * (j + 1))) & kMask));
    const uint32_t inc = uint32_t(wave_incl_scan(int(c0 | (c1 << 16))));
    const uint32_t tot = uint32_t(__builtin_amdgcn_readlane(int(inc), 63));
    first[j] = int((inc & 0xFFFFu) - c0);
    first[j + 1] = int((inc >> 16) - c1);
    total[j] = int(tot & 0xFFFFu);
    total[j + 1] = int(tot >> 16);
  }
#pragma unroll
  for (int j = 0; j < KS; ++j) {
    uint32_t m = (sel >> (B * j)) & kMask;
    int p = pos + first[j];
    const int col = base + 64 * B * j + B * lane;
    while (m != 0u) {
      const int e = __builtin_ctz(m);
      m &= m - 1u;
      if (p < k) out[p] = col + e;
      ++p;
    }
    pos += total[j];
  }
  return pos;
}

// Of the keys equal to T (bits of `eq`, same layout), the ones whose rank among the
// row's ties in column order is below kr; eq_run counts the ties met before this step.
template <int B, int KS>
__device__ __forceinline__ uint32_t take_ties(uint32_t eq, int kr, int &eq_run) {
  constexpr uint32_t kMask = (1u << B) - 1u;
  uint32_t take = 0u;
  if (__ballot(eq != 0u) == 0ull) return take;
#pragma unroll
  for (int j = 0; j < KS; ++j) {
    const uint32_t ej = (eq >> (B * j)) & kMask;
    if (__ballot(ej != 0u) != 0ull) {
      const int neq = __builtin_popcount(ej);
      const int inc = wave_incl_scan(neq);
      int r = eq_run + inc - neq;
      uint32_t m = ej;
      while (m != 0u) {
        const int e = __builtin_ctz(m);
        m &= m - 1u;
        take |= uint32_t(r < kr) << (B * j + e);
        ++r;
      }
      eq_run += __builtin_amdgcn_readlane(inc, 63);
    }
  }
  return take;
}

// Ordered emission of the keys above T, for rows with no ties to rank: lane L reads
// column base + 64 i + L of each step (key(c) fetches column c from LDS), so the keys
// selected by one ballot are already in column order, and each selected lane writes
// its column to pos plus the selected lanes below it. Groups at or past hi are not
// read (a wave-uniform test; hi is a multiple of 64 except at the row's end, where the
// zero keys of the padding are never selected). pos is wave-uniform.
template <int NI, typename Key>
__device__ __forceinline__ void emit_above(Key key, uint32_t T, int lo, int hi, int lane, int &pos, int k,
                                           int32_t *out) {
  lo = uniform(lo);
  hi = uniform(hi);
  auto place = [&](const uint32_t (&kv)[NI], int base) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const bool s = kv[i] > T;
      const uint64_t m = __ballot(s);
      if (m != 0ull) {
        const int cnt = __popcll(m);
        // slot: pos plus the selected lanes below this one (pos folded into the count)
        const uint32_t p = __builtin_amdgcn_mbcnt_hi(uint32_t(m >> 32), __builtin_amdgcn_mbcnt_lo(uint32_t(m), uint32_t(pos)));
        int32_t *const dst = reinterpret_cast<int32_t *>(reinterpret_cast<char *>(out) + (p << 2));
        if (pos + cnt <= k) {  // the usual case: every selected lane has a slot
          if (s) *dst = base + 64 * i + lane;
        } else if (s && p < uint32_t(k)) {
          *dst = base + 64 * i + lane;
        }
        pos += cnt;
      }
    }
  };
  int base = lo;
  for (; base + 64 * NI <= hi; base += 64 * NI) {  // whole steps: every load issued at once
    uint32_t kv[NI];
#pragma unroll
    for (int i = 0; i < NI; ++i) kv[i] = key(base + 64 * i + lane);
    place(kv, base);
  }
  if (base < hi) {  // the segment's last, partial step
    uint32_t kv[NI];
#pragma unroll
    for (int i = 0; i < NI; ++i) kv[i] = base + 64 * i < hi ? key(base + 64 * i + lane) : 0u;
    place(kv, base);
  }
}

// Phases 3 to 5 for a row whose keys sit in LDS, padded with zero keys up to a whole
// step (a zero key ranks below every real one: -inf maps to bin 3). The counting walk
// gives each lane four consecutive keys per step, read with one 16-byte load, so a
// step needs no bounds checks; candidate slots come from lane scans of per-lane
// counts. The emission places keys with one ballot per 64 columns when no ties are
// left to rank (emit_above: about six vector instructions per selected group against
// eleven per key for per-lane bit masks and lane scans over four-key groups; B = 32
// decode top-k 10.7 -> 10.4 us), and with the per-lane masks otherwise. Used when the
// selected bin is taken whole or fits the candidate list.
template <int NT>
__device__ __forceinline__ void finish_cached(Smem<NT> &sm, const uint32_t *keys, int n, int k, int32_t *out) {
  constexpr int kStep = 256;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int seg = (n + Cfg<NT>::kWaves * kStep - 1) / (Cfg<NT>::kWaves * kStep) * kStep;
  const int lo = min(n, wave * seg), hi = min(n, lo + seg);

  const uint32_t d1 = uint32_t(sm.sel[0]);
  const uint32_t top = (d1 << 21) | 0x1FFFFFu;  // largest key of bin d1
  int kr = k - sm.sel[1];
  const bool whole_bin = int(sm.hist[d1]) == kr;
  __syncthreads();  // every thread has read hist before it is cleared below

  // ---- phase 3 ----------------------------------------------------------------------
  for (int i = tid; i < kBins; i += NT) sm.hist[i] = 0u;
  int above = 0, match = 0;
  for (int base = lo; base < hi; base += kStep * kSubSteps) {
    uint32_t cm = 0u;  // keys of bin d1
#pragma unroll
    for (int j = 0; j < kSubSteps; ++j) {
      if (base + j * kStep < hi) {
        const v4i kv = *reinterpret_cast<const v4i *>(keys + base + j * kStep + 4 * lane);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const uint32_t key = uint32_t(kv[e]);
          const bool gt = key > top;
          above += __popcll(__ballot(gt));  // a wave total, counted by the scalar unit
          cm |= uint32_t(key >= (d1 << 21) && !gt) << (4 * j + e);  // key in bin d1
        }
      }
    }
    const int nc = __builtin_popcount(cm);
    match += nc;
    if (!whole_bin && __ballot(nc != 0) != 0ull) {
      const int incl = wave_incl_scan(nc);
      const int tot = __builtin_amdgcn_readlane(incl, 63);
      int slot = 0;
      if (lane == 0) slot = atomicAdd(&sm.ncand, tot);
      slot = __builtin_amdgcn_readfirstlane(slot) + incl - nc;
      while (cm != 0u) {
        const int b = __builtin_ctz(cm);
        cm &= cm - 1u;
        const uint32_t key = keys[base + (b >> 2) * kStep + 4 * lane + (b & 3)];
        // the list holds the bin's c1 <= kCand keys; only padding could add more,
        // and only for a row whose k-th key sorts below -inf (a NaN)
        atomicAdd(&sm.hist2[(key >> 10) & uint32_t(kBins - 1)], 1u);
        if (slot < Cfg<NT>::kCand) sm.cand[slot] = (uint32_t(wave) << 21) | (key & 0x1FFFFFu);
        ++slot;
      }
    }
  }
  above = uniform(above);
  match = wave_sum(match);
  if (lane == 0) {
    sm.wgt[wave] = whole_bin ? above + match : above;
    sm.weq[wave] = 0;
  }
  __syncthreads();

  // ---- phase 4 ----------------------------------------------------------------------
  uint32_t T;
  if (whole_bin) {
    T = (d1 << 21) - 1u;  // d1 >= 1: a whole bottom bin would mean n == k
    kr = 0;
  } else {
    select_digit<NT, kBins>(sm, sm.hist2, kr);
    const uint32_t p2 = (d1 << 11) | uint32_t(sm.sel[0]);
    kr -= sm.sel[1];
    const int nc = min(sm.ncand, Cfg<NT>::kCand);
    for (int i = tid; i < nc; i += NT) {
      const uint32_t key = (d1 << 21) | (sm.cand[i] & 0x1FFFFFu);
      if ((key >> 10) == p2) atomicAdd(&sm.hist[key & 1023u], 1u);
    }
    __syncthreads();
    select_digit<NT, 1024>(sm, sm.hist, kr);
    T = (p2 << 10) | uint32_t(sm.sel[0]);
    kr -= sm.sel[1];  // ties (keys equal to T) still to take, >= 1
    if (int(sm.hist[sm.sel[0]]) == kr) {
      // every key equal to T is taken (the usual case): the same set as keys > T - 1,
      // and the emission then has no ties to rank
      T -= 1u;
      kr = 0;
    }
    for (int i = tid; i < nc; i += NT) {
      const uint32_t c = sm.cand[i];
      const uint32_t key = (d1 << 21) | (c & 0x1FFFFFu);
      if (key > T)
        atomicAdd(&sm.wgt[c >> 21], 1);
      else if (key == T)
        atomicAdd(&sm.weq[c >> 21], 1);
    }
    __syncthreads();
  }

  // ---- phase 5 ----------------------------------------------------------------------
  int gt_before, eq_before;
  before_wave(sm, wave, lane, gt_before, eq_before);
  int pos = gt_before + min(eq_before, kr);
  int eq_run = eq_before;
  // rows with ties to place test keys for equality; the others do not
  auto walk = [&](auto ties) {
    for (int base = lo; base < hi; base += kStep * kSubSteps) {
      uint32_t sel = 0u, eq = 0u;
#pragma unroll
      for (int j = 0; j < kSubSteps; ++j) {
        if (base + j * kStep < hi) {
          const v4i kv = *reinterpret_cast<const v4i *>(keys + base + j * kStep + 4 * lane);
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            sel |= uint32_t(uint32_t(kv[e]) > T) << (4 * j + e);
            if constexpr (decltype(ties)::value) eq |= uint32_t(uint32_t(kv[e]) == T) << (4 * j + e);
          }
        }
      }
      // ties in column order: the first kr of the row's ties are taken
      if constexpr (decltype(ties)::value) sel |= take_ties<4, kSubSteps>(eq, kr, eq_run);
      pos = emit_bits<4, kSubSteps>(sel, base, lane, pos, k, out);
    }
  };
  if (kr > 0) {
    walk(std::true_type{});
  } else {
    int p = uniform(pos);
    emit_above<16>([&](int c) { return keys[c]; }, T, lo, hi, lane, p, k, out);
  }
}

// Phases 3 to 5 for a row of more keys than the key cache holds but at most twice as
// many (up to 65536): LDS holds the top 16 bits of every key (zero-padded to whole
// 512-key steps), which settle every key outside bin d1. The walk over them counts
// the keys above the bin and lists the columns of the bin's keys; one gather from
// global memory then fetches those keys' low 16 bits, kept beside their columns, which
// is all digits 2 and 3 need. Once T is known, the candidates sharing T's top 16 bits
// are re-labelled in LDS (one above T's prefix if above T, one below if below), so the
// emission walk decides every key from its 16 bits: above T's prefix, or equal (a tie).
template <int NT>
__device__ __forceinline__ void finish_half(Smem<NT> &sm, uint16_t *top16, const float *lr, int n, int k, int32_t *out) {
  constexpr int kStep = 512;  // eight keys per lane per 16-byte read
  constexpr int kCand = Cfg<NT>::kCand;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int seg = (n + Cfg<NT>::kWaves * kStep - 1) / (Cfg<NT>::kWaves * kStep) * kStep;
  const int lo = min(n, wave * seg), hi = min(n, lo + seg);

  const uint32_t d1 = uint32_t(sm.sel[0]);
  const uint32_t bin_low = d1 << 5, bin_top = (d1 << 5) | 31u;  // 16-bit prefixes of bin d1
  int kr = k - sm.sel[1];
  const bool whole_bin = int(sm.hist[d1]) == kr;
  __syncthreads();  // every thread has read hist before it is cleared below

  // ---- phase 3: counts above the bin, columns of the bin's keys ----------------------
  for (int i = tid; i < kBins; i += NT) sm.hist[i] = 0u;
  int above = 0, match = 0;
  for (int base = lo; base < hi; base += kStep * kSubSteps) {
    uint32_t inbin = 0u;
#pragma unroll
    for (int j = 0; j < kSubSteps; ++j) {
      if (base + j * kStep < hi) {
        const v4i raw = *reinterpret_cast<const v4i *>(top16 + base + j * kStep + 8 * lane);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const uint32_t t = (uint32_t(raw[e >> 1]) >> (16 * (e & 1))) & 0xFFFFu;
          // prefixes of bin d1 are [32 d1, 32 d1 + 31]: compared whole, no field extract
          const bool gt = t > bin_top;
          above += __popcll(__ballot(gt));  // a wave total, counted by the scalar unit
          inbin |= uint32_t(t >= bin_low && !gt) << (8 * j + e);
        }
      }
    }
    const int nc = __builtin_popcount(inbin);
    match += nc;
    if (!whole_bin && __ballot(nc != 0) != 0ull) {
      const int incl = wave_incl_scan(nc);
      const int tot = __builtin_amdgcn_readlane(incl, 63);
      int slot = 0;
      if (lane == 0) slot = atomicAdd(&sm.ncand, tot);
      slot = __builtin_amdgcn_readfirstlane(slot) + incl - nc;
      while (inbin != 0u) {
        const int b = __builtin_ctz(inbin);
        inbin &= inbin - 1u;
        if (slot < kCand) sm.cand[slot] = uint32_t(base + (b >> 3) * kStep + 8 * lane + (b & 7));
        ++slot;
      }
    }
  }
  above = uniform(above);
  match = wave_sum(match);
  if (lane == 0) {
    sm.wgt[wave] = whole_bin ? above + match : above;
    sm.weq[wave] = 0;
  }
  __syncthreads();

  // ---- phase 4: T; per-wave counts; ambiguous candidates re-labelled ------------------
  uint32_t T;
  if (whole_bin) {
    T = (d1 << 21) - 1u;  // d1 >= 1: a whole bottom bin would mean n == k
    kr = 0;
  } else {
    const int nc = min(sm.ncand, kCand);
    for (int i = tid; i < nc; i += NT) {
      const uint32_t col = sm.cand[i];
      const uint32_t key = order_key(lr[col]);
      atomicAdd(&sm.hist2[(key >> 10) & uint32_t(kBins - 1)], 1u);
      sm.cand[i] = (col << 16) | (key & 0xFFFFu);
    }
    __syncthreads();
    select_digit<NT, kBins>(sm, sm.hist2, kr);
    const uint32_t p2 = (d1 << 11) | uint32_t(sm.sel[0]);
    kr -= sm.sel[1];
    for (int i = tid; i < nc; i += NT) {
      const uint32_t c = sm.cand[i];
      const uint32_t key = (uint32_t(top16[c >> 16]) << 16) | (c & 0xFFFFu);
      if ((key >> 10) == p2) atomicAdd(&sm.hist[key & 1023u], 1u);
    }
    __syncthreads();
    select_digit<NT, 1024>(sm, sm.hist, kr);
    T = (p2 << 10) | uint32_t(sm.sel[0]);
    kr -= sm.sel[1];  // ties (keys equal to T) still to take, >= 1
    if (int(sm.hist[sm.sel[0]]) == kr) {
      T -= 1u;  // every key equal to T is taken: keys > T - 1, no ties to rank
      kr = 0;
    }
    const uint32_t tp = T >> 16;
    for (int i = tid; i < nc; i += NT) {
      const uint32_t c = sm.cand[i];
      const uint32_t col = c >> 16;
      const uint32_t t = top16[col];
      const uint32_t key = (t << 16) | (c & 0xFFFFu);
      const int w = int(col) / seg;
      if (key > T)
        atomicAdd(&sm.wgt[w], 1);
      else if (key == T)
        atomicAdd(&sm.weq[w], 1);
      if (t == tp) top16[col] = uint16_t(key > T ? min(tp + 1u, 0xFFFFu) : key < T ? max(tp, 1u) - 1u : tp);
    }
    __syncthreads();
  }

  // ---- phase 5: emission from the 16-bit keys --------------------------------------
  const uint32_t tp = T >> 16;
  int gt_before, eq_before;
  before_wave(sm, wave, lane, gt_before, eq_before);
  int pos = gt_before + min(eq_before, kr);
  int eq_run = eq_before;
  auto walk = [&](auto ties) {
    for (int base = lo; base < hi; base += kStep * kSubSteps) {
      uint32_t sel = 0u, eq = 0u;  // bit 8 j + e: column base + kStep j + 8 lane + e
#pragma unroll
      for (int j = 0; j < kSubSteps; ++j) {
        if (base + j * kStep < hi) {
          const v4i raw = *reinterpret_cast<const v4i *>(top16 + base + j * kStep + 8 * lane);
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const uint32_t t = (uint32_t(raw[e >> 1]) >> (16 * (e & 1))) & 0xFFFFu;
            sel |= uint32_t(t > tp) << (8 * j + e);
            if constexpr (decltype(ties)::value) eq |= uint32_t(t == tp) << (8 * j + e);
          }
        }
      }
      if constexpr (decltype(ties)::value) sel |= take_ties<8, kSubSteps>(eq, kr, eq_run);
      pos = emit_bits<8, kSubSteps>(sel, base, lane, pos, k, out);
    }
  };
  if (kr > 0)
    walk(std::true_type{});
  else
    walk(std::false_type{});
}

static_assert(sizeof(Smem<1024>) + kMaxCache * sizeof(uint32_t) <= 160 * 1024, "LDS of a workgroup");

template <int NT>
__global__ __launch_bounds__(NT) void topk_kernel(TopkArgs a, int cache_cap) {
  extern __shared__ __attribute__((aligned(16))) uint32_t s_keys[];  // cache_cap keys, rounded up to 256
  __shared__ Smem<NT> sm;

  const int tid = threadIdx.x;
  const int row = blockIdx.x;
  const int start = a.row_start ? min(max(a.row_start[row], 0), a.width) : 0;
  const int e_in = max(a.row_end[row], 0);
  const int end = min(a.end_div == 1 ? e_in : e_in / a.end_div + (e_in % a.end_div != 0), a.width);
  IDX_DEBUG_NOTE((a.row_start && (a.row_start[row] < 0 || a.row_start[row] > a.width)) || a.row_end[row] < 0 ||
                 (a.end_div == 1 ? e_in : e_in / a.end_div + (e_in % a.end_div != 0)) > a.width,
             IDX_DBG_LENGTH);
  const int n = max(end - start, 0);
  const int k = a.k;
  int32_t *out = a.out + int64_t(row) * a.out_row_stride;

  if (n <= k) {
    for (int i = tid; i < k; i += NT) out[i] = i < n ? i : -1;
    return;
  }
  const float *lr = a.logits + int64_t(row) * a.logits_row_stride + start;
  const bool cached = n <= cache_cap;
  const bool half = !cached && n <= 2 * cache_cap;  // top 16 bits of every key fit the cache
  uint16_t *s_top16 = reinterpret_cast<uint16_t *>(s_keys);

  // ---- phases 1 and 2 -------------------------------------------------------------------
  // kUnroll independent loads per thread are issued before any of them is used, so a
  // batch costs one memory round trip. A 16-byte aligned row is read four keys per
  // lane with range-checked buffer loads (zero past the row, no branch per key) and
  // cached with one 16-byte LDS store per four keys, zero keys filling the last step.
  for (int i = tid; i < kBins; i += NT) {
    sm.hist[i] = 0u;
    sm.hist2[i] = 0u;
  }
  if (tid == 0) sm.ncand = 0;
  __syncthreads();
  const int n_pad = half ? (n + 511) & ~511 : (n + 255) & ~255;  // whole steps of the cached walks
  // two counters per bin, side by side in hist | hist2 (different LDS banks), picked by
  // lane parity: lanes of one instruction that share a bin (logits crowd into few
  // bins) collide half as often; summed into hist below
  static_assert(offsetof(Smem<NT>, hist2) == offsetof(Smem<NT>, hist) + kBins * sizeof(uint32_t),
                "hist2 follows hist");
  uint32_t *pairs = sm.hist;
  const int lane = tid & 63;
  if ((reinterpret_cast<uintptr_t>(lr) & 15) == 0) {
    const buffer_rsrc rs = make_rsrc(lr, uint32_t(n) * 4u);
    constexpr int kGroups = kUnroll / 4;
    constexpr int kBatch = kUnroll * NT;  // keys per batch of loads
    auto issue = [&](v4i (&x)[kGroups], int base) {
#pragma unroll
      for (int u = 0; u < kGroups; ++u) x[u] = buffer_load16(rs, uint32_t(base + (u * NT + tid) * 4) * 4u);
    };
    auto consume = [&](const v4i (&x)[kGroups], int base) {
#pragma unroll
      for (int u = 0; u < kGroups; ++u) {
        const int i = base + (u * NT + tid) * 4;
        if (i < n_pad) {
          uint32_t kk[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) kk[e] = i + e < n ? order_key(__int_as_float(x[u][e])) : 0u;
          if (cached) *reinterpret_cast<v4i *>(s_keys + i) = v4i{int(kk[0]), int(kk[1]), int(kk[2]), int(kk[3])};
          if (half)
            *reinterpret_cast<uint2 *>(s_top16 + i) = make_uint2((kk[0] >> 16) | (kk[1] & 0xFFFF0000u),
                                                                 (kk[2] >> 16) | (kk[3] & 0xFFFF0000u));
          if (i < n) {
#pragma unroll
            for (int e = 0; e < 4; ++e) atomicAdd(&pairs[2 * (kk[e] >> 21) + (lane & 1)], i + e < n ? 1u : 0u);
          }
        }
      }
    };
    // two register sets: the next batch's loads are in flight while this one is used
    // (a row longer than one batch no longer pays a memory round trip per batch)
    v4i xa[kGroups], xb[kGroups];
    issue(xa, 0);
    for (int base = 0; base < n; base += 2 * kBatch) {
      if (base + kBatch < n) issue(xb, base + kBatch);
      consume(xa, base);
      if (base + 2 * kBatch < n) issue(xa, base + 2 * kBatch);
      if (base + kBatch < n) consume(xb, base + kBatch);
    }
  } else {
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
          if (half) s_top16[i] = uint16_t(key >> 16);
          atomicAdd(&pairs[2 * (key >> 21) + (lane & 1)], 1u);
        }
      }
    }
    // zero keys past the row up to a whole step of the cached walks
    if (cached)
      for (int i = n + tid; i < n_pad; i += NT) s_keys[i] = 0u;
    if (half)
      for (int i = n + tid; i < n_pad; i += NT) s_top16[i] = 0u;
  }
  __syncthreads();
  {
    constexpr int kPerT = kBins / NT;  // bins summed by each thread
    uint32_t sum[kPerT];
#pragma unroll
    for (int j = 0; j < kPerT; ++j) {
      const int b = tid * kPerT + j;
      sum[j] = pairs[2 * b] + pairs[2 * b + 1];
    }
    __syncthreads();
#pragma unroll
    for (int j = 0; j < kPerT; ++j) {
      sm.hist[tid * kPerT + j] = sum[j];
      sm.hist2[tid * kPerT + j] = 0u;
    }
  }
  __syncthreads();
  select_digit<NT, kBins>(sm, sm.hist, k);

  const int c1 = int(sm.hist[sm.sel[0]]);
  if (cached && (c1 == k - sm.sel[1] || c1 <= Cfg<NT>::kCand))
    finish_cached<NT>(sm, s_keys, n, k, out);
  else if (cached)
    finish_row<NT, 8>(sm, [&](int i) { return s_keys[i]; }, n, k, out, sm.cand, Cfg<NT>::kCand);
  else if (half && (c1 == k - sm.sel[1] || c1 <= Cfg<NT>::kCand))
    finish_half<NT>(sm, s_top16, lr, n, k, out);
  else
    finish_row<NT, 16>(sm, [&](int i) { return order_key(lr[i]); }, n, k, out, s_keys, cache_cap);
}

}  // namespace

hipError_t launch_topk(const TopkArgs &a, int num_cus, void *scratch, size_t scratch_bytes, hipStream_t stream) {
  // Few, long rows: several workgroups share each row (topk_coop.hip) when the
  // caller's scratch holds the rows' records and the rows are 16-byte aligned. Up to
  // 65536 keys a row fits one workgroup's LDS (whole keys or their top 16 bits) and the
  // single-workgroup kernel is as fast or faster: the units of a shared row meet
  // through device memory, about a microsecond a round trip (measured on an MI355X:
  // 64 rows x 65536, 35 us shared against 28 us; 16 rows x 131072, 22 us against 76 us;
  // one row of 2^20 keys, 41 us against 591 us).
  const bool rows16 = (reinterpret_cast<uintptr_t>(a.logits) & 15) == 0 && a.logits_row_stride % 4 == 0;
  if (scratch && a.width > kMaxCache * 2 && a.rows <= kCoopMaxRows && scratch_bytes >= topk_scratch_bytes(a.rows) &&
      rows16 && int64_t(a.rows) * (int64_t(a.width) + 4) < (int64_t(1) << 30)) {
    const int grid = topk_coop_grid(num_cus, a.rows, a.width);
    if (grid > a.rows) return launch_topk_coop(a, scratch, grid, stream);
  }
  // Many rows of at most 8192 columns: one 256-thread workgroup per row with the row's
  // keys in registers through the selection (topk_coop.hip), no key cache in LDS, so
  // five workgroups fit a compute unit instead of four (8192 rows of the causal
  // 8192-key chunk: 89 -> 63 us on an MI355X). With fewer rows the 1024-thread
  // workgroups below finish each row sooner (a 64-row candidate pool: 6.2 against
  // 8.6 us), and a 1024-thread register version for rows up to 32768 was slower than
  // the LDS cache on a 32-row decode step (15.0 against 11.7 us).
  if (rows16 && a.rows >= 1024 && a.width <= topk_solo_cap()) return launch_topk_solo(a, stream);
  // Many rows (narrow workgroups): a key cache of half the width, so rows longer than
  // it keep 16-bit key prefixes instead (finish_half) and four workgroups fit a CU's
  // LDS instead of three (8192 rows of 8192 keys: top-k 98 -> 86 us).
  const int cap = a.rows >= 1024 ? max(256, ((min(a.width, kMaxCache) / 2) + 255) & ~255) : min(a.width, kMaxCache);
  const size_t lds = size_t((cap + 255) & ~255) * sizeof(uint32_t);  // whole steps of the cached walk
  // the dynamic LDS limit is raised once per device (calls from several threads or
  // devices serialise on the flag)
  {
    constexpr int kDevices = 64;
    static std::mutex mu;
    static bool lds_raised[kDevices] = {};
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    std::lock_guard<std::mutex> lock(mu);
    if (dev < 0 || dev >= kDevices || !lds_raised[dev]) {
      e = hipFuncSetAttribute(reinterpret_cast<const void *>(&topk_kernel<1024>),
                              hipFuncAttributeMaxDynamicSharedMemorySize, int(kMaxCache * sizeof(uint32_t)));
      if (e != hipSuccess) return e;
      e = hipFuncSetAttribute(reinterpret_cast<const void *>(&topk_kernel<256>),
                              hipFuncAttributeMaxDynamicSharedMemorySize, int(kMaxCache * sizeof(uint32_t)));
      if (e != hipSuccess) return e;
      if (dev >= 0 && dev < kDevices) lds_raised[dev] = true;
    }
  }
  // few rows: the widest workgroup per row; many rows: narrower ones, more per CU
  if (a.rows >= 1024)
    topk_kernel<256><<<dim3(a.rows), 256, lds, stream>>>(a, cap);
  else
    topk_kernel<1024><<<dim3(a.rows), 1024, lds, stream>>>(a, cap);
  return hipGetLastError();
}

IDX_DEBUG_READER(debug_word_topk)

}  // namespace idx
