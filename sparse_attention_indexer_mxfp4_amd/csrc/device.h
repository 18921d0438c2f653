// Device-side building blocks shared by the indexer kernels (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace idx {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef int v4i __attribute__((ext_vector_type(4)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef float v2f __attribute__((ext_vector_type(2)));

// ---------------------------------------------------------------------------------
// Matrix cores: v_mfma_f32_16x16x128_f8f6f4 (gfx950), one 16x16 output tile with a
// 128-deep contraction per instruction.
//
// Operand layout (checked on the device): lane L of A supplies row L % 16 and lane
// L of B column L % 16, each with the 32 contraction elements of K-group L / 16
// (32 bytes of e4m3, or 16 bytes of packed e2m1). C lands with rows
// 4 * (L / 16) + j, j = 0..3, and column L % 16 in lane L. Which 32 of the 128
// contraction indices a K-group holds does not matter as long as A and B agree, so
// the kernels pick whatever byte order loads best. In the scaled fp4 form lane L's
// scale byte multiplies its own 32-element block by 2^(byte - 127).
// ---------------------------------------------------------------------------------
__device__ __forceinline__ v4f mfma_fp8(const v8i &a, const v8i &b) {
  const v4f zero = {0.f, 0.f, 0.f, 0.f};
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, zero, 0, 0, 0, 0, 0, 0);
}

__device__ __forceinline__ v4f mfma_fp4(const v8i &a, const v8i &b, int scale_a, int scale_b) {
  const v4f zero = {0.f, 0.f, 0.f, 0.f};
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, zero, 4, 4, 0, scale_a, 0, scale_b);
}

// Sum of x over the four lanes L, L^16, L^32, L^48 (the four K-groups / C row
// groups of an MFMA tile); every lane receives the total.
__device__ __forceinline__ float sum_row_groups(float x) {
  x += __shfl_xor(x, 16);
  x += __shfl_xor(x, 32);
  return x;
}

// Four partial sums per lane, p[kg] for the 16 keys kg*16 + L%16, reduced over the
// four lane groups and delivered transposed: lane L gets the total of
// p[L/16] over lanes L%16, L%16+16, L%16+32, L%16+48, i.e. the full sum for key L
// of a 64-key chunk. v_permlane32_swap exchanges the upper 32 lanes of its first
// operand with the lower 32 of its second, v_permlane16_swap the odd 16-lane rows of
// the first with the even rows of the second; three swaps and three adds replace
// eight cross-lane shuffles.
__device__ __forceinline__ float transpose_reduce4(const float (&p)[4]) {
  const auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(p[0]), __float_as_uint(p[2]), false, false);
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(p[1]), __float_as_uint(p[3]), false, false);
  const float s02 = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const float s13 = __uint_as_float(b[0]) + __uint_as_float(b[1]);
  const auto c = __builtin_amdgcn_permlane16_swap(__float_as_uint(s02), __float_as_uint(s13), false, false);
  return __uint_as_float(c[0]) + __uint_as_float(c[1]);
}

// max of x over the 16 lanes of a DPP row (every lane receives it): rotations by
// 8, 4, 2 and 1 lanes within the row
__device__ __forceinline__ float row16_max(float x) {
  x = fmaxf(x, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x128, 0xF, 0xF, false)));  // row_ror:8
  x = fmaxf(x, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x124, 0xF, 0xF, false)));  // row_ror:4
  x = fmaxf(x, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x122, 0xF, 0xF, false)));  // row_ror:2
  x = fmaxf(x, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x121, 0xF, 0xF, false)));  // row_ror:1
  return x;
}

// max of x over aligned groups of `group` lanes (16, 32 or 64); every lane receives
// its group's. Past a row, a swap with itself hands each lane its neighbouring row
// (permlane16) or half (permlane32).
__device__ __forceinline__ float group_max(float x, int group) {
  x = row16_max(x);
  if (group >= 32) {
    const auto s = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    x = fmaxf(__uint_as_float(s[0]), __uint_as_float(s[1]));
  }
  if (group >= 64) {
    const auto s = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    x = fmaxf(__uint_as_float(s[0]), __uint_as_float(s[1]));
  }
  return x;
}

// 4x4 transpose across the four 16-lane groups: on return r[i] in lane group g holds
// what r[g] held in lane group i (same lane within the group). Two permlane32 swaps
// then two permlane16 swaps, no arithmetic.
__device__ __forceinline__ void transpose4(float (&r)[4]) {
  const auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(r[0]), __float_as_uint(r[2]), false, false);
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(r[1]), __float_as_uint(r[3]), false, false);
  const auto c = __builtin_amdgcn_permlane16_swap(a[0], b[0], false, false);
  const auto d = __builtin_amdgcn_permlane16_swap(a[1], b[1], false, false);
  r[0] = __uint_as_float(c[0]);
  r[1] = __uint_as_float(c[1]);
  r[2] = __uint_as_float(d[0]);
  r[3] = __uint_as_float(d[1]);
}

__device__ __forceinline__ v4i load16(const void *p) { return *reinterpret_cast<const v4i *>(p); }

// ---------------------------------------------------------------------------------
// Buffer memory operations: a 128-bit resource (base address, size in bytes) held in
// scalar registers. An access whose byte offset is not below the size touches no
// memory: a load returns zeros and a store is dropped. Range checks cost nothing
// and leave the code free of branches.
// ---------------------------------------------------------------------------------
typedef __amdgpu_buffer_rsrc_t buffer_rsrc;

// a byte count clamped to what a resource can describe
__device__ __forceinline__ uint32_t range_bytes(int64_t bytes) {
  return bytes <= 0 ? 0u : (bytes >= int64_t(0x7FFFFFFF) ? 0x7FFFFFFFu : uint32_t(bytes));
}

__device__ __forceinline__ buffer_rsrc make_rsrc(const void *base, uint32_t bytes) {
  // dword 3: raw (untyped) 32-bit access, the value the gfx9 family expects
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), 0, int(bytes), 0x00020000);
}

__device__ __forceinline__ v4i buffer_load16(buffer_rsrc r, uint32_t off) {
  return __builtin_bit_cast(v4i, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
}

__device__ __forceinline__ float buffer_load_f32(buffer_rsrc r, uint32_t off) {
  return __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0));
}

__device__ __forceinline__ void buffer_store_f32(float x, buffer_rsrc r, uint32_t off) {
  __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(x), r, off, 0, 0);
}

// Streaming store (non-temporal cache policy): output that is not read again by the
// kernel should not push reusable lines (K tiles) out of L2.
__device__ __forceinline__ void buffer_store_f32_nt(float x, buffer_rsrc r, uint32_t off) {
  __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(x), r, off, 0, 2);
}

// max(x, 0) as one integer max on the bit pattern: negative floats are negative
// integers, so they (and -0.0) become +0.0 and non-negative floats pass unchanged.
// fmaxf would first canonicalise its input (a second VALU op) under IEEE mode.
__device__ __forceinline__ float relu(float x) { return __int_as_float(max(__float_as_int(x), 0)); }

// Makes x a value produced at this point of the program (an empty asm statement that
// reads and writes it): the computation of x can no longer be moved past it.
__device__ __forceinline__ void pin(float &x) { asm volatile("" : "+v"(x)); }

// A value the compiler may treat as wavefront-uniform (kept in a scalar register).
__device__ __forceinline__ int uniform(int x) { return __builtin_amdgcn_readfirstlane(x); }

__device__ __forceinline__ v8i cat(const v4i &lo, const v4i &hi) {
  v8i r;
  r[0] = lo[0]; r[1] = lo[1]; r[2] = lo[2]; r[3] = lo[3];
  r[4] = hi[0]; r[5] = hi[1]; r[6] = hi[2]; r[7] = hi[3];
  return r;
}

__device__ __forceinline__ v8i zero8() {
  v8i r = {0, 0, 0, 0, 0, 0, 0, 0};
  return r;
}

__device__ __forceinline__ float neg_inf() { return -__builtin_inff(); }

// -inf into row[from, to) by one wavefront (lane = lane index), 16-byte streaming
// stores; `from` is a multiple of 4 and the row is 16-byte aligned.
__device__ __forceinline__ void fill_neg_inf(float *row, int from, int to, int lane) {
  const float ninf = neg_inf();
  for (int c = from + 4 * lane; c < to; c += 256) {
    if (c + 4 <= to) {
      __builtin_nontemporal_store(v4f{ninf, ninf, ninf, ninf}, reinterpret_cast<v4f *>(row + c));
    } else {
      for (int i = 0; i < 4 && c + i < to; ++i) __builtin_nontemporal_store(ninf, row + c + i);
    }
  }
}

// One step of a reduce-scatter over the 16 lanes of a DPP row. x[0..2*HALF) holds
// partial sums; the DPP control pairs each lane with one that differs in the bit
// `upper` tests (and possibly lower bits). The lane keeps the half selected by that
// bit, adds the partner's copy of the same half, and on return x[0..HALF) holds it.
template <int CTRL, int HALF>
__device__ __forceinline__ void reduce_scatter_step(float (&x)[32], bool upper) {
#pragma unroll
  for (int j = 0; j < HALF; ++j) {
    const float keep = upper ? x[j + HALF] : x[j];
    const float send = upper ? x[j] : x[j + HALF];
    x[j] = keep + __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(send), CTRL, 0xF, 0xF, false));
  }
}

// ---------------------------------------------------------------------------------
// Integer scans and radix-select helpers (top-k).
// ---------------------------------------------------------------------------------

// Order-preserving 32-bit key of a float: larger float, larger key; -0.0 ranks with
// +0.0. The smallest key of a non-NaN float is that of -inf (0x007FFFFF), so 0 can
// stand for "no key".
__device__ __forceinline__ uint32_t order_key(float x) {
  // x + 0.0 turns -0.0 into +0.0 and leaves every other non-NaN float as it is
  // (fp32 denormals are kept: the library builds without flushing them)
  const uint32_t u = __float_as_uint(x + 0.0f);
  return u ^ (uint32_t(int32_t(u) >> 31) | 0x80000000u);
}

// number of set bits of mask below this lane
__device__ __forceinline__ int lane_prefix(uint64_t mask) {
  return __builtin_amdgcn_mbcnt_hi(uint32_t(mask >> 32), __builtin_amdgcn_mbcnt_lo(uint32_t(mask), 0u));
}

// Inclusive prefix sum over the 64 lanes with DPP moves (no LDS traffic): shifts of
// 1, 2, 4 and 8 lanes inside each 16-lane row, then the last lane of rows 0 and 2
// broadcast into rows 1 and 3, and lane 31 into rows 2 and 3. Lanes a move does not
// reach add 0.
__device__ __forceinline__ int wave_incl_scan(int x) {
  x += __builtin_amdgcn_update_dpp(0, x, 0x111, 0xF, 0xF, false);  // row_shr:1
  x += __builtin_amdgcn_update_dpp(0, x, 0x112, 0xF, 0xF, false);  // row_shr:2
  x += __builtin_amdgcn_update_dpp(0, x, 0x114, 0xF, 0xF, false);  // row_shr:4
  x += __builtin_amdgcn_update_dpp(0, x, 0x118, 0xF, 0xF, false);  // row_shr:8
  x += __builtin_amdgcn_update_dpp(0, x, 0x142, 0xA, 0xF, false);  // row_bcast:15
  x += __builtin_amdgcn_update_dpp(0, x, 0x143, 0xC, 0xF, false);  // row_bcast:31
  return x;
}

__device__ __forceinline__ int wave_sum(int x) { return __builtin_amdgcn_readlane(wave_incl_scan(x), 63); }

// Exclusive prefix sum of one value per thread over a workgroup of NT threads;
// returns the thread's offset and the workgroup total in *total. `scratch` holds
// NT / 64 ints of LDS. Contains one barrier; callers barrier again before reusing
// scratch.
template <int NT>
__device__ __forceinline__ int block_excl_scan(int v, int *scratch, int *total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int x = wave_incl_scan(v);
  if (lane == 63) scratch[wave] = x;
  __syncthreads();
  int before = 0, all = 0;
#pragma unroll
  for (int w = 0; w < NT / 64; ++w) {
    const int t = scratch[w];
    if (w < wave) before += t;
    all += t;
  }
  *total = all;
  return before + x - v;
}

// Radix-select step: wave 0 finds the bin d of hist[0..NBINS) holding the kr-th
// largest key (larger bin = larger key), i.e. (keys in bins above d) < kr <= (keys in
// bins at or above d), and stores d in sel[0] and the count above it in sel[1]; the
// caller synchronises before reading them. Two parallel steps, no serial walk: each
// lane sums its NBINS/64 bins and a lane scan with a ballot names the lane whose bins
// hold the kr-th key; then NBINS/64 lanes take one of that lane's bins each (highest
// first), and a second scan and ballot name the bin.
template <int NBINS>
__device__ __forceinline__ void select_bin(const uint32_t *hist, int kr, int *sel) {
  static_assert(NBINS % 256 == 0, "whole 16-byte loads per lane");
  constexpr int kPer = NBINS / 64;
  if ((threadIdx.x >> 6) == 0) {
    const int lane = threadIdx.x & 63;
    const int first = NBINS - (lane + 1) * kPer;  // this lane: bins [first, first + kPer), lane 0 highest
    int local = 0;
#pragma unroll
    for (int q = 0; q < kPer / 4; ++q) {
      const v4i x = *reinterpret_cast<const v4i *>(hist + first + 4 * q);
      local += (x[0] + x[1]) + (x[2] + x[3]);
    }
    const int incl = wave_incl_scan(local);
    const int run = incl - local;
    const uint64_t hit = __ballot(run < kr && incl >= kr);
    const int t = hit ? __builtin_ctzll(hit) : 0;  // one lane when 1 <= kr <= total
    const int run_t = __builtin_amdgcn_readlane(run, t);
    const int first_t = NBINS - (t + 1) * kPer;
    const int v = lane < kPer ? int(hist[first_t + kPer - 1 - lane]) : 0;
    const int iv = wave_incl_scan(v);
    const uint64_t hit2 = __ballot(lane < kPer && run_t + iv >= kr);
    const int j = hit2 ? __builtin_ctzll(hit2) : 0;
    if (lane == j) {
      sel[0] = first_t + kPer - 1 - j;
      sel[1] = run_t + iv - v;
    }
  }
}

// ---------------------------------------------------------------------------------
// Encoders of the K store and the query quantiser. Integer-exact, so they agree
// bit for bit with any other correct implementation of the same rounding.
// ---------------------------------------------------------------------------------

// fp32 -> e4m3fn (OCP) byte: nearest finite value, ties to even, saturating at
// +-448. NaN maps to the NaN code.
__device__ __forceinline__ uint32_t enc_e4m3(float x) {
  const uint32_t sign = (__float_as_uint(x) >> 24) & 0x80u;
  const float a = fabsf(x);
  if (!(a == a)) return sign | 0x7Fu;
  uint32_t code;
  if (a >= 448.0f) {
    code = 0x7Eu;
  } else if (a < 0.015625f) {
    // below 2^-6 the e4m3 grid is m * 2^-9, m = 0..7 (m = 8 is the smallest
    // normal, whose code is also 8); a * 512 is exact and rintf rounds to even
    code = uint32_t(rintf(a * 512.0f));
  } else {
    int e = int((__float_as_uint(a) >> 23) & 0xFFu) - 127;               // -6..8
    const float m = __uint_as_float((__float_as_uint(a) & 0x7FFFFFu) | 0x3F800000u);  // [1, 2)
    uint32_t qm = uint32_t(rintf(m * 8.0f));                              // 8..16
    if (qm == 16u) {
      qm = 8u;
      e += 1;
    }
    code = (uint32_t(e + 7) << 3) | (qm - 8u);
  }
  return sign | code;
}

// fp32 -> e2m1 nibble: nearest of {0, .5, 1, 1.5, 2, 3, 4, 6}, ties to the even
// code, saturating at +-6. The thresholds are the midpoints; a midpoint goes to
// whichever neighbour has the even code.
__device__ __forceinline__ uint32_t enc_e2m1(float x) {
  const float a = fabsf(x);
  const uint32_t c = uint32_t(a > 0.25f) + uint32_t(a >= 0.75f) + uint32_t(a > 1.25f) + uint32_t(a >= 1.75f) +
                     uint32_t(a > 2.5f) + uint32_t(a >= 3.5f) + uint32_t(a > 5.0f);
  return ((__float_as_uint(x) >> 28) & 0x8u) | c;
}

// Smallest e8m0 byte b in [0, 254] with amax <= 6 * 2^(b - 127), for finite
// amax >= 0. Writing amax = f * 2^(E - 127) with f in [1, 2): the bound holds at
// b = E - 2 when f <= 1.5 and needs b = E - 1 when f > 1.5; subnormal and zero
// amax give a negative value, clamped to 0.
__device__ __forceinline__ int e8m0_bits(float amax) {
  const uint32_t u = __float_as_uint(amax);
  const int E = int((u >> 23) & 0xFFu);
  const int b = E - 2 + int((u & 0x7FFFFFu) > 0x400000u);
  return b < 0 ? 0 : (b > 254 ? 254 : b);
}

// 2^(127 - b) for b in [0, 253] (normal fp32 throughout that range).
__device__ __forceinline__ float e8m0_inv_scale(int b) {
  const int ex = 254 - b;
  return __uint_as_float(uint32_t(ex < 1 ? 1 : ex) << 23);
}

__device__ __forceinline__ float bf16_to_f32(uint16_t h) { return __uint_as_float(uint32_t(h) << 16); }

// e4m3fn (OCP) byte -> fp32, exact (NaN codes are not expected).
__device__ __forceinline__ float dec_e4m3(uint32_t b) {
  const uint32_t e = (b >> 3) & 15u, m = b & 7u;
  const float mag = e ? __uint_as_float(((e + 120u) << 23) | (m << 20)) : float(m) * 0.001953125f;  // m * 2^-9
  return (b & 0x80u) ? -mag : mag;
}

}  // namespace idx
