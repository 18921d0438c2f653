// Quantisers that feed the indexer: the K store (quantise a key row and write it into
// its cache slot) and the query quantiser. Page "vllm.models.deepseek_v41.amd.rocm",
// rocm_mxfp4_indexer_k_store and rocm_mxfp4_indexer_q_quant (their quantise-and-write
// part).
//
// K store: sixteen lanes per 128-value key (four keys per wavefront), lane l of a key
// holding elements 8l .. 8l+7 from two 16-byte loads; maxima reduce over the 16 lanes
// (fp8) or over 4 lanes (an MXFP4 block of 32) with DPP moves. The fused variant
// applies RMSNorm and GPT-J RoPE before quantising (rocm_mxfp4_indexer_k_store on the
// same page hands the cache op the pre-norm key, its position, the rotary table and
// the norm weight). The fused query op (rocm_mxfp4_indexer_q_quant) rotates, quantises
// and scales the weights with the same lane layout. The plain query quantiser keeps
// one wavefront per 128-value row, lane L holding elements 2L and 2L+1.
//
//   fp8 K   scale = amax / 448 (IEEE fp32 division; 1.0 for an all-zero row), value
//           e4m3(k / scale) rounded to nearest even and saturated; written into the
//           block-flat page (values at entry*128, fp32 scale at P*128 + 4*entry).
//   fp8 q   e4m3(q), no scale.
//   MXFP4   per 32-value block, e8m0 byte b = smallest in [0, 254] with
//           amax <= 6 * 2^(b - 127); value e2m1(x * 2^(127 - b)) rounded to nearest
//           even; element 2i in the low nibble of byte i. The key goes to the run
//           layout: packed byte j of entry e at run*1024 + (j/16)*256 + (e%16)*16 + j%16,
//           scale i at P*64 + run*64 + i*16 + e%16 (run = e/16); the query goes to
//           [T, H, 64] bytes plus one int32 per head, byte i for block i.
#include "debug.h"
#include "device.h"
#include "launch.h"

namespace idx {
namespace {

constexpr int kRowsPerWG = 4;  // one wavefront per row, four per workgroup

__device__ __forceinline__ void load_pair(const void *base, int dtype, int64_t elem, float &x0, float &x1) {
  if (dtype == 0) {
    const float *p = static_cast<const float *>(base) + elem;
    x0 = p[0];
    x1 = p[1];
  } else {
    const uint16_t *p = static_cast<const uint16_t *>(base) + elem;
    x0 = bf16_to_f32(p[0]);
    x1 = bf16_to_f32(p[1]);
  }
}

__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) x = fmaxf(x, __shfl_xor(x, off));
  return x;
}

__device__ __forceinline__ float group16_max(float x) {
#pragma unroll
  for (int off = 8; off > 0; off >>= 1) x = fmaxf(x, __shfl_xor(x, off));
  return x;
}

constexpr int kKeysPerWG = 16;  // sixteen lanes per key

// sum over the 16 lanes of a DPP row (every lane receives it)
__device__ __forceinline__ float row16_sum(float x) {
  x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x128, 0xF, 0xF, false));  // row_ror:8
  x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x124, 0xF, 0xF, false));  // row_ror:4
  x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x122, 0xF, 0xF, false));  // row_ror:2
  x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x121, 0xF, 0xF, false));  // row_ror:1
  return x;
}

// max over the 4 lanes of a quad (every lane receives it)
__device__ __forceinline__ float quad_max(float x) {
  x = fmaxf(x, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x4E, 0xF, 0xF, false)));  // quad_perm [2,3,0,1]
  x = fmaxf(x, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0xB1, 0xF, 0xF, false)));  // quad_perm [1,0,3,2]
  return x;
}

// Elements 8l .. 8l+7 of a 128-value fp32 / bf16 row: 16-byte loads when `vec` (the
// rows are 16-byte aligned), element loads otherwise.
__device__ __forceinline__ void load_row8(const void *base, int dtype, int64_t e0, bool vec, float (&x)[8]) {
  if (dtype == 0) {
    const float *p = static_cast<const float *>(base) + e0;
    if (vec) {
      const v4f lo = *reinterpret_cast<const v4f *>(p), hi = *reinterpret_cast<const v4f *>(p + 4);
      x[0] = lo[0]; x[1] = lo[1]; x[2] = lo[2]; x[3] = lo[3];
      x[4] = hi[0]; x[5] = hi[1]; x[6] = hi[2]; x[7] = hi[3];
    } else {
#pragma unroll
      for (int j = 0; j < 8; ++j) x[j] = p[j];
    }
  } else {
    const uint16_t *p = static_cast<const uint16_t *>(base) + e0;
    if (vec) {
      const v4i r = *reinterpret_cast<const v4i *>(p);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        x[2 * j] = __uint_as_float(uint32_t(r[j]) << 16);
        x[2 * j + 1] = __uint_as_float(uint32_t(r[j]) & 0xFFFF0000u);
      }
    } else {
#pragma unroll
      for (int j = 0; j < 8; ++j) x[j] = bf16_to_f32(p[j]);
    }
  }
}

__device__ __forceinline__ bool rows_vec(const void *base, int dtype, int64_t row_stride) {
  const int esize = dtype == 0 ? 4 : 2;
  return (reinterpret_cast<uintptr_t>(base) & 15) == 0 && (row_stride * esize) % 16 == 0;
}

// RMSNorm over the 16 lanes of a row: x / sqrt(mean(x^2) + eps) * weight, in fp32
// (the mean is the lane sum times 2^-7, exact; the reciprocal root is a correctly
// rounded square root and division).
__device__ __forceinline__ void rms_norm8(float (&x)[8], const float *weight, int l, float eps) {
  float ss = 0.f;
#pragma unroll
  for (int j = 0; j < 8; ++j) ss = fmaf(x[j], x[j], ss);
  const float ms = row16_sum(ss) * 0.0078125f;
  const float r = __fdiv_rn(1.0f, __fsqrt_rn(ms + eps));
  const v4f w0 = *reinterpret_cast<const v4f *>(weight + 8 * l), w1 = *reinterpret_cast<const v4f *>(weight + 8 * l + 4);
  x[0] = x[0] * r * w0[0]; x[1] = x[1] * r * w0[1]; x[2] = x[2] * r * w0[2]; x[3] = x[3] * r * w0[3];
  x[4] = x[4] * r * w1[0]; x[5] = x[5] * r * w1[1]; x[6] = x[6] * r * w1[2]; x[7] = x[7] * r * w1[3];
}

// GPT-J RoPE of the trailing rope_dim channels: pair (d, d+1), d = 128 - rope_dim + 2i,
// rotated by (cos_i, sin_i) of table row `pos` to (a cos - b sin, b cos + a sin).
__device__ __forceinline__ void rope8(float (&x)[8], const float *cos_sin, int64_t pos, int rope_dim, int l) {
  const int lo = 128 - rope_dim, half = rope_dim >> 1;
  const float *row = cos_sin + pos * rope_dim;
#pragma unroll
  for (int j = 0; j < 8; j += 2) {
    const int d = 8 * l + j;
    if (d >= lo) {
      const int i = (d - lo) >> 1;
      const float c = row[i], s = row[half + i];
      const float a = x[j], b = x[j + 1];
      x[j] = a * c - b * s;
      x[j + 1] = b * c + a * s;
    }
  }
}

__device__ __forceinline__ int64_t clamp_pos(int64_t p, int max_position) {
  IDX_DEBUG_NOTE(p < 0 || p >= max_position, IDX_DBG_POSITION);
  return p < 0 ? 0 : (p >= max_position ? int64_t(max_position - 1) : p);
}

// Quantise a key row held as 8 values per lane and write it into its cache entry.
__device__ __forceinline__ void store_key(const float (&x)[8], int fmt, uint8_t *pb, int page_size, int e, int l,
                                          bool valid) {
  float m = 0.f;
#pragma unroll
  for (int j = 0; j < 8; ++j) m = fmaxf(m, fabsf(x[j]));
  if (fmt == 0) {
    const float amax = row16_max(m);
    const float scale = amax == 0.f ? 1.f : __fdiv_rn(amax, 448.0f);
    uint32_t w0 = 0, w1 = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      w0 |= enc_e4m3(__fdiv_rn(x[j], scale)) << (8 * j);
      w1 |= enc_e4m3(__fdiv_rn(x[4 + j], scale)) << (8 * j);
    }
    if (valid) {
      *reinterpret_cast<uint2 *>(pb + e * 128 + 8 * l) = make_uint2(w0, w1);
      if (l == 0) *reinterpret_cast<float *>(pb + page_size * 128 + 4 * e) = scale;
    }
  } else {
    // block b = l / 4 covers elements 32b .. 32b+31
    const float amax = quad_max(m);
    const int bits = e8m0_bits(amax);
    const float sc = e8m0_inv_scale(bits);
    uint32_t w = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) w |= (enc_e2m1(x[2 * j] * sc) | (enc_e2m1(x[2 * j + 1] * sc) << 4)) << (8 * j);
    if (valid) {
      // packed bytes 4l .. 4l+3 of the entry: chunk l/4, bytes 4(l%4) .. +3 of it
      const int run = e >> 4, u = e & 15;
      *reinterpret_cast<uint32_t *>(pb + run * 1024 + (l >> 2) * 256 + u * 16 + 4 * (l & 3)) = w;
      if ((l & 3) == 0) pb[page_size * 64 + run * 64 + (l >> 2) * 16 + u] = uint8_t(bits);
    }
  }
}

// K store, optionally preceded by RMSNorm and RoPE (NORM_ROPE). Every lane of a
// 16-lane row takes part in the DPP reductions, so no lane leaves before them; rows
// without a valid key only skip the loads and stores.
template <bool NORM_ROPE>
__global__ __launch_bounds__(256) void k_store_kernel(KStoreArgs a) {
  const int l = threadIdx.x & 15;  // lane within the key: elements 8l .. 8l+7
  const int i = blockIdx.x * kKeysPerWG + (threadIdx.x >> 4);
  bool valid = i < a.N;
  const int64_t slot = valid ? a.slots[i] : -1;
  const int64_t page = slot >= 0 ? slot / a.page_size : -1;
  IDX_DEBUG_NOTE(slot >= 0 && page >= a.num_pages, IDX_DBG_SLOT);
  valid = valid && slot >= 0 && page < a.num_pages;  // outside the pool: skipped like padding
  float x[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  if (valid) load_row8(a.k, a.k_dtype, int64_t(i) * a.k_row_stride + 8 * l, rows_vec(a.k, a.k_dtype, a.k_row_stride), x);
  if (NORM_ROPE) {
    rms_norm8(x, a.norm_weight, l, a.eps);
    if (valid && a.rope_dim > 0) rope8(x, a.cos_sin, clamp_pos(a.positions[i], a.max_position), a.rope_dim, l);
  }
  const int e = valid ? int(slot % a.page_size) : 0;
  uint8_t *pb = a.base + (valid ? page : 0) * a.page_stride;
  store_key(x, a.fmt, pb, a.page_size, e, l, valid);
}

// Query side of a step: RoPE, quantisation and the weight scale. Sixteen lanes per
// (token, head) row of 128 values.
__global__ __launch_bounds__(256) void q_rope_quant_kernel(QRopeArgs a) {
  const int l = threadIdx.x & 15;
  const int64_t row = int64_t(blockIdx.x) * kKeysPerWG + (threadIdx.x >> 4);  // t * H + h
  const bool valid = row < int64_t(a.T) * a.H;
  const int64_t t = valid ? row / a.H : 0;
  const int h = valid ? int(row % a.H) : 0;
  float x[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  if (valid) {
    load_row8(a.q, a.q_dtype, t * a.q_row_stride + int64_t(h) * 128 + 8 * l, rows_vec(a.q, a.q_dtype, a.q_row_stride), x);
    if (a.rope_dim > 0) rope8(x, a.cos_sin, clamp_pos(a.positions[t], a.max_position), a.rope_dim, l);
    if (l == 0) a.weights_out[row] = a.weights[t * a.weights_row_stride + h] * a.weight_scale;
  }
  if (a.fmt == 0) {
    uint32_t w0 = 0, w1 = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      w0 |= enc_e4m3(x[j]) << (8 * j);
      w1 |= enc_e4m3(x[4 + j]) << (8 * j);
    }
    if (valid) *reinterpret_cast<uint2 *>(a.q_out + row * 128 + 8 * l) = make_uint2(w0, w1);
  } else {
    float m = 0.f;
#pragma unroll
    for (int j = 0; j < 8; ++j) m = fmaxf(m, fabsf(x[j]));
    const float amax = quad_max(m);
    const int bits = e8m0_bits(amax);
    const float sc = e8m0_inv_scale(bits);
    uint32_t w = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) w |= (enc_e2m1(x[2 * j] * sc) | (enc_e2m1(x[2 * j + 1] * sc) << 4)) << (8 * j);
    if (valid) {
      *reinterpret_cast<uint32_t *>(a.q_out + row * 64 + 4 * l) = w;
      // byte b of the head's int32 is block b's scale (little-endian)
      if ((l & 3) == 0) reinterpret_cast<uint8_t *>(a.q_scale_out)[row * 4 + (l >> 2)] = uint8_t(bits);
    }
  }
}

__global__ __launch_bounds__(256) void q_quant_kernel(QQuantArgs a) {
  const int lane = threadIdx.x & 63;
  const int64_t row = int64_t(blockIdx.x) * kRowsPerWG + (threadIdx.x >> 6);  // t * H + h
  if (row >= int64_t(a.T) * a.H) return;
  const int64_t t = row / a.H;
  const int h = int(row % a.H);
  float x0, x1;
  load_pair(a.q, a.q_dtype, t * a.q_row_stride + int64_t(h) * 128 + 2 * lane, x0, x1);
  if (a.fmt == 0) {
    *reinterpret_cast<uint16_t *>(a.q_out + row * 128 + 2 * lane) = uint16_t(enc_e4m3(x0) | (enc_e4m3(x1) << 8));
  } else {
    const float amax = group16_max(fmaxf(fabsf(x0), fabsf(x1)));
    const int bits = e8m0_bits(amax);
    const float s = e8m0_inv_scale(bits);
    a.q_out[row * 64 + lane] = uint8_t(enc_e2m1(x0 * s) | (enc_e2m1(x1 * s) << 4));
    const int b1 = __shfl(bits, 16), b2 = __shfl(bits, 32), b3 = __shfl(bits, 48);
    if (lane == 0) a.q_scale_out[row] = int32_t(uint32_t(bits) | (uint32_t(b1) << 8) | (uint32_t(b2) << 16) | (uint32_t(b3) << 24));
  }
}

}  // namespace

hipError_t launch_k_store(const KStoreArgs &a, hipStream_t stream) {
  const int grid = (a.N + kKeysPerWG - 1) / kKeysPerWG;
  if (a.norm_weight)
    k_store_kernel<true><<<grid, 256, 0, stream>>>(a);
  else
    k_store_kernel<false><<<grid, 256, 0, stream>>>(a);
  return hipGetLastError();
}

hipError_t launch_q_rope_quant(const QRopeArgs &a, hipStream_t stream) {
  const int64_t rows = int64_t(a.T) * a.H;
  const int64_t grid = (rows + kKeysPerWG - 1) / kKeysPerWG;
  q_rope_quant_kernel<<<dim3(unsigned(grid)), 256, 0, stream>>>(a);
  return hipGetLastError();
}

hipError_t launch_q_quant(const QQuantArgs &a, hipStream_t stream) {
  const int64_t rows = int64_t(a.T) * a.H;
  const int64_t grid = (rows + kRowsPerWG - 1) / kRowsPerWG;
  q_quant_kernel<<<dim3(unsigned(grid)), 256, 0, stream>>>(a);
  return hipGetLastError();
}

IDX_DEBUG_READER(debug_word_quant)

}  // namespace idx
