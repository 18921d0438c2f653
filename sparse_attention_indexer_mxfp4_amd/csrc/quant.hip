// Quantisers that feed the indexer: the K store (quantise a key row and write it into
// its cache slot) and the query quantiser. Page "vllm.models.deepseek_v41.amd.rocm",
// rocm_mxfp4_indexer_k_store and rocm_mxfp4_indexer_q_quant (their quantise-and-write
// part). One wavefront per 128-value row; lane L holds elements 2L and 2L+1.
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

__global__ __launch_bounds__(256) void k_store_kernel(KStoreArgs a) {
  const int lane = threadIdx.x & 63;
  const int i = blockIdx.x * kRowsPerWG + (threadIdx.x >> 6);
  if (i >= a.N) return;
  const int64_t slot = a.slots[i];
  if (slot < 0) return;
  const int64_t page = slot / a.page_size;
  if (page >= a.num_pages) return;  // outside the pool: skipped like padding
  const int e = int(slot % a.page_size);
  uint8_t *pb = a.base + page * a.page_stride;
  float x0, x1;
  load_pair(a.k, a.k_dtype, int64_t(i) * a.k_row_stride + 2 * lane, x0, x1);

  if (a.fmt == 0) {
    const float amax = wave_max(fmaxf(fabsf(x0), fabsf(x1)));
    const float scale = amax == 0.f ? 1.f : __fdiv_rn(amax, 448.0f);
    const uint32_t c0 = enc_e4m3(__fdiv_rn(x0, scale));
    const uint32_t c1 = enc_e4m3(__fdiv_rn(x1, scale));
    *reinterpret_cast<uint16_t *>(pb + e * 128 + 2 * lane) = uint16_t(c0 | (c1 << 8));
    if (lane == 0) *reinterpret_cast<float *>(pb + a.page_size * 128 + 4 * e) = scale;
  } else {
    const float amax = group16_max(fmaxf(fabsf(x0), fabsf(x1)));
    const int bits = e8m0_bits(amax);
    const float s = e8m0_inv_scale(bits);
    const uint32_t byte = enc_e2m1(x0 * s) | (enc_e2m1(x1 * s) << 4);
    const int run = e >> 4, u = e & 15;
    pb[run * 1024 + (lane >> 4) * 256 + u * 16 + (lane & 15)] = uint8_t(byte);
    if ((lane & 15) == 0) pb[a.page_size * 64 + run * 64 + (lane >> 4) * 16 + u] = uint8_t(bits);
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
  const int grid = (a.N + kRowsPerWG - 1) / kRowsPerWG;
  k_store_kernel<<<grid, 256, 0, stream>>>(a);
  return hipGetLastError();
}

hipError_t launch_q_quant(const QQuantArgs &a, hipStream_t stream) {
  const int64_t rows = int64_t(a.T) * a.H;
  const int64_t grid = (rows + kRowsPerWG - 1) / kRowsPerWG;
  q_quant_kernel<<<dim3(unsigned(grid)), 256, 0, stream>>>(a);
  return hipGetLastError();
}

}  // namespace idx
