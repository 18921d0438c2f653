// Measurement kernels (include/idx_calib.h): a streaming copy and a streaming read
// for the HBM ceiling, and a register-operand loop of the dense 16x16x128 fp8 / fp4
// matrix instruction for the matrix-core ceiling.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../../include/idx_calib.h"

namespace {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;
constexpr int kUnroll = 4;          // 16-byte loads in flight per thread
constexpr int kWgPerCu = 8;         // streaming kernels
constexpr int kMfmaWgPerCu = 2;     // matrix loop: 8 waves per CU, 2 per SIMD
constexpr int kMaxSink = 8192;

int num_cus(int *out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return int(e);
  e = hipDeviceGetAttribute(out, hipDeviceAttributeMultiprocessorCount, dev);
  return int(e);
}

__global__ __launch_bounds__(kThreads) void copy_kernel(const v4i *__restrict__ src, v4i *__restrict__ dst,
                                                        size_t n) {
  const size_t stride = size_t(gridDim.x) * kThreads * kUnroll;
  for (size_t base = size_t(blockIdx.x) * kThreads * kUnroll + threadIdx.x; base < n; base += stride) {
    v4i x[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const size_t i = base + size_t(u) * kThreads;
      x[u] = i < n ? src[i] : v4i{0, 0, 0, 0};
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const size_t i = base + size_t(u) * kThreads;
      if (i < n) dst[i] = x[u];
    }
  }
}

__global__ __launch_bounds__(kThreads) void read_kernel(const v4i *__restrict__ src, size_t n, uint32_t *sink) {
  __shared__ uint32_t s_part[kThreads / 64];
  const size_t stride = size_t(gridDim.x) * kThreads * kUnroll;
  uint32_t h = 0;
  for (size_t base = size_t(blockIdx.x) * kThreads * kUnroll + threadIdx.x; base < n; base += stride) {
    v4i x[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const size_t i = base + size_t(u) * kThreads;
      x[u] = i < n ? src[i] : v4i{0, 0, 0, 0};
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) h ^= uint32_t(x[u][0] ^ x[u][1] ^ x[u][2] ^ x[u][3]);
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) h ^= uint32_t(__shfl_xor(int(h), off));
  if ((threadIdx.x & 63) == 0) s_part[threadIdx.x >> 6] = h;
  __syncthreads();
  if (threadIdx.x == 0) sink[blockIdx.x] = s_part[0] ^ s_part[1] ^ s_part[2] ^ s_part[3];
}

__device__ __forceinline__ uint32_t mix(uint32_t x) {
  x ^= x >> 16;
  x *= 0x7feb352du;
  x ^= x >> 15;
  x *= 0x846ca68bu;
  x ^= x >> 16;
  return x;
}

template <int FMT>
__device__ __forceinline__ v4f mma(const v8i &x, const v8i &y, const v4f &c) {
  if constexpr (FMT == 0)
    return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(x, y, c, 0, 0, 0, 0, 0, 0);
  else
    return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(x, y, c, 4, 4, 0, 127, 0, 127);
}

// FMT 0: e4m3 bytes with exponent fields kept below 7 (no NaN codes, sums stay finite)
// FMT 1: any e2m1 nibbles, unit block scales
template <int FMT>
__global__ __launch_bounds__(kThreads) void mfma_kernel(int iters, float *sink) {
  const uint32_t t = blockIdx.x * kThreads + threadIdx.x;
  const uint32_t mask = FMT == 0 ? 0xB7B7B7B7u : 0xFFFFFFFFu;
  v8i a[2], b[2];
#pragma unroll
  for (int s = 0; s < 2; ++s)
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      a[s][j] = int(mix(t * 32u + uint32_t(s * 16 + j)) & mask);
      b[s][j] = int(mix(t * 32u + uint32_t(s * 16 + j) + 0x9e3779b9u) & mask);
    }
  v4f acc[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) acc[j] = v4f{0.f, 0.f, 0.f, 0.f};
  // two trips per loop pass, so every operand choice is fixed at compile time (a choice
  // made from the trip count would move registers around every instruction)
  const int pairs = iters / 2;
  for (int it = 0; it < pairs; ++it) {
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const int c = j & 7;
      acc[c] = mma<FMT>(a[((j >> 3) + c) & 1], b[(c >> 1) & 1], acc[c]);
    }
  }
  if (iters & 1) {
#pragma unroll
    for (int c = 0; c < 8; ++c) acc[c] = mma<FMT>(a[c & 1], b[(c >> 1) & 1], acc[c]);
  }
  float s = 0.f;
#pragma unroll
  for (int j = 0; j < 8; ++j) s += (acc[j][0] + acc[j][1]) + (acc[j][2] + acc[j][3]);
  if ((threadIdx.x & 63) == 0) sink[t >> 6] = s;
}

}  // namespace

extern "C" {

int32_t idx_calib_copy(const void *src, void *dst, size_t bytes, hipStream_t stream) {
  if (!src || !dst || bytes % 16 || (reinterpret_cast<uintptr_t>(src) | reinterpret_cast<uintptr_t>(dst)) % 16)
    return int32_t(hipErrorInvalidValue);
  int cus = 0;
  if (int e = num_cus(&cus)) return e;
  copy_kernel<<<dim3(cus * kWgPerCu), kThreads, 0, stream>>>(static_cast<const v4i *>(src), static_cast<v4i *>(dst),
                                                             bytes / 16);
  return int32_t(hipGetLastError());
}

int32_t idx_calib_read_sink_words(void) { return kMaxSink; }

int32_t idx_calib_read(const void *src, size_t bytes, uint32_t *sink, hipStream_t stream) {
  if (!src || !sink || bytes % 16 || reinterpret_cast<uintptr_t>(src) % 16) return int32_t(hipErrorInvalidValue);
  int cus = 0;
  if (int e = num_cus(&cus)) return e;
  const int wgs = cus * kWgPerCu;
  if (wgs > kMaxSink) return int32_t(hipErrorInvalidConfiguration);
  read_kernel<<<dim3(wgs), kThreads, 0, stream>>>(static_cast<const v4i *>(src), bytes / 16, sink);
  return int32_t(hipGetLastError());
}

int32_t idx_calib_mfma_sink_words(void) { return kMaxSink; }

int32_t idx_calib_mfma(int32_t fmt, int32_t iters, float *sink, int64_t *flop_out, hipStream_t stream) {
  if (!sink || !flop_out || iters < 1 || (fmt != 0 && fmt != 1)) return int32_t(hipErrorInvalidValue);
  int cus = 0;
  if (int e = num_cus(&cus)) return e;
  const int wgs = cus * kMfmaWgPerCu;
  const int waves = wgs * (kThreads / 64);
  if (waves > kMaxSink) return int32_t(hipErrorInvalidConfiguration);
  *flop_out = int64_t(waves) * iters * 8 * (2LL * 16 * 16 * 128);
  if (fmt == 0)
    mfma_kernel<0><<<dim3(wgs), kThreads, 0, stream>>>(iters, sink);
  else
    mfma_kernel<1><<<dim3(wgs), kThreads, 0, stream>>>(iters, sink);
  return int32_t(hipGetLastError());
}

}  // extern "C"
