// Measurement kernels behind include/moda_probe.h: the attainable bf16
// matrix-core rate and HBM bandwidth of the GPU the benchmark runs on.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/moda.h"
#include "../../include/moda_probe.h"
#include "moda_device.h"

namespace moda {
namespace {

constexpr int kProbeThreads = 256;

// Four independent accumulator chains per wave keep the matrix core fed
// without waiting on any one product's result; operands live in registers and
// nothing touches memory inside the loop.  With random != 0 each chain has its
// own pseudo-random bf16 operands in [-1, 1) that differ per lane, so
// consecutive products switch data as real tiles do; with random == 0 every
// operand is the constant 1/64.  The matrix core's power draw depends on its
// data, so the two rates differ when the clock is power limited.
__device__ __forceinline__ uint32_t xorshift32(uint32_t x) {
  x ^= x << 13;
  x ^= x >> 17;
  x ^= x << 5;
  return x;
}

__global__ __launch_bounds__(kProbeThreads) void mfma_probe_kernel(float* __restrict__ sink, int iters, int random) {
  uint32_t x = (threadIdx.x + 1u) * 0x9e3779b9u ^ (blockIdx.x + 1u) * 0x85ebca6bu;
  bf16x8 a[4], b[4];
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    u32x4 w;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      x = xorshift32(x);
      const float lo = static_cast<float>(static_cast<int>(x >> 9) - (1 << 22)) * (1.0f / (1 << 22));
      x = xorshift32(x);
      const float hi = static_cast<float>(static_cast<int>(x >> 9) - (1 << 22)) * (1.0f / (1 << 22));
      w[j] = random ? pack_bf16x2(lo, hi) : 0x3c803c80u;  // 0x3c80 = bf16 1/64
    }
    if (k < 4)
      a[k] = __builtin_bit_cast(bf16x8, w);
    else
      b[k - 4] = __builtin_bit_cast(bf16x8, w);
  }
  f32x16 c0 = {}, c1 = {}, c2 = {}, c3 = {};
  for (int i = 0; i < iters; ++i) {
    c0 = mfma32(a[0], b[0], c0);
    c1 = mfma32(a[1], b[1], c1);
    c2 = mfma32(a[2], b[2], c2);
    c3 = mfma32(a[3], b[3], c3);
  }
  float s = 0.0f;
#pragma unroll
  for (int i = 0; i < 16; ++i) s += c0[i] + c1[i] + c2[i] + c3[i];
  sink[static_cast<int64_t>(blockIdx.x) * kProbeThreads + threadIdx.x] = s;
}

// Copy: block b moves one contiguous span of the buffer, its threads four
// 16-byte units apart per step, with non-temporal loads and stores (the data
// is touched once).  The span is the buffer split evenly over the blocks; a
// remainder of fewer units than blocks * 1024 is copied by a grid-stride tail.
__global__ __launch_bounds__(kProbeThreads) void copy_probe_kernel(const u32x4* __restrict__ src,
                                                                   u32x4* __restrict__ dst, int64_t n) {
  constexpr int U = 4;
  const int64_t span = n / gridDim.x / (kProbeThreads * U) * (kProbeThreads * U);
  const int64_t b0 = static_cast<int64_t>(blockIdx.x) * span;
  for (int64_t i = b0 + threadIdx.x; i < b0 + span; i += kProbeThreads * U) {
    u32x4 x[U];
#pragma unroll
    for (int u = 0; u < U; ++u) x[u] = __builtin_nontemporal_load(src + i + u * kProbeThreads);
#pragma unroll
    for (int u = 0; u < U; ++u) __builtin_nontemporal_store(x[u], dst + i + u * kProbeThreads);
  }
  for (int64_t i = span * gridDim.x + static_cast<int64_t>(blockIdx.x) * kProbeThreads + threadIdx.x; i < n;
       i += static_cast<int64_t>(gridDim.x) * kProbeThreads)
    dst[i] = src[i];
}

// Read: grid-stride, four independent non-temporal 16-byte loads per step.
__global__ __launch_bounds__(kProbeThreads) void read_probe_kernel(const u32x4* __restrict__ src, int64_t n,
                                                                   uint32_t* __restrict__ sink) {
  const int64_t stride = static_cast<int64_t>(gridDim.x) * kProbeThreads;
  int64_t i = static_cast<int64_t>(blockIdx.x) * kProbeThreads + threadIdx.x;
  u32x4 acc = {0u, 0u, 0u, 0u};
  for (; i + 3 * stride < n; i += 4 * stride)
    acc ^= __builtin_nontemporal_load(src + i) ^ __builtin_nontemporal_load(src + i + stride) ^
           __builtin_nontemporal_load(src + i + 2 * stride) ^ __builtin_nontemporal_load(src + i + 3 * stride);
  for (; i < n; i += stride) acc ^= src[i];
  sink[static_cast<int64_t>(blockIdx.x) * kProbeThreads + threadIdx.x] = acc.x ^ acc.y ^ acc.z ^ acc.w;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

}  // namespace
}  // namespace moda

extern "C" {

int moda_probe_mfma_bf16(float* sink, int blocks, int iters, int random, moda_probe_stream_t stream) {
  if (!sink) return MODA_ERR_NULL;
  if (blocks <= 0 || iters <= 0 || (random != 0 && random != 1)) return MODA_ERR_SHAPE;
  if (!moda::aligned16(sink)) return MODA_ERR_ALIGN;
  hipLaunchKernelGGL(moda::mfma_probe_kernel, dim3(blocks), dim3(moda::kProbeThreads), 0,
                     static_cast<hipStream_t>(stream), sink, iters, random);
  return hipGetLastError() == hipSuccess ? MODA_OK : MODA_ERR_HIP;
}

int moda_probe_copy(const void* src, void* dst, size_t bytes, int blocks, moda_probe_stream_t stream) {
  if (!src || !dst) return MODA_ERR_NULL;
  if (bytes == 0 || bytes % 16 != 0 || blocks <= 0 || bytes / 16 > static_cast<size_t>(INT64_MAX / 8))
    return MODA_ERR_SHAPE;
  if (!moda::aligned16(src) || !moda::aligned16(dst)) return MODA_ERR_ALIGN;
  hipLaunchKernelGGL(moda::copy_probe_kernel, dim3(blocks), dim3(moda::kProbeThreads), 0,
                     static_cast<hipStream_t>(stream), static_cast<const moda::u32x4*>(src),
                     static_cast<moda::u32x4*>(dst), static_cast<int64_t>(bytes / 16));
  return hipGetLastError() == hipSuccess ? MODA_OK : MODA_ERR_HIP;
}

int moda_probe_read(const void* src, size_t bytes, int blocks, unsigned int* sink, moda_probe_stream_t stream) {
  if (!src || !sink) return MODA_ERR_NULL;
  if (bytes == 0 || bytes % 16 != 0 || blocks <= 0 || bytes / 16 > static_cast<size_t>(INT64_MAX / 8))
    return MODA_ERR_SHAPE;
  if (!moda::aligned16(src) || !moda::aligned16(sink)) return MODA_ERR_ALIGN;
  hipLaunchKernelGGL(moda::read_probe_kernel, dim3(blocks), dim3(moda::kProbeThreads), 0,
                     static_cast<hipStream_t>(stream), static_cast<const moda::u32x4*>(src),
                     static_cast<int64_t>(bytes / 16), sink);
  return hipGetLastError() == hipSuccess ? MODA_OK : MODA_ERR_HIP;
}

}  // extern "C"
