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
// without waiting on any one product's result; operands are loop invariant
// and live in registers.  Values stay small (1/64 * 1/64 * 16 per product
// and element), so the sums stay finite for any iteration count used.
__global__ __launch_bounds__(kProbeThreads) void mfma_probe_kernel(float* __restrict__ sink, int iters) {
  const uint32_t one64 = 0x3c803c80u;  // two bf16 1/64
  const u32x4 w = {one64, one64, one64, one64};
  const bf16x8 a = __builtin_bit_cast(bf16x8, w);
  bf16x8 b = a;
  asm volatile("" : "+v"(b));  // not a compile-time constant
  f32x16 c0 = {}, c1 = {}, c2 = {}, c3 = {};
  for (int i = 0; i < iters; ++i) {
    c0 = mfma32(a, b, c0);
    c1 = mfma32(a, b, c1);
    c2 = mfma32(a, b, c2);
    c3 = mfma32(a, b, c3);
  }
  float s = 0.0f;
#pragma unroll
  for (int i = 0; i < 16; ++i) s += c0[i] + c1[i] + c2[i] + c3[i];
  sink[static_cast<int64_t>(blockIdx.x) * kProbeThreads + threadIdx.x] = s;
}

// Grid-stride copy, four independent 16-byte loads in flight per thread.
__global__ __launch_bounds__(kProbeThreads) void copy_probe_kernel(const u32x4* __restrict__ src,
                                                                   u32x4* __restrict__ dst, int64_t n) {
  const int64_t stride = static_cast<int64_t>(gridDim.x) * kProbeThreads;
  int64_t i = static_cast<int64_t>(blockIdx.x) * kProbeThreads + threadIdx.x;
  for (; i + 3 * stride < n; i += 4 * stride) {
    const u32x4 x0 = src[i], x1 = src[i + stride], x2 = src[i + 2 * stride], x3 = src[i + 3 * stride];
    dst[i] = x0;
    dst[i + stride] = x1;
    dst[i + 2 * stride] = x2;
    dst[i + 3 * stride] = x3;
  }
  for (; i < n; i += stride) dst[i] = src[i];
}

__global__ __launch_bounds__(kProbeThreads) void read_probe_kernel(const u32x4* __restrict__ src, int64_t n,
                                                                   uint32_t* __restrict__ sink) {
  const int64_t stride = static_cast<int64_t>(gridDim.x) * kProbeThreads;
  int64_t i = static_cast<int64_t>(blockIdx.x) * kProbeThreads + threadIdx.x;
  u32x4 acc = {0u, 0u, 0u, 0u};
  for (; i + 3 * stride < n; i += 4 * stride)
    acc ^= src[i] ^ src[i + stride] ^ src[i + 2 * stride] ^ src[i + 3 * stride];
  for (; i < n; i += stride) acc ^= src[i];
  sink[static_cast<int64_t>(blockIdx.x) * kProbeThreads + threadIdx.x] = acc.x ^ acc.y ^ acc.z ^ acc.w;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

}  // namespace
}  // namespace moda

extern "C" {

int moda_probe_mfma_bf16(float* sink, int blocks, int iters, moda_probe_stream_t stream) {
  if (!sink) return MODA_ERR_NULL;
  if (blocks <= 0 || iters <= 0) return MODA_ERR_SHAPE;
  if (!moda::aligned16(sink)) return MODA_ERR_ALIGN;
  hipLaunchKernelGGL(moda::mfma_probe_kernel, dim3(blocks), dim3(moda::kProbeThreads), 0,
                     static_cast<hipStream_t>(stream), sink, iters);
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
