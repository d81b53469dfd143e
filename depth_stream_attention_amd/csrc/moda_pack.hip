// Depth-stream layout kernels: the full pack [B,T,L,Hk,d] -> [B,T,Hk,L,d]
// and the per-layer slot write [B,T,Hk,d] -> slot `slot` of [B,T,Hk,L,d].
//
// The "Mixture-of-Depths Attention" summary (papercache.org, 3.2) keeps a
// position's L depth states contiguous so a query reads them as one block;
// with the KV head moved outside the slot index, the L*d elements of one
// (token, KV head) pair are one run that the forward stages once for the G
// query heads of that group.  Writing a layer's KV into its slot is the
// "write" step of 2.2 in the same summary.
//
// Both are pure permutations (no arithmetic): HBM-bound copies.  One
// workgroup handles one (b, t) position; threads walk the destination in
// order, so stores are fully coalesced and loads come in d-element runs.
// The copy unit is the widest of 16/8/4/2/1 bytes dividing a d-row.
#include "moda_device.h"
#include "moda_launch.h"

namespace moda {
namespace {

constexpr int kPackThreads = 256;

template <typename U>
__global__ __launch_bounds__(kPackThreads) void pack_kernel(const U* __restrict__ src, U* __restrict__ dst, int L,
                                                            int Hk, int upr) {
  const int64_t bt = blockIdx.x;
  const int per_pos = Hk * L * upr;  // units per (b, t) position
  const U* s = src + bt * per_pos;
  U* o = dst + bt * per_pos;
  for (int idx = threadIdx.x; idx < per_pos; idx += kPackThreads) {
    const int c = idx % upr;
    const int row = idx / upr;  // destination row = hk * L + l
    const int l = row % L, hk = row / L;
    o[idx] = s[(l * Hk + hk) * upr + c];
  }
}

template <typename U>
__global__ __launch_bounds__(kPackThreads) void append_kernel(const U* __restrict__ kv, U* __restrict__ dst, int slot,
                                                              int L, int Hk, int upr) {
  const int64_t bt = blockIdx.x;
  const int per_pos = Hk * upr;
  const U* s = kv + bt * per_pos;
  U* o = dst + bt * static_cast<int64_t>(Hk) * L * upr;
  for (int idx = threadIdx.x; idx < per_pos; idx += kPackThreads) {
    const int c = idx % upr, hk = idx / upr;
    o[(static_cast<int64_t>(hk) * L + slot) * upr + c] = s[idx];
  }
}

template <typename U>
hipError_t pack_as(const void* src, void* dst, int B, int T, int L, int Hk, int row_bytes, void* stream) {
  const int upr = row_bytes / static_cast<int>(sizeof(U));
  hipLaunchKernelGGL((pack_kernel<U>), dim3(static_cast<unsigned>(static_cast<int64_t>(B) * T)), dim3(kPackThreads),
                     0, static_cast<hipStream_t>(stream), static_cast<const U*>(src), static_cast<U*>(dst), L, Hk,
                     upr);
  return hipGetLastError();
}

template <typename U>
hipError_t append_as(const void* kv, void* dst, int slot, int B, int T, int L, int Hk, int row_bytes,
                     void* stream) {
  const int upr = row_bytes / static_cast<int>(sizeof(U));
  hipLaunchKernelGGL((append_kernel<U>), dim3(static_cast<unsigned>(static_cast<int64_t>(B) * T)),
                     dim3(kPackThreads), 0, static_cast<hipStream_t>(stream), static_cast<const U*>(kv),
                     static_cast<U*>(dst), slot, L, Hk, upr);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_pack_depth(const void* src, void* dst, int B, int T, int L, int Hk, int d, int elem_bytes,
                             void* stream) {
  const int row_bytes = d * elem_bytes;
  if (row_bytes % 16 == 0) return pack_as<u32x4>(src, dst, B, T, L, Hk, row_bytes, stream);
  if (row_bytes % 8 == 0) return pack_as<u32x2>(src, dst, B, T, L, Hk, row_bytes, stream);
  if (row_bytes % 4 == 0) return pack_as<uint32_t>(src, dst, B, T, L, Hk, row_bytes, stream);
  if (row_bytes % 2 == 0) return pack_as<uint16_t>(src, dst, B, T, L, Hk, row_bytes, stream);
  return pack_as<uint8_t>(src, dst, B, T, L, Hk, row_bytes, stream);
}

hipError_t launch_append_depth_slot(const void* kv, void* dst, int slot, int B, int T, int L, int Hk, int d,
                                    int elem_bytes, void* stream) {
  const int row_bytes = d * elem_bytes;
  if (row_bytes % 16 == 0) return append_as<u32x4>(kv, dst, slot, B, T, L, Hk, row_bytes, stream);
  if (row_bytes % 8 == 0) return append_as<u32x2>(kv, dst, slot, B, T, L, Hk, row_bytes, stream);
  if (row_bytes % 4 == 0) return append_as<uint32_t>(kv, dst, slot, B, T, L, Hk, row_bytes, stream);
  if (row_bytes % 2 == 0) return append_as<uint16_t>(kv, dst, slot, B, T, L, Hk, row_bytes, stream);
  return append_as<uint8_t>(kv, dst, slot, B, T, L, Hk, row_bytes, stream);
}

}  // namespace moda
