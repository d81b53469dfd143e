// Internal launchers behind the C ABI (include/moda.h).  Arguments reaching
// these have already been validated on the host.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moda {

struct FwdArgs {
  const void *q, *k, *v, *kd, *vd;
  int B, T, Hq, Hk, d, L, causal;
  void* out;
  float* lse;
  void* stream;
};

hipError_t launch_fwd_bf16(const FwdArgs& a);
hipError_t launch_fwd_f32(const FwdArgs& a);
int64_t fwd_bf16_grid_blocks(int B, int T, int Hq, int Hk);
int64_t fwd_f32_grid_blocks(int B, int T, int Hq);

hipError_t launch_pack_depth(const void* src, void* dst, int B, int T, int L, int Hk, int d, int elem_bytes,
                             void* stream);
hipError_t launch_append_depth_slot(const void* kv, void* dst, int slot, int B, int T, int L, int Hk, int d,
                                    int elem_bytes, void* stream);

}  // namespace moda
