// Internal launchers behind the C ABI (include/moda.h).  Arguments reaching
// these have already been validated on the host.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/moda.h"

namespace moda {

struct FwdArgs {
  const void *q, *k, *v, *kd, *vd;
  int B, T, Hq, Hk, d, L, causal;
  int Lcap;  // depth slots per (token, KV head) in memory; the first L are attended
  void* out;
  float* lse;
  void* stream;
};

struct DecodeArgs {
  const void *q, *k, *v, *kd, *vd;  // q [B][Hq][d]; caches [B][T][Hk][d]; depth [B][Hk][L][d]
  int B, T, Hq, Hk, d, L;
  int Lcap;    // depth slots per (batch, KV head) in memory; the first L are attended
  void* out;   // [B][Hq][d]
  float* lse;  // [B][Hq]
  void* workspace;
  void* stream;
};

struct BwdArgs {
  const void *q, *k, *v, *kd, *vd;  // forward inputs; depth packed [B][T][Hk][L][d]
  const void* out;                  // forward output [B][T][Hq][d]
  const float* lse;                 // forward lse [B][Hq][T], natural log
  const void* dout;                 // output gradient [B][T][Hq][d]
  int B, T, Hq, Hk, d, L, causal;
  void *dq, *dk, *dv, *dkd, *dvd;   // gradients in the input layouts
  void* workspace;
  void* stream;
};

struct KvProjArgs {
  const void *x, *w;        // x [B*T][Dm]; w [2*Hk*d][Dm] (K rows, then V rows)
  int B, T, Dm, Hk, d;
  void *k_out, *v_out;      // [B*T][Hk][d] or both NULL
  void *k_depth, *v_depth;  // packed [B*T][Hk][S][d] or both NULL
  int S, slot;
  void* stream;
};

hipError_t launch_fwd_bf16(const FwdArgs& a);
hipError_t launch_fwd_f32(const FwdArgs& a);
int64_t fwd_bf16_grid_blocks(int B, int T, int Hq, int Hk, int d);
int fwd_bf16_rows_per_block(int T, int d);  // expanded query rows per workgroup of the bf16 forward
int64_t fwd_f32_grid_blocks(int B, int T, int Hq);

hipError_t launch_decode_bf16(const DecodeArgs& a);
size_t decode_workspace_bytes(int B, int T, int Hq, int Hk, int d, int L);
int64_t decode_grid_blocks(int B, int T, int Hk, int L);

// Scratch of the allocation-free decode (a static device array per device):
// its capacity, and its address on the current device, which the first call
// on each device looks up.
constexpr size_t kDecodeScratchBytes = MODA_DECODE_NOALLOC_SCRATCH_BYTES;
hipError_t decode_scratch(void** ptr);

hipError_t launch_bwd_bf16(const BwdArgs& a);
size_t bwd_workspace_bytes(int B, int T, int Hq, int d, int L);
int64_t bwd_grid_blocks(int B, int T, int Hq, int Hk);

hipError_t launch_kv_project(const KvProjArgs& a);
int64_t kv_project_grid_blocks(int B, int T, int Hk, int d);

hipError_t launch_pack_depth(const void* src, void* dst, int B, int T, int L, int Hk, int d, int elem_bytes,
                             void* stream);
hipError_t launch_append_depth_slot(const void* kv, void* dst, int slot, int B, int T, int L, int Hk, int d,
                                    int elem_bytes, void* stream);

}  // namespace moda
