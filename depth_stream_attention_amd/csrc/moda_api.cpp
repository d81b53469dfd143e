// C ABI of libmoda.so (declared and documented in include/moda.h).
//
// Every entry point validates its arguments on the host first and returns an
// error code before touching HIP; only then does it enqueue kernels on the
// caller's stream.  Nothing is allocated and nothing is synchronised.
#include "../../include/moda.h"

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <climits>

#include "moda_launch.h"

namespace {

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

bool is_pow2_in(int x, int lo, int hi) { return x >= lo && x <= hi && (x & (x - 1)) == 0; }

int validate_fwd(bool bf16, const void* q, const void* k, const void* v, const void* kd, const void* vd, int B, int T,
                 int Hq, int Hk, int d, int Lcap, int L, int causal, const void* out, const float* lse) {
  if (!q || !k || !v || !out || !lse) return MODA_ERR_NULL;
  if (L > 0 && (!kd || !vd)) return MODA_ERR_NULL;
  if (B <= 0 || T <= 0 || Hq <= 0 || Hk <= 0 || d <= 0 || L < 0 || Lcap < L) return MODA_ERR_SHAPE;
  if (Hq % Hk != 0) return MODA_ERR_SHAPE;
  if (causal != 0 && causal != 1) return MODA_ERR_SHAPE;
  if (d != 64 && d != 128) return MODA_ERR_UNSUPPORTED;
  const int G = Hq / Hk;
  if (!is_pow2_in(G, 1, 32)) return MODA_ERR_UNSUPPORTED;
  // Launch-size limits of this build: expanded rows and workgroup counts in int32.
  if (static_cast<int64_t>(T) * G > INT_MAX / 2) return MODA_ERR_UNSUPPORTED;
  if (moda::fwd_bf16_grid_blocks(B, T, Hq, Hk, d) > INT_MAX || moda::fwd_f32_grid_blocks(B, T, Hq) > INT_MAX)
    return MODA_ERR_UNSUPPORTED;
  // The bf16 kernel addresses one (batch, KV head) sequence and one
  // workgroup's depth slabs (at most one token per expanded row of the
  // workgroup) with 32-bit byte offsets.
  if (bf16 && (static_cast<int64_t>(T + 64) * Hk * d * 2 >= (int64_t{1} << 31) ||
               static_cast<int64_t>(moda::fwd_bf16_rows_per_block(T, d) + 1) * Hk * Lcap * d * 2 >=
                   (int64_t{1} << 31)))
    return MODA_ERR_UNSUPPORTED;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out) || !aligned16(lse)) return MODA_ERR_ALIGN;
  if (L > 0 && (!aligned16(kd) || !aligned16(vd))) return MODA_ERR_ALIGN;
  return MODA_OK;
}

// Everything moda_attn_decode checks except its workspace.
int validate_decode_args(const void* q, const void* k, const void* v, const void* kd, const void* vd, int B, int T,
                         int Hq, int Hk, int d, int Lcap, int L, const void* out, const float* lse) {
  if (!q || !k || !v || !out || !lse) return MODA_ERR_NULL;
  if (L > 0 && (!kd || !vd)) return MODA_ERR_NULL;
  if (B <= 0 || T <= 0 || Hq <= 0 || Hk <= 0 || d <= 0 || L < 0 || Lcap < L) return MODA_ERR_SHAPE;
  if (Hq % Hk != 0) return MODA_ERR_SHAPE;
  if (d != 64 && d != 128) return MODA_ERR_UNSUPPORTED;
  if (!is_pow2_in(Hq / Hk, 1, 32)) return MODA_ERR_UNSUPPORTED;
  // One chunk of keys (or the depth slab) is addressed with 32-bit byte offsets.
  if (static_cast<int64_t>(1024) * Hk * d * 2 >= (int64_t{1} << 31) ||
      static_cast<int64_t>(B) * Hk * Lcap * d * 2 >= (int64_t{1} << 62))
    return MODA_ERR_UNSUPPORTED;
  if (moda::decode_grid_blocks(B, T, Hk, L) > INT_MAX || static_cast<int64_t>(B) * Hq > INT_MAX)
    return MODA_ERR_UNSUPPORTED;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out) || !aligned16(lse)) return MODA_ERR_ALIGN;
  if (L > 0 && (!aligned16(kd) || !aligned16(vd))) return MODA_ERR_ALIGN;
  return MODA_OK;
}

int validate_decode(const void* q, const void* k, const void* v, const void* kd, const void* vd, int B, int T,
                    int Hq, int Hk, int d, int Lcap, int L, const void* out, const float* lse, const void* ws,
                    size_t ws_bytes) {
  if (!ws) return MODA_ERR_NULL;
  const int rc = validate_decode_args(q, k, v, kd, vd, B, T, Hq, Hk, d, Lcap, L, out, lse);
  if (rc != MODA_OK) return rc;
  if (ws_bytes < moda::decode_workspace_bytes(B, T, Hq, Hk, d, L)) return MODA_ERR_SHAPE;
  if (!aligned16(ws)) return MODA_ERR_ALIGN;
  return MODA_OK;
}

int validate_bwd(const void* q, const void* k, const void* v, const void* kd, const void* vd, const void* out,
                 const float* lse, const void* dout, int B, int T, int Hq, int Hk, int d, int L, int causal,
                 const void* dq, const void* dk, const void* dv, const void* dkd, const void* dvd, const void* ws,
                 size_t ws_bytes) {
  if (!q || !k || !v || !out || !lse || !dout || !dq || !dk || !dv || !ws) return MODA_ERR_NULL;
  if (L > 0 && (!kd || !vd || !dkd || !dvd)) return MODA_ERR_NULL;
  if (B <= 0 || T <= 0 || Hq <= 0 || Hk <= 0 || d <= 0 || L < 0) return MODA_ERR_SHAPE;
  if (Hq % Hk != 0) return MODA_ERR_SHAPE;
  if (causal != 0 && causal != 1) return MODA_ERR_SHAPE;
  if (d != 64 && d != 128) return MODA_ERR_UNSUPPORTED;
  if (!is_pow2_in(Hq / Hk, 1, 32)) return MODA_ERR_UNSUPPORTED;
  // One (batch) sequence of q or dO, and of one KV head's keys, is addressed
  // with 32-bit byte offsets; grids and expanded rows stay in int32.
  if (static_cast<int64_t>(T + 128) * Hq * d * 2 >= (int64_t{1} << 31)) return MODA_ERR_UNSUPPORTED;
  if (static_cast<int64_t>(T) * (Hq / Hk) > INT_MAX / 2) return MODA_ERR_UNSUPPORTED;
  if (moda::bwd_grid_blocks(B, T, Hq, Hk) > INT_MAX) return MODA_ERR_UNSUPPORTED;
  if (ws_bytes < moda::bwd_workspace_bytes(B, T, Hq, d, L)) return MODA_ERR_SHAPE;
  for (const void* p : {q, k, v, out, static_cast<const void*>(lse), dout, dq, dk, dv, ws})
    if (!aligned16(p)) return MODA_ERR_ALIGN;
  if (L > 0)
    for (const void* p : {kd, vd, dkd, dvd})
      if (!aligned16(p)) return MODA_ERR_ALIGN;
  return MODA_OK;
}

int validate_kv_project(const void* x, const void* w, int B, int T, int Dm, int Hk, int d, const void* k_out,
                        const void* v_out, const void* k_depth, const void* v_depth, int S, int slot) {
  if (!x || !w) return MODA_ERR_NULL;
  const bool seq = k_out || v_out, depth = k_depth || v_depth;
  if (!seq && !depth) return MODA_ERR_NULL;               // nothing to write
  if ((seq && (!k_out || !v_out)) || (depth && (!k_depth || !v_depth))) return MODA_ERR_NULL;
  if (B <= 0 || T <= 0 || Dm <= 0 || Hk <= 0 || d <= 0) return MODA_ERR_SHAPE;
  if (depth && (S <= 0 || slot < 0 || slot >= S)) return MODA_ERR_SHAPE;
  if (d != 64 && d != 128) return MODA_ERR_UNSUPPORTED;
  if (Dm % 64 != 0) return MODA_ERR_UNSUPPORTED;        // whole 64-element chunks of the hidden size
  if (static_cast<int64_t>(256) * Dm * 2 >= (int64_t{1} << 31)) return MODA_ERR_UNSUPPORTED;
  if (static_cast<int64_t>(B) * T > INT_MAX / 2 || moda::kv_project_grid_blocks(B, T, Hk, d) > INT_MAX)
    return MODA_ERR_UNSUPPORTED;
  for (const void* p : {x, w, k_out, v_out, k_depth, v_depth})
    if (p && !aligned16(p)) return MODA_ERR_ALIGN;
  return MODA_OK;
}

int validate_layout(const void* src, const void* dst, int B, int T, int L, int Hk, int d, int elem_bytes) {
  if (!src || !dst) return MODA_ERR_NULL;
  if (B <= 0 || T <= 0 || L <= 0 || Hk <= 0 || d <= 0) return MODA_ERR_SHAPE;
  if (elem_bytes != 1 && elem_bytes != 2 && elem_bytes != 4 && elem_bytes != 8) return MODA_ERR_SHAPE;
  if (static_cast<int64_t>(B) * T > INT_MAX) return MODA_ERR_UNSUPPORTED;
  if (static_cast<int64_t>(Hk) * L * d * elem_bytes > INT_MAX) return MODA_ERR_UNSUPPORTED;
  if (!aligned16(src) || !aligned16(dst)) return MODA_ERR_ALIGN;
  return MODA_OK;
}

int fwd_common(bool bf16, const void* q, const void* k, const void* v, const void* kd, const void* vd, int B, int T,
               int Hq, int Hk, int d, int Lcap, int L, int causal, void* out, float* lse, moda_stream_t stream) {
  const int rc = validate_fwd(bf16, q, k, v, kd, vd, B, T, Hq, Hk, d, Lcap, L, causal, out, lse);
  if (rc != MODA_OK) return rc;
  moda::FwdArgs a{q, k, v, L > 0 ? kd : nullptr, L > 0 ? vd : nullptr, B, T, Hq, Hk, d, L, causal, Lcap,
                  out, lse, stream};
  const hipError_t e = bf16 ? moda::launch_fwd_bf16(a) : moda::launch_fwd_f32(a);
  return e == hipSuccess ? MODA_OK : MODA_ERR_HIP;
}

int decode_common(const void* q, const void* k_cache, const void* v_cache, const void* k_depth, const void* v_depth,
                  int B, int T, int Hq, int Hk, int d, int S, int L, void* out, float* lse, void* workspace,
                  size_t workspace_bytes, moda_stream_t stream) {
  const int rc = validate_decode(q, k_cache, v_cache, k_depth, v_depth, B, T, Hq, Hk, d, S, L, out, lse, workspace,
                                 workspace_bytes);
  if (rc != MODA_OK) return rc;
  moda::DecodeArgs a{q, k_cache, v_cache, L > 0 ? k_depth : nullptr, L > 0 ? v_depth : nullptr,
                     B, T, Hq, Hk, d, L, S, out, lse, workspace, stream};
  return moda::launch_decode_bf16(a) == hipSuccess ? MODA_OK : MODA_ERR_HIP;
}

}  // namespace

extern "C" {

int moda_attn_fwd(const void* q, const void* k_seq, const void* v_seq, const void* k_depth, const void* v_depth,
                  int B, int T, int Hq, int Hk, int d, int L, int causal, void* out, float* lse,
                  moda_stream_t stream) {
  return fwd_common(true, q, k_seq, v_seq, k_depth, v_depth, B, T, Hq, Hk, d, L, L, causal, out, lse, stream);
}

int moda_attn_fwd_ring(const void* q, const void* k_seq, const void* v_seq, const void* k_depth,
                       const void* v_depth, int B, int T, int Hq, int Hk, int d, int S, int L, int causal,
                       void* out, float* lse, moda_stream_t stream) {
  return fwd_common(true, q, k_seq, v_seq, k_depth, v_depth, B, T, Hq, Hk, d, S, L, causal, out, lse, stream);
}

int moda_attn_fwd_f32(const void* q, const void* k_seq, const void* v_seq, const void* k_depth,
                      const void* v_depth, int B, int T, int Hq, int Hk, int d, int L, int causal, void* out,
                      float* lse, moda_stream_t stream) {
  return fwd_common(false, q, k_seq, v_seq, k_depth, v_depth, B, T, Hq, Hk, d, L, L, causal, out, lse, stream);
}

int moda_attn_decode(const void* q, const void* k_cache, const void* v_cache, const void* k_depth,
                     const void* v_depth, int B, int T, int Hq, int Hk, int d, int L, void* out, float* lse,
                     void* workspace, size_t workspace_bytes, moda_stream_t stream) {
  return decode_common(q, k_cache, v_cache, k_depth, v_depth, B, T, Hq, Hk, d, L, L, out, lse, workspace,
                       workspace_bytes, stream);
}

int moda_attn_decode_ring(const void* q, const void* k_cache, const void* v_cache, const void* k_depth,
                          const void* v_depth, int B, int T, int Hq, int Hk, int d, int S, int L, void* out,
                          float* lse, void* workspace, size_t workspace_bytes, moda_stream_t stream) {
  return decode_common(q, k_cache, v_cache, k_depth, v_depth, B, T, Hq, Hk, d, S, L, out, lse, workspace,
                       workspace_bytes, stream);
}

int moda_attn_bwd(const void* q, const void* k_seq, const void* v_seq, const void* k_depth, const void* v_depth,
                  const void* out, const float* lse, const void* dout, int B, int T, int Hq, int Hk, int d, int L,
                  int causal, void* dq, void* dk_seq, void* dv_seq, void* dk_depth, void* dv_depth, void* workspace,
                  size_t workspace_bytes, moda_stream_t stream) {
  const int rc = validate_bwd(q, k_seq, v_seq, k_depth, v_depth, out, lse, dout, B, T, Hq, Hk, d, L, causal, dq,
                              dk_seq, dv_seq, dk_depth, dv_depth, workspace, workspace_bytes);
  if (rc != MODA_OK) return rc;
  const bool depth = L > 0;
  moda::BwdArgs a{q, k_seq, v_seq, depth ? k_depth : nullptr, depth ? v_depth : nullptr, out, lse, dout,
                  B, T, Hq, Hk, d, L, causal, dq, dk_seq, dv_seq, depth ? dk_depth : nullptr,
                  depth ? dv_depth : nullptr, workspace, stream};
  return moda::launch_bwd_bf16(a) == hipSuccess ? MODA_OK : MODA_ERR_HIP;
}

size_t moda_attn_bwd_workspace(int B, int T, int Hq, int Hk, int d, int L) {
  if (B <= 0 || T <= 0 || Hq <= 0 || Hk <= 0 || d <= 0 || L < 0) return 0;
  if (Hq % Hk != 0) return 0;
  return moda::bwd_workspace_bytes(B, T, Hq, d, L);
}

int moda_kv_project(const void* x, const void* w_kv, int B, int T, int Dm, int Hk, int d, void* k_out, void* v_out,
                    void* k_depth, void* v_depth, int S, int slot, moda_stream_t stream) {
  const int rc = validate_kv_project(x, w_kv, B, T, Dm, Hk, d, k_out, v_out, k_depth, v_depth, S, slot);
  if (rc != MODA_OK) return rc;
  moda::KvProjArgs a{x, w_kv, B, T, Dm, Hk, d, k_out, v_out, k_depth, v_depth, S, slot, stream};
  return moda::launch_kv_project(a) == hipSuccess ? MODA_OK : MODA_ERR_HIP;
}

int moda_attn_decode_noalloc(const void* q, const void* k_cache, const void* v_cache, const void* k_depth,
                             const void* v_depth, int B, int T, int Hq, int Hk, int d, int L, void* out,
                             float* lse, moda_stream_t stream) {
  const int rc = validate_decode_args(q, k_cache, v_cache, k_depth, v_depth, B, T, Hq, Hk, d, L, L, out, lse);
  if (rc != MODA_OK) return rc;
  if (moda::decode_workspace_bytes(B, T, Hq, Hk, d, L) > moda::kDecodeScratchBytes) return MODA_ERR_TOO_LARGE;
  void* ws = nullptr;
  if (moda::decode_scratch(&ws) != hipSuccess) return MODA_ERR_HIP;
  moda::DecodeArgs a{q, k_cache, v_cache, L > 0 ? k_depth : nullptr, L > 0 ? v_depth : nullptr,
                     B, T, Hq, Hk, d, L, L, out, lse, ws, stream};
  return moda::launch_decode_bf16(a) == hipSuccess ? MODA_OK : MODA_ERR_HIP;
}

size_t moda_attn_decode_workspace(int B, int T, int Hq, int Hk, int d, int L) {
  if (B <= 0 || T <= 0 || Hq <= 0 || Hk <= 0 || d <= 0 || L < 0) return 0;
  if (Hq % Hk != 0) return 0;
  return moda::decode_workspace_bytes(B, T, Hq, Hk, d, L);
}

int moda_pack_depth(const void* src, void* dst, int B, int T, int L, int Hk, int d, int elem_bytes,
                    moda_stream_t stream) {
  const int rc = validate_layout(src, dst, B, T, L, Hk, d, elem_bytes);
  if (rc != MODA_OK) return rc;
  return moda::launch_pack_depth(src, dst, B, T, L, Hk, d, elem_bytes, stream) == hipSuccess ? MODA_OK
                                                                                               : MODA_ERR_HIP;
}

int moda_append_depth_slot(const void* kv_l, void* dst, int slot, int B, int T, int L, int Hk, int d,
                           int elem_bytes, moda_stream_t stream) {
  const int rc = validate_layout(kv_l, dst, B, T, L, Hk, d, elem_bytes);
  if (rc != MODA_OK) return rc;
  if (slot < 0 || slot >= L) return MODA_ERR_SHAPE;
  return moda::launch_append_depth_slot(kv_l, dst, slot, B, T, L, Hk, d, elem_bytes, stream) == hipSuccess
             ? MODA_OK
             : MODA_ERR_HIP;
}

int moda_block_span(int row0, int rows, int G, int* t_start, int* t_end) {
  if (!t_start || !t_end) return MODA_ERR_NULL;
  if (row0 < 0 || rows <= 0 || G <= 0) return MODA_ERR_SHAPE;
  if (static_cast<int64_t>(row0) + rows - 1 > INT_MAX) return MODA_ERR_SHAPE;
  *t_start = row0 / G;
  *t_end = (row0 + rows - 1) / G + 1;
  return MODA_OK;
}

const char* moda_error_string(int code) {
  switch (code) {
    case MODA_OK: return "success";
    case MODA_ERR_NULL: return "a required pointer is NULL";
    case MODA_ERR_SHAPE: return "a size is out of range or inconsistent";
    case MODA_ERR_UNSUPPORTED: return "no kernel for this head dimension, group size or problem size";
    case MODA_ERR_ALIGN: return "a pointer is not 16-byte aligned";
    case MODA_ERR_HIP: return "the HIP launch failed";
    case MODA_ERR_TOO_LARGE: return "the problem needs more scratch than the allocation-free entry point holds";
    default: return "unknown error";
  }
}

}  // extern "C"
