// Device building blocks shared by the bf16 MoDA kernels (gfx950): LDS tile
// geometry and swizzles, buffer descriptors, the MFMA score and PV steps and
// the online-softmax state.  Included by the kernel sources only.
#ifndef MODA_TILE_H
#define MODA_TILE_H

#include "moda_device.h"

namespace moda {
namespace {

constexpr int kBN = 64;  // rows (keys or depth slots) per LDS tile

// LDS pointers are kept in address space 3 (32-bit) so tile addressing is
// plain 32-bit arithmetic.
typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(3))) uint8_t lds_u8;
typedef __attribute__((ext_vector_type(4))) short s16x4;
typedef __attribute__((address_space(3))) s16x4 lds_s16x4_t;
typedef __attribute__((address_space(3))) bf16x8 lds_bf16x8_t;

// The LDS object at byte address addr.  (Built from the integer: the null
// pointer of the LDS address space is not address 0.)
template <typename T>
__device__ __forceinline__ T* lds_at(uint32_t addr) {
  return reinterpret_cast<T*>(static_cast<uintptr_t>(addr));
}
__device__ __forceinline__ uint32_t lds_addr(const lds_u8* p) {
  return static_cast<uint32_t>(reinterpret_cast<uintptr_t>(p));
}

// Tile geometry for head dimension D: kBN rows (keys or depth slots) of D*2
// bytes = CH chunks of 16 bytes.  One direct-to-LDS load instruction of a
// wave fills 1 KiB = RPI rows.
template <int D>
struct Tile {
  static constexpr int ROW_BYTES = D * 2;
  static constexpr int CH = D / 8;
  static constexpr int RPI = 64 / CH;
  static constexpr int BYTES = kBN * ROW_BYTES;  // one K or V tile
  static constexpr int RPB = 256 / ROW_BYTES;    // rows sharing one 256-byte bank row
  // Chunk swizzles: logical chunk c of row r lives at physical chunk c ^ swz(r).
  __device__ static __forceinline__ int swz_k(int row) { return (row / RPB) % CH; }
  __device__ static __forceinline__ int swz_v(int row) { return 4 * ((row / RPB) % (CH / 4)); }
};

constexpr uint32_t kOutOfRange = 0x80000000u;  // > every descriptor range (host-checked)
constexpr int kBufFlags = 0x00020000;         // raw buffer, 32-bit dwords

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const uint16_t* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(base), static_cast<short>(0),
                                           static_cast<int>(bytes), kBufFlags);
}

// A raw buffer descriptor as four scalar dwords (the same fields as
// make_rsrc: base address, stride 0, `bytes` records of one byte).
__device__ __forceinline__ u32x4 raw_rsrc(const uint16_t* base, uint32_t bytes) {
  const uint64_t a = reinterpret_cast<uint64_t>(base);
  return u32x4{static_cast<uint32_t>(a), static_cast<uint32_t>(a >> 32) & 0xffffu, bytes,
               static_cast<uint32_t>(kBufFlags)};
}

// One direct-to-LDS load of 16 bytes per lane (the wave fills 1 KiB at LDS
// byte address `lds`), issued as inline asm so that the compiler does not know
// a load into LDS is in flight.  Knowing it, the compiler makes every
// transposed LDS read (a builtin) wait for all such loads first -- in a double
// buffered pipeline that is the next tile's load, in the middle of the current
// tile.  Visibility is the pipeline's own explicit vmcnt wait and barrier.
// The compiler's hazard checks do not look inside inline asm.  The s_nop
// covers the M0 write -> LDS-DMA hazard (the compiler sets M0 just before the
// statement).  The other hazard of the statement, a VALU write of a descriptor
// SGPR fewer than 5 wait states before it (the compiler reloads spilled SGPRs
// with v_readlane; read early, a descriptor dword is stale and the load goes
// to a wrong address), is left to the surrounding code: the build scans the
// compiled kernels for it and refuses to link a library that has it.  rsrc
// and lds are scalar operands: they must be the same in every lane of the
// wave.
__device__ __forceinline__ void dma16(const u32x4& rsrc, uint32_t lds, uint32_t voff) {
  asm volatile("s_nop 0\n\tbuffer_load_dwordx4 %0, %1, 0 offen lds" ::"v"(voff), "s"(rsrc), "{m0}"(lds) : "memory");
}

// Running softmax state of one query row held by a lane pair (l, l ^ 32).
template <int D>
struct RowState {
  f32x16 o[D / 32];  // O^T accumulator: d = 32*dt + 8*(i/4) + 4*half + (i%4)
  float m;           // base-2 exponent offset of the row (same in both lanes)
  float l;           // this lane's share of the running denominator
};

// The row's exponent offset m only moves when a block's max exceeds it by more
// than this (base 2), so unnormalised weights stay below 2^8 and the costly
// rescale of the output accumulator is rare.  Any offset gives the same
// quotient; the final division and lse use the offset actually applied.
constexpr float kRescaleSlack = 8.0f;

// acc *= alpha, element by element in the accumulator's own registers.  As
// plain code the multiply gets fresh destination registers and, once the
// conditional rescale merges back, every tile pays a copy of the whole
// accumulator; tying each element's input and output keeps it in place.
// Inline asm is invisible to the compiler's hazard checks, so the waits are
// explicit: before the first multiply, enough wait states for an MFMA result
// (the accumulator may have been written by one shortly before) and for the
// v_exp result alpha; after the last one, the wait a VALU result needs before
// an MFMA reads it as its accumulator.
__device__ __forceinline__ void scale_in_place(f32x16& acc, float alpha, bool first, bool last) {
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    float x = acc[i];
    if (first && i == 0)
      asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7\n\tv_mul_f32 %0, %0, %1" : "+v"(x) : "v"(alpha));
    else if (last && i == 15)
      asm volatile("v_mul_f32 %0, %0, %1\n\ts_nop 3" : "+v"(x) : "v"(alpha));
    else
      asm volatile("v_mul_f32 %0, %0, %1" : "+v"(x) : "v"(alpha));
    acc[i] = x;
  }
}

// Max and sum of N values as balanced trees (three-input max steps), so the
// dependent chain is a few instructions long rather than N.
template <int N>
__device__ __forceinline__ float tree_max(const float (&s)[N]) {
  float a[(N + 2) / 3];
#pragma unroll
  for (int i = 0; i < (N + 2) / 3; ++i) {
    a[i] = s[3 * i];
    if (3 * i + 1 < N) a[i] = fmaxf(a[i], s[3 * i + 1]);
    if (3 * i + 2 < N) a[i] = fmaxf(a[i], s[3 * i + 2]);
  }
  if constexpr ((N + 2) / 3 == 1) {
    return a[0];
  } else {
    return tree_max<(N + 2) / 3>(a);
  }
}

template <int N>
__device__ __forceinline__ float tree_sum(const float (&s)[N]) {
  static_assert((N & (N - 1)) == 0, "power of two");
  if constexpr (N == 1) {
    return s[0];
  } else {
    float a[N / 2];
#pragma unroll
    for (int i = 0; i < N / 2; ++i) a[i] = s[i] + s[i + N / 2];
    return tree_sum<N / 2>(a);
  }
}

// Fold N raw scores (-inf = masked) into the state and return the weights,
// packed to bf16 in groups of 8 (one PV B operand per group).
template <int D, int N>
__device__ __forceinline__ void online_update(RowState<D>& st, float (&s)[N], bf16x8 (&pb)[N / 8], float scale) {
  const float mx = pair_max(tree_max<N>(s));
  const float m_blk = mx * scale;  // -inf stays -inf (scale > 0)
  if (__any(m_blk > st.m + kRescaleSlack)) {
    const float m_new = fmaxf(st.m, m_blk);
    const float alpha = fast_exp2(st.m - (m_new == -INFINITY ? 0.0f : m_new));
    st.l *= alpha;
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt) scale_in_place(st.o[dt], alpha, dt == 0, dt == D / 32 - 1);
    st.m = m_new;
  }
  const float base = (st.m == -INFINITY) ? 0.0f : st.m;
#pragma unroll
  for (int i = 0; i < N; ++i) s[i] = fast_exp2(fmaf(s[i], scale, -base));
  st.l += tree_sum<N>(s);
#pragma unroll
  for (int h = 0; h < N / 8; ++h) {
    u32x4 w;
#pragma unroll
    for (int k = 0; k < 4; ++k) w[k] = pack_bf16x2(s[8 * h + 2 * k], s[8 * h + 2 * k + 1]);
    pb[h] = __builtin_bit_cast(bf16x8, w);
  }
}

// S^T block: 32 keys x the wave's 32 query rows.  kt[sl] holds the lane's
// read address of slice sl for the block's first row; lane l supplies key row
// l%32, logical chunk 2*sl + l/32.
template <int D>
__device__ __forceinline__ f32x16 qk_block(const bf16x8 (&qf)[D / 16], const uint32_t (&kt)[D / 16], int row_bytes_off) {
  f32x16 s = {};
#pragma unroll
  for (int sl = 0; sl < D / 16; ++sl) {
    const bf16x8 a = *lds_at<lds_bf16x8_t>(kt[sl] + row_bytes_off);
    s = mfma32(a, qf[sl], s);
  }
  return s;
}

// O^T += V^T * P^T for one 16-key group whose first V row is `off` bytes past
// the addresses in vt.  The B operand pb holds, in lane half hf, the weights
// of keys 4*hf + {0..3} and 8 + 4*hf + {0..3} of the group.  The A operand is
// read with two transposing LDS reads: lane i of each 16-lane group points at
// row key_b + i/4, columns d0 + 4*(i%4) .. +3, and receives V[key_b + k][d0 + i]
// for k = 0..3.
template <int D>
__device__ __forceinline__ void pv_group(RowState<D>& st, const bf16x8& pb, const uint32_t (&vt)[D / 32], int off) {
  using TL = Tile<D>;
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt) {
    const s16x4 lo4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(lds_at<lds_s16x4_t>(vt[dt] + off));
    const s16x4 hi4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(lds_at<lds_s16x4_t>(vt[dt] + off + 8 * TL::ROW_BYTES));
    const bf16x8 a = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo4, hi4, 0, 1, 2, 3, 4, 5, 6, 7));
    st.o[dt] = mfma32(a, pb, st.o[dt]);
  }
}

// Transposed LDS reads issued as inline asm.  As a compiler builtin every such
// read first waits for all outstanding direct-to-LDS loads (the compiler
// cannot tell that those fill another buffer), which exposes the next tile's
// load latency in every tile.  The compiler does not track these reads, so
// their consumers must follow lds_ready() on the same values.
__device__ __forceinline__ s16x4 read_tr_async(uint32_t addr) {
  s16x4 r;
  asm volatile("ds_read_b64_tr_b16 %0, %1" : "=v"(r) : "v"(addr));
  return r;
}
// The same at a compile-time byte offset, which goes into the instruction's
// offset field instead of costing an address add.
template <int OFF>
__device__ __forceinline__ s16x4 read_tr_async_at(uint32_t addr) {
  static_assert(OFF >= 0 && OFF < 65536, "LDS instruction offset field");
  s16x4 r;
  asm volatile("ds_read_b64_tr_b16 %0, %1 offset:%2" : "=v"(r) : "v"(addr), "i"(OFF));
  return r;
}
// Wait until every LDS read of this wave has returned; afterwards the values
// passed here may be used (each is re-defined after the wait).
__device__ __forceinline__ void lds_wait() { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); }
// Re-define values after lds_wait(), so that their consumers cannot be placed
// before it.
template <int N>
__device__ __forceinline__ void lds_tie(bf16x8 (&x)[N]) {
#pragma unroll
  for (int i = 0; i < N; ++i) asm volatile("" : "+v"(x[i]));
}
template <int N>
__device__ __forceinline__ void lds_ready(bf16x8 (&x)[N]) {
  lds_wait();
  lds_tie(x);
}

// Ask the scheduler to alternate the region's N matrix products with its vector
// instructions (one product, then up to K vector ops).
template <int N, int K>
__device__ __forceinline__ void interleave() {
#pragma unroll
  for (int i = 0; i < N; ++i) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    __builtin_amdgcn_sched_group_barrier(0x002, K, 0);
  }
}

// Publish the tile this wave's DMA loads filled: wait for them, then barrier.
__device__ __forceinline__ void publish_tile() {
  __builtin_amdgcn_s_waitcnt(0x0f70);  // vmcnt(0)
  __syncthreads();
}

}  // namespace
}  // namespace moda

#endif  // MODA_TILE_H
