// Device-side types and small helpers shared by the MoDA HIP kernels (gfx950).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moda {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;
typedef __attribute__((ext_vector_type(16))) float f32x16;
typedef __attribute__((ext_vector_type(2))) float f32x2;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(4))) uint32_t u32x4;
typedef __attribute__((ext_vector_type(2))) uint32_t u32x2;

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// 32x32x16 bf16 matrix-core product with fp32 accumulation: acc += A * B.
// A lane l supplies row (l % 32) of A, B lane l supplies column (l % 32) of B;
// both carry 8 consecutive elements of the contraction index chosen by l / 32.
// acc element i of lane l is C[8*(i/4) + 4*(l/32) + (i%4)][l % 32].
__device__ __forceinline__ f32x16 mfma32(const bf16x8& a, const bf16x8& b, const f32x16& acc) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc, 0, 0, 0);
}

// Two fp32 values -> two bf16 (round to nearest even), packed in one dword.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  f32x2 f = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f, bf16x2));
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Lanes l and l ^ 32 exchange through v_permlane32_swap (upper half of the
// first operand <-> lower half of the second).  With both operands holding x,
// afterwards each lane has x[l] in one and x[l ^ 32] in the other, so their
// max / sum needs no select.  Issued as inline asm: the compiler builtin,
// given two equal inputs, folds its two results into one.  The leading
// s_nop covers the VALU-write -> permlane-read hazard.
__device__ __forceinline__ void swap_halves(float& a, float& b) {
  asm volatile("s_nop 1\n\tv_permlane32_swap_b32 %0, %1" : "+v"(a), "+v"(b));
}
// Returns x through an empty asm statement, hiding its value from the
// optimiser at this point: values derived from it are then computed here
// instead of being hoisted out of a loop and held in registers across it.
__device__ __forceinline__ int opaque(int x) {
  asm volatile("" : "+v"(x));
  return x;
}
__device__ __forceinline__ int opaque_s(int x) {  // the same for a wave-uniform value
  asm volatile("" : "+s"(x));
  return x;
}
__device__ __forceinline__ float pair_max(float x) {
  float a = x, b = x;
  swap_halves(a, b);
  return fmaxf(a, b);
}
__device__ __forceinline__ float pair_sum(float x) {
  float a = x, b = x;
  swap_halves(a, b);
  return a + b;
}

}  // namespace moda
