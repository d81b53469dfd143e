// MoDA forward in fp32 (fp32 inputs, fp32 arithmetic, fp32 output).
//
// Same operation as the bf16 kernel: one softmax per query row over the
// row's causally visible sequence keys and the L depth slots of its own token
// ("Mixture-of-Depths Attention" summary, papercache.org, 2.2 MoDA; MoDA
// reading notes, cc.laoqi.cc, 二.2), with the online update of 二.5 / 3.3
// (running max, running sum, one final division).
//
// This path serves fp32 callers and small problems; it runs on the vector
// ALUs.  One wave owns one query row: in each 64-candidate block lane j
// computes the full logit of candidate j, the wave reduces max and sum with
// cross-lane shuffles, and every lane then accumulates its own d columns of
// the output over the block's candidates.  Sequence candidates come first,
// then the token's depth slots, through the same running state.
#include "moda_device.h"
#include "moda_launch.h"

namespace moda {
namespace {

constexpr int kWaves = 4;

__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x = fmaxf(x, __shfl_xor(x, o, 64));
  return x;
}
__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x += __shfl_xor(x, o, 64);
  return x;
}

template <int D>
struct F32Row {
  float q[D];       // the query row (same in every lane)
  float o[D / 64];  // this lane's output columns d = lane + 64*e
  float m, l;
};

// Fold candidates [0, n) of one block into the row state.  Candidate j's key
// row is at key + j*stride and its value row at val + j*stride.
template <int D>
__device__ __forceinline__ void f32_block(F32Row<D>& st, const float* __restrict__ key,
                                          const float* __restrict__ val, int64_t stride, int n, int lane,
                                          float scale) {
  float s = -INFINITY;
  if (lane < n) {
    const float* kr = key + lane * stride;
    float acc = 0.0f;
#pragma unroll
    for (int c = 0; c < D; c += 4) {
      const float4 kk = *reinterpret_cast<const float4*>(kr + c);
      acc = fmaf(st.q[c], kk.x, acc);
      acc = fmaf(st.q[c + 1], kk.y, acc);
      acc = fmaf(st.q[c + 2], kk.z, acc);
      acc = fmaf(st.q[c + 3], kk.w, acc);
    }
    s = acc * scale;
  }
  const float m_new = fmaxf(st.m, wave_max(s));  // finite: n >= 1
  const float alpha = expf(st.m - m_new);
  const float p = (lane < n) ? expf(s - m_new) : 0.0f;
  st.l = st.l * alpha + wave_sum(p);
  st.m = m_new;
#pragma unroll
  for (int e = 0; e < D / 64; ++e) st.o[e] *= alpha;
  for (int j = 0; j < n; ++j) {
    const float pj = __shfl(p, j, 64);
    const float* vr = val + j * stride;
#pragma unroll
    for (int e = 0; e < D / 64; ++e) st.o[e] = fmaf(pj, vr[lane + 64 * e], st.o[e]);
  }
}

template <int D>
__global__ __launch_bounds__(kWaves * 64) void moda_fwd_f32_kernel(
    const float* __restrict__ q, const float* __restrict__ k, const float* __restrict__ v,
    const float* __restrict__ kd, const float* __restrict__ vd, int B, int T, int Hq, int Hk, int L, int Lcap,
    int causal, float scale, float* __restrict__ out, float* __restrict__ lse) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t row = static_cast<int64_t>(blockIdx.x) * kWaves + wave;  // rows in (b, t, h) order
  if (row >= static_cast<int64_t>(B) * T * Hq) return;                  // whole wave leaves together
  const int h = static_cast<int>(row % Hq);
  const int t = static_cast<int>((row / Hq) % T);
  const int b = static_cast<int>(row / (static_cast<int64_t>(Hq) * T));
  const int G = Hq / Hk;
  const int hk = h / G;

  F32Row<D> st;
  const float* qr = q + row * D;
#pragma unroll
  for (int c = 0; c < D; c += 4) {
    const float4 x = *reinterpret_cast<const float4*>(qr + c);
    st.q[c] = x.x;
    st.q[c + 1] = x.y;
    st.q[c + 2] = x.z;
    st.q[c + 3] = x.w;
  }
#pragma unroll
  for (int e = 0; e < D / 64; ++e) st.o[e] = 0.0f;
  st.m = -INFINITY;
  st.l = 0.0f;

  const int64_t kv_stride = static_cast<int64_t>(Hk) * D;
  const float* kb = k + (static_cast<int64_t>(b) * T * Hk + hk) * D;
  const float* vb = v + (static_cast<int64_t>(b) * T * Hk + hk) * D;
  const int nseq = causal ? t + 1 : T;
  for (int j0 = 0; j0 < nseq; j0 += 64)
    f32_block<D>(st, kb + j0 * kv_stride, vb + j0 * kv_stride, kv_stride, min(64, nseq - j0), lane, scale);
  if (L > 0) {
    const int64_t slab = ((static_cast<int64_t>(b) * T + t) * Hk + hk) * Lcap * D;
    for (int i0 = 0; i0 < L; i0 += 64)
      f32_block<D>(st, kd + slab + static_cast<int64_t>(i0) * D, vd + slab + static_cast<int64_t>(i0) * D, D,
                   min(64, L - i0), lane, scale);
  }

  const float inv = 1.0f / st.l;
  float* orow = out + row * D;
#pragma unroll
  for (int e = 0; e < D / 64; ++e) orow[lane + 64 * e] = st.o[e] * inv;
  if (lane == 0) lse[(static_cast<int64_t>(b) * Hq + h) * T + t] = st.m + logf(st.l);
}

template <int D>
hipError_t launch_d(const FwdArgs& a) {
  const int64_t rows = static_cast<int64_t>(a.B) * a.T * a.Hq;
  const unsigned blocks = static_cast<unsigned>((rows + kWaves - 1) / kWaves);
  hipLaunchKernelGGL((moda_fwd_f32_kernel<D>), dim3(blocks), dim3(kWaves * 64), 0,
                     static_cast<hipStream_t>(a.stream), static_cast<const float*>(a.q),
                     static_cast<const float*>(a.k), static_cast<const float*>(a.v),
                     static_cast<const float*>(a.kd), static_cast<const float*>(a.vd), a.B, a.T, a.Hq, a.Hk, a.L, a.Lcap,
                     a.causal, 1.0f / sqrtf(static_cast<float>(D)), static_cast<float*>(a.out), a.lse);
  return hipGetLastError();
}

}  // namespace

int64_t fwd_f32_grid_blocks(int B, int T, int Hq) {
  return (static_cast<int64_t>(B) * T * Hq + kWaves - 1) / kWaves;
}

hipError_t launch_fwd_f32(const FwdArgs& a) { return a.d == 64 ? launch_d<64>(a) : launch_d<128>(a); }

}  // namespace moda
