// MoDA decode: one new token per sequence attends jointly to its KV cache and
// to its own L depth slots (one softmax over both sets; the sequence set of
// the last token of a causal layer is the whole cache).  Operation from
// "Mixture-of-Depths Attention" (papercache.org summary, 2.2 MoDA) and the
// MoDA reading notes (cc.laoqi.cc, 二.2 unified softmax; 二.4 on the decode
// cost of the depth cache).
//
// Split-K over the cache: workgroup (b, hk, c) reduces chunk c of the keys for
// the G query heads of KV head hk -- chunks of 128 to 1024 sequence keys (sized
// from the problem), plus one chunk holding the L depth slots -- to a partial (offset m, sum l, unnormalised
// o) per head in the caller's workspace.  A second kernel merges the chunks of
// each head by their offsets (the log-sum-exp identity), in a fixed order.
//
// Decode reads every cache element once and uses it G times, so the path is
// bound by HBM bandwidth.  Each workgroup is one wave: the G heads are rows of
// the 32-row MFMA tile (rows G..31 are zero and discarded), K/V tiles of 32
// keys (16 KiB per K/V pair at d = 128, so five waves fit a CU's LDS) are
// staged by direct-to-LDS loads, double buffered, and the score/PV steps are
// the forward kernel's.
#include <mutex>

#include "moda_launch.h"
#include "moda_tile.h"

// Per-device scratch of the allocation-free decode entry point: it holds the
// per-chunk partial results that moda_attn_decode keeps in the caller's
// workspace.  Every GPU the library runs on holds one copy until the process
// ends, and every call on that GPU shares it.
static __device__ __align__(256) float scratch[moda::kDecodeScratchBytes / sizeof(float)];

namespace moda {
namespace {

constexpr int kRows = 32;  // keys per LDS tile: one 32-key MFMA block

// Bytes of one K (or V) tile of kRows rows.
template <int D>
constexpr int kTileBytes = kRows * Tile<D>::ROW_BYTES;

// Sequence keys per workgroup: the largest of 1024, 512, 256 that still gives
// at least 512 workgroups (fewer, longer chunks amortise each workgroup's
// start-up and the merge; small problems need the parallelism), else 128.
int decode_chunk(int B, int T, int Hk) {
  for (int c = 1024; c >= 256; c >>= 1)
    if (static_cast<int64_t>(B) * Hk * ((T + c - 1) / c) >= 512) return c;
  return 128;
}
int decode_seq_chunks(int B, int T, int Hk) {
  const int c = decode_chunk(B, T, Hk);
  return (T + c - 1) / c;
}
int decode_chunks(int B, int T, int Hk, int L) { return decode_seq_chunks(B, T, Hk) + (L > 0 ? 1 : 0); }

// Direct-to-LDS loads of the K and V rows [first, first + kRows) of one chunk
// into buf (K at buf, V at buf + kTileBytes).  One wave loads the whole tile:
// instruction x fills rows pr = x*RPI + lane/CH, physical chunk lane % CH, with
// logical chunk pc ^ swz(pr).  Rows past the chunk's end fall outside the
// descriptors' ranges and read as zero.
template <int D>
__device__ __forceinline__ void dma_rows(const u32x4& rk, const u32x4& rv, uint32_t stride,
                                         int first, lds_u8* buf, int lane) {
  using TL = Tile<D>;
  lane = opaque(lane);  // recompute the per-lane offsets here rather than hold 2 * 64 / RPI registers
#pragma unroll
  for (int x = 0; x < kRows / TL::RPI; ++x) {
    const int pr = x * TL::RPI + lane / TL::CH;
    const int pc = lane % TL::CH;
    const uint32_t row = static_cast<uint32_t>(first + pr) * stride;
    const uint32_t ok = row + ((pc ^ TL::swz_k(pr)) * 16);
    const uint32_t ov = row + ((pc ^ TL::swz_v(pr)) * 16);
    const uint32_t dk = lds_addr(buf + x * 1024);
    dma16(rk, dk, ok);
    dma16(rv, dk + kTileBytes<D>, ov);
  }
}

// Partial results of one chunk for the G heads of one (b, hk).
//   ws_o  [B][Hq][nc][D] fp32: sum over the chunk's keys of 2^(s - m) * v
//   ws_ml [B][Hq][nc][2] fp32: (m, l), m the base-2 offset and l the sum of 2^(s - m)
template <int D>
__global__ __launch_bounds__(64) __attribute__((amdgpu_waves_per_eu(1, 4))) void moda_decode_partial_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ kc, const uint16_t* __restrict__ vc,
    const uint16_t* __restrict__ kd, const uint16_t* __restrict__ vd, int T, int Hq, int Hk, int L, int Lcap,
    int lgG, int chunk, int nc_seq, float scale_log2, float* __restrict__ ws_o, float* __restrict__ ws_ml) {
  using TL = Tile<D>;
  __shared__ __attribute__((aligned(1024))) uint8_t smem_raw[4 * kTileBytes<D>];  // two (K, V) tile buffers
  lds_u8* const smem = (lds_u8*)smem_raw;

  const int G = 1 << lgG;
  const int nc = nc_seq + (L > 0 ? 1 : 0);
  const int lane = threadIdx.x;
  const int r = lane & 31, half = lane >> 5;
  const int c = blockIdx.x % nc;
  const int bh = blockIdx.x / nc;
  const int hk = bh % Hk, b = bh / Hk;

  // This chunk's rows: sequence keys [key0, key0 + nkeys) of head hk, or the L depth slots.
  const bool depth = c == nc_seq;
  const uint16_t* kbase;
  const uint16_t* vbase;
  uint32_t stride;
  int nkeys;
  if (depth) {
    const int64_t slab = (static_cast<int64_t>(b) * Hk + hk) * Lcap * D;
    kbase = kd + slab;
    vbase = vd + slab;
    stride = D * 2;
    nkeys = L;
  } else {
    const int key0 = c * chunk;
    const int64_t first = (static_cast<int64_t>(b) * T + key0) * Hk * D + static_cast<int64_t>(hk) * D;
    kbase = kc + first;
    vbase = vc + first;
    stride = static_cast<uint32_t>(Hk) * D * 2;
    nkeys = min(chunk, T - key0);
  }
  const uint32_t range = static_cast<uint32_t>(nkeys - 1) * stride + D * 2;
  const u32x4 rk = raw_rsrc(kbase, range);
  const u32x4 rv = raw_rsrc(vbase, range);
  const int ntile = (nkeys + kRows - 1) / kRows;

  // Q^T fragments: row r is head hk*G + r (zero for r >= G).
  const bool row_ok = r < G;
  const int h = hk * G + r;
  bf16x8 qf[D / 16];
  {
    const uint16_t* qrow = q + (static_cast<int64_t>(b) * Hq + (row_ok ? h : 0)) * D;
#pragma unroll
    for (int sl = 0; sl < D / 16; ++sl) {
      u32x4 val = {0u, 0u, 0u, 0u};
      if (row_ok) val = *reinterpret_cast<const u32x4*>(qrow + sl * 16 + half * 8);
      qf[sl] = __builtin_bit_cast(bf16x8, val);
    }
  }

  // Per-lane LDS read offsets (the forward kernel's layout).
  uint32_t kr[D / 16], vr[D / 32];
#pragma unroll
  for (int sl = 0; sl < D / 16; ++sl) kr[sl] = r * TL::ROW_BYTES + (((2 * sl + half) ^ TL::swz_k(r)) * 16);
  {
    const int i = lane & 15, qd = (lane >> 4) & 1, hf = lane >> 5;
    const int row0 = 4 * hf + (i >> 2);
    const int sw = TL::swz_v(row0);
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt) {
      const int lc = (32 * dt + 16 * qd) / 8 + ((i & 3) >> 1);
      vr[dt] = row0 * TL::ROW_BYTES + 8 * (i & 1) + ((lc ^ sw) * 16);
    }
  }

  RowState<D> st;
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt) st.o[dt] = f32x16{};
  st.m = -INFINITY;
  st.l = 0.0f;

  dma_rows<D>(rk, rv, stride, 0, smem, lane);
  for (int t = 0; t < ntile; ++t) {
    lds_u8* cur = smem + opaque_s((t & 1) * 2 * kTileBytes<D>);
    lds_u8* nxt = smem + opaque_s(((t + 1) & 1) * 2 * kTileBytes<D>);
    publish_tile();
    if (t + 1 < ntile) dma_rows<D>(rk, rv, stride, (t + 1) * kRows, nxt, lane);
    const uint32_t base = lds_addr(cur);
    uint32_t ka[D / 16], va[D / 32];
#pragma unroll
    for (int sl = 0; sl < D / 16; ++sl) ka[sl] = base + kr[sl];
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt) va[dt] = base + kTileBytes<D> + vr[dt];
    const f32x16 sacc = qk_block<D>(qf, ka, 0);
    const int kt0 = t * kRows;
    float s[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int key = kt0 + 8 * (i >> 2) + 4 * half + (i & 3);
      s[i] = key < nkeys ? sacc[i] : -INFINITY;
    }
    bf16x8 pb[2];
    online_update<D, 16>(st, s, pb, scale_log2);
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) pv_group<D>(st, pb[hh], va, 16 * hh * TL::ROW_BYTES);
  }

  const float l_tot = pair_sum(st.l);
  if (row_ok) {
    const int64_t slot = (static_cast<int64_t>(b) * Hq + h) * nc + c;
    float* orow = ws_o + slot * D;
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
      for (int a = 0; a < 4; ++a) {
        const int d0 = dt * 32 + a * 8 + half * 4;
        f32x4 w = {st.o[dt][4 * a], st.o[dt][4 * a + 1], st.o[dt][4 * a + 2], st.o[dt][4 * a + 3]};
        *reinterpret_cast<f32x4*>(orow + d0) = w;
      }
    if (half == 0) {
      ws_ml[slot * 2] = st.m;
      ws_ml[slot * 2 + 1] = l_tot;
    }
  }
}

// Merge of the chunks of one (b, h): M = max m_c, Z = sum l_c 2^(m_c - M),
// out = sum o_c 2^(m_c - M) / Z, lse = (M + log2 Z) ln 2.  Wave w takes the
// chunks c = w mod 4 in increasing order and the four partial sums are added
// in wave order, so the result does not depend on timing.
constexpr int kMergeWaves = 4;

template <int D>
__global__ __launch_bounds__(kMergeWaves * 64) void moda_decode_merge_kernel(
    const float* __restrict__ ws_o, const float* __restrict__ ws_ml, int nc, uint16_t* __restrict__ out,
    float* __restrict__ lse) {
  constexpr int PER = D / 64;  // output elements per lane
  __shared__ float part[kMergeWaves][D + 2];
  const int bh = blockIdx.x;  // b * Hq + h
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const float* ml = ws_ml + static_cast<int64_t>(bh) * nc * 2;
  const float* o = ws_o + static_cast<int64_t>(bh) * nc * D;

  // M: every lane scans a strided share of the chunks, then a wave and a block reduction.
  float M = -INFINITY;
  for (int c = threadIdx.x; c < nc; c += kMergeWaves * 64) M = fmaxf(M, ml[2 * c]);
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) M = fmaxf(M, __shfl_xor(M, off));
  if (lane == 0) part[wave][D] = M;
  __syncthreads();
  M = part[0][D];
#pragma unroll
  for (int w = 1; w < kMergeWaves; ++w) M = fmaxf(M, part[w][D]);
  __syncthreads();
  const float base = M == -INFINITY ? 0.0f : M;

  float acc[PER], Z = 0.0f;
#pragma unroll
  for (int e = 0; e < PER; ++e) acc[e] = 0.0f;
#pragma unroll 4
  for (int c = wave; c < nc; c += kMergeWaves) {
    const float w = fast_exp2(ml[2 * c] - base);
    Z = fmaf(ml[2 * c + 1], w, Z);
#pragma unroll
    for (int e = 0; e < PER; ++e) acc[e] = fmaf(o[static_cast<int64_t>(c) * D + lane * PER + e], w, acc[e]);
  }
#pragma unroll
  for (int e = 0; e < PER; ++e) part[wave][lane * PER + e] = acc[e];
  if (lane == 0) part[wave][D + 1] = Z;
  __syncthreads();
  if (wave == 0) {
#pragma unroll
    for (int e = 0; e < PER; ++e) {
      acc[e] = part[0][lane * PER + e];
#pragma unroll
      for (int w = 1; w < kMergeWaves; ++w) acc[e] += part[w][lane * PER + e];
    }
    Z = part[0][D + 1];
#pragma unroll
    for (int w = 1; w < kMergeWaves; ++w) Z += part[w][D + 1];
    const float inv = 1.0f / Z;
    uint16_t* orow = out + static_cast<int64_t>(bh) * D;
    if constexpr (PER == 2) {
      *reinterpret_cast<uint32_t*>(orow + lane * 2) = pack_bf16x2(acc[0] * inv, acc[1] * inv);
    } else {
      orow[lane] = static_cast<uint16_t>(pack_bf16x2(acc[0] * inv, 0.0f) & 0xffffu);
    }
    if (lane == 0) lse[bh] = (M + __log2f(Z)) * kLn2;
  }
}

template <int D>
hipError_t launch_decode_d(const DecodeArgs& a) {
  const int lgG = __builtin_ctz(a.Hq / a.Hk);
  const int chunk = decode_chunk(a.B, a.T, a.Hk);
  const int nc_seq = decode_seq_chunks(a.B, a.T, a.Hk);
  const int nc = decode_chunks(a.B, a.T, a.Hk, a.L);
  const float scale_log2 = kLog2e / sqrtf(static_cast<float>(D));
  float* ws_o = static_cast<float*>(a.workspace);
  float* ws_ml = ws_o + static_cast<int64_t>(a.B) * a.Hq * nc * D;
  hipLaunchKernelGGL((moda_decode_partial_kernel<D>), dim3(static_cast<unsigned>(a.B * a.Hk * nc)), dim3(64), 0,
                     static_cast<hipStream_t>(a.stream), static_cast<const uint16_t*>(a.q),
                     static_cast<const uint16_t*>(a.k), static_cast<const uint16_t*>(a.v),
                     static_cast<const uint16_t*>(a.kd), static_cast<const uint16_t*>(a.vd), a.T, a.Hq, a.Hk, a.L,
                     a.Lcap, lgG, chunk, nc_seq, scale_log2, ws_o, ws_ml);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((moda_decode_merge_kernel<D>), dim3(static_cast<unsigned>(a.B * a.Hq)),
                     dim3(kMergeWaves * 64), 0,
                     static_cast<hipStream_t>(a.stream), ws_o, ws_ml, nc, static_cast<uint16_t*>(a.out), a.lse);
  return hipGetLastError();
}

}  // namespace

size_t decode_workspace_bytes(int B, int T, int Hq, int Hk, int d, int L) {
  return static_cast<size_t>(B) * Hq * decode_chunks(B, T, Hk, L) * (d + 2) * sizeof(float);
}

int64_t decode_grid_blocks(int B, int T, int Hk, int L) {
  return static_cast<int64_t>(B) * Hk * decode_chunks(B, T, Hk, L);
}

hipError_t launch_decode_bf16(const DecodeArgs& a) {
  return a.d == 64 ? launch_decode_d<64>(a) : launch_decode_d<128>(a);
}

namespace {
constexpr int kMaxDevices = 64;
std::mutex scratch_mu;
void* scratch_ptr[kMaxDevices];  // device address of `scratch` on each device, once looked up
}  // namespace

hipError_t decode_scratch(void** ptr) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(scratch_mu);
  if (!scratch_ptr[dev]) {
    // The array's name is a host-side stand-in; the kernels need this
    // device's own address of it, looked up once with the device current.
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    scratch_ptr[dev] = p;
  }
  *ptr = scratch_ptr[dev];
  return hipSuccess;
}

}  // namespace moda
