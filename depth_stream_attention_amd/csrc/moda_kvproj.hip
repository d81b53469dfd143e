// Depth write path: the KV projection of a layer's hidden states, written by
// the GEMM's epilogue straight into one slot of the packed depth stream (gfx950).
//
// A layer adds its KV to the depth stream of every token: the attention
// branch its own K, V, the FFN branch a KV projection of the FFN input (MoDA
// reading notes, cc.laoqi.cc, 二.3; "Mixture-of-Depths Attention" summary,
// papercache.org, 2.2, the write step).  Both are one product
//   [K | V] (tokens x 2*Hk*d) = X (tokens x Dm) * W^T,  W = [2*Hk*d][Dm]
// whose rows are the output channels (K channels, then V channels).  Instead
// of writing [B,T,Hk,d] and copying it into slot `slot` of the packed
// [B,T,Hk,S,d] stream afterwards, the epilogue stores each result once into
// the slot (and, when asked, also into the layer's sequence K/V buffers).
//
// Decomposition: a workgroup owns 128 channels x 128 tokens, 4 waves each 64
// channels x 64 tokens = 2 x 2 blocks of 32x32 on v_mfma_f32_32x32x16_bf16.
// The products are formed transposed, C^T = W X^T (A = weight rows, B = token
// rows), so that each lane owns one token and four consecutive channels per
// register group: the epilogue stores 8 bytes per lane per group.  Dm is
// walked in 64-element chunks, double-buffered in LDS by direct-to-LDS buffer
// loads (16 bytes per lane, rows XOR-swizzled so the operand reads are free of
// bank conflicts); the chunk offset is the scalar offset of the loads, so the
// per-lane offsets are loop invariant.
#include "moda_launch.h"
#include "moda_tile.h"

namespace moda {
namespace {

constexpr int kKW = 4;                 // waves
constexpr int kKThreads = kKW * 64;
constexpr int kTileRows = 128;         // channels and tokens per workgroup
constexpr int kKC = 64;                // Dm elements per LDS chunk
constexpr int kRowBytes = kKC * 2;     // 128 bytes per tile row
constexpr int kTileBytes = kTileRows * kRowBytes;  // 16 KiB per operand tile
constexpr int kStageBytes = 2 * kTileBytes;        // weight tile, then token tile
constexpr int kLoadsPerWave = kTileBytes / 1024 / kKW;  // 1 KiB per wave-wide load

// Two tile rows share one 256-byte LDS line; 16 consecutive rows read with one
// logical chunk meet 8 distinct swizzles in each half of the line.
__device__ __forceinline__ int swz(int row) { return (row >> 1) & 7; }

template <bool SEQ, bool DEPTH>
__global__ __launch_bounds__(kKThreads) __attribute__((amdgpu_waves_per_eu(2, 2))) void moda_kv_project_kernel(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ w, int M, int Dm, int Hk, int d, int S, int slot,
    int n_tiles_c, uint16_t* __restrict__ k_out, uint16_t* __restrict__ v_out, uint16_t* __restrict__ k_depth,
    uint16_t* __restrict__ v_depth) {
  __shared__ __attribute__((aligned(1024))) uint8_t smem_raw[2 * kStageBytes];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int half = lane >> 5;
  // Channel tiles vary fastest, so consecutive workgroups share their tokens.
  const int ct = blockIdx.x % n_tiles_c;
  const int mt = blockIdx.x / n_tiles_c;
  const int n0 = ct * kTileRows;
  const int m0 = mt * kTileRows;
  const int cw0 = (wave & 1) * 64;   // the wave's channels within the tile
  const int tw0 = (wave >> 1) * 64;  // the wave's tokens within the tile

  // Buffer descriptors: weight rows n0.., token rows m0.. (rows past M read as zero).
  const uint32_t row_bytes = static_cast<uint32_t>(Dm) * 2;
  const int64_t xrange = static_cast<int64_t>(M - m0) * row_bytes;
  const __amdgpu_buffer_rsrc_t rw = make_rsrc(w + static_cast<int64_t>(n0) * Dm, kTileRows * row_bytes);
  const __amdgpu_buffer_rsrc_t rx = make_rsrc(x + static_cast<int64_t>(m0) * Dm,
                                              static_cast<uint32_t>(xrange < 0x7fffffff ? xrange : 0x7fffffff));
  // Load instruction j of this wave fills tile rows pr = (wave*L + j)*8 + lane/8,
  // physical chunk lane%8 (logical chunk (lane%8) ^ swz(pr)).
  uint32_t dma_off[kLoadsPerWave];
#pragma unroll
  for (int j = 0; j < kLoadsPerWave; ++j) {
    const int pr = (wave * kLoadsPerWave + j) * 8 + lane / 8;
    dma_off[j] = static_cast<uint32_t>(pr) * row_bytes + (((lane & 7) ^ swz(pr)) * 16);
  }
  auto dma = [&](int chunk, int stage) {
    lds_u8* base = (lds_u8*)smem_raw + stage * kStageBytes;
    const int soff = chunk * kKC * 2;
#pragma unroll
    for (int j = 0; j < kLoadsPerWave; ++j) {
      lds_u8* dst = base + (wave * kLoadsPerWave + j) * 1024;
      const uint32_t off = dma_off[j];
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rw, (lds_void_t*)dst, 16, off, soff, 0, 0);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rx, (lds_void_t*)(dst + kTileBytes), 16, off, soff, 0, 0);
    }
  };

  // Operand read offsets: block b of the wave's rows, 16-element slice sl:
  // row = base + 32*b + lane%32, logical chunk 2*sl + lane/32.
  uint32_t rd_w[2][4], rd_x[2][4];
#pragma unroll
  for (int b = 0; b < 2; ++b)
#pragma unroll
    for (int sl = 0; sl < 4; ++sl) {
      const int rw_row = cw0 + 32 * b + (lane & 31);
      const int rx_row = tw0 + 32 * b + (lane & 31);
      rd_w[b][sl] = rw_row * kRowBytes + (((2 * sl + half) ^ swz(rw_row)) * 16);
      rd_x[b][sl] = kTileBytes + rx_row * kRowBytes + (((2 * sl + half) ^ swz(rx_row)) * 16);
    }

  f32x16 acc[2][2];  // [channel block][token block]
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int b = 0; b < 2; ++b) acc[a][b] = f32x16{};

  const int nch = Dm / kKC;
  dma(0, 0);
  for (int c = 0; c < nch; ++c) {
    publish_tile();
    if (c + 1 < nch) dma(c + 1, (c + 1) & 1);
    const uint32_t base = lds_addr((lds_u8*)smem_raw) + opaque_s((c & 1) * kStageBytes);
#pragma unroll
    for (int sl = 0; sl < 4; ++sl) {
      bf16x8 fa[2], fb[2];
#pragma unroll
      for (int b = 0; b < 2; ++b) {
        fa[b] = *lds_at<lds_bf16x8_t>(base + rd_w[b][sl]);
        fb[b] = *lds_at<lds_bf16x8_t>(base + rd_x[b][sl]);
      }
#pragma unroll
      for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int b = 0; b < 2; ++b) acc[a][b] = mfma32(fa[a], fb[b], acc[a][b]);
    }
  }

  // Epilogue: acc[a][b] element i of this lane is channel n0 + cw0 + 32a + 8(i/4) +
  // 4*half + i%4 of token m0 + tw0 + 32b + lane%32.  Four consecutive channels never
  // cross a head, so each group is one 8-byte store per destination.
  const int HD = Hk * d;
#pragma unroll
  for (int b = 0; b < 2; ++b) {
    const int tok = m0 + tw0 + 32 * b + (lane & 31);
    if (tok >= M) continue;
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int ch = n0 + cw0 + 32 * a + 8 * g + 4 * half;
        const bool is_v = ch >= HD;
        const int r = is_v ? ch - HD : ch;
        const int hk = r / d, cc = r - hk * d;
        u32x2 val = {pack_bf16x2(acc[a][b][4 * g], acc[a][b][4 * g + 1]),
                     pack_bf16x2(acc[a][b][4 * g + 2], acc[a][b][4 * g + 3])};
        const int64_t th = static_cast<int64_t>(tok) * Hk + hk;
        if (SEQ) *reinterpret_cast<u32x2*>((is_v ? v_out : k_out) + th * d + cc) = val;
        if (DEPTH) *reinterpret_cast<u32x2*>((is_v ? v_depth : k_depth) + (th * S + slot) * d + cc) = val;
      }
  }
}

template <bool SEQ, bool DEPTH>
hipError_t launch(const KvProjArgs& a) {
  const int M = a.B * a.T;
  const int n_tiles_c = 2 * a.Hk * a.d / kTileRows;
  const int64_t blocks = static_cast<int64_t>((M + kTileRows - 1) / kTileRows) * n_tiles_c;
  hipLaunchKernelGGL((moda_kv_project_kernel<SEQ, DEPTH>), dim3(static_cast<unsigned>(blocks)), dim3(kKThreads), 0,
                     static_cast<hipStream_t>(a.stream), static_cast<const uint16_t*>(a.x),
                     static_cast<const uint16_t*>(a.w), M, a.Dm, a.Hk, a.d, a.S, a.slot, n_tiles_c,
                     static_cast<uint16_t*>(a.k_out), static_cast<uint16_t*>(a.v_out),
                     static_cast<uint16_t*>(a.k_depth), static_cast<uint16_t*>(a.v_depth));
  return hipGetLastError();
}

}  // namespace

int64_t kv_project_grid_blocks(int B, int T, int Hk, int d) {
  const int64_t M = static_cast<int64_t>(B) * T;
  return (M + kTileRows - 1) / kTileRows * (2 * static_cast<int64_t>(Hk) * d / kTileRows);
}

hipError_t launch_kv_project(const KvProjArgs& a) {
  const bool seq = a.k_out != nullptr, depth = a.k_depth != nullptr;
  if (seq && depth) return launch<true, true>(a);
  if (seq) return launch<true, false>(a);
  return launch<false, true>(a);
}

}  // namespace moda
