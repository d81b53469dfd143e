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
// Decomposition: a workgroup of 8 waves (two per SIMD) owns 256 channels x 256
// tokens; wave w computes channels 128*(w%2) .. +128 x tokens 64*(w/2) .. +64 as
// 8 x 4 blocks of 16x16 on v_mfma_f32_16x16x32_bf16 (twelve operand reads per
// 32 products; the scheduler places them, measured 3.5-5% faster than 32x32
// blocks with the reads fetched one slice ahead by hand).  The products are
// formed transposed, C^T = W X^T (A = weight rows, B = token rows).  Dm is walked in 64-element chunks, double-buffered in
// LDS by direct-to-LDS buffer loads (16 bytes per lane, rows XOR-swizzled so
// the operand reads are free of bank conflicts); the chunk offset is the
// loads' scalar offset, so the per-lane offsets are loop invariant.  The
// epilogue rounds to bf16 and stages the 256 x 256 tile through LDS as
// [token][channel] rows, so that each 16-byte global store holds 8 consecutive
// channels of one token and a wave stores whole 512-byte token rows.
#include "moda_launch.h"
#include "moda_tile.h"

namespace moda {
namespace {

constexpr int kKW = 8;                 // waves
constexpr int kKThreads = kKW * 64;
constexpr int kTileRows = 256;         // channels and tokens per workgroup
constexpr int kKC = 64;                // Dm elements per LDS chunk
constexpr int kRowBytes = kKC * 2;     // 128 bytes per operand tile row
constexpr int kTileBytes = kTileRows * kRowBytes;  // 32 KiB per operand tile
constexpr int kStageBytes = 2 * kTileBytes;        // weight tile, then token tile
constexpr int kLoadsPerWave = kTileBytes / 1024 / kKW;  // 1 KiB per wave-wide load
constexpr int kEpiRow = kTileRows * 2 + 16;        // staged output row: 256 channels + 16 bytes of skew
constexpr int kSmemBytes = (2 * kStageBytes > kTileRows * kEpiRow) ? 2 * kStageBytes : kTileRows * kEpiRow;

// Two tile rows share one 256-byte LDS line; 16 consecutive rows read with one
// logical chunk meet 8 distinct swizzles in each half of the line.  The
// swizzle repeats every 16 rows, so 16-row steps are immediate offsets.
__device__ __forceinline__ int swz(int row) { return (row >> 1) & 7; }

template <bool SEQ, bool DEPTH>
__global__ __launch_bounds__(kKThreads) __attribute__((amdgpu_waves_per_eu(2, 2))) void moda_kv_project_kernel(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ w, int M, int Dm, int Hk, int d, int S, int slot,
    int n_tiles_c, uint16_t* __restrict__ k_out, uint16_t* __restrict__ v_out, uint16_t* __restrict__ k_depth,
    uint16_t* __restrict__ v_depth) {
  __shared__ __attribute__((aligned(1024))) uint8_t smem_raw[kSmemBytes];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int HD = Hk * d;
  const int N = 2 * HD;
  // Workgroups are dealt round-robin to the 8 XCDs (each with its own L2), so
  // the channel tiles of one token tile are given workgroup ids that are equal
  // mod 8: they run on one XCD and read the token tile from HBM once.
  const int ct = (blockIdx.x / 8) % n_tiles_c;
  const int mt = (blockIdx.x / (8 * n_tiles_c)) * 8 + blockIdx.x % 8;
  if (mt * kTileRows >= M) return;  // padding workgroup of the last group of 8 token tiles
  const int n0 = ct * kTileRows;
  const int m0 = mt * kTileRows;
  const int cw0 = (wave & 1) * 128;  // the wave's channels within the tile
  const int tw0 = (wave >> 1) * 64;  // the wave's tokens within the tile

  // Buffer descriptors: weight rows n0.. (rows past N read as zero), token rows m0..
  // (rows past M read as zero).
  const uint32_t row_bytes = static_cast<uint32_t>(Dm) * 2;
  const int64_t xrange = static_cast<int64_t>(M - m0) * row_bytes;
  const __amdgpu_buffer_rsrc_t rw =
      make_rsrc(w + static_cast<int64_t>(n0) * Dm, static_cast<uint32_t>(min(N - n0, kTileRows)) * row_bytes);
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

  // Operand read offsets of 32-element slice sl for the wave's first 16-row
  // block: row = base + lane%16, logical chunk 4*sl + lane/16; block a adds 16*a
  // rows (the swizzle repeats every 16 rows).
  uint32_t rd_w[2], rd_x[2];
#pragma unroll
  for (int sl = 0; sl < 2; ++sl) {
    const int rw_row = cw0 + (lane & 15);
    const int rx_row = tw0 + (lane & 15);
    rd_w[sl] = rw_row * kRowBytes + (((4 * sl + (lane >> 4)) ^ swz(rw_row)) * 16);
    rd_x[sl] = kTileBytes + rx_row * kRowBytes + (((4 * sl + (lane >> 4)) ^ swz(rx_row)) * 16);
  }

  f32x4 acc[8][4];  // [channel block][token block], 16x16 each
#pragma unroll
  for (int a = 0; a < 8; ++a)
#pragma unroll
    for (int b = 0; b < 4; ++b) acc[a][b] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};

  const int nch = Dm / kKC;
  dma(0, 0);
  for (int c = 0; c < nch; ++c) {
    publish_tile();
    if (c + 1 < nch) dma(c + 1, (c + 1) & 1);
    const uint32_t base = lds_addr((lds_u8*)smem_raw) + opaque_s((c & 1) * kStageBytes);
#pragma unroll
    for (int sl = 0; sl < 2; ++sl) {
      bf16x8 fw[8], fx[4];
#pragma unroll
      for (int a = 0; a < 8; ++a) fw[a] = *lds_at<lds_bf16x8_t>(base + rd_w[sl] + 16 * a * kRowBytes);
#pragma unroll
      for (int b = 0; b < 4; ++b) fx[b] = *lds_at<lds_bf16x8_t>(base + rd_x[sl] + 16 * b * kRowBytes);
#pragma unroll
      for (int a = 0; a < 8; ++a)
#pragma unroll
        for (int b = 0; b < 4; ++b) acc[a][b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fw[a], fx[b], acc[a][b], 0, 0, 0);
    }
  }

  // Epilogue.  acc[a][b] element i of this lane is channel cw0 + 16a + 4*(lane/16) + i
  // of token tw0 + 16b + lane%16 (tile coordinates).  Stage the bf16 tile as
  // [token][channel] rows in LDS (every wave is done with the operand tiles first).
  __syncthreads();
  const uint32_t epi = lds_addr((lds_u8*)smem_raw);
#pragma unroll
  for (int b = 0; b < 4; ++b) {
    const int tr = tw0 + 16 * b + (lane & 15);
#pragma unroll
    for (int a = 0; a < 8; ++a) {
      const int cc = cw0 + 16 * a + 4 * (lane >> 4);
      const f32x4 v4 = acc[a][b];
      const float v0 = v4[0], v1 = v4[1], v2 = v4[2], v3 = v4[3];
      u32x2 val = {pack_bf16x2(v0, v1), pack_bf16x2(v2, v3)};
      *lds_at<__attribute__((address_space(3))) u32x2>(epi + tr * kEpiRow + cc * 2) = val;
    }
  }
  __syncthreads();
  // Each thread stores 16-byte pieces (8 channels of one token); consecutive
  // threads take consecutive pieces of a token row.  Eight consecutive channels
  // never cross a head.
  for (int j = threadIdx.x; j < kTileRows * (kTileRows / 8); j += kKThreads) {
    const int tr = j / (kTileRows / 8), pc = j % (kTileRows / 8);
    const int tok = m0 + tr, ch = n0 + 8 * pc;
    if (tok >= M || ch >= N) continue;
    const u32x4 val = *lds_at<__attribute__((address_space(3))) u32x4>(epi + tr * kEpiRow + pc * 16);
    const bool is_v = ch >= HD;
    const int r = is_v ? ch - HD : ch;
    const int hk = r / d, cc = r - hk * d;
    const int64_t th = static_cast<int64_t>(tok) * Hk + hk;
    if (SEQ) *reinterpret_cast<u32x4*>((is_v ? v_out : k_out) + th * d + cc) = val;
    if (DEPTH) *reinterpret_cast<u32x4*>((is_v ? v_depth : k_depth) + (th * S + slot) * d + cc) = val;
  }
}

template <bool SEQ, bool DEPTH>
hipError_t launch(const KvProjArgs& a) {
  const int M = a.B * a.T;
  const int n_tiles_c = (2 * a.Hk * a.d + kTileRows - 1) / kTileRows;
  const int64_t groups = ((M + kTileRows - 1) / kTileRows + 7) / 8;  // groups of 8 token tiles
  const int64_t blocks = groups * 8 * n_tiles_c;
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
  return ((M + kTileRows - 1) / kTileRows + 7) / 8 * 8 * ((2 * static_cast<int64_t>(Hk) * d + kTileRows - 1) / kTileRows);
}

hipError_t launch_kv_project(const KvProjArgs& a) {
  const bool seq = a.k_out != nullptr, depth = a.k_depth != nullptr;
  if (seq && depth) return launch<true, true>(a);
  if (seq) return launch<true, false>(a);
  return launch<false, true>(a);
}

}  // namespace moda
