// MoDA fused forward, bf16 inputs, fp32 accumulation, bf16 output (gfx950).
//
// One softmax per query row runs over the causally visible sequence keys of
// the row's KV head and over the L depth slots stored for the row's own token
// ("Mixture-of-Depths Attention" summary, papercache.org, 2.2 MoDA and 3.3
// Algorithm 1; MoDA reading notes, cc.laoqi.cc, 二.2 and 二.5).
//
// Work decomposition
//   * Group-aware rows: for one (batch b, KV head hk), expanded row
//     i_q = t*G + g is token t, query head hk*G + g.  Consecutive rows of one
//     token are its G heads, which share every K/V element they read.
//   * A workgroup of W waves owns BM = 32*W consecutive expanded rows (BM/G
//     tokens) of one (b, hk); each wave owns 32 rows (32/G tokens).  With
//     d = 128, W = 4 (two workgroups per CU) for sequences shorter than 32768
//     tokens, W = 8 (one per CU, each staged K/V tile serving 256 rows) from
//     there on; with d = 64, W = 4 at three or four workgroups per CU.  The
//     block's tokens are [t_start, t_end) with t_start = floor(row0/G) and
//     t_end = floor(last/G) + 1; sequence keys at or past t_end are never read.
//   * Every workgroup runs one pipeline of K/V tiles in LDS, double buffered.
//     Tiles are staged by direct-to-LDS buffer loads (16 bytes per lane, no
//     staging registers) issued as inline asm: the loads of tile i+1 are
//     issued right after the barrier that publishes tile i, and each wave
//     waits for its own loads before the next barrier.  Two kinds of tile:
//       - sequence tiles of 64 keys, shared by all W waves;
//       - depth tiles: 16 rows per wave, 16 consecutive slots of one of the
//         wave's own tokens, read from the packed [B][T][Hk][L][d] stream (each
//         (token, KV head) slab is one contiguous run, each depth element is
//         read from HBM exactly once and used by the G rows of its token
//         only), spread evenly among the sequence tiles.  With d = 128 and
//         G <= 16 a depth tile's scores are one 16x16x32 block per wave (the
//         16 slots against the 16-row half of the wave that holds the token),
//         permuted into the 32x32 layout of the sequence scores.
//     Both kinds fold into the same running (max, sum, output) state of each
//     row, so the softmax is one joint softmax over both candidate sets.
//   * Scores are computed transposed, S^T = K * Q^T, on 32x32x16 bf16 MFMA with
//     Q^T held in registers, so each lane owns one query row: the row max
//     needs one cross-lane exchange (lane ^ 32) and the rescale of the output
//     accumulator is per lane.  O^T += V^T * P^T takes the score registers,
//     packed to bf16, directly as the B operand; its A operand (V^T) is read
//     from the row-major V tile with the transposing ds_read_b64_tr_b16, whose
//     key order is chosen to match the score register layout.
//   * LDS tiles are unpadded; 16-byte chunks are XOR-swizzled per row (K:
//     chunk ^ row, V: chunk ^ 4*row, over the rows that share one LDS pass)
//     so that the MFMA operand reads are bank-conflict free.
//   * Softmax runs in base 2 with log2(e)/sqrt(d) folded into the exponent's
//     FMA; the output rescale is skipped unless a row max grows by more than
//     2^8.  lse is converted back to the natural log at the end.
//   * Causal workgroups are issued heaviest first (last row block first).
#include <type_traits>

#include "moda_launch.h"
#include "moda_tile.h"

namespace moda {
namespace {

constexpr int kRowsPerWave = 32;
// W waves per workgroup (4, or 8 for long sequences): W * 32 expanded rows.
template <int W>
constexpr int kBM = W * kRowsPerWave;
// With d = 128, sequences at least this long run 8-wave workgroups (one per
// CU), which stage each K/V tile once for 256 rows; shorter ones run two 4-wave
// workgroups per CU.  With d = 64 the kernel needs few enough registers for
// three waves per SIMD (four without the depth stage), so every length runs
// 4-wave workgroups, three (four) per CU.
constexpr int kLongT = 32768;
__host__ __device__ constexpr int waves_for(int T, int d) { return (d == 128 && T >= kLongT) ? 8 : 4; }
// Waves per SIMD the kernel is compiled for (its register budget).
template <int D, int W, bool DEPTH>
constexpr int kWavesPerEU = (D == 64 && W == 4) ? (DEPTH ? 3 : 4) : 2;
constexpr int kDepthRowsPerWave = 16;                     // slots of one token per wave in a depth tile

// Direct-to-LDS load instructions per wave per K (or V) tile.
template <int D, int W>
constexpr int kNX = Tile<D>::CH / W;  // sequence-tile loads per wave per matrix
template <int D>
constexpr int kNXD = kDepthRowsPerWave * Tile<D>::ROW_BYTES / 1024;  // depth-tile loads per wave per matrix
// LDS holds the two pipeline buffers as [K0 | K1 | V0 | V1], each region kHalf
// bytes (a depth tile has W * 16 rows, a sequence tile kBN rows): buffer P's K
// starts at P * kHalf and its V at (2 + P) * kHalf.  With the V-region offset
// folded into the per-lane V read offsets, every read address of either buffer
// is a per-lane register plus an instruction immediate below 64 KiB.
template <int D, int W>
constexpr int kHalf = (W * kDepthRowsPerWave > kBN ? W * kDepthRowsPerWave : kBN) * Tile<D>::ROW_BYTES;

// Per-workgroup staging geometry.  All global tile reads are raw buffer loads
// against four descriptors whose ranges end exactly at the last valid row, so
// rows past the end of the sequence read as zero; padding depth slots (slot
// >= L) get an offset beyond every range and read as zero too.
//   seq K/V : base &x[b][0][hk][0], key j at byte j * Hk*d*2.
//   depth   : base &x[b][t_b][hk][0][0] with t_b the workgroup's first token;
//             token t_b + u, slot i at byte (u*Hk*L + i) * d*2.
struct Geo {
  u32x4 kd, vd;  // raw buffer descriptors (see raw_rsrc)
  int L;
  uint32_t key_bytes;   // Hk*d*2: stride between consecutive keys of one KV head
  uint32_t tok_bytes;   // Hk*Lcap*d*2: stride between consecutive tokens' depth slabs
  int tok_wave;         // tokens per wave (32 / G)
};

// Direct-to-LDS loads of depth tile `idx` into `buf` (K at buf, V at
// buf + 2 * kHalf).  For every wave w the tile holds token w*tok_wave + dtok of
// the workgroup, slots [16*dch, 16*dch + 16), at tile rows [16w, 16w + 16).
// Instruction x of wave w fills tile rows pr = (w*NXD + x)*RPI + lane/CH,
// physical chunk pc = lane % CH, with logical chunk pc ^ swz(pr).  Padding
// slots (>= L) get an offset past the descriptor range and read as zero.
template <int D, int W>
__device__ __forceinline__ void dma_depth(const Geo& g, int idx, int nchunk, lds_u8* buf, int wave, int lane) {
  using TL = Tile<D>;
  lane = opaque(lane);  // per-lane offsets below are recomputed per tile, not held across the loop
  const int dtok = idx / nchunk;
  const int dch = idx - dtok * nchunk;
#pragma unroll
  for (int x = 0; x < kNXD<D>; ++x) {
    const int pr = (wave * kNXD<D> + x) * TL::RPI + lane / TL::CH;
    const int pc = lane % TL::CH;
    const int slot = dch * kDepthRowsPerWave + (pr % kDepthRowsPerWave);
    const uint32_t row_off = static_cast<uint32_t>(wave * g.tok_wave + dtok) * g.tok_bytes +
                             static_cast<uint32_t>(slot) * TL::ROW_BYTES;
    const bool valid = slot < g.L;
    const uint32_t ok = valid ? row_off + ((pc ^ TL::swz_k(pr)) * 16) : kOutOfRange;  // selects, not branches
    const uint32_t ov = valid ? row_off + ((pc ^ TL::swz_v(pr)) * 16) : kOutOfRange;
    const uint32_t dk = lds_addr(buf + (wave * kNXD<D> + x) * 1024);
    dma16(g.kd, dk, ok);
    dma16(g.vd, dk + 2 * kHalf<D, W>, ov);
  }
}

// Per-lane LDS and DMA offsets, computed once.  In the tile loop every LDS
// read address is (buffer base + one of these) plus a compile-time immediate
// (the 32-key block, 16-key group or second half of a transposed read), so a
// tile costs one add per distinct register instead of a full address
// computation per read, and the sequence-tile loads need no address work.
template <int D, int W>
struct LaneOffs {
  uint32_t kr[D / 16];                        // K read of slice sl, tile rows 0..31 (rows 32..63: + 32 rows)
  uint32_t vr[D / 32];                        // V transposed read of d tile dt, keys 0..15 (others: + rows)
  uint32_t dk[kNX<D, W>], dv[kNX<D, W>];  // sequence-tile loads, relative to the tile's first key
};

template <int D, int W>
__device__ __forceinline__ void init_offsets(LaneOffs<D, W>& lo, int lane, int wave, uint32_t key_bytes) {
  using TL = Tile<D>;
  const int r = lane & 31, half = lane >> 5;
#pragma unroll
  for (int sl = 0; sl < D / 16; ++sl) lo.kr[sl] = r * TL::ROW_BYTES + (((2 * sl + half) ^ TL::swz_k(r)) * 16);
  const int i = lane & 15, q = (lane >> 4) & 1, hf = lane >> 5;
  const int row0 = 4 * hf + (i >> 2);  // the second read is 8 rows further (same swizzle)
  const int sw = TL::swz_v(row0);
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt) {
    const int lc = (32 * dt + 16 * q) / 8 + ((i & 3) >> 1);  // logical chunk of column d0 + 4*(i%4)
    lo.vr[dt] = 2 * kHalf<D, W> + row0 * TL::ROW_BYTES + 8 * (i & 1) + ((lc ^ sw) * 16);
  }
  // Load instruction x of wave w fills tile rows pr = (w*NX + x)*RPI + lane/CH,
  // physical chunk pc = lane % CH, with logical chunk pc ^ swz(pr).
#pragma unroll
  for (int x = 0; x < kNX<D, W>; ++x) {
    const int pr = (wave * kNX<D, W> + x) * TL::RPI + lane / TL::CH;
    const int pc = lane % TL::CH;
    lo.dk[x] = static_cast<uint32_t>(pr) * key_bytes + ((pc ^ TL::swz_k(pr)) * 16);
    lo.dv[x] = static_cast<uint32_t>(pr) * key_bytes + ((pc ^ TL::swz_v(pr)) * 16);
  }
}

// Direct-to-LDS loads of sequence tile `idx` into `buf` (K at buf, V at
// buf + 2 * kHalf), through descriptors rebased to the tile's first key (scalar
// work), so the per-lane offsets are loop invariant.  Keys past the sequence
// end fall outside the range and read as zero.
template <int D, int W>
__device__ __forceinline__ void dma_seq(const uint16_t* kb, const uint16_t* vb, uint32_t seq_range,
                                        uint32_t key_bytes, int Hk, int idx, lds_u8* buf, int wave,
                                        const LaneOffs<D, W>& lo) {
  using TL = Tile<D>;
  const int64_t first = static_cast<int64_t>(idx) * kBN * Hk * D;  // elements
  const uint32_t range = seq_range - static_cast<uint32_t>(idx * kBN) * key_bytes;
  const u32x4 rk = raw_rsrc(kb + first, range);
  const u32x4 rv = raw_rsrc(vb + first, range);
#pragma unroll
  for (int x = 0; x < kNX<D, W>; ++x) {
    const uint32_t dk = lds_addr(buf + (wave * kNX<D, W> + x) * 1024);
    dma16(rk, dk, lo.dk[x]);
    dma16(rv, dk + 2 * kHalf<D, W>, lo.dv[x]);
  }
}

// Absolute LDS addresses of this tile's K and V reads: one add per register.
template <int D>
struct TileAddr {
  uint32_t k[D / 16];
  uint32_t v[D / 32];
};

template <int D, int W>
__device__ __forceinline__ TileAddr<D> tile_addr(const lds_u8* buf, const LaneOffs<D, W>& lo) {
  TileAddr<D> a;
  const uint32_t base = lds_addr(buf);
#pragma unroll
  for (int sl = 0; sl < D / 16; ++sl) a.k[sl] = base + lo.kr[sl];
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt) a.v[dt] = base + lo.vr[dt];
  return a;
}

// One 64-key sequence tile: both 32-key blocks of S^T, then one online update
// of the state for all 64 keys (one row max, one rescale test), then O^T +=
// V^T P^T over the tile's four 16-key groups.  MASK applies the causal /
// sequence-end mask (branch-free selects); interior tiles take MASK = false.
template <int D, bool MASK, bool CAUSAL>
__device__ __forceinline__ void seq_tile(RowState<D>& st, const bf16x8 (&qf)[D / 16], const TileAddr<D>& ta,
                                         int kt0, int T, int my_t, int half, float scale) {
  using TL = Tile<D>;
  f32x16 sq[2];
  sq[0] = qk_block<D>(qf, ta.k, 0);
  sq[1] = qk_block<D>(qf, ta.k, 32 * TL::ROW_BYTES);
  // One online update for the whole 64-key tile: one row max, one rescale test.
  float s[32];
#pragma unroll
  for (int j = 0; j < 2; ++j)
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      s[16 * j + i] = sq[j][i];
      if (MASK) {
        const int key = kt0 + 32 * j + 8 * (i >> 2) + 4 * half + (i & 3);
        const bool vis = key < T && (!CAUSAL || key <= my_t);
        s[16 * j + i] = vis ? s[16 * j + i] : -INFINITY;
      }
    }
  bf16x8 pb[4];
  online_update<D, 32>(st, s, pb, scale);
#pragma unroll
  for (int g = 0; g < 4; ++g) pv_group<D>(st, pb[g], ta.v, 16 * g * TL::ROW_BYTES);
}

template <int D, bool DEPTH, bool CAUSAL, int W>
__global__ __launch_bounds__(W * 64) __attribute__((amdgpu_waves_per_eu(kWavesPerEU<D, W, DEPTH>, kWavesPerEU<D, W, DEPTH>))) void moda_fwd_bf16_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
    const uint16_t* __restrict__ kd, const uint16_t* __restrict__ vd, int B, int T, int Hq, int Hk, int L,
    int Lcap, int lgG, int nrb, float scale_log2, uint16_t* __restrict__ out, float* __restrict__ lse) {
  using TL = Tile<D>;
  constexpr int kBMW = kBM<W>;
  constexpr int HALF = kHalf<D, W>;
  __shared__ __attribute__((aligned(1024))) uint8_t smem_raw[4 * HALF];
  lds_u8* const smem = (lds_u8*)smem_raw;

  const int G = 1 << lgG;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform: keeps per-wave control scalar
  const int r = lane & 31, half = lane >> 5;
  const int nbh = B * Hk;
  const int bid = blockIdx.x;
  const int rb = CAUSAL ? (nrb - 1 - bid / nbh) : (bid / nbh);
  const int bh = bid % nbh;
  const int b = bh / Hk, hk = bh % Hk;
  const int row0 = rb * kBMW;
  const int TG = T << lgG;
  const int tb = row0 >> lgG;  // the workgroup's first token

  Geo g;
  g.L = DEPTH ? L : 0;
  g.tok_wave = (kRowsPerWave >> lgG) > 0 ? (kRowsPerWave >> lgG) : 1;
  g.key_bytes = static_cast<uint32_t>(Hk) * D * 2;
  g.tok_bytes = static_cast<uint32_t>(Hk) * (DEPTH ? Lcap : 0) * D * 2;
  const uint16_t* kb = k + (static_cast<int64_t>(b) * T * Hk + hk) * D;
  const uint16_t* vb = v + (static_cast<int64_t>(b) * T * Hk + hk) * D;
  const uint32_t seq_range = (static_cast<uint32_t>(T - 1) * Hk + 1) * D * 2;
  if (DEPTH) {
    const int64_t slab0 = ((static_cast<int64_t>(b) * T + tb) * Hk + hk) * static_cast<int64_t>(Lcap) * D;
    const int64_t range = ((static_cast<int64_t>(T - 1 - tb) * Hk + 1) * Lcap) * D * 2;
    const uint32_t dr = static_cast<uint32_t>(range < 0x7fffffff ? range : 0x7fffffff);
    g.kd = raw_rsrc(kd + slab0, dr);
    g.vd = raw_rsrc(vd + slab0, dr);
  }
  LaneOffs<D, W> lo;
  init_offsets<D, W>(lo, lane, wave, g.key_bytes);

  const int wrow0 = row0 + wave * kRowsPerWave;
  const int my_row = wrow0 + r;
  const bool row_ok = my_row < TG;
  const int my_t = my_row >> lgG;
  const int my_g = my_row & (G - 1);
  const int wt0 = wrow0 >> lgG;                                    // wave's first token
  const int wt1 = (min(wrow0 + kRowsPerWave, TG) - 1) >> lgG;      // wave's last valid token
  const int blk_last = (min(row0 + kBMW, TG) - 1) >> lgG;           // block's last valid token
  const int kv_end = CAUSAL ? blk_last + 1 : T;
  const int ns = (kv_end + kBN - 1) / kBN;                         // sequence tiles
  const int nchunk = DEPTH ? (L + kDepthRowsPerWave - 1) / kDepthRowsPerWave : 1;  // 16-slot chunks per token
  const int nd = DEPTH ? g.tok_wave * nchunk : 0;                                  // depth tiles

  // Q^T fragments (B operand): lane holds row my_row, d = 16*sl + 8*half + [0, 8).
  bf16x8 qf[D / 16];
  {
    const uint16_t* qrow = q + ((static_cast<int64_t>(b) * T + my_t) * Hq + hk * G + my_g) * D;
#pragma unroll
    for (int sl = 0; sl < D / 16; ++sl) {
      u32x4 val = {0u, 0u, 0u, 0u};
      if (row_ok) val = *reinterpret_cast<const u32x4*>(qrow + sl * 16 + half * 8);
      qf[sl] = __builtin_bit_cast(bf16x8, val);
    }
  }

  RowState<D> st;
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt) st.o[dt] = f32x16{};
  st.m = -INFINITY;
  st.l = 0.0f;

  // In depth tile d this wave's 16 rows (token wt0 + d / nchunk, slots from
  // 16 * (d % nchunk)) sit at tile rows [16*wave, 16*wave + 16): 32-key block
  // wave/2, score registers [8*(wave%2), 8*(wave%2) + 8).
  const int dj = wave >> 1, dh = wave & 1;

  // With d = 128 and G <= 16 a depth tile's scores are one 16x16 block per
  // wave (v_mfma_f32_16x16x32_bf16): the wave's 16 slots against the 16-row
  // half of its rows that holds the token (G <= 16 rows, a power of two, so
  // they never straddle the halves).  The B operand is Q^T of that half in
  // the 16x16 layout -- lane l: row 16*qh + l%16, d = 32c + 8*(l/16) + [0, 8)
  // -- read from global memory (the rows are L2-resident since the prologue)
  // whenever the half changes, one depth tile ahead.  The 32x32 block of the
  // sequence path would spend 32 keys x 32 rows on the same 16 slots x G rows.
  constexpr bool kDepth16 = DEPTH && D == 128;
  const bool depth16 = kDepth16 && lgG <= 4;
  bf16x8 q16[D / 32];
  auto half_of = [&](int d) { return ((d / nchunk) << lgG) >> 4; };
  auto load_q16 = [&](int qh) __attribute__((always_inline)) {
    const int row = wrow0 + 16 * qh + (lane & 15);
    const bool ok = row < TG;
    const uint16_t* qr = q + ((static_cast<int64_t>(b) * T + (row >> lgG)) * Hq + hk * G + (row & (G - 1))) * D +
                         8 * (lane >> 4);
#pragma unroll
    for (int c = 0; c < D / 32; ++c) {
      u32x4 val = {0u, 0u, 0u, 0u};
      if (ok) val = *reinterpret_cast<const u32x4*>(qr + 32 * c);
      q16[c] = __builtin_bit_cast(bf16x8, val);
    }
  };
  if (depth16 && nd > 0) load_q16(0);

  // The LDS buffer of pipeline position pos is smem + (pos & 1) * 2 * BYTES.
  // Sequence tiles run in pairs with a constant buffer each (seq_run); the
  // depth tiles, one per run, take the buffer at run time, with its base
  // hidden from the optimiser so that their address adds stay in place
  // instead of becoming hoisted copies of every offset.
  auto buf_of = [&](int pos) -> lds_u8* {
    return smem + opaque_s((pos & 1) * HALF);
  };

  // ---- tile pipeline ------------------------------------------------------------
  // Sequence tiles wholly before the workgroup's first token (and the sequence
  // end) are unmasked for every wave; the few after them overlap the
  // workgroup's own tokens and take the masked path.  The nd depth tiles are
  // spread evenly among the unmasked ones -- depth tile d follows sequence
  // tile s_end(d) - 1, about (d+1)*n_int/nd - 1 -- so each depth load (a
  // once-read HBM stream) is prefetched under a full sequence tile of MFMA
  // work.  Every loop body is
  // straight-line per wave, so the accumulator keeps its registers.
  const int n_int = CAUSAL ? min(ns, (tb + 1) / kBN) : T / kBN;
  int pos = 0;  // pipeline position: selects the LDS buffer
  int sq = 0;   // next sequence tile
  // One sequence tile in LDS buffer P (= pos % 2, a constant here, so the
  // tile's read addresses are the per-lane offsets plus instruction
  // immediates); the next tile -- sequence tile sq + 1 of the run ending at
  // s_end, else depth tile d if d < nd -- is loaded into buffer 1 - P.
  auto seq_step = [&](auto parity, auto maskc, int s_end, int d) __attribute__((always_inline)) {
    constexpr int P = decltype(parity)::value;
    constexpr bool MASK = decltype(maskc)::value != 0;
    lds_u8* const nxt = smem + opaque_s((1 - P) * HALF);
    publish_tile();
    if (sq + 1 < s_end || (d >= nd && sq + 1 < ns))
      dma_seq<D, W>(kb, vb, seq_range, g.key_bytes, Hk, sq + 1, nxt, wave, lo);
    else if (DEPTH && d < nd)
      dma_depth<D, W>(g, d, nchunk, nxt, wave, lane);
    const int kt0 = sq * kBN;
    ++sq;
    ++pos;
    if (MASK && CAUSAL && kt0 > wt1) return;  // nothing visible to this wave
    seq_tile<D, MASK, CAUSAL>(st, qf, tile_addr<D, W>(smem + P * HALF, lo), kt0, T, my_t, half,
                              scale_log2);
  };
  // Sequence tiles sq .. s_end - 1 in pairs (buffer 0, then buffer 1), after
  // at most one tile that brings pos to an even value.
  auto seq_run = [&](auto maskc, int s_end, int d) __attribute__((always_inline)) {
    using P0 = std::integral_constant<int, 0>;
    using P1 = std::integral_constant<int, 1>;
    if (sq < s_end && (pos & 1)) seq_step(P1(), maskc, s_end, d);
    while (sq + 1 < s_end) {
      seq_step(P0(), maskc, s_end, d);
      seq_step(P1(), maskc, s_end, d);
    }
    if (sq < s_end) seq_step(P0(), maskc, s_end, d);
  };
  // Depth tile d follows sequence tile s_end(d) - 1.  Each workgroup shifts its
  // schedule earlier by its own fraction (one of 64, from a hash of the
  // workgroup id) of the depth-tile spacing: workgroups that run at the same
  // time have nearly equal n_int and nd and would otherwise issue their depth
  // loads, each a burst of HBM reads, in the same steps.
  const int d_off = (static_cast<int>((static_cast<uint32_t>(bid) * 2654435761u) >> 26) * n_int) >> 6;
  auto s_end_of = [&](int d) { return ((d + 1) * n_int - d_off) / max(nd, 1); };
  if (DEPTH && nd > 0 && s_end_of(0) == 0)
    dma_depth<D, W>(g, 0, nchunk, smem, wave, lane);
  else
    dma_seq<D, W>(kb, vb, seq_range, g.key_bytes, Hk, 0, smem, wave, lo);

  if constexpr (DEPTH) {
    for (int d = 0; d < nd; ++d) {
      const int s_end = s_end_of(d);
      seq_run(std::integral_constant<int, 0>(), s_end, d);
      // depth tile d: each wave sees only its own token's slots
      lds_u8* cur = buf_of(pos);
      lds_u8* nxt = buf_of(pos + 1);
      publish_tile();
      if (d + 1 < nd) {
        if (sq < s_end_of(d + 1))
          dma_seq<D, W>(kb, vb, seq_range, g.key_bytes, Hk, sq, nxt, wave, lo);
        else
          dma_depth<D, W>(g, d + 1, nchunk, nxt, wave, lane);
      } else if (sq < ns) {
        dma_seq<D, W>(kb, vb, seq_range, g.key_bytes, Hk, sq, nxt, wave, lo);
      }
      ++pos;
      const TileAddr<D> ta = tile_addr<D, W>(cur, lo);
      const int dtok = d / nchunk;
      const int slot0 = (d - dtok * nchunk) * kDepthRowsPerWave;
      const bool mine = my_t == wt0 + dtok;
      const int hf = opaque(half);
      // s[i]: slot slot0 + 8*(i/4) + 4*hf + i%4 of this lane's row (the
      // weights' order in the PV operand).
      float s[8];
      if (kDepth16 && depth16) {
        // S^T (16 slots x 16 rows): A = the wave's 16 depth rows, row l%16,
        // logical chunk 4c + l/16; lane l gets slots 4*(l/16) + [0, 4) of row
        // 16*qh + l%16.
        const int kr = 16 * wave + (lane & 15);
        const uint32_t kbase = lds_addr(cur) + kr * TL::ROW_BYTES;
        f32x4 s4 = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int c = 0; c < D / 32; ++c) {
          const bf16x8 a = *lds_at<lds_bf16x8_t>(kbase + (((4 * c + (lane >> 4)) ^ TL::swz_k(kr)) * 16));
          s4 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, q16[c], s4, 0, 0, 0);
        }
        if (d + 1 < nd && half_of(d + 1) != half_of(d)) load_q16(half_of(d + 1));
        // To the 32x32 layout: lane L (row L%32, hf = L/32) needs slots 4hf + [0, 4)
        // and 8 + 4hf + [0, 4) of its row, held by lanes 16hf + L%16 and
        // 32 + 16hf + L%16.  Swapping 16-lane rows (odd of the first operand with
        // even of the second), then 32-lane halves, leaves exactly those in the
        // two operands (rows of the other half are masked below).
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          // (Elements go through scalars: __builtin_bit_cast of a vector
          // element reads element 0.)
          const float si = s4[i];
          const uint32_t x = __builtin_bit_cast(uint32_t, si);
          const auto r16 = __builtin_amdgcn_permlane16_swap(x, static_cast<uint32_t>(opaque(static_cast<int>(x))),
                                                            false, false);
          const auto r32 = __builtin_amdgcn_permlane32_swap(r16[0], r16[1], false, false);
          const uint32_t lo32 = r32[0], hi32 = r32[1];
          s[i] = __builtin_bit_cast(float, lo32);
          s[4 + i] = __builtin_bit_cast(float, hi32);
        }
      } else {
        const f32x16 sacc = qk_block<D>(qf, ta.k, 32 * dj * TL::ROW_BYTES);
#pragma unroll
        for (int i = 0; i < 8; ++i) s[i] = sacc[8 * dh + i];
      }
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int slot = slot0 + 8 * (i >> 2) + 4 * hf + (i & 3);
        s[i] = (mine && slot < L) ? s[i] : -INFINITY;
      }
      bf16x8 pb[1];
      online_update<D, 8>(st, s, pb, scale_log2);
      pv_group<D>(st, pb[0], ta.v, (32 * dj + 16 * dh) * TL::ROW_BYTES);
    }
  }
  seq_run(std::integral_constant<int, 0>(), n_int, nd);  // unmasked sequence tiles (all of them without depth)
  seq_run(std::integral_constant<int, 1>(), ns, nd);     // masked sequence tiles

  // ---- epilogue --------------------------------------------------------------
  const float l_tot = pair_sum(st.l);
  if (row_ok) {
    const float inv = 1.0f / l_tot;
    const int h = hk * G + my_g;
    uint16_t* orow = out + ((static_cast<int64_t>(b) * T + my_t) * Hq + h) * D;
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
      for (int a = 0; a < 4; ++a) {
        const int d0 = dt * 32 + a * 8 + half * 4;
        u32x2 w = {pack_bf16x2(st.o[dt][4 * a] * inv, st.o[dt][4 * a + 1] * inv),
                   pack_bf16x2(st.o[dt][4 * a + 2] * inv, st.o[dt][4 * a + 3] * inv)};
        *reinterpret_cast<u32x2*>(orow + d0) = w;
      }
    if (half == 0) lse[(static_cast<int64_t>(b) * Hq + h) * T + my_t] = (st.m + __log2f(l_tot)) * kLn2;
  }
}

template <int D, bool DEPTH, bool CAUSAL, int W>
hipError_t launch(const FwdArgs& a) {
  const int lgG = __builtin_ctz(a.Hq / a.Hk);
  const int TG = a.T * (a.Hq / a.Hk);
  const int nrb = (TG + kBM<W> - 1) / kBM<W>;
  const int64_t nblocks = static_cast<int64_t>(nrb) * a.B * a.Hk;
  const float scale_log2 = kLog2e / sqrtf(static_cast<float>(D));
  hipLaunchKernelGGL((moda_fwd_bf16_kernel<D, DEPTH, CAUSAL, W>), dim3(static_cast<unsigned>(nblocks)),
                     dim3(W * 64), 0, static_cast<hipStream_t>(a.stream),
                     static_cast<const uint16_t*>(a.q), static_cast<const uint16_t*>(a.k),
                     static_cast<const uint16_t*>(a.v), static_cast<const uint16_t*>(a.kd),
                     static_cast<const uint16_t*>(a.vd), a.B, a.T, a.Hq, a.Hk, a.L, a.Lcap, lgG, nrb, scale_log2,
                     static_cast<uint16_t*>(a.out), a.lse);
  return hipGetLastError();
}

template <int D, int W>
hipError_t launch_dw(const FwdArgs& a) {
  if (a.L > 0) return a.causal ? launch<D, true, true, W>(a) : launch<D, true, false, W>(a);
  return a.causal ? launch<D, false, true, W>(a) : launch<D, false, false, W>(a);
}

template <int D>
hipError_t launch_d(const FwdArgs& a) {
  if constexpr (D == 128) {
    if (waves_for(a.T, D) == 8) return launch_dw<D, 8>(a);
  }
  return launch_dw<D, 4>(a);
}

}  // namespace

int fwd_bf16_rows_per_block(int T, int d) { return waves_for(T, d) * kRowsPerWave; }

int64_t fwd_bf16_grid_blocks(int B, int T, int Hq, int Hk, int d) {
  const int64_t TG = static_cast<int64_t>(T) * (Hq / Hk);
  const int bm = fwd_bf16_rows_per_block(T, d);
  return (TG + bm - 1) / bm * B * Hk;
}

hipError_t launch_fwd_bf16(const FwdArgs& a) { return a.d == 64 ? launch_d<64>(a) : launch_d<128>(a); }

}  // namespace moda
