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
//   * A workgroup owns BM = 128 consecutive expanded rows (128/G tokens) of one
//     (b, hk); each of its 4 waves owns 32 rows (32/G tokens).  The block's
//     tokens are [t_start, t_end) with t_start = floor(row0/G) and
//     t_end = floor(last/G) + 1; sequence keys at or past t_end are never read.
//   * Every workgroup runs one pipeline of 64-row tiles staged in LDS, double
//     buffered: while the waves compute on tile i, the global loads of tile
//     i+1 are in flight in registers; one barrier per tile.  Two kinds:
//       - sequence tiles of 64 keys, shared by all 4 waves;
//       - depth tiles: 16 rows per wave, 16 consecutive slots of one of the
//         wave's own tokens, read from the packed [B][T][Hk][L][d] stream
//         (each (token, KV head) slab is one contiguous run, each depth
//         element is read from HBM exactly once and used by the G rows of its
//         token only), spread evenly among the sequence tiles.
//     Both kinds fold into the same running (max, sum, output) state of each
//     row, so the softmax is one joint softmax over both candidate sets.
//   * Scores are computed transposed, S^T = K * Q^T, on 32x32x16 bf16 MFMA with
//     Q^T held in registers, so each lane owns one query row: the row max
//     needs one cross-lane exchange (lane ^ 32) and the rescale of the output
//     accumulator is per lane.  O^T += V^T * P^T takes the score registers,
//     packed to bf16, directly as the B operand; V is written to LDS
//     transposed (d-major) with the key order permuted to match the score
//     register layout, so every MFMA operand is one 16-byte LDS read.
//   * Softmax runs in base 2 with log2(e)/sqrt(d) folded into the exponent's
//     FMA; the output rescale is skipped when no row max of the wave moved.
//     lse is converted back to the natural log at the end.
//   * Causal workgroups are issued heaviest first (last row block first).
#include "moda_device.h"
#include "moda_launch.h"

namespace moda {
namespace {

constexpr int kWaves = 4;
constexpr int kThreads = kWaves * 64;
constexpr int kRowsPerWave = 32;
constexpr int kBM = kWaves * kRowsPerWave;  // expanded rows per workgroup
constexpr int kBN = 64;                     // rows (keys or depth slots) per tile
constexpr int kDepthRowsPerWave = kBN / kWaves;

template <int D>
struct Smem {
  static constexpr int KS = D + 8;    // K row stride (elements): +16 B breaks bank aliasing
  static constexpr int VS = kBN + 8;  // V^T row stride
  static constexpr int kK = kBN * KS;
  static constexpr int kV = D * VS;
  static constexpr int kBuf = kK + kV;
  static constexpr int kElems = 2 * kBuf;
};

// Position of tile key `kk` inside a d-row of the transposed V tile.  Within
// each 16-key group, key 8a + 4b + c is stored at 8b + 4a + c: the 8 keys that
// lane half b holds in its score registers for one PV product become 8
// consecutive elements (one 16-byte read).
__device__ __forceinline__ int vpos(int kk) {
  const int a = (kk >> 3) & 1, bb = (kk >> 2) & 1;
  return (kk & ~15) | (bb << 3) | (a << 2) | (kk & 3);
}

// Per-workgroup staging geometry.  All global tile reads are raw buffer loads
// against four descriptors whose ranges end exactly at the last valid row, so
// rows past the end of the sequence read as zero; padding depth slots (slot
// >= L) get an offset beyond every range and read as zero too.
//   seq K/V : base &x[b][0][hk][0], key j at byte j * Hk*d*2.
//   depth   : base &x[b][t_b][hk][0][0] with t_b the workgroup's first token;
//             token t_b + u, slot i at byte (u*Hk*L + i) * d*2.
struct Geo {
  __amdgpu_buffer_rsrc_t k, v, kd, vd;
  int L;
  uint32_t key_bytes;   // Hk*d*2: stride between consecutive keys of one KV head
  uint32_t tok_bytes;   // Hk*L*d*2: stride between consecutive tokens' depth slabs
  int tok_wave;         // tokens per wave (32 / G)
};

constexpr uint32_t kOutOfRange = 0x80000000u;  // > every descriptor range (host-checked)
constexpr int kBufFlags = 0x00020000;         // raw buffer, 32-bit dwords

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const uint16_t* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(base), static_cast<short>(0),
                                           static_cast<int>(bytes), kBufFlags);
}

// Byte offset of 16-byte column chunk `ch` of tile row r.  A depth tile holds,
// for every wave w, token w*tok_wave + dtok of the workgroup and slots
// [16*dch, 16*dch + 16) at tile rows [16w, 16w + 16); a sequence tile holds
// 64 keys starting at kt0.
template <int D>
__device__ __forceinline__ uint32_t tile_row_bytes(const Geo& g, bool depth, int kt0, int dtok, int dch, int r,
                                                   int ch) {
  if (!depth) return static_cast<uint32_t>(kt0 + r) * g.key_bytes + ch * 16;
  const int w = r / kDepthRowsPerWave;
  const int slot = dch * kDepthRowsPerWave + (r % kDepthRowsPerWave);
  const uint32_t off = static_cast<uint32_t>(w * g.tok_wave + dtok) * g.tok_bytes +
                       static_cast<uint32_t>(slot) * (D * 2) + ch * 16;
  return slot < g.L ? off : kOutOfRange;  // a select, not a branch
}

// Register staging of one tile: each thread holds up to KCH 16-byte K chunks
// and one (4-row, 8-column) V block per VIT item.
template <int D>
struct Stage {
  static constexpr int CH = D / 8;                                  // 16-byte chunks per row
  static constexpr int KCH = (kBN * CH + kThreads - 1) / kThreads;  // K chunks per thread
  static constexpr int VIT = ((kBN / 4) * CH + kThreads - 1) / kThreads;
  u32x4 kc[KCH];
  u32x4 vr[VIT][4];
};

// Issue the global loads of depth tile `idx` (DEPTH_TILE) or sequence tile
// `idx` into the thread's staging registers.
template <int D, bool DEPTH_TILE>
__device__ __forceinline__ void load_tile(Stage<D>& s, const Geo& g, int idx, int nchunk, int tid) {
  constexpr int CH = Stage<D>::CH;
  constexpr bool depth = DEPTH_TILE;
  const int dtok = depth ? idx / nchunk : 0;
  const int dch = depth ? idx - dtok * nchunk : 0;
  const int kt0 = depth ? 0 : idx * kBN;
  const __amdgpu_buffer_rsrc_t rk = depth ? g.kd : g.k;
  const __amdgpu_buffer_rsrc_t rv = depth ? g.vd : g.v;
  constexpr bool k_full = Stage<D>::KCH * kThreads == kBN * CH;          // every thread has every K chunk
  constexpr bool v_full = Stage<D>::VIT * kThreads == (kBN / 4) * CH;    // every thread has every V item
#pragma unroll
  for (int x = 0; x < Stage<D>::KCH; ++x) {
    const int c = tid + x * kThreads;
    uint32_t off = tile_row_bytes<D>(g, depth, kt0, dtok, dch, c / CH, c % CH);
    if (!k_full) off = c < kBN * CH ? off : kOutOfRange;
    s.kc[x] = __builtin_amdgcn_raw_buffer_load_b128(rk, off, 0, 0);
  }
#pragma unroll
  for (int x = 0; x < Stage<D>::VIT; ++x) {
    const int item = tid + x * kThreads;
    const int quad = item % (kBN / 4), oc = item / (kBN / 4);
#pragma unroll
    for (int y = 0; y < 4; ++y) {
      uint32_t off = tile_row_bytes<D>(g, depth, kt0, dtok, dch, quad * 4 + y, oc);
      if (!v_full) off = item < (kBN / 4) * CH ? off : kOutOfRange;
      s.vr[x][y] = __builtin_amdgcn_raw_buffer_load_b128(rv, off, 0, 0);
    }
  }
}

template <int D>
__device__ __forceinline__ void store_tile(const Stage<D>& s, uint16_t* ks, uint16_t* vt, int tid) {
  constexpr int CH = Stage<D>::CH;
  constexpr int KS = Smem<D>::KS, VS = Smem<D>::VS;
  constexpr bool k_full = Stage<D>::KCH * kThreads == kBN * CH;
  constexpr bool v_full = Stage<D>::VIT * kThreads == (kBN / 4) * CH;
#pragma unroll
  for (int x = 0; x < Stage<D>::KCH; ++x) {
    const int c = tid + x * kThreads;
    if (k_full || c < kBN * CH) *reinterpret_cast<u32x4*>(ks + (c / CH) * KS + (c % CH) * 8) = s.kc[x];
  }
#pragma unroll
  for (int x = 0; x < Stage<D>::VIT; ++x) {
    const int item = tid + x * kThreads;
    if (!v_full && item >= (kBN / 4) * CH) continue;
    const int quad = item % (kBN / 4), oc = item / (kBN / 4);
    const int pos = vpos(quad * 4);
    const u32x4* r = s.vr[x];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int w = e >> 1;
      uint32_t lo, hi;
      if (e & 1) {
        lo = (r[0][w] >> 16) | (r[1][w] & 0xffff0000u);
        hi = (r[2][w] >> 16) | (r[3][w] & 0xffff0000u);
      } else {
        lo = (r[0][w] & 0xffffu) | (r[1][w] << 16);
        hi = (r[2][w] & 0xffffu) | (r[3][w] << 16);
      }
      *reinterpret_cast<u32x2*>(vt + (oc * 8 + e) * VS + pos) = u32x2{lo, hi};
    }
  }
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

// Fold N raw scores (-inf = masked) into the state and return the weights,
// packed to bf16 in groups of 8 (one PV B operand per group).
template <int D, int N>
__device__ __forceinline__ void online_update(RowState<D>& st, float (&s)[N], bf16x8 (&pb)[N / 8], float scale) {
  float mx = s[0];
#pragma unroll
  for (int i = 1; i < N; ++i) mx = fmaxf(mx, s[i]);
  mx = pair_max(mx);
  const float m_blk = mx * scale;  // -inf stays -inf (scale > 0)
  if (__any(m_blk > st.m + kRescaleSlack)) {
    const float m_new = fmaxf(st.m, m_blk);
    const float alpha = fast_exp2(st.m - (m_new == -INFINITY ? 0.0f : m_new));
    st.l *= alpha;
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
      for (int i = 0; i < 16; ++i) st.o[dt][i] *= alpha;
    st.m = m_new;
  }
  const float base = (st.m == -INFINITY) ? 0.0f : st.m;
  float sum = 0.0f;
#pragma unroll
  for (int i = 0; i < N; ++i) {
    s[i] = fast_exp2(fmaf(s[i], scale, -base));
    sum += s[i];
  }
  st.l += sum;
#pragma unroll
  for (int h = 0; h < N / 8; ++h) {
    u32x4 w;
#pragma unroll
    for (int k = 0; k < 4; ++k) w[k] = pack_bf16x2(s[8 * h + 2 * k], s[8 * h + 2 * k + 1]);
    pb[h] = __builtin_bit_cast(bf16x8, w);
  }
}

// S^T block: 32 keys (rows of ks starting at key0) x the wave's 32 query rows.
template <int D>
__device__ __forceinline__ f32x16 qk_block(const bf16x8 (&qf)[D / 16], const uint16_t* ks, int key0, int r,
                                           int half) {
  constexpr int KS = Smem<D>::KS;
  f32x16 s = {};
#pragma unroll
  for (int sl = 0; sl < D / 16; ++sl) {
    const bf16x8 a = *reinterpret_cast<const bf16x8*>(ks + (key0 + r) * KS + sl * 16 + half * 8);
    s = mfma32(a, qf[sl], s);
  }
  return s;
}

// O^T += V^T * P^T for one 16-key group starting at tile key key0 + 16*h.
template <int D>
__device__ __forceinline__ void pv_group(RowState<D>& st, const bf16x8& pb, const uint16_t* vt, int key16, int r,
                                         int half) {
  constexpr int VS = Smem<D>::VS;
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt) {
    const bf16x8 a = *reinterpret_cast<const bf16x8*>(vt + (dt * 32 + r) * VS + key16 + 8 * half);
    st.o[dt] = mfma32(a, pb, st.o[dt]);
  }
}

// One 64-key sequence tile: two 32-key blocks of S^T, each folded into the
// state and multiplied into O^T.  MASK applies the causal / sequence-end mask
// (branch-free selects); interior tiles take the MASK = false path.
template <int D, bool MASK, bool CAUSAL>
__device__ __forceinline__ void seq_tile(RowState<D>& st, const bf16x8 (&qf)[D / 16], const uint16_t* ks,
                                         const uint16_t* vt, int kt0, int T, int my_t, int r, int half,
                                         float scale) {
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const f32x16 sacc = qk_block<D>(qf, ks, 32 * j, r, half);
    float s[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      s[i] = sacc[i];
      if (MASK) {
        const int key = kt0 + 32 * j + 8 * (i >> 2) + 4 * half + (i & 3);
        const bool vis = key < T && (!CAUSAL || key <= my_t);
        s[i] = vis ? s[i] : -INFINITY;
      }
    }
    bf16x8 pb[2];
    online_update<D, 16>(st, s, pb, scale);
#pragma unroll
    for (int h = 0; h < 2; ++h) pv_group<D>(st, pb[h], vt, 32 * j + 16 * h, r, half);
  }
}

template <int D, bool DEPTH, bool CAUSAL>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2, 2))) void moda_fwd_bf16_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
    const uint16_t* __restrict__ kd, const uint16_t* __restrict__ vd, int B, int T, int Hq, int Hk, int L,
    int lgG, int nrb, float scale_log2, uint16_t* __restrict__ out, float* __restrict__ lse) {
  using S = Smem<D>;
  __shared__ __attribute__((aligned(16))) uint16_t smem[S::kElems];

  const int G = 1 << lgG;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform: keeps per-wave control scalar
  const int r = lane & 31, half = lane >> 5;
  const int nbh = B * Hk;
  const int bid = blockIdx.x;
  const int rb = CAUSAL ? (nrb - 1 - bid / nbh) : (bid / nbh);
  const int bh = bid % nbh;

  const int b = bh / Hk, hk = bh % Hk;
  const int row0 = rb * kBM;
  const int TG = T << lgG;
  const int tb = row0 >> lgG;  // the workgroup's first token

  Geo g;
  g.L = DEPTH ? L : 0;
  g.tok_wave = (kRowsPerWave >> lgG) > 0 ? (kRowsPerWave >> lgG) : 1;
  g.key_bytes = static_cast<uint32_t>(Hk) * D * 2;
  g.tok_bytes = static_cast<uint32_t>(Hk) * (DEPTH ? L : 0) * D * 2;
  {
    const uint16_t* kb = k + (static_cast<int64_t>(b) * T * Hk + hk) * D;
    const uint16_t* vb = v + (static_cast<int64_t>(b) * T * Hk + hk) * D;
    const uint32_t seq_range = (static_cast<uint32_t>(T - 1) * Hk + 1) * D * 2;
    g.k = make_rsrc(kb, seq_range);
    g.v = make_rsrc(vb, seq_range);
    if (DEPTH) {
      const int64_t slab0 = ((static_cast<int64_t>(b) * T + tb) * Hk + hk) * static_cast<int64_t>(L) * D;
      const int64_t range = ((static_cast<int64_t>(T - 1 - tb) * Hk + 1) * L) * D * 2;
      const uint32_t dr = static_cast<uint32_t>(range < 0x7fffffff ? range : 0x7fffffff);
      g.kd = make_rsrc(kd + slab0, dr);
      g.vd = make_rsrc(vd + slab0, dr);
    } else {
      g.kd = g.k;
      g.vd = g.v;
    }
  }

  const int wrow0 = row0 + wave * kRowsPerWave;
  const int my_row = wrow0 + r;
  const bool row_ok = my_row < TG;
  const int my_t = my_row >> lgG;
  const int my_g = my_row & (G - 1);
  const int wt0 = wrow0 >> lgG;                                    // wave's first token
  const int wt1 = (min(wrow0 + kRowsPerWave, TG) - 1) >> lgG;      // wave's last valid token
  const int blk_last = (min(row0 + kBM, TG) - 1) >> lgG;           // block's last valid token
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

  // In depth tile it this wave's 16 rows (token wt0 + it / nchunk, slots from
  // 16 * (it % nchunk)) sit at tile rows [16*wave, 16*wave + 16): 32-key block
  // wave/2, score registers [8*(wave%2), 8*(wave%2) + 8).
  const int dj = wave >> 1, dh = wave & 1;

  // ---- tile pipeline ------------------------------------------------------------
  // Sequence tiles wholly before the workgroup's first token (and the sequence
  // end) are unmasked for every wave; the few after them overlap the
  // workgroup's own tokens and take the masked path.  The nd depth tiles are
  // spread evenly among the unmasked ones -- depth tile d follows sequence
  // tile (d+1)*n_int/nd - 1 -- so each depth load (a once-read HBM stream) is
  // prefetched under a full sequence tile of MFMA work.  Every loop body is
  // straight-line per wave, so the accumulator keeps its registers.
  const int tb_first = row0 >> lgG;
  const int n_int = CAUSAL ? min(ns, (tb_first + 1) / kBN) : T / kBN;
  Stage<D> stage;
  int pos = 0;  // pipeline position: selects the LDS buffer
  int sq = 0;   // next sequence tile
  if (DEPTH && nd > 0 && n_int / max(nd, 1) == 0)
    load_tile<D, true>(stage, g, 0, nchunk, tid);
  else
    load_tile<D, false>(stage, g, 0, nchunk, tid);

  if constexpr (DEPTH) {
    for (int d = 0; d < nd; ++d) {
      const int s_end = ((d + 1) * n_int) / nd;
      for (; sq < s_end; ++sq, ++pos) {
        uint16_t* ks = smem + (pos & 1) * S::kBuf;
        uint16_t* vt = ks + S::kK;
        store_tile<D>(stage, ks, vt, tid);
        __syncthreads();
        if (sq + 1 < s_end)
          load_tile<D, false>(stage, g, sq + 1, nchunk, tid);
        else
          load_tile<D, true>(stage, g, d, nchunk, tid);
        seq_tile<D, false, CAUSAL>(st, qf, ks, vt, sq * kBN, T, my_t, r, half, scale_log2);
      }
      // depth tile d: each wave sees only its own token's slots
      uint16_t* ks = smem + (pos & 1) * S::kBuf;
      uint16_t* vt = ks + S::kK;
      store_tile<D>(stage, ks, vt, tid);
      __syncthreads();
      if (d + 1 < nd) {
        if (sq < ((d + 2) * n_int) / nd)
          load_tile<D, false>(stage, g, sq, nchunk, tid);
        else
          load_tile<D, true>(stage, g, d + 1, nchunk, tid);
      } else if (sq < ns) {
        load_tile<D, false>(stage, g, sq, nchunk, tid);
      }
      ++pos;
      const f32x16 sacc = qk_block<D>(qf, ks, 32 * dj, r, half);
      const int dtok = d / nchunk;
      const int slot0 = (d - dtok * nchunk) * kDepthRowsPerWave;
      const bool mine = my_t == wt0 + dtok;
      float s[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int slot = slot0 + 8 * (i >> 2) + 4 * half + (i & 3);
        s[i] = (mine && slot < L) ? sacc[8 * dh + i] : -INFINITY;
      }
      bf16x8 pb[1];
      online_update<D, 8>(st, s, pb, scale_log2);
      pv_group<D>(st, pb[0], vt, 32 * dj + 16 * dh, r, half);
    }
  }
  for (; sq < n_int; ++sq, ++pos) {  // unmasked sequence tiles (all of them when there is no depth)
    uint16_t* ks = smem + (pos & 1) * S::kBuf;
    uint16_t* vt = ks + S::kK;
    store_tile<D>(stage, ks, vt, tid);
    __syncthreads();
    if (sq + 1 < ns) load_tile<D, false>(stage, g, sq + 1, nchunk, tid);
    seq_tile<D, false, CAUSAL>(st, qf, ks, vt, sq * kBN, T, my_t, r, half, scale_log2);
  }
  for (; sq < ns; ++sq, ++pos) {  // masked sequence tiles
    uint16_t* ks = smem + (pos & 1) * S::kBuf;
    uint16_t* vt = ks + S::kK;
    store_tile<D>(stage, ks, vt, tid);
    __syncthreads();
    if (sq + 1 < ns) load_tile<D, false>(stage, g, sq + 1, nchunk, tid);
    const int kt0 = sq * kBN;
    if (CAUSAL && kt0 > wt1) continue;  // nothing visible to this wave
    seq_tile<D, true, CAUSAL>(st, qf, ks, vt, kt0, T, my_t, r, half, scale_log2);
  }

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

template <int D, bool DEPTH, bool CAUSAL>
hipError_t launch(const FwdArgs& a) {
  const int lgG = __builtin_ctz(a.Hq / a.Hk);
  const int TG = a.T * (a.Hq / a.Hk);
  const int nrb = (TG + kBM - 1) / kBM;
  const int64_t nblocks = static_cast<int64_t>(nrb) * a.B * a.Hk;
  const float scale_log2 = kLog2e / sqrtf(static_cast<float>(D));
  hipLaunchKernelGGL((moda_fwd_bf16_kernel<D, DEPTH, CAUSAL>), dim3(static_cast<unsigned>(nblocks)),
                     dim3(kThreads), 0, static_cast<hipStream_t>(a.stream),
                     static_cast<const uint16_t*>(a.q), static_cast<const uint16_t*>(a.k),
                     static_cast<const uint16_t*>(a.v), static_cast<const uint16_t*>(a.kd),
                     static_cast<const uint16_t*>(a.vd), a.B, a.T, a.Hq, a.Hk, a.L, lgG, nrb, scale_log2,
                     static_cast<uint16_t*>(a.out), a.lse);
  return hipGetLastError();
}

template <int D>
hipError_t launch_d(const FwdArgs& a) {
  if (a.L > 0) return a.causal ? launch<D, true, true>(a) : launch<D, true, false>(a);
  return a.causal ? launch<D, false, true>(a) : launch<D, false, false>(a);
}

}  // namespace

int64_t fwd_bf16_grid_blocks(int B, int T, int Hq, int Hk) {
  const int64_t TG = static_cast<int64_t>(T) * (Hq / Hk);
  return (TG + kBM - 1) / kBM * B * Hk;
}

hipError_t launch_fwd_bf16(const FwdArgs& a) { return a.d == 64 ? launch_d<64>(a) : launch_d<128>(a); }

}  // namespace moda
