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
//     (b, hk); each of its 4 waves owns 32 rows.  The block's tokens are
//     [t_start, t_end) with t_start = floor(row0/G), t_end = floor(last/G)+1.
//   * Sequence loop: 64-key tiles of K and V are staged in LDS once per block
//     and read by all 4 waves.  Tiles past the block's last token are never
//     touched; tiles that are fully visible to a wave skip the mask.
//   * Scores are computed transposed, S^T = K * Q^T, on 32x32x16 bf16 MFMA with
//     Q^T held in registers, so each lane owns one query row: the row max
//     needs one cross-lane exchange (lane ^ 32) and the rescale of the output
//     accumulator is per lane.  O^T += V^T * P^T reuses the score registers as
//     the B operand directly; V is written to LDS transposed (d-major) with the
//     key order permuted to match the score register layout, so every MFMA
//     operand is one 16-byte LDS read.
//   * Depth stage: after the sequence loop each wave stages, token by token,
//     its own tokens' packed depth slab [L][d] (32 slots at a time) in LDS,
//     and folds it into the SAME running (max, sum, output) state; a slot is
//     visible only to the G rows of its token.  Each depth element is read
//     from HBM exactly once.
//   * Softmax runs in base 2 with log2(e)/sqrt(d) folded into one FMA; lse is
//     converted back to the natural log at the end.
//   * Causal workgroups are issued heaviest first (last row block first).
#include "moda_device.h"
#include "moda_launch.h"

namespace moda {
namespace {

constexpr int kWaves = 4;
constexpr int kThreads = kWaves * 64;
constexpr int kRowsPerWave = 32;
constexpr int kBM = kWaves * kRowsPerWave;  // expanded rows per workgroup
constexpr int kBN = 64;                     // sequence keys per tile
constexpr int kBD = 32;                     // depth slots per depth tile

template <int D>
struct Smem {
  static constexpr int KS = D + 8;     // K row stride (elements): +16 B breaks bank aliasing
  static constexpr int VS = kBN + 8;   // V^T row stride for sequence tiles
  static constexpr int VSD = kBD + 8;  // V^T row stride for depth tiles
  static constexpr int kSeqK = kBN * KS;
  static constexpr int kSeqV = D * VS;
  static constexpr int kDepK = kBD * KS;
  static constexpr int kDepV = D * VSD;
  static constexpr int kDepWave = kDepK + kDepV;
  static constexpr int kSeqTotal = kSeqK + kSeqV;
  static constexpr int kDepTotal = kWaves * kDepWave;
  static constexpr int kElems = kSeqTotal > kDepTotal ? kSeqTotal : kDepTotal;
};

// Position of tile key `kk` inside a d-row of the transposed V tile.  Within
// each 16-key group, key 8a + 4b + c is stored at 8b + 4a + c: the 8 keys that
// lane half b holds in its score registers for one PV product become 8
// consecutive elements (one 16-byte read).
__device__ __forceinline__ int vpos(int kk) {
  const int a = (kk >> 3) & 1, bb = (kk >> 2) & 1;
  return (kk & ~15) | (bb << 3) | (a << 2) | (kk & 3);
}

// Stage `nrows` rows (keys or slots) of K as row-major [row][d] and of V as
// transposed [d][vpos(row)], zero-filling rows >= valid.  Row r of K (V) is
// at kg + r*stride (vg + r*stride).  Threads [t0, t0 + nthr) take part.
template <int D, int NROWS, int VSTRIDE>
__device__ __forceinline__ void stage_kv(const uint16_t* __restrict__ kg, const uint16_t* __restrict__ vg,
                                         int64_t stride, int valid, uint16_t* ks, uint16_t* vt,
                                         int tid, int nthr) {
  constexpr int KS = D + 8;
  constexpr int CH = D / 8;  // 16-byte chunks per row
  for (int c = tid; c < NROWS * CH; c += nthr) {
    const int row = c / CH, ch = c % CH;
    u32x4 val = {0u, 0u, 0u, 0u};
    if (row < valid) val = *reinterpret_cast<const u32x4*>(kg + row * stride + ch * 8);
    *reinterpret_cast<u32x4*>(ks + row * KS + ch * 8) = val;
  }
  for (int it = tid; it < (NROWS / 4) * CH; it += nthr) {
    const int quad = it % (NROWS / 4), oc = it / (NROWS / 4);
    u32x4 r[4];
#pragma unroll
    for (int x = 0; x < 4; ++x) {
      const int row = quad * 4 + x;
      r[x] = u32x4{0u, 0u, 0u, 0u};
      if (row < valid) r[x] = *reinterpret_cast<const u32x4*>(vg + row * stride + oc * 8);
    }
    const int pos = vpos(quad * 4);
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
      *reinterpret_cast<u32x2*>(vt + (oc * 8 + e) * VSTRIDE + pos) = u32x2{lo, hi};
    }
  }
}

// Running softmax state of one query row held by a lane pair (l, l ^ 32).
template <int D>
struct RowState {
  f32x16 o[D / 32];  // O^T accumulator: d = 32*dt + 8*(i/4) + 4*half + (i%4)
  float m;           // running max of the base-2 scaled logits (same in both lanes)
  float l;           // this lane's share of the running denominator
};

// Fold one 32-key block of scores (already scaled to base 2, -inf = masked)
// into the state.  x[i] belongs to key 8*(i/4) + 4*half + (i%4) of the block.
// Returns the unnormalised weights, packed to bf16, as the two B operands of
// the PV product (keys 0..15 and 16..31 of the block).
template <int D>
__device__ __forceinline__ void online_update(RowState<D>& st, float (&x)[16], bf16x8 (&pb)[2]) {
  float mx = x[0];
#pragma unroll
  for (int i = 1; i < 16; ++i) mx = fmaxf(mx, x[i]);
  mx = fmaxf(mx, wave_xor32(mx));
  const float m_new = fmaxf(st.m, mx);
  const float base = (m_new == -INFINITY) ? 0.0f : m_new;
  const float alpha = fast_exp2(st.m - base);
  float sum = 0.0f;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    x[i] = fast_exp2(x[i] - base);
    sum += x[i];
  }
  st.l = st.l * alpha + sum;
  st.m = m_new;
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
    for (int i = 0; i < 16; ++i) st.o[dt][i] *= alpha;
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    u32x4 w;
#pragma unroll
    for (int k = 0; k < 4; ++k) w[k] = pack_bf16x2(x[8 * h + 2 * k], x[8 * h + 2 * k + 1]);
    pb[h] = __builtin_bit_cast(bf16x8, w);
  }
}

// O^T += V^T * P^T for one 32-key block (two 16-key products per d tile).
template <int D, int VSTRIDE>
__device__ __forceinline__ void pv_block(RowState<D>& st, const bf16x8 (&pb)[2], const uint16_t* vt,
                                         int key0, int r, int half) {
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const bf16x8 a = *reinterpret_cast<const bf16x8*>(vt + (dt * 32 + r) * VSTRIDE + key0 + 16 * h + 8 * half);
      st.o[dt] = mfma32(a, pb[h], st.o[dt]);
    }
}

// S^T block: 32 keys (rows of ks starting at key0) x 32 query rows.
template <int D>
__device__ __forceinline__ f32x16 qk_block(const bf16x8 (&qf)[D / 16], const uint16_t* ks, int key0, int r,
                                           int half) {
  constexpr int KS = D + 8;
  f32x16 s = {};
#pragma unroll
  for (int sl = 0; sl < D / 16; ++sl) {
    const bf16x8 a = *reinterpret_cast<const bf16x8*>(ks + (key0 + r) * KS + sl * 16 + half * 8);
    s = mfma32(a, qf[sl], s);
  }
  return s;
}

template <int D, bool DEPTH, bool CAUSAL>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2, 2))) void moda_fwd_bf16_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
    const uint16_t* __restrict__ kd, const uint16_t* __restrict__ vd, int B, int T, int Hq, int Hk, int L,
    int lgG, int nrb, float scale_log2, uint16_t* __restrict__ out, float* __restrict__ lse) {
  using S = Smem<D>;
  __shared__ __attribute__((aligned(16))) uint16_t smem[S::kElems];

  const int G = 1 << lgG;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int r = lane & 31, half = lane >> 5;
  const int nbh = B * Hk;
  const int bid = blockIdx.x;
  const int rb = CAUSAL ? (nrb - 1 - bid / nbh) : (bid / nbh);
  const int bh = bid % nbh;
  const int b = bh / Hk, hk = bh % Hk;
  const int TG = T << lgG;
  const int row0 = rb * kBM;
  const int wrow0 = row0 + wave * kRowsPerWave;
  const int my_row = wrow0 + r;
  const bool row_ok = my_row < TG;
  const int my_t = my_row >> lgG;
  const int my_g = my_row & (G - 1);
  const bool wave_live = wrow0 < TG;
  const int wt0 = wrow0 >> lgG;                                        // wave's first token
  const int wt1 = (min(wrow0 + kRowsPerWave, TG) - 1) >> lgG;          // wave's last valid token
  const int blk_last = (min(row0 + kBM, TG) - 1) >> lgG;               // block's last valid token
  const int kv_end = CAUSAL ? blk_last + 1 : T;
  const int ntiles = (kv_end + kBN - 1) / kBN;

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

  const int64_t kv_stride = static_cast<int64_t>(Hk) * D;
  const uint16_t* kbase = k + (static_cast<int64_t>(b) * T * Hk + hk) * D;
  const uint16_t* vbase = v + (static_cast<int64_t>(b) * T * Hk + hk) * D;
  uint16_t* ks = smem;
  uint16_t* vt = smem + S::kSeqK;

  // ---- sequence loop -------------------------------------------------------
  for (int tile = 0; tile < ntiles; ++tile) {
    const int kt0 = tile * kBN;
    __syncthreads();
    stage_kv<D, kBN, S::VS>(kbase + kt0 * kv_stride, vbase + kt0 * kv_stride, kv_stride, min(kBN, T - kt0), ks,
                           vt, tid, kThreads);
    __syncthreads();
    if (!wave_live || (CAUSAL && kt0 > wt1)) continue;  // nothing visible to this wave
    const bool need_mask = (kt0 + kBN > T) || (CAUSAL && kt0 + kBN - 1 > wt0);
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      f32x16 s = qk_block<D>(qf, ks, 32 * j, r, half);
      float x[16];
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        x[i] = s[i] * scale_log2;
        if (need_mask) {
          const int key = kt0 + 32 * j + 8 * (i >> 2) + 4 * half + (i & 3);
          const bool vis = key < T && (!CAUSAL || key <= my_t);
          if (!vis) x[i] = -INFINITY;
        }
      }
      bf16x8 pb[2];
      online_update<D>(st, x, pb);
      pv_block<D, S::VS>(st, pb, vt, 32 * j, r, half);
    }
  }

  // ---- depth stage ---------------------------------------------------------
  if constexpr (DEPTH) {
    const int tok_per_wave = (kRowsPerWave >> lgG) > 0 ? (kRowsPerWave >> lgG) : 1;
    const int nchunks = (L + kBD - 1) / kBD;
    uint16_t* kds = smem + wave * S::kDepWave;
    uint16_t* vdt = kds + S::kDepK;
    for (int kt = 0; kt < tok_per_wave; ++kt) {
      const int tw = wt0 + kt;  // this wave's token for this step
      const bool tok_ok = wave_live && tw < T && tw <= wt1;
      const int64_t slab = ((static_cast<int64_t>(b) * T + (tok_ok ? tw : 0)) * Hk + hk) * L;
      for (int ch = 0; ch < nchunks; ++ch) {
        const int i0 = ch * kBD;
        __syncthreads();
        const int valid = tok_ok ? min(kBD, L - i0) : 0;
        stage_kv<D, kBD, S::VSD>(kd + (slab + i0) * D, vd + (slab + i0) * D, D, valid, kds, vdt, lane, 64);
        __syncthreads();
        if (!tok_ok) continue;
        f32x16 s = qk_block<D>(qf, kds, 0, r, half);
        float x[16];
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int slot = i0 + 8 * (i >> 2) + 4 * half + (i & 3);
          const bool vis = (my_t == tw) && slot < L;
          x[i] = vis ? s[i] * scale_log2 : -INFINITY;
        }
        bf16x8 pb[2];
        online_update<D>(st, x, pb);
        pv_block<D, S::VSD>(st, pb, vdt, 0, r, half);
      }
    }
  }

  // ---- epilogue --------------------------------------------------------------
  const float l_tot = st.l + wave_xor32(st.l);
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
