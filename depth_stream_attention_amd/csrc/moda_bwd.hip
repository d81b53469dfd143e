// MoDA backward, bf16 inputs, fp32 accumulation, bf16 gradients (gfx950).
//
// The forward's one softmax per query row runs over the row's causally
// visible sequence keys and the L depth slots of its own token ("Mixture-of-
// Depths Attention" summary, papercache.org, 2.2; MoDA reading notes,
// cc.laoqi.cc, 二.2).  Its gradients follow from the saved natural-log lse:
// with P = exp(s q.k - lse) for every candidate of a row, dP = dO.v,
// Dsum = sum_c dO*O (equal to sum_n P_n dP_n) and dS = P (dP - Dsum),
//   dq = s sum_n dS_n k_n,   dk_n = s sum_rows dS q,   dv_n = sum_rows P dO.
// Rows are recomputed from lse; nothing of the forward but out and lse is kept.
//
// Four launches, no atomics, every output written by exactly one lane:
//   1. rows:  Dsum per row and lse in base 2, both re-laid out as expanded
//             rows [B][Hk][T*G] (row t*G + g is token t, head hk*G + g), the
//             order the tiled kernels read.
//   2. depth: per (token, KV head): the G rows of the token against its L depth
//             slots.  Depth slots are seen by their own token only, so this
//             produces dK_depth and dV_depth completely and the depth share of
//             dq (fp32, in the workspace).  16x16 MFMA tiles: 16 of the G
//             rows on one side (G = 32 in two halves), 16 slots on the other.
//   3. dq:    the forward's decomposition (128 expanded rows per workgroup, 32
//             per wave, lane = query row) over 64-key sequence tiles:
//             S^T = K Q^T, dP^T = V dO^T, dS^T, then dQ^T += K^T dS^T.  Adds the
//             depth share and writes dq.
//   4. dkv:   128 sequence keys per workgroup over 64-row tiles of Q, dO, lse
//             and Dsum; each 32 keys (lane = key) are shared by two waves, one
//             forming S = Q K^T, P and dV^T += dO^T P, the other, a tile later,
//             dP = dO V^T, dS from the P passed through LDS, and dK^T += Q^T dS.
// Tiles are staged by direct-to-LDS buffer loads into a double-buffered
// (dkv: triple-buffered) pipeline.  Every tile that is read both row-wise (as an MFMA operand) and
// transposed (ds_read_b64_tr_b16) uses one XOR swizzle that keeps both read
// patterns free of bank conflicts.
#include <algorithm>
#include <type_traits>

#include "moda_launch.h"
#include "moda_tile.h"

namespace moda {
namespace {

typedef __attribute__((address_space(3))) f32x4 lds_f32x4_t;
typedef __attribute__((address_space(3))) u32x4 lds_u32x4_t;

constexpr int kWaves = 4;
constexpr int kThreads = kWaves * 64;
constexpr int kRowsPerWave = 32;
constexpr int kBM = kWaves * kRowsPerWave;  // expanded rows per dq workgroup
constexpr int kKB = kWaves * 32;            // sequence keys per dkv workgroup

// Direct-to-LDS load instructions per wave per 64-row tile of one tensor.
template <int D>
constexpr int kNX = Tile<D>::CH / kWaves;

// 16x16 matrix-core products, fp32 accumulation.  Lane l supplies row (l % 16)
// of A and column (l % 16) of B with the contraction elements chosen by
// l / 16 (8 of them for x32, 4 for x16); acc element i of lane l is
// C[4*(l/16) + i][l % 16].
__device__ __forceinline__ f32x4 mfma16x32(const bf16x8& a, const bf16x8& b, const f32x4& acc) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, acc, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma16x16(const s16x4& a, const s16x4& b, const f32x4& acc) {
  return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, b, acc, 0, 0, 0);
}

__device__ __forceinline__ s16x4 pack4(float a, float b, float c, float d) {
  u32x2 w = {pack_bf16x2(a, b), pack_bf16x2(c, d)};
  return __builtin_bit_cast(s16x4, w);
}

__device__ __forceinline__ s16x4 read_tr(uint32_t addr) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16(lds_at<lds_s16x4_t>(addr));
}

// ---- 64-row tiles read both row-wise and transposed -----------------------------
//
// Logical 16-byte chunk c of tile row r lives at physical chunk c ^ swz_u(r),
// swz_u(r) = 4*(u % (CH/4)) + (u / (CH/4)) % 4 with u = r / RPB (RPB rows share
// one 256-byte bank row).  Row-wise operand reads (16 consecutive rows, one
// logical chunk per 16 lanes) see 16 distinct values of swz_u; transposed reads
// (4 consecutive rows x 4 consecutive chunks per 32 lanes) see 4 distinct
// values of swz_u / 4.  Both therefore cover all 64 banks.  swz_u repeats
// every 16 rows, so 16-row and 32-row steps are immediate offsets.
template <int D>
__device__ __forceinline__ int swz_u(int row) {
  using TL = Tile<D>;
  const int u = row / TL::RPB;
  return 4 * (u % (TL::CH / 4)) + (u / (TL::CH / 4)) % 4;
}

// Per-lane LDS read offsets within one 64-row tile (see qk_block and acc_group).
template <int D>
struct TileReads {
  uint32_t nr[D / 16];  // row-wise read of slice sl: row lane%32, logical chunk 2*sl + lane/32
  uint32_t lo[D / 32];  // transposed read of d tile dt, rows 4*hf + i/4
  uint32_t hi[D / 32];  // the same 8 rows further down (its own swizzle)
};

template <int D>
__device__ __forceinline__ void init_reads(TileReads<D>& tr, int lane) {
  using TL = Tile<D>;
  const int r = lane & 31, half = lane >> 5;
#pragma unroll
  for (int sl = 0; sl < D / 16; ++sl) tr.nr[sl] = r * TL::ROW_BYTES + (((2 * sl + half) ^ swz_u<D>(r)) * 16);
  const int i = lane & 15, q = (lane >> 4) & 1, hf = lane >> 5;
  const int row0 = 4 * hf + (i >> 2), row1 = row0 + 8;
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt) {
    const int lc = (32 * dt + 16 * q) / 8 + ((i & 3) >> 1);  // logical chunk of column 32*dt + 16*q + 4*(i%4)
    tr.lo[dt] = row0 * TL::ROW_BYTES + 8 * (i & 1) + ((lc ^ swz_u<D>(row0)) * 16);
    tr.hi[dt] = row1 * TL::ROW_BYTES + 8 * (i & 1) + ((lc ^ swz_u<D>(row1)) * 16);
  }
}

// Absolute addresses of one tile's reads (one add per register).
template <int D>
__device__ __forceinline__ TileReads<D> at(const TileReads<D>& o, uint32_t base) {
  TileReads<D> a;
#pragma unroll
  for (int sl = 0; sl < D / 16; ++sl) a.nr[sl] = base + o.nr[sl];
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt) {
    a.lo[dt] = base + o.lo[dt];
    a.hi[dt] = base + o.hi[dt];
  }
  return a;
}

// acc^T += X^T * W for one 16-row group of the tile (`off` bytes in): X is the
// tile (rows x d), read transposed as the A operand; W is the B operand pb,
// which in lane half hf holds the weights of group rows 4*hf + {0..3} and
// 8 + 4*hf + {0..3} (the layout of a 32x32 accumulator's 16-row group).
template <int D>
__device__ __forceinline__ void acc_group(f32x16 (&acc)[D / 32], const bf16x8& pb, const TileReads<D>& ta,
                                          int off) {
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt) {
    const s16x4 lo4 = read_tr(ta.lo[dt] + off);
    const s16x4 hi4 = read_tr(ta.hi[dt] + off);
    const bf16x8 a = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo4, hi4, 0, 1, 2, 3, 4, 5, 6, 7));
    acc[dt] = mfma32(a, pb, acc[dt]);
  }
}

// 16 accumulator values -> two bf16x8 B operands (group h = values 8h .. 8h+7).
__device__ __forceinline__ void pack16(const float (&x)[16], bf16x8 (&pb)[2]) {
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    u32x4 w;
#pragma unroll
    for (int k = 0; k < 4; ++k) w[k] = pack_bf16x2(x[8 * h + 2 * k], x[8 * h + 2 * k + 1]);
    pb[h] = __builtin_bit_cast(bf16x8, w);
  }
}

// ---- 1. row statistics ------------------------------------------------------------

template <int D>
__global__ __launch_bounds__(256) void moda_bwd_rows_kernel(const uint16_t* __restrict__ out,
                                                            const uint16_t* __restrict__ dout,
                                                            const float* __restrict__ lse, int64_t n_rows, int T,
                                                            int Hq, int Hk, int lgG, float* __restrict__ ws_l2,
                                                            float* __restrict__ ws_dd) {
  constexpr int LPR = D / 8;  // lanes per row, 8 elements each
  const int64_t row = (static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x) / LPR;
  const int c = threadIdx.x % LPR;
  float acc = 0.0f;
  if (row < n_rows) {
    const u32x4 o = *reinterpret_cast<const u32x4*>(out + row * D + c * 8);
    const u32x4 g = *reinterpret_cast<const u32x4*>(dout + row * D + c * 8);
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      acc = fmaf(__uint_as_float(o[k] << 16), __uint_as_float(g[k] << 16), acc);
      acc = fmaf(__uint_as_float(o[k] & 0xffff0000u), __uint_as_float(g[k] & 0xffff0000u), acc);
    }
  }
#pragma unroll
  for (int m = 1; m < LPR; m <<= 1) acc += __shfl_xor(acc, m, 64);
  if (row < n_rows && c == 0) {
    const int G = 1 << lgG;
    const int h = static_cast<int>(row % Hq);
    const int64_t bt = row / Hq;
    const int t = static_cast<int>(bt % T);
    const int64_t b = bt / T;
    const int hk = h >> lgG, g = h & (G - 1);
    const int64_t e = ((b * Hk + hk) * T + t) * G + g;
    ws_dd[e] = acc;
    ws_l2[e] = lse[(b * Hq + h) * T + t] * kLog2e;
  }
}

// ---- 2. depth slots ------------------------------------------------------------------
//
// One wave per (token t, KV head hk) unit at a time.  Its G rows (padded to 16)
// and 16 depth slots per step meet in 16x16 tiles:
//   S   = Q Kd^T and dP = dO Vd^T   (lane = slot; rows down the registers)
//   S^T and dP^T                    (lane = row;  slots down the registers)
//   dVd^T = dO^T P, dKd^T = Q^T dS  (A read transposed from LDS, B = P, dS as computed)
//   dQ^T += Kd^T dS^T               (A read transposed from LDS, B = dS^T as computed)
// Both orientations of the scores are formed so that every B operand is an
// accumulator exactly as the MFMA left it.  The unit's rows of Q and dO and
// the step's Kd rows are kept in LDS (16 rows each, per wave) for the
// transposed reads.

template <int D>
struct Blk16 {
  static constexpr int ROW_BYTES = D * 2;
  static constexpr int CH = D / 8;
  static constexpr int RPB = 256 / ROW_BYTES;
  static constexpr int BYTES = 16 * ROW_BYTES;
  // Row-wise reads (16 rows, one logical chunk per 16 lanes) meet 16 distinct
  // swizzles; transposed reads (8 rows x one 32-byte chunk pair per 32 lanes)
  // meet 8 distinct values of swz / 2.
  __device__ static __forceinline__ int swz(int row) {
    const int u = row / RPB;
    return 2 * (u % (CH / 2)) + (u / (CH / 2)) % 2;
  }
};

template <int D, int NH>
__global__ __launch_bounds__(kThreads) void moda_bwd_depth_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ dout, const uint16_t* __restrict__ kd,
    const uint16_t* __restrict__ vd, const float* __restrict__ ws_l2, const float* __restrict__ ws_dd, int T, int Hq,
    int Hk, int L, int lgG, int64_t n_units, float scale, float scale_log2, float* __restrict__ dq_depth,
    uint16_t* __restrict__ dkd, uint16_t* __restrict__ dvd) {
  // NH = 16-row halves of the unit's G rows (1 for G <= 16, 2 for G = 32): each
  // half forms its own scores; the slot gradients sum both halves' products.
  using BK = Blk16<D>;
  constexpr int KC = D / 32;  // 16x16x32 contraction steps over d
  constexpr int DC = D / 16;  // 16-wide d tiles of the outputs
  constexpr int PER_WAVE = (2 * NH + 1) * BK::BYTES;  // Q and dO rows of every half, one Kd step
  __shared__ __attribute__((aligned(16))) uint8_t smem_raw[kWaves * PER_WAVE];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const uint32_t qs = lds_addr((lds_u8*)smem_raw) + wave * PER_WAVE;  // half h: qs + h * BYTES
  const uint32_t os = qs + NH * BK::BYTES, ks = os + NH * BK::BYTES;
  const int G = 1 << lgG;
  const int r16 = lane & 15, grp = lane >> 4;

  uint32_t nrm[KC];  // row r16, logical chunk 4*kc + grp
#pragma unroll
  for (int kc = 0; kc < KC; ++kc) nrm[kc] = r16 * BK::ROW_BYTES + (((4 * kc + grp) ^ BK::swz(r16)) * 16);
  uint32_t trd[DC];  // transposed read of d tile dc: lane r16 of group grp -> row 4*grp + r16/4, column 16*dc + 4*(r16%4)
  {
    const int row = 4 * grp + (r16 >> 2);
#pragma unroll
    for (int dc = 0; dc < DC; ++dc) {
      const int lc = 2 * dc + ((r16 & 3) >> 1);
      trd[dc] = row * BK::ROW_BYTES + ((lc ^ BK::swz(row)) * 16) + 8 * (r16 & 1);
    }
  }

  const int64_t stride = static_cast<int64_t>(gridDim.x) * kWaves;
  for (int64_t u = static_cast<int64_t>(blockIdx.x) * kWaves + wave; u < n_units; u += stride) {
    const int hk = static_cast<int>(u % Hk);
    const int64_t bt = u / Hk;  // b*T + t
    const int t = static_cast<int>(bt % T);
    const int64_t b = bt / T;
    const int64_t row0 = (bt * Hq + static_cast<int64_t>(hk) * G) * D;  // element offset of the unit's first row

    bf16x8 qf[NH][KC], of[NH][KC];
#pragma unroll
    for (int h = 0; h < NH; ++h)
#pragma unroll
      for (int kc = 0; kc < KC; ++kc) {
        u32x4 a = {0u, 0u, 0u, 0u}, c = {0u, 0u, 0u, 0u};
        if (16 * h + r16 < G) {
          a = *reinterpret_cast<const u32x4*>(q + row0 + (16 * h + r16) * D + (4 * kc + grp) * 8);
          c = *reinterpret_cast<const u32x4*>(dout + row0 + (16 * h + r16) * D + (4 * kc + grp) * 8);
        }
        qf[h][kc] = __builtin_bit_cast(bf16x8, a);
        of[h][kc] = __builtin_bit_cast(bf16x8, c);
        *lds_at<lds_bf16x8_t>(qs + h * BK::BYTES + nrm[kc]) = qf[h][kc];
        *lds_at<lds_bf16x8_t>(os + h * BK::BYTES + nrm[kc]) = of[h][kc];
      }
    const int64_t e0 = ((b * Hk + hk) * T + t) * G;  // expanded index of the unit's row 0
    float l2T[NH], ddT[NH], l2S[NH][4], ddS[NH][4];
#pragma unroll
    for (int h = 0; h < NH; ++h) {
      l2T[h] = 16 * h + r16 < G ? ws_l2[e0 + 16 * h + r16] : INFINITY;
      ddT[h] = 16 * h + r16 < G ? ws_dd[e0 + 16 * h + r16] : 0.0f;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int rr = 16 * h + 4 * grp + i;
        l2S[h][i] = rr < G ? ws_l2[e0 + rr] : INFINITY;
        ddS[h][i] = rr < G ? ws_dd[e0 + rr] : 0.0f;
      }
    }

    f32x4 dqa[NH][DC];
#pragma unroll
    for (int h = 0; h < NH; ++h)
#pragma unroll
      for (int dc = 0; dc < DC; ++dc) dqa[h][dc] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    const int64_t slab = u * static_cast<int64_t>(L) * D;  // packed [B][T][Hk][L][d]: slab index = u

    // Depth K/V rows of one 16-slot step (zero past slot L), the next step's
    // loads issued before this step's products.
    auto load_step = [&](int c0, bf16x8 (&kx)[KC], bf16x8 (&vx)[KC]) {
      const int slot = c0 + r16;
#pragma unroll
      for (int kc = 0; kc < KC; ++kc) {
        u32x4 a = {0u, 0u, 0u, 0u}, c = {0u, 0u, 0u, 0u};
        if (slot < L) {
          a = *reinterpret_cast<const u32x4*>(kd + slab + static_cast<int64_t>(slot) * D + (4 * kc + grp) * 8);
          c = *reinterpret_cast<const u32x4*>(vd + slab + static_cast<int64_t>(slot) * D + (4 * kc + grp) * 8);
        }
        kx[kc] = __builtin_bit_cast(bf16x8, a);
        vx[kc] = __builtin_bit_cast(bf16x8, c);
      }
    };
    bf16x8 kn[KC], vn[KC];
    load_step(0, kn, vn);
    for (int c0 = 0; c0 < L; c0 += 16) {
      const int slot = c0 + r16;
      const bool valid = slot < L;
      bf16x8 kf[KC], vf[KC];
#pragma unroll
      for (int kc = 0; kc < KC; ++kc) {
        kf[kc] = kn[kc];
        vf[kc] = vn[kc];
      }
      if (c0 + 16 < L) load_step(c0 + 16, kn, vn);
#pragma unroll
      for (int kc = 0; kc < KC; ++kc) *lds_at<lds_bf16x8_t>(ks + nrm[kc]) = kf[kc];
      s16x4 P4[NH], DS4[NH], DST4[NH];
#pragma unroll
      for (int h = 0; h < NH; ++h) {
        f32x4 S = {}, dP = {}, ST = {}, dPT = {};
#pragma unroll
        for (int kc = 0; kc < KC; ++kc) {
          S = mfma16x32(qf[h][kc], kf[kc], S);     // [row 16h+4*grp+i][slot r16]
          dP = mfma16x32(of[h][kc], vf[kc], dP);
          ST = mfma16x32(kf[kc], qf[h][kc], ST);   // [slot 4*grp+i][row 16h+r16]
          dPT = mfma16x32(vf[kc], of[h][kc], dPT);
        }
        float p[4], ds[4], dst[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          p[i] = valid ? fast_exp2(fmaf(S[i], scale_log2, -l2S[h][i])) : 0.0f;
          ds[i] = p[i] * (dP[i] - ddS[h][i]);
          const bool vt = c0 + 4 * grp + i < L;
          const float pt = vt ? fast_exp2(fmaf(ST[i], scale_log2, -l2T[h])) : 0.0f;
          dst[i] = pt * (dPT[i] - ddT[h]);
        }
        P4[h] = pack4(p[0], p[1], p[2], p[3]);
        DS4[h] = pack4(ds[0], ds[1], ds[2], ds[3]);
        DST4[h] = pack4(dst[0], dst[1], dst[2], dst[3]);
      }
      uint16_t* dk_row = dkd + slab + static_cast<int64_t>(slot) * D + 4 * grp;
      uint16_t* dv_row = dvd + slab + static_cast<int64_t>(slot) * D + 4 * grp;
#pragma unroll
      for (int dc = 0; dc < DC; ++dc) {
        f32x4 gv = {0.0f, 0.0f, 0.0f, 0.0f}, gk = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int h = 0; h < NH; ++h) {
          gv = mfma16x16(read_tr(os + h * BK::BYTES + trd[dc]), P4[h], gv);   // [d 16dc+4grp+i][slot r16]
          gk = mfma16x16(read_tr(qs + h * BK::BYTES + trd[dc]), DS4[h], gk);
          dqa[h][dc] = mfma16x16(read_tr(ks + trd[dc]), DST4[h], dqa[h][dc]);  // [d 16dc+4grp+i][row 16h+r16]
        }
        if (valid) {
          u32x2 wv = {pack_bf16x2(gv[0], gv[1]), pack_bf16x2(gv[2], gv[3])};
          u32x2 wk = {pack_bf16x2(gk[0] * scale, gk[1] * scale), pack_bf16x2(gk[2] * scale, gk[3] * scale)};
          *reinterpret_cast<u32x2*>(dv_row + 16 * dc) = wv;
          *reinterpret_cast<u32x2*>(dk_row + 16 * dc) = wk;
        }
      }
    }
#pragma unroll
    for (int h = 0; h < NH; ++h)
      if (16 * h + r16 < G) {
        float* dqr = dq_depth + row0 + (16 * h + r16) * D + 4 * grp;
#pragma unroll
        for (int dc = 0; dc < DC; ++dc) *reinterpret_cast<f32x4*>(dqr + 16 * dc) = dqa[h][dc] * scale;
      }
  }
}

// ---- 3. dq over the sequence keys ------------------------------------------------------

// Direct-to-LDS staging of a 64-key tile of K and V: the forward's scheme with
// the swizzle that serves both read patterns.
template <int D>
struct KvDma {
  uint32_t k[kNX<D>], v[kNX<D>];
};

template <int D>
__device__ __forceinline__ void init_kv_dma(KvDma<D>& o, int lane, int wave, uint32_t key_bytes) {
  using TL = Tile<D>;
  constexpr int NX = kNX<D>;
#pragma unroll
  for (int x = 0; x < NX; ++x) {
    const int pr = (wave * NX + x) * TL::RPI + lane / TL::CH;
    const int pc = lane % TL::CH;
    o.k[x] = static_cast<uint32_t>(pr) * key_bytes + ((pc ^ swz_u<D>(pr)) * 16);
    o.v[x] = o.k[x];
  }
}

template <int D>
__device__ __forceinline__ void dma_kv(const uint16_t* kb, const uint16_t* vb, uint32_t seq_range, uint32_t key_bytes,
                                       int Hk, int idx, lds_u8* buf, int wave, const KvDma<D>& o) {
  using TL = Tile<D>;
  constexpr int NX = kNX<D>;
  const int64_t first = static_cast<int64_t>(idx) * kBN * Hk * D;
  const uint32_t range = seq_range - static_cast<uint32_t>(idx * kBN) * key_bytes;
  const u32x4 rk = raw_rsrc(kb + first, range);
  const u32x4 rv = raw_rsrc(vb + first, range);
#pragma unroll
  for (int x = 0; x < NX; ++x) {
    const uint32_t dst = lds_addr(buf + (wave * NX + x) * 1024);
    dma16(rk, dst, o.k[x]);
    dma16(rv, dst + TL::BYTES, o.v[x]);
  }
}

// One 64-key tile: for both 32-key blocks S^T, dP^T, dS^T, then dQ^T += K^T dS^T.
// ka, va address buffer 0's K and V; the tile sits B bytes further.
template <int D, bool MASK, bool CAUSAL, int B>
__device__ __forceinline__ void dq_tile(f32x16 (&dqa)[D / 32], const bf16x8 (&qf)[D / 16], const bf16x8 (&df)[D / 16],
                                        const TileReads<D>& ka, const TileReads<D>& va, int kt0, int T, int my_t,
                                        int half, float scale_log2, float l2, float dd) {
  using TL = Tile<D>;
  f32x16 sq[2], dp[2];
  sq[0] = qk_block<D>(qf, ka.nr, B);
  sq[1] = qk_block<D>(qf, ka.nr, B + 32 * TL::ROW_BYTES);
  dp[0] = qk_block<D>(df, va.nr, B);
  dp[1] = qk_block<D>(df, va.nr, B + 32 * TL::ROW_BYTES);
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    float ds[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      float x = fmaf(sq[j][i], scale_log2, -l2);
      if (MASK) {
        const int key = kt0 + 32 * j + 8 * (i >> 2) + 4 * half + (i & 3);
        const bool vis = key < T && (!CAUSAL || key <= my_t);
        x = vis ? x : -INFINITY;
      }
      ds[i] = fast_exp2(x) * (dp[j][i] - dd);
    }
    bf16x8 pb[2];
    pack16(ds, pb);
#pragma unroll
    for (int h = 0; h < 2; ++h) acc_group<D>(dqa, pb[h], ka, B + (32 * j + 16 * h) * TL::ROW_BYTES);
  }
}

// Waves per SIMD the dq kernel is compiled for: at d = 64 it fits three
// (at most 168 VGPRs, 32 KiB of LDS per workgroup).
template <int D>
constexpr int kDqWavesPerEU = D == 64 ? 3 : 2;

template <int D, bool CAUSAL>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(kDqWavesPerEU<D>, kDqWavesPerEU<D>))) void moda_bwd_dq_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
    const uint16_t* __restrict__ dout, const float* __restrict__ ws_l2, const float* __restrict__ ws_dd,
    const float* __restrict__ dq_depth, int B, int T, int Hq, int Hk, int lgG, int nrb, float scale,
    float scale_log2, uint16_t* __restrict__ dq) {
  using TL = Tile<D>;
  __shared__ __attribute__((aligned(1024))) uint8_t smem_raw[4 * TL::BYTES];
  lds_u8* const smem = (lds_u8*)smem_raw;

  const int G = 1 << lgG;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int r = lane & 31, half = lane >> 5;
  const int nbh = B * Hk;
  const int bid = blockIdx.x;
  const int rb = CAUSAL ? (nrb - 1 - bid / nbh) : (bid / nbh);
  const int bh = bid % nbh;
  const int b = bh / Hk, hk = bh % Hk;
  const int row0 = rb * kBM;
  const int TG = T << lgG;
  const int tb = row0 >> lgG;

  const uint32_t key_bytes = static_cast<uint32_t>(Hk) * D * 2;
  const uint16_t* kb = k + (static_cast<int64_t>(b) * T * Hk + hk) * D;
  const uint16_t* vb = v + (static_cast<int64_t>(b) * T * Hk + hk) * D;
  const uint32_t seq_range = (static_cast<uint32_t>(T - 1) * Hk + 1) * D * 2;
  KvDma<D> dm;
  init_kv_dma<D>(dm, lane, wave, key_bytes);
  TileReads<D> ro;
  init_reads<D>(ro, lane);

  const int wrow0 = row0 + wave * kRowsPerWave;
  const int my_row = wrow0 + r;
  const bool row_ok = my_row < TG;
  const int my_t = my_row >> lgG;
  const int my_g = my_row & (G - 1);
  const int wt1 = (min(wrow0 + kRowsPerWave, TG) - 1) >> lgG;
  const int blk_last = (min(row0 + kBM, TG) - 1) >> lgG;
  const int kv_end = CAUSAL ? blk_last + 1 : T;
  const int ns = (kv_end + kBN - 1) / kBN;

  // Q^T and dO^T fragments (B operands): lane holds row my_row, d = 16*sl + 8*half + [0, 8).
  const int64_t qoff = ((static_cast<int64_t>(b) * T + my_t) * Hq + hk * G + my_g) * D;
  bf16x8 qf[D / 16], df[D / 16];
#pragma unroll
  for (int sl = 0; sl < D / 16; ++sl) {
    u32x4 a = {0u, 0u, 0u, 0u}, c = {0u, 0u, 0u, 0u};
    if (row_ok) {
      a = *reinterpret_cast<const u32x4*>(q + qoff + sl * 16 + half * 8);
      c = *reinterpret_cast<const u32x4*>(dout + qoff + sl * 16 + half * 8);
    }
    qf[sl] = __builtin_bit_cast(bf16x8, a);
    df[sl] = __builtin_bit_cast(bf16x8, c);
  }
  const int64_t e = (static_cast<int64_t>(b) * Hk + hk) * TG + my_row;
  const float l2 = row_ok ? ws_l2[e] : 0.0f;
  const float dd = row_ok ? ws_dd[e] : 0.0f;

  f32x16 dqa[D / 32];
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt) dqa[dt] = f32x16{};

  // Tiles run in pairs (LDS buffer 0, then buffer 1, after at most one tile
  // that evens the position), so every read address is a per-lane offset of
  // buffer 0 plus an instruction immediate.  The last unmasked tile of an odd
  // run is taken as masked (the mask keeps all of it), so that both runs
  // start at an even position.
  const uint32_t lds0 = lds_addr(smem);
  const TileReads<D> ka0 = at<D>(ro, lds0), va0 = at<D>(ro, lds0 + TL::BYTES);
  const int n_int0 = CAUSAL ? min(ns, (tb + 1) / kBN) : T / kBN;
  const int n_int = n_int0 & ~1;
  int sq = 0;
  auto tile = [&](auto parity, auto maskc) __attribute__((always_inline)) {
    constexpr int P = decltype(parity)::value;
    constexpr bool MASK = decltype(maskc)::value != 0;
    publish_tile();
    if (sq + 1 < ns)
      dma_kv<D>(kb, vb, seq_range, key_bytes, Hk, sq + 1, smem + opaque_s((1 - P) * (2 * TL::BYTES)), wave, dm);
    const int kt0 = sq * kBN;
    ++sq;
    if (MASK && CAUSAL && kt0 > wt1) return;
    dq_tile<D, MASK, CAUSAL, P * 2 * TL::BYTES>(dqa, qf, df, ka0, va0, kt0, T, my_t, half, scale_log2, l2, dd);
  };
  using P0 = std::integral_constant<int, 0>;
  using P1 = std::integral_constant<int, 1>;
  using U = std::integral_constant<int, 0>;
  using M = std::integral_constant<int, 1>;
  dma_kv<D>(kb, vb, seq_range, key_bytes, Hk, 0, smem, wave, dm);
  while (sq + 1 < n_int) {  // unmasked tiles
    tile(P0(), U());
    tile(P1(), U());
  }
  while (sq + 1 < ns) {  // masked tiles
    tile(P0(), M());
    tile(P1(), M());
  }
  if (sq < ns) tile(P0(), M());

  if (row_ok) {
    uint16_t* orow = dq + qoff;
    const float* drow = dq_depth ? dq_depth + qoff : nullptr;
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
      for (int a = 0; a < 4; ++a) {
        const int d0 = dt * 32 + a * 8 + half * 4;
        f32x4 x = {dqa[dt][4 * a] * scale, dqa[dt][4 * a + 1] * scale, dqa[dt][4 * a + 2] * scale,
                   dqa[dt][4 * a + 3] * scale};
        if (drow) x += *reinterpret_cast<const f32x4*>(drow + d0);
        u32x2 w = {pack_bf16x2(x[0], x[1]), pack_bf16x2(x[2], x[3])};
        *reinterpret_cast<u32x2*>(orow + d0) = w;
      }
  }
}

// ---- 4. dk, dv over the sequence keys --------------------------------------------------

// Eight waves; waves w and w + 4 own the same 32 keys.  The P wave holds K^T
// of its keys and the dV^T accumulator: per 64-row tile it forms S = Q K^T,
// P = exp2(S*scale*log2e - lse2) (masked), writes P (bf16, in the register
// layout of its accumulators) to LDS, and adds dO^T P into dV^T.  The dS wave
// holds V^T and the dK^T accumulator: one tile later it forms dP = dO V^T,
// reads P back (the same lane's layout), forms dS = P (dP - Dsum) from that
// bf16 P (dS is rounded to bf16 for its product anyway), and adds Q^T dS
// into dK^T.  Each wave holds one key operand and one accumulator (96
// registers), so two waves share a SIMD; one barrier per tile publishes the
// next row tile and the P of the previous one.  Row tiles rotate through three
// stage buffers (tile i for the P waves, tile i-1 for the dS waves, tile i+1
// loading), P through three transfer slots.

// Direct-to-LDS staging of a 64-row tile of Q and dO (expanded rows: row
// t*G + g at token offset t, head g) plus the tile's 64 lse2 and Dsum values.
template <int D>
struct RowDma {
  uint32_t o[kNX<D>];
};

template <int D>
__device__ __forceinline__ void init_row_dma(RowDma<D>& o, int lane, int wave, int Hq, int lgG) {
  using TL = Tile<D>;
  constexpr int NX = kNX<D>;
#pragma unroll
  for (int x = 0; x < NX; ++x) {
    const int pr = (wave * NX + x) * TL::RPI + lane / TL::CH;
    const int pc = lane % TL::CH;
    const uint32_t row_bytes = static_cast<uint32_t>((pr >> lgG) * Hq + (pr & ((1 << lgG) - 1))) * D * 2;
    o.o[x] = row_bytes + ((pc ^ swz_u<D>(pr)) * 16);
  }
}

// A transposed A operand (two async reads) at a compile-time byte offset.
template <int D, int OFF>
__device__ __forceinline__ bf16x8 read_tr8(const TileReads<D>& ta, int dt) {
  const s16x4 lo4 = read_tr_async_at<OFF>(ta.lo[dt]);
  const s16x4 hi4 = read_tr_async_at<OFF>(ta.hi[dt]);
  return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo4, hi4, 0, 1, 2, 3, 4, 5, 6, 7));
}

template <int D>
struct XferSlot {
  static constexpr int PAIR = 4 * 1024;  // 16 dwords per lane: 4 chunks of 64 lanes x 16 bytes
  static constexpr int BYTES = 4 * PAIR;
};

// dO^T (P wave) or Q^T (dS wave) operands of one 32-row block, half h and d
// tile dt at tt[h * NT + dt], from the stage at `stage` + SRC (async reads).
template <int D, int J, int SRC>
__device__ __forceinline__ void fetch_tr_block(bf16x8 (&tt)[2 * (D / 32)], const TileReads<D>& ta) {
  using TL = Tile<D>;
  constexpr int NT = D / 32;
#pragma unroll
  for (int dt = 0; dt < NT; ++dt) {
    tt[dt] = read_tr8<D, SRC + (32 * J) * TL::ROW_BYTES>(ta, dt);
    tt[NT + dt] = read_tr8<D, SRC + (32 * J + 16) * TL::ROW_BYTES>(ta, dt);
  }
}

// LDS layout: the three stages' Q tiles, then their dO
// tiles, then their lse2 and Dsum rows, then the three transfer slots.  From a
// role's base every tile it reads (row-wise or transposed) lies within the
// 64 KiB reach of an instruction's immediate offset.
template <int D>
struct RowStages {
  static constexpr int TB = Tile<D>::BYTES;
  static constexpr int Q = 0;                      // + stage * TB
  static constexpr int DO = 3 * TB;                // + stage * TB
  static constexpr int ST = 6 * TB;                // + stage * SB: lse2[64], then Dsum[64]
  static constexpr int SB = 2 * kBN * 4;
  static constexpr int XF = ST + 3 * SB;           // + slot * XferSlot::BYTES
  static constexpr int BYTES = XF + 3 * XferSlot<D>::BYTES;
};

// Direct-to-LDS loads of row tile idx into stage r.
template <int D>
__device__ __forceinline__ void dma_rows(const uint16_t* qb, const uint16_t* ob, const float* l2b, const float* ddb,
                                          int T, int Hq, int lgG, int TG, int idx, lds_u8* smem, int r, int wave,
                                          int lane, const RowDma<D>& o) {
  using LY = RowStages<D>;
  constexpr int NX = kNX<D>;
  const int r0 = idx * kBN;
  const int t0 = r0 >> lgG;
  const int64_t first = static_cast<int64_t>(t0) * Hq * D;
  const uint32_t range = static_cast<uint32_t>((static_cast<int64_t>(T - 1 - t0) * Hq + (1 << lgG)) * D * 2);
  const __amdgpu_buffer_rsrc_t rq = make_rsrc(qb + first, range);
  const __amdgpu_buffer_rsrc_t ro = make_rsrc(ob + first, range);
  lds_u8* const qdst = smem + opaque_s(LY::Q + r * LY::TB + wave * NX * 1024);
  lds_u8* const odst = smem + opaque_s(LY::DO + r * LY::TB + wave * NX * 1024);
#pragma unroll
  for (int x = 0; x < NX; ++x) {
    const uint32_t off = o.o[x];
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rq, (lds_void_t*)(qdst + x * 1024), 16, off, 0, 0, 0);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(ro, (lds_void_t*)(odst + x * 1024), 16, off, 0, 0, 0);
  }
  if (wave < 2) {
    const float* src = (wave == 0 ? l2b : ddb) + r0;
    const uint32_t frange = static_cast<uint32_t>(TG - r0) * 4;
    const __amdgpu_buffer_rsrc_t rf =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<float*>(src), static_cast<short>(0), static_cast<int>(frange),
                                          kBufFlags);
    lds_u8* const sdst = smem + opaque_s(LY::ST + r * LY::SB + wave * kBN * 4);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rf, (lds_void_t*)sdst, 4, static_cast<uint32_t>(lane) * 4, 0, 0, 0);
  }
}

// P of one 32-row block from its scores: exp2(s * scale * log2e - lse2), masked.
template <int J, bool MASK>
__device__ __forceinline__ void p_weights(const f32x16& s, const f32x4 (&l2)[4], int r0, int lgG, int my_key,
                                          int half, float scale_log2, bf16x8 (&pb)[2]) {
  float p[16];
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      float x = fmaf(s[4 * a + c], scale_log2, -l2[a][c]);
      if (MASK) x = my_key <= ((r0 + 32 * J + 8 * a + 4 * half + c) >> lgG) ? x : -INFINITY;
      p[4 * a + c] = fast_exp2(x);
    }
  pack16(p, pb);
}

// dS = P (dP - Dsum) of one 32-row block, P as the P wave stored it (bf16).
__device__ __forceinline__ void ds_weights(const f32x16& dp, const f32x4 (&dd)[4], const u32x4 (&pw)[2],
                                           bf16x8 (&db)[2]) {
  float ds[16];
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const int i = 4 * a + c;
      const uint32_t w = pw[i >> 3][(i & 7) >> 1];
      const float pv = __builtin_bit_cast(float, (i & 1) ? (w & 0xffff0000u) : (w << 16));
      ds[i] = pv * (dp[i] - dd[a][c]);
    }
  pack16(ds, db);
}

// One row tile on the P side, its two 32-row blocks as a software pipeline:
// block 1's score products run beside block 0's weights, block 0's dV products
// beside block 1's weights.  ta holds row-wise read addresses into stage 0's
// Q tile and transposed ones into its dO tile; the tile's stage lies B bytes
// further in both, its lse2 row S bytes past stat0 and its transfer slot X
// bytes past xfer0 (all constants, so that every LDS address is a per-lane
// offset plus an instruction immediate).
template <int D, bool MASK, int B, int S, int X>
__device__ __forceinline__ void p_tile(f32x16 (&acc)[D / 32], const bf16x8 (&kf)[D / 16], const TileReads<D>& ta,
                                       uint32_t stat0, uint32_t xfer0, int r0, int lgG, int my_key, int half,
                                       float scale_log2) {
  constexpr int NT = D / 32;
  constexpr int RB = Tile<D>::ROW_BYTES;
  const uint32_t stat = stat0 + S, xfer = xfer0 + X;
  bf16x8 aq[D / 16], tt[2 * NT], pb0[2], pb1[2];
  f32x4 l2[4];
#pragma unroll
  for (int sl = 0; sl < D / 16; ++sl) aq[sl] = *lds_at<lds_bf16x8_t>(ta.nr[sl] + B);
#pragma unroll
  for (int a = 0; a < 4; ++a) l2[a] = *lds_at<lds_f32x4_t>(stat + (8 * a + 4 * half) * 4);
  __builtin_amdgcn_sched_barrier(0);
  f32x16 s0 = {}, s1 = {};
#pragma unroll
  for (int sl = 0; sl < D / 16; ++sl) s0 = mfma32(aq[sl], kf[sl], s0);
#pragma unroll
  for (int sl = 0; sl < D / 16; ++sl) aq[sl] = *lds_at<lds_bf16x8_t>(ta.nr[sl] + B + 32 * RB);
  fetch_tr_block<D, 0, B>(tt, ta);
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int sl = 0; sl < D / 16; ++sl) s1 = mfma32(aq[sl], kf[sl], s1);
  p_weights<0, MASK>(s0, l2, r0, lgG, my_key, half, scale_log2, pb0);
  interleave<D / 16, MASK ? 8 : 5>();
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int h = 0; h < 2; ++h) *lds_at<lds_bf16x8_t>(xfer + h * 1024) = pb0[h];
#pragma unroll
  for (int a = 0; a < 4; ++a) l2[a] = *lds_at<lds_f32x4_t>(stat + (32 + 8 * a + 4 * half) * 4);
  lds_ready(tt);
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int h = 0; h < 2; ++h)
#pragma unroll
    for (int dt = 0; dt < NT; ++dt) acc[dt] = mfma32(tt[h * NT + dt], pb0[h], acc[dt]);
  p_weights<1, MASK>(s1, l2, r0, lgG, my_key, half, scale_log2, pb1);
  interleave<2 * NT, MASK ? 8 : 5>();
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int h = 0; h < 2; ++h) *lds_at<lds_bf16x8_t>(xfer + (2 + h) * 1024) = pb1[h];
  fetch_tr_block<D, 1, B>(tt, ta);
  lds_ready(tt);
#pragma unroll
  for (int h = 0; h < 2; ++h)
#pragma unroll
    for (int dt = 0; dt < NT; ++dt) acc[dt] = mfma32(tt[h * NT + dt], pb1[h], acc[dt]);
}

// One row tile on the dS side, pipelined like p_tile.  ta holds row-wise read
// addresses into stage 0's dO tile and transposed ones into its Q tile; B, S
// and X as in p_tile (S addresses the tile's lse2 row, Dsum follows it).
template <int D, int B, int S, int X>
__device__ __forceinline__ void ds_tile(f32x16 (&acc)[D / 32], const bf16x8 (&vf)[D / 16], const TileReads<D>& ta,
                                        uint32_t stat0, uint32_t xfer0, int half) {
  constexpr int NT = D / 32;
  constexpr int RB = Tile<D>::ROW_BYTES;
  const uint32_t stat = stat0 + S + kBN * 4, xfer = xfer0 + X;
  bf16x8 ao[D / 16], tt[2 * NT], db0[2], db1[2];
  f32x4 dd[4];
  u32x4 pw[2];
#pragma unroll
  for (int sl = 0; sl < D / 16; ++sl) ao[sl] = *lds_at<lds_bf16x8_t>(ta.nr[sl] + B);
#pragma unroll
  for (int a = 0; a < 4; ++a) dd[a] = *lds_at<lds_f32x4_t>(stat + (8 * a + 4 * half) * 4);
#pragma unroll
  for (int h = 0; h < 2; ++h) pw[h] = *lds_at<lds_u32x4_t>(xfer + h * 1024);
  __builtin_amdgcn_sched_barrier(0);
  f32x16 dp0 = {}, dp1 = {};
#pragma unroll
  for (int sl = 0; sl < D / 16; ++sl) dp0 = mfma32(ao[sl], vf[sl], dp0);
#pragma unroll
  for (int sl = 0; sl < D / 16; ++sl) ao[sl] = *lds_at<lds_bf16x8_t>(ta.nr[sl] + B + 32 * RB);
  fetch_tr_block<D, 0, B>(tt, ta);
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int sl = 0; sl < D / 16; ++sl) dp1 = mfma32(ao[sl], vf[sl], dp1);
  ds_weights(dp0, dd, pw, db0);
  interleave<D / 16, 7>();
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int a = 0; a < 4; ++a) dd[a] = *lds_at<lds_f32x4_t>(stat + (32 + 8 * a + 4 * half) * 4);
#pragma unroll
  for (int h = 0; h < 2; ++h) pw[h] = *lds_at<lds_u32x4_t>(xfer + (2 + h) * 1024);
  lds_ready(tt);
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int h = 0; h < 2; ++h)
#pragma unroll
    for (int dt = 0; dt < NT; ++dt) acc[dt] = mfma32(tt[h * NT + dt], db0[h], acc[dt]);
  ds_weights(dp1, dd, pw, db1);
  interleave<2 * NT, 7>();
  __builtin_amdgcn_sched_barrier(0);
  fetch_tr_block<D, 1, B>(tt, ta);
  lds_ready(tt);
#pragma unroll
  for (int h = 0; h < 2; ++h)
#pragma unroll
    for (int dt = 0; dt < NT; ++dt) acc[dt] = mfma32(tt[h * NT + dt], db1[h], acc[dt]);
}

constexpr int kKvWaves = 8;
constexpr int kKvThreads = kKvWaves * 64;

template <int D, bool CAUSAL>
__global__ __launch_bounds__(kKvThreads) __attribute__((amdgpu_waves_per_eu(2, 2))) void moda_bwd_dkv_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
    const uint16_t* __restrict__ dout, const float* __restrict__ ws_l2, const float* __restrict__ ws_dd, int B, int T,
    int Hq, int Hk, int lgG, float scale, float scale_log2, uint16_t* __restrict__ dk, uint16_t* __restrict__ dv) {
  using LY = RowStages<D>;
  using XS = XferSlot<D>;
  __shared__ __attribute__((aligned(1024))) uint8_t smem_raw[LY::BYTES];
  lds_u8* const smem = (lds_u8*)smem_raw;

  const int G = 1 << lgG;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const bool p_role = wave < 4;
  const int pair = wave & 3;
  const int half = lane >> 5;
  const int nbh = B * Hk;
  const int kb = blockIdx.x / nbh;  // key block; causal: the heaviest (first) blocks go first
  const int bh = blockIdx.x % nbh;
  const int b = bh / Hk, hk = bh % Hk;
  const int k0 = kb * kKB;
  const int kw0 = k0 + pair * 32;
  const int my_key = kw0 + (lane & 31);
  const int TG = T << lgG;

  // K^T (P wave) or V^T (dS wave) fragments: lane holds key my_key, d = 16*sl + 8*half + [0, 8).
  const int64_t koff = ((static_cast<int64_t>(b) * T + my_key) * Hk + hk) * D;
  const uint16_t* src = p_role ? k : v;
  bf16x8 frag[D / 16];
#pragma unroll
  for (int sl = 0; sl < D / 16; ++sl) {
    u32x4 a = {0u, 0u, 0u, 0u};
    if (my_key < T) a = *reinterpret_cast<const u32x4*>(src + koff + sl * 16 + half * 8);
    frag[sl] = __builtin_bit_cast(bf16x8, a);
  }

  const uint16_t* qb = q + (static_cast<int64_t>(b) * T * Hq + hk * G) * D;
  const uint16_t* ob = dout + (static_cast<int64_t>(b) * T * Hq + hk * G) * D;
  const float* l2b = ws_l2 + (static_cast<int64_t>(b) * Hk + hk) * TG;
  const float* ddb = ws_dd + (static_cast<int64_t>(b) * Hk + hk) * TG;
  RowDma<D> dm;
  init_row_dma<D>(dm, lane, pair, Hq, lgG);
  TileReads<D> ro;
  init_reads<D>(ro, lane);

  f32x16 acc[D / 32];
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt) acc[dt] = f32x16{};

  const int nt = (TG + kBN - 1) / kBN;
  const int i0 = CAUSAL ? (k0 << lgG) / kBN : 0;
  const int i_m = CAUSAL ? min(nt, (((k0 + kKB - 1) << lgG) + kBN - 1) / kBN) : i0;
  const uint32_t lds0 = lds_addr(smem);
  // Stage-0 read addresses: the P side reads Q row-wise and dO transposed, the
  // dS side dO row-wise and Q transposed.
  TileReads<D> ra;
  {
    const uint32_t rowb = lds0 + (p_role ? LY::Q : LY::DO), trb = lds0 + (p_role ? LY::DO : LY::Q);
#pragma unroll
    for (int sl = 0; sl < D / 16; ++sl) ra.nr[sl] = rowb + ro.nr[sl];
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt) {
      ra.lo[dt] = trb + ro.lo[dt];
      ra.hi[dt] = trb + ro.hi[dt];
    }
  }
  const uint32_t stat0 = lds0 + LY::ST;
  const uint32_t xfer0 = lds0 + static_cast<uint32_t>(LY::XF + pair * XS::PAIR) + static_cast<uint32_t>(lane) * 16;
  // No row of tile it sees the pair's keys.
  auto skip = [&](int it) __attribute__((always_inline)) { return CAUSAL && ((it * kBN + kBN - 1) >> lgG) < kw0; };

  // Row tiles are taken last to first, so every workgroup starts at the same
  // tile and the workgroups that run side by side on one XCD (the same
  // (b, hk)) read the same Q/dO rows at about the same time.  Step u
  // (u = 0 .. nt - i0) publishes tile nt - 1 - u, starts loading the next
  // one, lets the P waves work on tile nt - 1 - u and the dS waves on tile
  // nt - u.  The tile of step u lives in stage and slot u % 3; the steps are
  // unrolled by three so that the residue, and with it every LDS offset, is a
  // constant.  The unmasked steps are rounded down to a multiple of three and
  // the rest run masked (the mask is exact on any tile, so the extra masked
  // steps only cost a select).
  using IC0 = std::integral_constant<int, 0>;
  using IC1 = std::integral_constant<int, 1>;
  using IC2 = std::integral_constant<int, 2>;
  const int n_it = nt - i0 + 1;
  const int n_unm = CAUSAL ? (nt - i_m) / 3 * 3 : n_it;
  auto p_step = [&](auto res, auto maskc, int u) __attribute__((always_inline)) {
    constexpr int R = decltype(res)::value;
    constexpr bool MASK = decltype(maskc)::value != 0;
    const int it = nt - 1 - u;
    publish_tile();
    if (it - 1 >= i0) dma_rows<D>(qb, ob, l2b, ddb, T, Hq, lgG, TG, it - 1, smem, (R + 1) % 3, pair, lane, dm);
    if (it < i0 || skip(it)) return;
    p_tile<D, MASK, R * LY::TB, R * LY::SB, R * XS::BYTES>(acc, frag, ra, stat0, xfer0, it * kBN, lgG, my_key, half,
                                                           scale_log2);
  };
  auto ds_step = [&](auto res, auto maskc, int u) __attribute__((always_inline)) {
    constexpr int R = (decltype(res)::value + 2) % 3;  // the previous tile's stage and slot
    publish_tile();
    const int jt = nt - u;
    if (u == 0 || skip(jt)) return;
    ds_tile<D, R * LY::TB, R * LY::SB, R * XS::BYTES>(acc, frag, ra, stat0, xfer0, half);
  };
  // Steps [u, end) in threes, then at most two more (u % 3 == 0 on entry).
  auto run = [&](auto step, auto maskc, int& u, int end) __attribute__((always_inline)) {
    for (; u + 2 < end; u += 3) {
      step(IC0(), maskc, u);
      step(IC1(), maskc, u + 1);
      step(IC2(), maskc, u + 2);
    }
    if (u < end) step(IC0(), maskc, u++);
    if (u < end) step(IC1(), maskc, u++);
  };

  if (p_role && i0 < nt) dma_rows<D>(qb, ob, l2b, ddb, T, Hq, lgG, TG, nt - 1, smem, 0, pair, lane, dm);
  int u = 0;
  if (p_role) {
    run(p_step, IC0(), u, n_unm);
    run(p_step, IC1(), u, n_it);
  } else {
    run(ds_step, IC0(), u, n_unm);
    run(ds_step, IC1(), u, n_it);
  }

  if (my_key < T) {
    uint16_t* row = (p_role ? dv : dk) + koff;
    const float f = p_role ? 1.0f : scale;
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
      for (int a = 0; a < 4; ++a) {
        const int d0 = dt * 32 + a * 8 + half * 4;
        u32x2 w = {pack_bf16x2(acc[dt][4 * a] * f, acc[dt][4 * a + 1] * f),
                   pack_bf16x2(acc[dt][4 * a + 2] * f, acc[dt][4 * a + 3] * f)};
        *reinterpret_cast<u32x2*>(row + d0) = w;
      }
  }
}

// ---- host side ----------------------------------------------------------------------------

struct BwdLayout {
  size_t l2, dd, dqd, total;
};

size_t align256(size_t x) { return (x + 255) & ~static_cast<size_t>(255); }

BwdLayout bwd_layout(int B, int T, int Hq, int d, int L) {
  BwdLayout w;
  const size_t rows = static_cast<size_t>(B) * T * Hq;
  w.l2 = 0;
  w.dd = align256(rows * 4);
  w.dqd = w.dd + align256(rows * 4);
  w.total = w.dqd + (L > 0 ? align256(rows * d * 4) : 0);
  return w;
}

constexpr int kDepthBlocks = 4096;  // workgroups of the depth launch (each wave strides over units)

template <int D>
hipError_t launch_bwd_d(const BwdArgs& a) {
  const int G = a.Hq / a.Hk;
  const int lgG = __builtin_ctz(G);
  const int TG = a.T * G;
  const hipStream_t st = static_cast<hipStream_t>(a.stream);
  const BwdLayout w = bwd_layout(a.B, a.T, a.Hq, D, a.L);
  uint8_t* ws = static_cast<uint8_t*>(a.workspace);
  float* l2 = reinterpret_cast<float*>(ws + w.l2);
  float* dd = reinterpret_cast<float*>(ws + w.dd);
  float* dqd = a.L > 0 ? reinterpret_cast<float*>(ws + w.dqd) : nullptr;
  const float scale = 1.0f / sqrtf(static_cast<float>(D));
  const float scale_log2 = kLog2e * scale;
  const uint16_t* q = static_cast<const uint16_t*>(a.q);
  const uint16_t* k = static_cast<const uint16_t*>(a.k);
  const uint16_t* v = static_cast<const uint16_t*>(a.v);
  const uint16_t* dout = static_cast<const uint16_t*>(a.dout);

  const int64_t rows = static_cast<int64_t>(a.B) * a.T * a.Hq;
  const int64_t rows_per_block = 256 / (D / 8);
  hipLaunchKernelGGL((moda_bwd_rows_kernel<D>), dim3(static_cast<unsigned>((rows + rows_per_block - 1) / rows_per_block)),
                     dim3(256), 0, st, static_cast<const uint16_t*>(a.out), dout, a.lse, rows, a.T, a.Hq, a.Hk, lgG, l2,
                     dd);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;

  if (a.L > 0) {
    const int64_t units = static_cast<int64_t>(a.B) * a.T * a.Hk;
    const int64_t blocks = std::min<int64_t>((units + kWaves - 1) / kWaves, kDepthBlocks);
    if (G <= 16)
      hipLaunchKernelGGL((moda_bwd_depth_kernel<D, 1>), dim3(static_cast<unsigned>(blocks)), dim3(kThreads), 0, st, q,
                         dout, static_cast<const uint16_t*>(a.kd), static_cast<const uint16_t*>(a.vd), l2, dd, a.T,
                         a.Hq, a.Hk, a.L, lgG, units, scale, scale_log2, dqd, static_cast<uint16_t*>(a.dkd),
                         static_cast<uint16_t*>(a.dvd));
    else
      hipLaunchKernelGGL((moda_bwd_depth_kernel<D, 2>), dim3(static_cast<unsigned>(blocks)), dim3(kThreads), 0, st, q,
                         dout, static_cast<const uint16_t*>(a.kd), static_cast<const uint16_t*>(a.vd), l2, dd, a.T,
                         a.Hq, a.Hk, a.L, lgG, units, scale, scale_log2, dqd, static_cast<uint16_t*>(a.dkd),
                         static_cast<uint16_t*>(a.dvd));
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }

  const int nrb = (TG + kBM - 1) / kBM;
  const unsigned dq_blocks = static_cast<unsigned>(static_cast<int64_t>(nrb) * a.B * a.Hk);
  if (a.causal)
    hipLaunchKernelGGL((moda_bwd_dq_kernel<D, true>), dim3(dq_blocks), dim3(kThreads), 0, st, q, k, v, dout, l2, dd,
                       dqd, a.B, a.T, a.Hq, a.Hk, lgG, nrb, scale, scale_log2, static_cast<uint16_t*>(a.dq));
  else
    hipLaunchKernelGGL((moda_bwd_dq_kernel<D, false>), dim3(dq_blocks), dim3(kThreads), 0, st, q, k, v, dout, l2, dd,
                       dqd, a.B, a.T, a.Hq, a.Hk, lgG, nrb, scale, scale_log2, static_cast<uint16_t*>(a.dq));
  e = hipGetLastError();
  if (e != hipSuccess) return e;

  const int nkb = (a.T + kKB - 1) / kKB;
  const unsigned kv_blocks = static_cast<unsigned>(static_cast<int64_t>(nkb) * a.B * a.Hk);
  if (a.causal)
    hipLaunchKernelGGL((moda_bwd_dkv_kernel<D, true>), dim3(kv_blocks), dim3(kKvThreads), 0, st, q, k, v, dout, l2, dd,
                       a.B, a.T, a.Hq, a.Hk, lgG, scale, scale_log2, static_cast<uint16_t*>(a.dk),
                       static_cast<uint16_t*>(a.dv));
  else
    hipLaunchKernelGGL((moda_bwd_dkv_kernel<D, false>), dim3(kv_blocks), dim3(kKvThreads), 0, st, q, k, v, dout, l2, dd,
                       a.B, a.T, a.Hq, a.Hk, lgG, scale, scale_log2, static_cast<uint16_t*>(a.dk),
                       static_cast<uint16_t*>(a.dv));
  return hipGetLastError();
}

}  // namespace

size_t bwd_workspace_bytes(int B, int T, int Hq, int d, int L) { return bwd_layout(B, T, Hq, d, L).total; }

int64_t bwd_grid_blocks(int B, int T, int Hq, int Hk) {
  const int64_t TG = static_cast<int64_t>(T) * (Hq / Hk);
  const int64_t dq = (TG + kBM - 1) / kBM * B * Hk;
  const int64_t kv = (static_cast<int64_t>(T) + kKB - 1) / kKB * B * Hk;
  const int64_t rows = (static_cast<int64_t>(B) * T * Hq + 15) / 16;
  return std::max(std::max(dq, kv), rows);
}

hipError_t launch_bwd_bf16(const BwdArgs& a) { return a.d == 64 ? launch_bwd_d<64>(a) : launch_bwd_d<128>(a); }

}  // namespace moda
