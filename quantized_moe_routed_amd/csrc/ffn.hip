// Expert FFN on fp16 matrix cores, for tiles of up to 16 routed slots of one
// expert (decode-size batches, and every batch until the large-tile kernel
// takes the heavy experts).
//
// A workgroup owns one tile (16 slots of one expert) and 16*NT output
// columns; its 4 waves split the contraction: wave w takes the code units
// w, w+4, w+8, ... of the rows (a unit is 8 blocks of Q2SM or 2 blocks of
// Q8_0, 64 bytes per row) and the m-term chunks w, w+4, ... of 32 blocks.
// Per block each wave issues one v_mfma_f32_16x16x32_f16 per output tile (two
// when the activation carries a lo plane), with the weights' codes as exact
// small fp16 integers (fmt.h), and folds the block scale in fp32:
//     acc += (2^-6 d_b) * P_b.
// The m-term sum_b m_b (sigma S_b) of 2-bit blocks is accumulated by the
// matrix cores over the block index.  The four partial sums are then added in wave order through
// LDS, so the result does not depend on scheduling; no atomics.
//
// gate/up: h = silu(g) * u for every (slot, column) of the tile, written as
// the down projection's operand (fp16 hi/lo, in its code order, row scale
// 2^-6) together with the block sums of h.
// down:    y_slot[slot][col] = the down projection of h.
#include "device.h"
#include "fmt.h"
#include "launch.h"

namespace moe {

constexpr int kFfnThreads = 256;
constexpr int kFfnWaves = 4;

template <int FG, int NT, bool LO>
__global__ __launch_bounds__(kFfnThreads) void ffn_gateup_kernel(
    const uint16_t* __restrict__ xq_hi, const uint16_t* __restrict__ xq_lo, const uint16_t* __restrict__ sq_hi,
    const uint16_t* __restrict__ sq_lo, const float* __restrict__ sigma, int H, int I, int k, int nb32H, QMat gate,
    QMat up, const int32_t* __restrict__ slot_list, const int4* __restrict__ tiles,
    const int32_t* __restrict__ n_tiles, int fd, uint16_t* __restrict__ h_hi, uint16_t* __restrict__ h_lo,
    uint16_t* __restrict__ hs_hi, uint16_t* __restrict__ hs_lo, int nb32I) {
  const int tile = blockIdx.y;
  if (tile >= *n_tiles) return;
  __shared__ float red[kFfnWaves][NT][2][4][kWave];
  __shared__ float hbuf[16][16 * NT + 1];
  __shared__ float s_sig[16];

  const int4 tl = tiles[tile];
  const int le = tl.x, p0 = tl.y, rows = tl.z;
  const int n0 = blockIdx.x * 16 * NT;
  const int tid = threadIdx.x, lane = tid % kWave, wave = tid / kWave;
  const int c16 = lane & 15, g = lane >> 4;
  const int nb = H / 32;
  constexpr int UB = Codes<FG>::kUnitBlocks;
  const int n_units = (nb + UB - 1) / UB;
  const int64_t rbytes = Codes<FG>::row_bytes(H);

  const bool mvalid = c16 < rows;
  const int tok = mvalid ? slot_list[p0 + c16] / k : 0;
  const uint16_t* ah = xq_hi + (int64_t)tok * H + 8 * g;
  const uint16_t* al = LO ? xq_lo + (int64_t)tok * H + 8 * g : nullptr;
  if (tid < 16) s_sig[tid] = tid < rows ? sigma[slot_list[p0 + tid] / k] : 1.0f;

  const uint8_t* cp[NT][2];
  int64_t srow[NT][2];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    const int64_t row = (int64_t)le * I + n0 + 16 * nt + c16;
    cp[nt][0] = reinterpret_cast<const uint8_t*>(gate.codes) + row * rbytes + 16 * g;
    cp[nt][1] = reinterpret_cast<const uint8_t*>(up.codes) + row * rbytes + 16 * g;
    srow[nt][0] = srow[nt][1] = row * nb;
  }
  const f32x4_t zero4 = {0.0f, 0.0f, 0.0f, 0.0f};
  f32x4_t acc[NT][2], accm[NT][2];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt)
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) acc[nt][mt] = accm[nt][mt] = zero4;

  for (int u = wave; u < n_units; u += kFfnWaves) {
    uint4 cw[NT][2];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      cw[nt][0] = *reinterpret_cast<const uint4*>(cp[nt][0] + (int64_t)u * 64);
      cw[nt][1] = *reinterpret_cast<const uint4*>(cp[nt][1] + (int64_t)u * 64);
    }
#pragma unroll
    for (int i = 0; i < UB; ++i) {
      const int b = u * UB + i;
      if (b >= nb) break;
      const uint4 zero = make_uint4(0u, 0u, 0u, 0u);
      const uint4 a_hi = mvalid ? *reinterpret_cast<const uint4*>(ah + 32 * b) : zero;
      uint4 a_lo = zero;
      if (LO) a_lo = mvalid ? *reinterpret_cast<const uint4*>(al + 32 * b) : zero;
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
#pragma unroll
        for (int mt = 0; mt < 2; ++mt) {
          const uint4 bf = Codes<FG>::frag(cw[nt][mt], i);
          f32x4_t p = mfma16(a_hi, bf, zero4);
          if (LO) p = mfma16(a_lo, bf, p);
          const float d = Codes<FG>::d(mt ? up.scales : gate.scales, srow[nt][mt] + b) * kScaleD;
#pragma unroll
          for (int r = 0; r < 4; ++r) acc[nt][mt][r] = fmaf(d, p[r], acc[nt][mt][r]);
        }
      }
    }
  }
  // m-term over the block index, 32 blocks per product
  const int n_mc = Codes<FG>::kHasM ? (nb + 31) / 32 : 0;
  for (int c = wave; c < n_mc; c += kFfnWaves) {
    const uint4 zero = make_uint4(0u, 0u, 0u, 0u);
    const int64_t so = (int64_t)tok * nb32H + 32 * c + 8 * g;
    const uint4 s_hi = mvalid ? *reinterpret_cast<const uint4*>(sq_hi + so) : zero;
    const uint4 s_lo = mvalid ? *reinterpret_cast<const uint4*>(sq_lo + so) : zero;
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
#pragma unroll
      for (int mt = 0; mt < 2; ++mt) {
        const uint4 bm = m_frag<FG>(mt ? up.scales : gate.scales, srow[nt][mt], 32 * c + 8 * g, nb);
        accm[nt][mt] = mfma16(s_hi, bm, accm[nt][mt]);
        accm[nt][mt] = mfma16(s_lo, bm, accm[nt][mt]);
      }
    }
  }
#pragma unroll
  for (int nt = 0; nt < NT; ++nt)
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
      for (int r = 0; r < 4; ++r) red[wave][nt][mt][r][lane] = acc[nt][mt][r] + accm[nt][mt][r];
  __syncthreads();

  // partial sums in wave order; thread tid owns element (r, lane) of every output tile
  {
    const int r = tid / kWave, l = tid % kWave;
    const int m = 4 * (l >> 4) + r;
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      float gs = red[0][nt][0][r][l], us = red[0][nt][1][r][l];
#pragma unroll
      for (int w = 1; w < kFfnWaves; ++w) {
        gs += red[w][nt][0][r][l];
        us += red[w][nt][1][r][l];
      }
      const int cl = 16 * nt + (l & 15);
      float h = 0.0f;
      if (m < rows) {
        const float inv = 1.0f / s_sig[m];   // a power of two: exact
        h = silu(gs * inv) * (us * inv);
        const int col = n0 + cl;
        const int blk = col >> 5, kk = col & 31, gg = kk >> 3;
        const int e = elem_of_rt(fd, kk & 7);
        const float hv = h * ldexpf(1.0f, -pos_rt(fd, e));   // kSigmaH * 2^(6 - pos)
        uint32_t hi, lo;
        split_f16(hv, hi, lo);
        const int64_t at = (int64_t)(p0 + m) * I + 32 * blk + 8 * gg + e;
        h_hi[at] = (uint16_t)hi;
        h_lo[at] = (uint16_t)lo;
      }
      hbuf[m][cl] = h;
    }
  }
  __syncthreads();
  // block sums of h for the NT/2 blocks of this tile (index order), and zero padding
  if (tid < 16 * (NT / 2)) {
    const int m = tid % 16, blk = tid / 16;
    if (m < rows) {
      float s = 0.0f;
      for (int i = 0; i < 32; ++i) s += hbuf[m][32 * blk + i];
      uint32_t hi, lo;
      split_f16(s * kSigmaH, hi, lo);
      const int64_t at = (int64_t)(p0 + m) * nb32I + n0 / 32 + blk;
      hs_hi[at] = (uint16_t)hi;
      hs_lo[at] = (uint16_t)lo;
    }
  }
  if (blockIdx.x == 0) {
    const int nbI = I / 32;
    for (int j = tid; j < 16 * (nb32I - nbI); j += kFfnThreads) {
      const int m = j % 16, b = nbI + j / 16;
      if (m < rows) {
        hs_hi[(int64_t)(p0 + m) * nb32I + b] = 0;
        hs_lo[(int64_t)(p0 + m) * nb32I + b] = 0;
      }
    }
  }
}

template <int FD, int NT>
__global__ __launch_bounds__(kFfnThreads) void ffn_down_kernel(
    const uint16_t* __restrict__ h_hi, const uint16_t* __restrict__ h_lo, const uint16_t* __restrict__ hs_hi,
    const uint16_t* __restrict__ hs_lo, int H, int I, int nb32I, QMat down, const int32_t* __restrict__ slot_list,
    const int4* __restrict__ tiles, const int32_t* __restrict__ n_tiles, float* __restrict__ y) {
  const int tile = blockIdx.y;
  if (tile >= *n_tiles) return;
  __shared__ float red[kFfnWaves][NT][4][kWave];

  const int4 tl = tiles[tile];
  const int le = tl.x, p0 = tl.y, rows = tl.z;
  const int n0 = blockIdx.x * 16 * NT;
  const int tid = threadIdx.x, lane = tid % kWave, wave = tid / kWave;
  const int c16 = lane & 15, g = lane >> 4;
  const int nb = I / 32;
  constexpr int UB = Codes<FD>::kUnitBlocks;
  const int n_units = (nb + UB - 1) / UB;
  const int64_t rbytes = Codes<FD>::row_bytes(I);

  const bool mvalid = c16 < rows;
  const uint16_t* ah = h_hi + (int64_t)(p0 + (mvalid ? c16 : 0)) * I + 8 * g;
  const uint16_t* al = h_lo + (int64_t)(p0 + (mvalid ? c16 : 0)) * I + 8 * g;

  const uint8_t* cp[NT];
  int64_t srow[NT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    const int64_t row = (int64_t)le * H + n0 + 16 * nt + c16;
    cp[nt] = reinterpret_cast<const uint8_t*>(down.codes) + row * rbytes + 16 * g;
    srow[nt] = row * nb;
  }
  const f32x4_t zero4 = {0.0f, 0.0f, 0.0f, 0.0f};
  f32x4_t acc[NT], accm[NT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) acc[nt] = accm[nt] = zero4;

  for (int u = wave; u < n_units; u += kFfnWaves) {
    uint4 cw[NT];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) cw[nt] = *reinterpret_cast<const uint4*>(cp[nt] + (int64_t)u * 64);
#pragma unroll
    for (int i = 0; i < UB; ++i) {
      const int b = u * UB + i;
      if (b >= nb) break;
      const uint4 zero = make_uint4(0u, 0u, 0u, 0u);
      const uint4 a_hi = mvalid ? *reinterpret_cast<const uint4*>(ah + 32 * b) : zero;
      const uint4 a_lo = mvalid ? *reinterpret_cast<const uint4*>(al + 32 * b) : zero;
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        const uint4 bf = Codes<FD>::frag(cw[nt], i);
        f32x4_t p = mfma16(a_hi, bf, zero4);
        p = mfma16(a_lo, bf, p);
        const float d = Codes<FD>::d(down.scales, srow[nt] + b) * kScaleD;
#pragma unroll
        for (int r = 0; r < 4; ++r) acc[nt][r] = fmaf(d, p[r], acc[nt][r]);
      }
    }
  }
  const int n_mc = Codes<FD>::kHasM ? (nb + 31) / 32 : 0;
  for (int c = wave; c < n_mc; c += kFfnWaves) {
    const uint4 zero = make_uint4(0u, 0u, 0u, 0u);
    const int64_t so = (int64_t)(p0 + (mvalid ? c16 : 0)) * nb32I + 32 * c + 8 * g;
    const uint4 s_hi = mvalid ? *reinterpret_cast<const uint4*>(hs_hi + so) : zero;
    const uint4 s_lo = mvalid ? *reinterpret_cast<const uint4*>(hs_lo + so) : zero;
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      const uint4 bm = m_frag<FD>(down.scales, srow[nt], 32 * c + 8 * g, nb);
      accm[nt] = mfma16(s_hi, bm, accm[nt]);
      accm[nt] = mfma16(s_lo, bm, accm[nt]);
    }
  }
#pragma unroll
  for (int nt = 0; nt < NT; ++nt)
#pragma unroll
    for (int r = 0; r < 4; ++r) red[wave][nt][r][lane] = acc[nt][r] + accm[nt][r];
  __syncthreads();
  {
    const int r = tid / kWave, l = tid % kWave;
    const int m = 4 * (l >> 4) + r;
    if (m < rows) {
      const int64_t slot = slot_list[p0 + m];
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        float v = red[0][nt][r][l];
#pragma unroll
        for (int w = 1; w < kFfnWaves; ++w) v += red[w][nt][r][l];
        y[slot * H + n0 + 16 * nt + (l & 15)] = v * (1.0f / kSigmaH);
      }
    }
  }
}

template <int FG, int NT, bool LO>
static void launch_gateup_t(dim3 grid, const FfnArgs& a, hipStream_t s) {
  ffn_gateup_kernel<FG, NT, LO><<<grid, kFfnThreads, 0, s>>>(
      a.xq_hi, a.xq_lo, a.sq_hi, a.sq_lo, a.sigma, a.H, a.I, a.k, a.nb32H, a.gate, a.up, a.slot_list, a.tiles,
      a.n_tiles, a.fd, a.h_hi, a.h_lo, a.hs_hi, a.hs_lo, a.nb32I);
}

template <int FD, int NT>
static void launch_down_t(dim3 grid, const FfnArgs& a, hipStream_t s) {
  ffn_down_kernel<FD, NT><<<grid, kFfnThreads, 0, s>>>(a.h_hi, a.h_lo, a.hs_hi, a.hs_lo, a.H, a.I, a.nb32I, a.down,
                                                      a.slot_list, a.tiles, a.n_tiles, a.y);
}

hipError_t launch_ffn_small(const FfnArgs& a, int nt_cols, hipStream_t s) {
  const bool lo = a.xq_lo != nullptr;
  hipError_t err;
  trace_pre("ffn_gateup", s);
  {
    const dim3 grid(a.I / (16 * nt_cols), a.max_tiles);
#define MOE_GU(F, N)                                      \
  if (lo) launch_gateup_t<F, N, true>(grid, a, s);        \
  else launch_gateup_t<F, N, false>(grid, a, s)
    if (a.fg == FMT_Q2SM) {
      if (nt_cols == 2) { MOE_GU(FMT_Q2SM, 2); } else { MOE_GU(FMT_Q2SM, 4); }
    } else {
      if (nt_cols == 2) { MOE_GU(FMT_Q8_0, 2); } else { MOE_GU(FMT_Q8_0, 4); }
    }
#undef MOE_GU
  }
  trace_post("ffn_gateup", s);
  if ((err = hipGetLastError()) != hipSuccess) return err;
  trace_pre("ffn_down", s);
  {
    const dim3 grid(a.H / (16 * nt_cols), a.max_tiles);
    if (a.fd == FMT_Q2SM) {
      if (nt_cols == 2) launch_down_t<FMT_Q2SM, 2>(grid, a, s);
      else launch_down_t<FMT_Q2SM, 4>(grid, a, s);
    } else {
      if (nt_cols == 2) launch_down_t<FMT_Q8_0, 2>(grid, a, s);
      else launch_down_t<FMT_Q8_0, 4>(grid, a, s);
    }
  }
  trace_post("ffn_down", s);
  return hipGetLastError();
}

}  // namespace moe
