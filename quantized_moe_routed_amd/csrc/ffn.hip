// Expert FFN on fp16 matrix cores, for tiles of up to 4 routed slots of one
// expert (decode-size batches, and every batch until the large-tile kernel
// takes the heavy experts).
//
// A workgroup owns one tile (up to 4 slots of one expert) and 32 output
// columns; its 8 waves split the contraction: wave w takes a contiguous
// range of the code units of the rows (a unit is 8 blocks of Q2SM or 2 blocks
// of Q8_0: 64 bytes of codes per row) and the m-term chunks w, w+8, ... of 32
// blocks.  A wave issues the code and scale loads of several units at once,
// the first of them before anything else, so a workgroup keeps tens of
// kilobytes in flight; the tile's activation rows are staged in LDS once, so
// the inner loop reads no activations from memory.  Per block each wave issues one
// v_mfma_f32_16x16x32_f16 per output tile (two when the activation carries a
// lo plane), with the weights' codes as exact small fp16 integers (fmt.h),
// and folds the block scale in fp32:
//     acc += (2^-6 d_b) * P_b.
// The m-term sum_b m_b (sigma S_b) of 2-bit blocks is accumulated by the
// matrix cores over the block index.  The eight partial sums are then added in
// wave order through LDS, so the result does not depend on scheduling; no
// atomics.
//
// gate/up: h = silu(g) * u for every (slot, column) of the tile, written as
// the down projection's operand (fp16 hi/lo, in its code order, row scale
// 2^-6) together with the block sums of h.
// down:    y_slot[slot][col] = the down projection of h.
#include "device.h"
#include "fmt.h"
#include "launch.h"

namespace moe {

constexpr int kFfnThreads = 512;
constexpr int kFfnWaves = kFfnThreads / 64;
constexpr int kNT = 2;            // 16-column output tiles per workgroup
constexpr int kStageRows = 4;     // slots per tile; their activation rows are staged in LDS

enum { MODE_GATEUP = 0, MODE_DOWN = 1 };

struct FfnTileArgs {
  const uint16_t *a_hi, *a_lo;      // activation operand planes, row stride K
  const uint16_t *s_hi, *s_lo;      // block-sum planes, row stride nb32
  const float* sigma;               // per-token row scale (gate/up); NULL: kSigmaH (down)
  int K, N, nb32, k;
  QMat w0, w1;                      // gate, up (gate/up) or down (w0 only)
  const int32_t* slot_list;
  const int4* tiles;
  const int32_t* n_tiles;
  int fd, I, nb32I;                 // gate/up: down format, I, padded block count of h
  int stage_rows;                   // rows of the LDS staging area: min(kStageRows, T)
  FragConsts kc;
  uint16_t *h_hi, *h_lo, *hs_hi, *hs_lo;
  float* y;
};

template <int F>
__device__ __forceinline__ uint4 load_d(const uint8_t* srow, int u) {
  if constexpr (F == FMT_Q2SM) {
    return *reinterpret_cast<const uint4*>(srow + 16 * (int64_t)u);
  } else {
    return make_uint4(*reinterpret_cast<const uint32_t*>(srow + 4 * (int64_t)u), 0u, 0u, 0u);
  }
}

template <int F>
__device__ __forceinline__ float d_of(const uint4& dw, int i) {
  uint32_t w;
  if constexpr (F == FMT_Q2SM) {
    w = (i >> 1) == 0 ? dw.x : (i >> 1) == 1 ? dw.y : (i >> 1) == 2 ? dw.z : dw.w;
  } else {
    w = dw.x;
  }
  return half_bits_to_float((i & 1) ? (w >> 16) : (w & 0xFFFFu)) * kScaleD;
}

// ONE: every tile holds a single slot (one token in the batch), so only the
// first component of each output fragment is ever needed.
template <int F, int NM, bool LO, int MODE, bool ONE>
__global__ __launch_bounds__(kFfnThreads, 4) void ffn_small_kernel(FfnTileArgs a) {
  constexpr int UB = Codes<F>::kUnitBlocks;
  constexpr int CH = NM == 2 ? 2 : (F == FMT_Q8_0 ? 4 : 1);   // units whose loads are issued together
  extern __shared__ __align__(16) uint8_t smem[];
  __shared__ float s_sig[16];
  __shared__ int32_t s_row[16];

  const int tile = blockIdx.y;
  if (tile >= *a.n_tiles) return;
  const int4 tl = a.tiles[tile];
  const int le = tl.x, p0 = tl.y, rows = tl.z;
  const int n0 = blockIdx.x * 16 * kNT;
  const int tid = threadIdx.x, lane = tid % kWave, wave = tid / kWave;
  const int c16 = lane & 15, g = lane >> 4;
  const int K = a.K, nb = K / 32;
  const int n_units = (nb + UB - 1) / UB;
  const int64_t rbytes = Codes<F>::row_bytes(K);
  const int64_t sbytes = Codes<F>::scale_row_bytes(K);

  // weight rows of this workgroup's output columns
  const uint8_t* cp[kNT][NM];
  const uint8_t* sp[kNT][NM];
#pragma unroll
  for (int nt = 0; nt < kNT; ++nt) {
    const int64_t row = (int64_t)le * a.N + n0 + 16 * nt + c16;
#pragma unroll
    for (int mt = 0; mt < NM; ++mt) {
      const QMat& w = mt ? a.w1 : a.w0;
      cp[nt][mt] = reinterpret_cast<const uint8_t*>(w.codes) + row * rbytes + 16 * g;
      sp[nt][mt] = reinterpret_cast<const uint8_t*>(w.scales) + row * sbytes;
    }
  }
  const f32x4_t zero4 = {0.0f, 0.0f, 0.0f, 0.0f};
  const uint4 zero = make_uint4(0u, 0u, 0u, 0u);
  // this wave's code units: a contiguous range (contiguous bytes of every row it reads)
  const int per_wave = (n_units + kFfnWaves - 1) / kFfnWaves;
  const int u_beg = min(wave * per_wave, n_units), u_end = min(u_beg + per_wave, n_units);
  uint4 cw[CH][kNT][NM], dw[CH][kNT][NM];
  auto load_chunk = [&](int u0) {
#pragma unroll
    for (int j = 0; j < CH; ++j) {
      const int u = min(u0 + j, n_units - 1);   // past the range: loaded, never used
#pragma unroll
      for (int nt = 0; nt < kNT; ++nt)
#pragma unroll
        for (int mt = 0; mt < NM; ++mt) {
          cw[j][nt][mt] = *reinterpret_cast<const uint4*>(cp[nt][mt] + (int64_t)u * 64);
          dw[j][nt][mt] = load_d<F>(sp[nt][mt], u);
        }
    }
  };
  if (u_beg < u_end) load_chunk(u_beg);   // the first weight loads go out before the activation set-up

  // operand rows: tokens (gate/up) or grouped positions (down)
  if (tid < 16) {
    int r = 0;
    float sg = kSigmaH;
    if (tid < rows) {
      r = MODE == MODE_GATEUP ? a.slot_list[p0 + tid] / a.k : p0 + tid;
      if (MODE == MODE_GATEUP) sg = a.sigma[r];
    }
    s_row[tid] = r;
    s_sig[tid] = sg;
  }
  uint16_t* st_hi = reinterpret_cast<uint16_t*>(smem);
  uint16_t* st_lo = st_hi + a.stage_rows * K;
  uint16_t* st_zero = st_lo + (LO ? a.stage_rows * K : 0);   // one row of zeros for rows without a slot
  for (int j = tid; j < K / 8; j += kFfnThreads) reinterpret_cast<uint4*>(st_zero)[j] = make_uint4(0u, 0u, 0u, 0u);
  __syncthreads();
  {
    const int per_row = K / 8;
    for (int j = tid; j < rows * per_row; j += kFfnThreads) {
      const int m = j / per_row, c = j % per_row;
      const int64_t src = (int64_t)s_row[m] * K + 8 * c;
      reinterpret_cast<uint4*>(st_hi)[m * per_row + c] = *reinterpret_cast<const uint4*>(a.a_hi + src);
      if (LO) reinterpret_cast<uint4*>(st_lo)[m * per_row + c] = *reinterpret_cast<const uint4*>(a.a_lo + src);
    }
    __syncthreads();
  }
  // A fragment rows: 0..3 the hi plane of slots 0..3, 4..7 their lo plane, 8..15 zero
  const int slot_m = c16 & 3;
  const bool mvalid = slot_m < rows && (c16 < 4 || (LO && c16 < 8));
  const int arow = s_row[slot_m < rows ? slot_m : 0];
  const uint16_t* pa = (mvalid ? (c16 < 4 ? st_hi : st_lo) + slot_m * K : st_zero) + 8 * g;
  // the m-term operand: rows 0..3 hi, 4..7 lo of the block sums
  const bool svalid = slot_m < rows && c16 < 8;
  const uint16_t* ps = (c16 < 4 ? a.s_hi : a.s_lo) + (int64_t)arow * a.nb32 + 8 * g;

  f32x4_t acc[kNT][NM];
#pragma unroll
  for (int nt = 0; nt < kNT; ++nt)
#pragma unroll
    for (int mt = 0; mt < NM; ++mt) acc[nt][mt] = zero4;
  const uint32_t k1024v = to_vgpr(a.kc.k1024);

  // main loop over this wave's code units; activations from LDS
  {
    for (int u0 = u_beg; u0 < u_end; u0 += CH) {
      if (u0 != u_beg) load_chunk(u0);
#pragma unroll
      for (int j = 0; j < CH; ++j) {
        const int u = u0 + j;
        if (u >= u_end) break;
#pragma unroll
        for (int i = 0; i < UB; ++i) {
          const int b = u * UB + i;
          if (b >= nb) break;
          const uint4 av = *reinterpret_cast<const uint4*>(pa + 32 * b);
#pragma unroll
          for (int nt = 0; nt < kNT; ++nt) {
#pragma unroll
            for (int mt = 0; mt < NM; ++mt) {
              const uint4 bf = Codes<F>::frag(cw[j][nt][mt], i, a.kc, k1024v);
              const f32x4_t p = mfma16(av, bf, zero4);
              const float d = d_of<F>(dw[j][nt][mt], i);
              // output row 4(l/16)+r holds slot r (hi or lo plane) for the first two lane groups
              acc[nt][mt][0] = fmaf(d, p[0], acc[nt][mt][0]);
              if (!ONE) {
                acc[nt][mt][1] = fmaf(d, p[1], acc[nt][mt][1]);
                acc[nt][mt][2] = fmaf(d, p[2], acc[nt][mt][2]);
                acc[nt][mt][3] = fmaf(d, p[3], acc[nt][mt][3]);
              }
            }
          }
        }
      }
    }
  }
  // m-term over the block index, 32 blocks per product (2-bit blocks only)
  if constexpr (Codes<F>::kHasM) {
    const int n_mc = (nb + 31) / 32;
    const int mlen = n_units * UB;   // entries of the m row
    for (int c = wave; c < n_mc; c += kFfnWaves) {
      const uint4 sv = svalid ? *reinterpret_cast<const uint4*>(ps + 32 * c) : zero;
      const int b0 = 32 * c + 8 * g;
#pragma unroll
      for (int nt = 0; nt < kNT; ++nt)
#pragma unroll
        for (int mt = 0; mt < NM; ++mt) {
          const uint4 bm = b0 < mlen ? *reinterpret_cast<const uint4*>(sp[nt][mt] + 2 * (int64_t)(mlen + b0)) : zero;
          acc[nt][mt] = mfma16(sv, bm, acc[nt][mt]);   // same units as the d-term: sigma * value
        }
    }
  }
  // partial sums of the four waves, added in wave order (the staging area is reused)
  __syncthreads();
  float* red = reinterpret_cast<float*>(smem);   // [wave][nt][mt][r][lane]
  auto R = [&](int w, int nt, int mt, int r, int l) -> float& {
    return red[(((w * kNT + nt) * NM + mt) * 4 + r) * kWave + l];
  };
#pragma unroll
  for (int nt = 0; nt < kNT; ++nt)
#pragma unroll
    for (int mt = 0; mt < NM; ++mt)
#pragma unroll
      for (int r = 0; r < 4; ++r) R(wave, nt, mt, r, lane) = acc[nt][mt][r];
  __syncthreads();
  // thread t < 64 owns output (slot m, column l) of each 16-column tile: the sum over the waves
  // of the hi row (lane l, component m) and the lo row (lane l+16, component m)
  const int m = tid >> 4, l = tid & 15;
  const bool owner = tid < 64;
  if constexpr (MODE == MODE_DOWN) {
    if (owner && m < rows) {
      const int64_t slot = a.slot_list[p0 + m];
#pragma unroll
      for (int nt = 0; nt < kNT; ++nt) {
        float v = R(0, nt, 0, m, l) + R(0, nt, 0, m, l + 16);
#pragma unroll
        for (int w = 1; w < kFfnWaves; ++w) v += R(w, nt, 0, m, l) + R(w, nt, 0, m, l + 16);
        a.y[slot * a.N + n0 + 16 * nt + l] = v * (1.0f / kSigmaH);
      }
    }
  } else {
    float* hbuf = red + kFfnWaves * kNT * NM * 4 * kWave;   // [4][33]
    const float inv = 1.0f / s_sig[m & 3];                   // a power of two: exact
#pragma unroll
    for (int nt = 0; nt < kNT; ++nt) {
      float gs = R(0, nt, 0, m, l) + R(0, nt, 0, m, l + 16), us = R(0, nt, 1, m, l) + R(0, nt, 1, m, l + 16);
#pragma unroll
      for (int w = 1; w < kFfnWaves; ++w) {
        gs += R(w, nt, 0, m, l) + R(w, nt, 0, m, l + 16);
        us += R(w, nt, 1, m, l) + R(w, nt, 1, m, l + 16);
      }
      const int cl = 16 * nt + l;
      float h = 0.0f;
      if (owner && m < rows) {
        h = silu(gs * inv) * (us * inv);
        const int col = n0 + cl;
        const int blk = col >> 5, kk = col & 31, gg = kk >> 3;
        const int e = elem_of_rt(a.fd, kk & 7);
        const float hv = h * ldexpf(1.0f, -pos_rt(a.fd, e));   // kSigmaH * 2^(6 - pos)
        uint32_t hi, lo;
        split_f16(hv, hi, lo);
        const int64_t at = (int64_t)(p0 + m) * a.I + 32 * blk + 8 * gg + e;
        a.h_hi[at] = (uint16_t)hi;
        a.h_lo[at] = (uint16_t)lo;
      }
      if (owner) hbuf[m * 33 + cl] = h;
    }
    __syncthreads();
    // block sum of h over this tile's 32 columns (index order), and the zero padding
    if (tid < 16) {
      if (tid < rows) {
        float sacc = 0.0f;
        for (int i = 0; i < 32; ++i) sacc += hbuf[tid * 33 + i];
        uint32_t hi, lo;
        split_f16(sacc * kSigmaH, hi, lo);
        const int64_t at = (int64_t)(p0 + tid) * a.nb32I + n0 / 32;
        a.hs_hi[at] = (uint16_t)hi;
        a.hs_lo[at] = (uint16_t)lo;
      }
    }
    if (blockIdx.x == 0) {
      const int nbI = a.I / 32;
      for (int j = tid; j < 16 * (a.nb32I - nbI); j += kFfnThreads) {
        const int mm = j % 16, bb = nbI + j / 16;
        if (mm < rows) {
          a.hs_hi[(int64_t)(p0 + mm) * a.nb32I + bb] = 0;
          a.hs_lo[(int64_t)(p0 + mm) * a.nb32I + bb] = 0;
        }
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Large tiles (experts with many slots): a workgroup owns up to 128 slots of one
// expert and 64 output columns; its 4 waves form a 2 x 2 grid, each with 64
// slots (four 16-row fragments) by 32 columns (two 16-column tiles) per
// matrix, over the whole contraction.  Activation fragments are read straight
// from memory (rows past the tile read row 0; their outputs are never
// stored), codes and scales as in the small kernel, the next unit's and the
// next block's loads issued before the current ones are used.
constexpr int kLargeRows = 128;
constexpr int kLargeCols = 64;

template <int F, int NM, bool LO, int MODE>
__global__ __launch_bounds__(256) void ffn_large_kernel(FfnTileArgs a) {
  constexpr int UB = Codes<F>::kUnitBlocks;
  const int tile = blockIdx.y;
  if (tile >= *a.n_tiles) return;
  const int4 tl = a.tiles[tile];
  const int le = tl.x, p0 = tl.y, rows = tl.z;
  const int tid = threadIdx.x, lane = tid % kWave, wave = tid / kWave;
  const int wm = wave >> 1, wn = wave & 1;
  const int r0 = 64 * wm;
  if (r0 >= rows) return;   // this wave has no slots (the kernel has no barrier)
  const int n_mi = min(4, (rows - r0 + 15) / 16);
  const int n0 = blockIdx.x * kLargeCols + 32 * wn;
  const int c16 = lane & 15, g = lane >> 4;
  const int K = a.K, nb = K / 32;
  const int n_units = (nb + UB - 1) / UB;
  const int64_t rbytes = Codes<F>::row_bytes(K);
  const int64_t sbytes = Codes<F>::scale_row_bytes(K);

  const uint16_t* ah[4];
  const uint16_t* al[4];
  int64_t so[4];
#pragma unroll
  for (int mi = 0; mi < 4; ++mi) {
    const int r = r0 + 16 * mi + c16;
    const int rr = r < rows ? r : 0;
    const int64_t arow = MODE == MODE_GATEUP ? a.slot_list[p0 + rr] / a.k : p0 + rr;
    ah[mi] = a.a_hi + arow * K + 8 * g;
    al[mi] = LO ? a.a_lo + arow * K + 8 * g : nullptr;
    so[mi] = arow * a.nb32 + 8 * g;
  }
  const uint8_t* cp[kNT][NM];
  const uint8_t* sp[kNT][NM];
#pragma unroll
  for (int nt = 0; nt < kNT; ++nt) {
    const int64_t row = (int64_t)le * a.N + n0 + 16 * nt + c16;
#pragma unroll
    for (int mt = 0; mt < NM; ++mt) {
      const QMat& w = mt ? a.w1 : a.w0;
      cp[nt][mt] = reinterpret_cast<const uint8_t*>(w.codes) + row * rbytes + 16 * g;
      sp[nt][mt] = reinterpret_cast<const uint8_t*>(w.scales) + row * sbytes;
    }
  }
  const f32x4_t zero4 = {0.0f, 0.0f, 0.0f, 0.0f};
  const uint4 zero = make_uint4(0u, 0u, 0u, 0u);
  f32x4_t acc[4][kNT][NM];
#pragma unroll
  for (int mi = 0; mi < 4; ++mi)
#pragma unroll
    for (int nt = 0; nt < kNT; ++nt)
#pragma unroll
      for (int mt = 0; mt < NM; ++mt) acc[mi][nt][mt] = zero4;
  const uint32_t k1024v = to_vgpr(a.kc.k1024);

  uint4 cw[kNT][NM], dw[kNT][NM], cwn[kNT][NM], dwn[kNT][NM];
  auto load_unit = [&](int u, uint4 (&c)[kNT][NM], uint4 (&d)[kNT][NM]) {
#pragma unroll
    for (int nt = 0; nt < kNT; ++nt)
#pragma unroll
      for (int mt = 0; mt < NM; ++mt) {
        c[nt][mt] = *reinterpret_cast<const uint4*>(cp[nt][mt] + (int64_t)u * 64);
        d[nt][mt] = load_d<F>(sp[nt][mt], u);
      }
  };
  uint4 ahv[4], alv[4], ahn[4], aln[4];
  auto load_a = [&](int b, uint4 (&hv)[4], uint4 (&lv)[4]) {
#pragma unroll
    for (int mi = 0; mi < 4; ++mi) {
      if (mi < n_mi) {
        hv[mi] = *reinterpret_cast<const uint4*>(ah[mi] + 32 * (int64_t)b);
        if (LO) lv[mi] = *reinterpret_cast<const uint4*>(al[mi] + 32 * (int64_t)b);
      }
    }
  };
  load_unit(0, cw, dw);
  load_a(0, ahv, alv);
  for (int u = 0; u < n_units; ++u) {
    if (u + 1 < n_units) load_unit(u + 1, cwn, dwn);
#pragma unroll
    for (int i = 0; i < UB; ++i) {
      const int b = u * UB + i;
      if (b >= nb) break;
      if (b + 1 < nb) load_a(b + 1, ahn, aln);
#pragma unroll
      for (int nt = 0; nt < kNT; ++nt) {
#pragma unroll
        for (int mt = 0; mt < NM; ++mt) {
          const uint4 bf = Codes<F>::frag(cw[nt][mt], i, a.kc, k1024v);
          const float d = d_of<F>(dw[nt][mt], i);
#pragma unroll
          for (int mi = 0; mi < 4; ++mi) {
            if (mi < n_mi) {
              f32x4_t p = mfma16(ahv[mi], bf, zero4);
              if (LO) p = mfma16(alv[mi], bf, p);
#pragma unroll
              for (int r = 0; r < 4; ++r) acc[mi][nt][mt][r] = fmaf(d, p[r], acc[mi][nt][mt][r]);
            }
          }
        }
      }
#pragma unroll
      for (int mi = 0; mi < 4; ++mi) {
        ahv[mi] = ahn[mi];
        if (LO) alv[mi] = aln[mi];
      }
    }
#pragma unroll
    for (int nt = 0; nt < kNT; ++nt)
#pragma unroll
      for (int mt = 0; mt < NM; ++mt) {
        cw[nt][mt] = cwn[nt][mt];
        dw[nt][mt] = dwn[nt][mt];
      }
  }
  if constexpr (Codes<F>::kHasM) {
    const int n_mc = (nb + 31) / 32;
    const int mlen = n_units * UB;
    for (int c = 0; c < n_mc; ++c) {
      const int b0 = 32 * c + 8 * g;
      uint4 bm[kNT][NM];
#pragma unroll
      for (int nt = 0; nt < kNT; ++nt)
#pragma unroll
        for (int mt = 0; mt < NM; ++mt)
          bm[nt][mt] = b0 < mlen ? *reinterpret_cast<const uint4*>(sp[nt][mt] + 2 * (int64_t)(mlen + b0)) : zero;
#pragma unroll
      for (int mi = 0; mi < 4; ++mi) {
        if (mi < n_mi) {
          const uint4 shi = *reinterpret_cast<const uint4*>(a.s_hi + so[mi] + 32 * c);
          const uint4 slo = *reinterpret_cast<const uint4*>(a.s_lo + so[mi] + 32 * c);
#pragma unroll
          for (int nt = 0; nt < kNT; ++nt)
#pragma unroll
            for (int mt = 0; mt < NM; ++mt) {
              acc[mi][nt][mt] = mfma16(shi, bm[nt][mt], acc[mi][nt][mt]);
              acc[mi][nt][mt] = mfma16(slo, bm[nt][mt], acc[mi][nt][mt]);
            }
        }
      }
    }
  }
  // epilogue: lane holds rows r0 + 16 mi + 4g + r, columns n0 + 16 nt + c16
#pragma unroll
  for (int mi = 0; mi < 4; ++mi) {
    if (mi >= n_mi) break;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int row = r0 + 16 * mi + 4 * g + r;
      const bool valid = row < rows;
      if constexpr (MODE == MODE_DOWN) {
        if (valid) {
          const int64_t slot = a.slot_list[p0 + row];
#pragma unroll
          for (int nt = 0; nt < kNT; ++nt)
            a.y[slot * a.N + n0 + 16 * nt + c16] = acc[mi][nt][0][r] * (1.0f / kSigmaH);
        }
      } else {
        float hsum = 0.0f;
        if (valid) {
          const float inv = 1.0f / a.sigma[a.slot_list[p0 + row] / a.k];   // a power of two: exact
#pragma unroll
          for (int nt = 0; nt < kNT; ++nt) {
            const float h = silu(acc[mi][nt][0][r] * inv) * (acc[mi][nt][1][r] * inv);
            const int col = n0 + 16 * nt + c16;
            const int blk = col >> 5, kk = col & 31, gg = kk >> 3;
            const int e = elem_of_rt(a.fd, kk & 7);
            uint32_t hi, lo;
            split_f16(h * ldexpf(1.0f, -pos_rt(a.fd, e)), hi, lo);
            const int64_t at = (int64_t)(p0 + row) * a.I + 32 * blk + 8 * gg + e;
            a.h_hi[at] = (uint16_t)hi;
            a.h_lo[at] = (uint16_t)lo;
            hsum += h;
          }
        }
        // block sum over the wave's 32 columns of this row: 16 lanes, fixed order
#pragma unroll
        for (int m = 1; m < 16; m <<= 1) hsum += __shfl_xor(hsum, m, kWave);
        if (valid && c16 == 0) {
          uint32_t hi, lo;
          split_f16(hsum * kSigmaH, hi, lo);
          const int64_t at = (int64_t)(p0 + row) * a.nb32I + n0 / 32;
          a.hs_hi[at] = (uint16_t)hi;
          a.hs_lo[at] = (uint16_t)lo;
        }
      }
    }
  }
  if (MODE == MODE_GATEUP && blockIdx.x == 0 && wn == 0) {
    const int nbI = a.I / 32, npad = a.nb32I - nbI;
    for (int j = lane; j < 64 * npad; j += kWave) {
      const int row = r0 + j % 64, bb = nbI + j / 64;
      if (row < rows) {
        a.hs_hi[(int64_t)(p0 + row) * a.nb32I + bb] = 0;
        a.hs_lo[(int64_t)(p0 + row) * a.nb32I + bb] = 0;
      }
    }
  }
}

template <int F, int NM, bool LO, int MODE, bool ONE>
static hipError_t launch_small_t(const FfnTileArgs& t, int max_tiles, hipStream_t s) {
  const size_t stage = (size_t)t.stage_rows * t.K * 2 * (LO ? 2 : 1) + (size_t)t.K * 2;
  const size_t red = (size_t)kFfnWaves * kNT * NM * 4 * kWave * 4 + 16 * 33 * 4;
  const size_t lds = stage > red ? stage : red;
  auto kern = ffn_small_kernel<F, NM, LO, MODE, ONE>;
  if (lds > 64 * 1024) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
  }
  kern<<<dim3(t.N / (16 * kNT), max_tiles), kFfnThreads, lds, s>>>(t);
  return hipGetLastError();
}

template <int F, int NM, bool LO, int MODE>
static hipError_t launch_large_t(const FfnTileArgs& t, int max_tiles, hipStream_t s) {
  ffn_large_kernel<F, NM, LO, MODE><<<dim3(t.N / kLargeCols, max_tiles), 256, 0, s>>>(t);
  return hipGetLastError();
}

hipError_t launch_ffn(const FfnArgs& a, hipStream_t s) {
  hipError_t err = hipSuccess;
  FfnTileArgs t{};
  t.slot_list = a.slot_list;
  t.k = a.k;
  t.stage_rows = a.T < kStageRows ? a.T : kStageRows;
  t.kc = frag_consts();
  // gate/up: activations (hi [+ lo]) x gate, up  ->  h
  t.a_hi = a.xq_hi; t.a_lo = a.xq_lo; t.s_hi = a.sq_hi; t.s_lo = a.sq_lo; t.sigma = a.sigma;
  t.K = a.H; t.N = a.I; t.nb32 = a.nb32H; t.w0 = a.gate; t.w1 = a.up;
  t.fd = a.fd; t.I = a.I; t.nb32I = a.nb32I;
  t.h_hi = a.h_hi; t.h_lo = a.h_lo; t.hs_hi = a.hs_hi; t.hs_lo = a.hs_lo;
  const bool lo = a.xq_lo != nullptr;
  const bool one = a.T == 1;
#define MOE_SMALL(F, NM, LO, MODE) \
  (one ? launch_small_t<F, NM, LO, MODE, true>(t, a.max_small, s) : launch_small_t<F, NM, LO, MODE, false>(t, a.max_small, s))
#define MOE_LARGE(F, NM, LO, MODE) launch_large_t<F, NM, LO, MODE>(t, a.max_large, s)
  t.tiles = a.small; t.n_tiles = a.n_small;
  trace_pre("ffn_gateup", s);
  if (a.fg == FMT_Q2SM)
    err = lo ? MOE_SMALL(FMT_Q2SM, 2, true, MODE_GATEUP) : MOE_SMALL(FMT_Q2SM, 2, false, MODE_GATEUP);
  else
    err = lo ? MOE_SMALL(FMT_Q8_0, 2, true, MODE_GATEUP) : MOE_SMALL(FMT_Q8_0, 2, false, MODE_GATEUP);
  trace_post("ffn_gateup", s);
  if (err != hipSuccess) return err;
  if (a.max_large > 0) {
    t.tiles = a.large; t.n_tiles = a.n_large;
    trace_pre("ffn_gateup_large", s);
    if (a.fg == FMT_Q2SM)
      err = lo ? MOE_LARGE(FMT_Q2SM, 2, true, MODE_GATEUP) : MOE_LARGE(FMT_Q2SM, 2, false, MODE_GATEUP);
    else
      err = lo ? MOE_LARGE(FMT_Q8_0, 2, true, MODE_GATEUP) : MOE_LARGE(FMT_Q8_0, 2, false, MODE_GATEUP);
    trace_post("ffn_gateup_large", s);
    if (err != hipSuccess) return err;
  }
  // down: h (hi + lo) x down  ->  y_slot
  t.a_hi = a.h_hi; t.a_lo = a.h_lo; t.s_hi = a.hs_hi; t.s_lo = a.hs_lo; t.sigma = nullptr;
  t.K = a.I; t.N = a.H; t.nb32 = a.nb32I; t.w0 = a.down; t.w1 = a.down;
  t.y = a.y;
  t.tiles = a.small; t.n_tiles = a.n_small;
  trace_pre("ffn_down", s);
  err = a.fd == FMT_Q2SM ? MOE_SMALL(FMT_Q2SM, 1, true, MODE_DOWN) : MOE_SMALL(FMT_Q8_0, 1, true, MODE_DOWN);
  trace_post("ffn_down", s);
  if (err != hipSuccess) return err;
  if (a.max_large > 0) {
    t.tiles = a.large; t.n_tiles = a.n_large;
    trace_pre("ffn_down_large", s);
    err = a.fd == FMT_Q2SM ? MOE_LARGE(FMT_Q2SM, 1, true, MODE_DOWN) : MOE_LARGE(FMT_Q8_0, 1, true, MODE_DOWN);
    trace_post("ffn_down_large", s);
  }
#undef MOE_SMALL
#undef MOE_LARGE
  return err;
}

}  // namespace moe
