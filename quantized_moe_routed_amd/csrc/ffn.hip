// Expert FFN on fp16 matrix cores, for tiles of up to 8 routed slots of one
// expert (decode-size batches, and every batch until the large-tile kernel
// takes the heavy experts).
//
// A workgroup owns one tile (up to 8 slots of one expert) and 32 output
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
// gate/up: h = silu(g) * u for every (slot, column) of the tile, written in
// fp32 in the down projection's K order, with the block sum and the largest
// |h| of each slot's 32 columns.
// down:    y_slot[slot][col] = the down projection of h.  Tiles of several
// slots: each wave stages its own range of the tile's h rows, every row scaled
// by the power of two of its largest |h| (row_scale over the row's block
// maxima, the rule of the activation operand) and split into the fp16 hi and
// lo planes, and the row's block sums likewise; the row scale is divided out
// in the epilogue.  One-slot tiles (single-token batches): gate/up writes each
// 32-column block of h already as the fp16 hi + lo operand, scaled by the
// power of two of that block's own largest |h|, with the inverse of that
// scale and the block's unscaled sum; down stages the planes as they are,
// multiplies each block's weight scale by the block's inverse factor in the
// fold, and adds the m-term sum_b m_b S_b on the vector units in fp32.
#include "device.h"
#include "fmt.h"
#include "launch.h"
#include "ffn.h"
#include "smallsel.h"

namespace moe {

constexpr int kFfnThreads = 512;
constexpr int kFfnWaves = kFfnThreads / 64;
constexpr int kNT = 2;            // 16-column output tiles per workgroup
constexpr int kStageRows = kSmallRowsMax;   // slots per tile at most; their activation rows are staged in LDS
// LDS of the unit-by-unit staging: per wave one unit (UB blocks) of 8 hi rows, 8 lo rows and a zero row
constexpr size_t half_stage_bytes(int ub) { return (size_t)kFfnWaves * (2 * kStageRows + 1) * ub * 32 * 2; }

// ONE: every tile holds a single slot (one token in the batch), so only the
// first component of each output fragment is ever needed.
// SEL (gate/up of batches of at most kSelMaxTokens tokens): the workgroup first selects, groups
// and numbers the tiles itself from the logits (smallsel.h); workgroup (0, 0) also stores the
// routing results and the tile list for the later launches.  (As a workgroup of its own, in a grid
// row past the tiles, it would be dispatched only once a tile's workgroup had finished, and its
// selection would then end the launch several microseconds after the last tile.)
// Bytes of the activation staging area (rows hi [+ lo], then a row of zeros), rounded to 16: the
// one-token selection keeps its candidates past it, and the one-slot reduction its sums past those.
__host__ __device__ constexpr size_t sel_cand_offset(int stage_rows, int K, bool lo) {
  return ((size_t)stage_rows * K * 2 * (lo ? 2 : 1) + (size_t)K * 2 + 15) & ~(size_t)15;
}
__host__ __device__ constexpr size_t one_red_offset(bool sel, int stage_rows, int K, bool lo) {
  return sel_cand_offset(stage_rows, K, lo) + (sel ? kSelScratchBytes : 0);
}



// PRE (down of several slots): the operand rows come prepared (the conversion launch wrote each row
// of h scaled and split, with its block sums and row scale), staged as they are; without PRE each
// wave converts its own range of the fp32 rows while staging (CONV).
// HALF (2-bit gate/up of several slots with a lo plane, at most two code units per wave): each
// wave stages one code unit of its rows at a time in a window of its own, and the second after
// the first unit is multiplied, so that 8 slots' rows take half the LDS of staging the whole range.
template <int F, int NM, bool LO, int MODE, bool ONE, bool SEL, bool PRE = false, bool HALF = false>
__global__ __launch_bounds__(kFfnThreads, 4) void ffn_small_kernel(FfnTileArgs a) {
  static_assert(!HALF || (MODE == MODE_GATEUP && !ONE && !SEL && LO && F == FMT_Q2SM && NM == 2),
                "unit-by-unit staging: 2-bit gate/up of several slots with a lo plane");
  constexpr int UB = Codes<F>::kUnitBlocks;
  constexpr bool CONV = MODE == MODE_DOWN && !ONE && !PRE;   // down of several slots: converts fp32 h while staging
  constexpr bool BSC = MODE == MODE_DOWN && ONE;     // down of one slot: block-scaled operand planes
  constexpr int CH = NM == 2 ? 2 : (F == FMT_Q8_0 ? 4 : 1);   // units whose loads are issued together
  extern __shared__ __align__(16) uint8_t smem[];
  __shared__ float s_sig[16];

  const int tile = blockIdx.y;
  int4 tl, tk0, tk1;   // the tile; the operand rows of its slots 0..3 and 4..7
  if constexpr (SEL) {
    const bool writer = blockIdx.x == 0 && blockIdx.y == 0;
    if constexpr (ONE) {
      // wave 0 selects (its candidates sit past the staging area) and hands the tile to the other
      // waves through LDS: a selection in every wave would put four copies of the same work on
      // each SIMD
      __shared__ int4 s_tl;
      __shared__ int s_n;
      tl = tk0 = tk1 = make_int4(0, 0, 0, 0);
      if (threadIdx.x < kWave) {
        uint64_t* cand = reinterpret_cast<uint64_t*>(smem + sel_cand_offset(a.stage_rows, a.K, LO));
        const int n = one_token_select(a.sel, writer, tile, cand, tl);
        if (threadIdx.x == 0) {
          s_tl = tl;
          s_n = n;
        }
      }
      __syncthreads();
      if (tile >= s_n) return;
      tl = s_tl;
    } else {
      __shared__ SelLds sl;
      small_select<kFfnThreads>(a.sel, sl, writer, tile, reinterpret_cast<uint64_t*>(smem));
      if (tile >= sl.n_tiles) return;
      tl = sl.tile;
      tk0 = sl.tok[0];
      tk1 = sl.tok[1];
    }
  } else {
    if (tile >= *a.n_tiles) return;
    tl = a.tiles[tile];
    // operand rows of the tile: tokens (gate/up, listed with the tile) or grouped positions (down)
    if constexpr (MODE == MODE_GATEUP) {
      tk0 = a.tile_tok[2 * tile];
      tk1 = a.tile_tok[2 * tile + 1];
    } else {
      tk0 = make_int4(tl.y, tl.y + 1, tl.y + 2, tl.y + 3);
      tk1 = make_int4(tl.y + 4, tl.y + 5, tl.y + 6, tl.y + 7);
    }
  }
  const int le = tl.x, p0 = tl.y, rows = tl.z;
  auto row_of = [&](int m) {
    const int j = m & 3;
    const int a0 = j == 0 ? tk0.x : j == 1 ? tk0.y : j == 2 ? tk0.z : tk0.w;
    const int a1 = j == 0 ? tk1.x : j == 1 ? tk1.y : j == 2 ? tk1.z : tk1.w;
    return m < 4 ? a0 : a1;
  };
  const int n0 = blockIdx.x * 16 * kNT;
  const int tid = threadIdx.x, lane = tid % kWave, wave = tid / kWave;
  const int c16 = lane & 15, g = lane >> 4;
  const int K = a.K, nb = K / 32;
  const int n_units = (nb + UB - 1) / UB;
  const int64_t rbytes = Codes<F>::row_bytes(K);
  const int64_t sbytes = Codes<F>::scale_row_bytes(K);

  // weight rows of this workgroup's output columns: the expert's matrices (uniform bases) and the
  // lane's byte offsets within them (one matrix is well under 4 GiB)
  const uint8_t* cb[NM];
  const uint8_t* sb[NM];
#pragma unroll
  for (int mt = 0; mt < NM; ++mt) {
    const QMat& w = mt ? a.w1 : a.w0;
    cb[mt] = reinterpret_cast<const uint8_t*>(w.codes) + (int64_t)le * a.N * rbytes;
    sb[mt] = reinterpret_cast<const uint8_t*>(w.scales) + (int64_t)le * a.N * sbytes;
  }
  // (row-group layout: a 16-column tile is one row group, unit u of it 1 KiB at 1 KiB * u)
  uint32_t co[kNT], so[kNT];
#pragma unroll
  for (int nt = 0; nt < kNT; ++nt) {
    const int col = n0 + 16 * nt + c16;
    co[nt] = (uint32_t)code_off(col, 0, n_units) + 16u * (uint32_t)g;
    so[nt] = (uint32_t)Codes<F>::d_off(col, 0, n_units);
  }
  // codes of unit u; d values of unit u (m values of a 2-bit unit follow its d values of 16 rows)
  auto cp = [&](int nt, int mt, int u) { return cb[mt] + (co[nt] + 1024u * (uint32_t)u); };
  auto dp = [&](int nt, int mt, int u) { return sb[mt] + (so[nt] + (uint32_t)Codes<F>::kScaleUnit * (uint32_t)u); };
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
          cw[j][nt][mt] = *reinterpret_cast<const uint4*>(cp(nt, mt, u));
          dw[j][nt][mt] = load_d<F>(dp(nt, mt, u));
        }
    }
  };
  // Each wave moves its own slice of the tile's activation rows (the values of its code units) to
  // LDS with direct loads, ahead of its codes so that they are not queued behind the weight stream;
  // no other wave reads that slice, so no barrier is needed before the main loop.
  // (HALF: wave w's window of one code unit, WV values per row: 8 hi rows, 8 lo rows, a zero row)
  constexpr int WV = UB * 32;
  const int RS = HALF ? WV : K;   // row stride of the staging area
  // (the staging loops' fields, kept in registers: the staging loads are inline assembly with a
  // memory clobber, after which a field read through the argument block would be loaded again,
  // a scalar load and its wait before every staging load)
  const uint16_t* const ahi = a.a_hi;
  const uint16_t* const alo = a.a_lo;
  [[maybe_unused]] const float* const hf = a.hf;
  const int srows = a.stage_rows;
  uint16_t* st_hi = reinterpret_cast<uint16_t*>(smem) + (HALF ? (size_t)wave * (2 * kStageRows + 1) * WV : 0);
  uint16_t* st_lo = st_hi + (HALF ? kStageRows * WV : srows * K);
  uint16_t* st_zero = HALF ? st_hi + 2 * kStageRows * WV
                           : st_lo + (LO ? srows * K : 0);   // one row of zeros for rows without a slot
  // the rows' scales (prepared down operand: per grouped position), loaded now and stored in LDS
  // after the main loop, so that no wait for them holds back the loads below
  [[maybe_unused]] float sig_row = 1.0f;
  if constexpr (MODE == MODE_GATEUP || PRE)
    if (tid < kStageRows && tid < rows) sig_row = a.sigma[row_of(tid)];
  const int k0 = 32 * UB * u_beg, k1 = min(32 * UB * u_end, K);
  if constexpr (HALF) {
    for (int e = 8 * lane; e < WV; e += 8 * kWave) *reinterpret_cast<uint4*>(st_zero + e) = make_uint4(0u, 0u, 0u, 0u);
  } else {
    for (int e = k0 + 8 * lane; e < k1; e += 8 * kWave)
      *reinterpret_cast<uint4*>(st_zero + e) = make_uint4(0u, 0u, 0u, 0u);
  }
  // HALF: code unit u of the rows into this wave's window (lanes past the unit or the row load nothing)
  [[maybe_unused]] auto stage_unit = [&, ahi, alo](int u) {
    const uint32_t w0 = (uint32_t)(uintptr_t)st_hi;
    const int e = 32 * UB * u + 8 * lane;
    if (8 * lane < WV && e < K) {
#pragma unroll
      for (int pl = 0; pl < 2; ++pl) {
        const uint16_t* base = (pl ? alo : ahi) + e;
        for (int m = 0; m < rows; ++m)
          dma16(base + (int64_t)row_of(m) * K,
                __builtin_amdgcn_readfirstlane(w0 + (uint32_t)((pl * kStageRows + m) * WV * 2)));
      }
    }
  };
  // down: the fp32 h of this wave's range [k0, k1) of every row goes by direct loads into the LDS
  // bytes that its fp16 pairs will occupy: pass q (values 256 q .. 256 q + n - 1 of the range, n at
  // most 256) puts its first n / 2 values into the hi plane's bytes of the pass and the rest into
  // the lo plane's, so that converting a pass reads and writes only that pass's bytes.  The rows'
  // block maxima come into registers (lane l: row l / LPR, blocks l % LPR + LPR j), ahead of the
  // weights; once they are in, each wave converts its own range in place, with no barrier.
  constexpr int LPR = kWave / kStageRows;                 // lanes per row of the block maxima
  constexpr int HMJ = 64 / LPR;                           // maxima per lane issued early (nb <= 64)
  [[maybe_unused]] float hmv[HMJ];
  [[maybe_unused]] int64_t slot_out = 0;                  // down: the output slot of the lane's row
  // one slot: lane l holds the inverse scale and the sum of block b0 + (l % 32) of the wave's range
  [[maybe_unused]] float fbl = 1.0f, sbl = 0.0f;
  if constexpr (MODE == MODE_DOWN) {
    // the output slot of the row this thread stores in the epilogue
    // (an opaque zero keeps a one-slot tile's index in a vector register: a uniform value would be
    // moved to a scalar register right after its load, which would wait for every earlier load)
    int z = 0;
    asm volatile("" : "+v"(z));
    slot_out = a.slot_list[p0 + z + (ONE ? 0 : min(tid >> 4, rows - 1))];
  }
  if constexpr (BSC) {
    const int64_t bi = (int64_t)p0 * a.nb32 + min(k0 / 32 + lane % 32, a.nb32 - 1);
    fbl = a.hmf[bi];
    if constexpr (Codes<F>::kHasM) sbl = a.hsf[bi];
  }
  if constexpr (CONV) {
    const uint32_t lds0 = (uint32_t)(uintptr_t)smem;
    for (int m = 0; m < rows; ++m)
      for (int q0 = 0; q0 < k1 - k0; q0 += 4 * kWave) {
        const int hq = min(4 * kWave, k1 - k0 - q0) / 2;   // values of the pass in each plane
        if (4 * lane < hq)
          for (int pl = 0; pl < 2; ++pl) {
            const float* src = hf + (int64_t)(p0 + m) * K + k0 + q0 + pl * hq + 4 * lane;
            const uint32_t dst = lds0 + (uint32_t)((((pl ? srows : 0) + m) * K + k0 + q0) * 2);
            dma16(src, __builtin_amdgcn_readfirstlane(dst));
          }
      }
    const int mr = lane / LPR;
    const float* pm = a.hmf + (int64_t)(p0 + (mr < rows ? mr : 0)) * a.nb32 + lane % LPR;
#pragma unroll
    for (int j = 0; j < HMJ; ++j) hmv[j] = pm[min(LPR * j, a.nb32 - LPR)];   // (past the row: dropped below)
  } else if constexpr (HALF) {
    if (u_beg < u_end) stage_unit(u_beg);
  } else {   // gate/up, and one-slot down: the prepared fp16 planes as they are

    const uint32_t lds0 = (uint32_t)(uintptr_t)smem;
    for (int pl = 0; pl < (LO ? 2 : 1); ++pl)
      for (int m = 0; m < rows; ++m)
        for (int c0 = k0; c0 < k1; c0 += 512) {   // 1 KiB per instruction
          const int e = c0 + 8 * lane;
          if (e < k1) {
            const uint16_t* src = (pl ? alo : ahi) + (int64_t)(BSC ? p0 + m : row_of(m)) * K + e;
            const uint32_t dst = lds0 + (uint32_t)((((pl ? srows : 0) + m) * K + c0) * 2);
            dma16(src, __builtin_amdgcn_readfirstlane(dst));
          }
        }
  }
  // m values of a group of up to 4 of this wave's units (lane group g: unit ug + g); the first
  // group's m values and block sums are fetched right after the row slices, ahead of the codes
  uint4 mv[kNT][NM];
  // (every load is issued, from a clamped unit, and its value dropped when out of range: no load
  // sits behind a branch, so the loads issued after the row slices are known)
  auto load_m = [&](int ug) {
    const int u = ug + g;
    const bool in = u < u_end;
    const int uc = min(u, n_units - 1);
#pragma unroll
    for (int nt = 0; nt < kNT; ++nt)
#pragma unroll
      for (int mt = 0; mt < NM; ++mt) {
        const uint4 v = *reinterpret_cast<const uint4*>(dp(nt, mt, uc) + 256u);
        mv[nt][mt] = in ? v : zero;
      }
  };
  if constexpr (Codes<F>::kHasM) load_m(u_beg);

  // A fragment rows: 0..7 the hi plane of slots 0..7, 8..15 their lo plane (zero without one)
  const int slot_m = c16 & 7;
  const bool mvalid = slot_m < rows && (c16 < 8 || LO);
  const int arow = row_of(slot_m < rows ? slot_m : 0);
  const uint16_t* pa = (mvalid ? (c16 < 8 ? st_hi : st_lo) + slot_m * RS : st_zero) + 8 * g;
  // the m-term operand: rows 0..7 hi, 8..15 lo of the block sums
  const bool svalid = slot_m < rows;
  const uint16_t* ps = (c16 < 8 ? a.s_hi : a.s_lo) + (int64_t)arow * a.nb32;
  // m-term operands of a group of up to 4 of this wave's units (lane group g: unit ug + g): the m
  // values of the lane's column and the block sums of the slots (rows 0..7 hi, 8..15 lo); down
  // loads the fp32 sums of h (sraw) and scales and splits them once the row's scale is known
  uint4 sv = zero;
  [[maybe_unused]] float sraw[8];
  [[maybe_unused]] bool sin = false;
  [[maybe_unused]] const float* psf = a.hsf + (int64_t)arow * a.nb32;
  auto load_s = [&](int ug) {
    const int u = ug + g;
    sin = u < u_end && svalid;
    if constexpr (BSC) {
      (void)u;
    } else if constexpr (CONV) {
      const float4* p = reinterpret_cast<const float4*>(psf + UB * min(u, n_units - 1));
      const float4 v0 = p[0], v1 = p[1];
      sraw[0] = v0.x; sraw[1] = v0.y; sraw[2] = v0.z; sraw[3] = v0.w;
      sraw[4] = v1.x; sraw[5] = v1.y; sraw[6] = v1.z; sraw[7] = v1.w;
    } else {
      const uint4 v = *reinterpret_cast<const uint4*>(ps + UB * min(u, n_units - 1));
      sv = sin ? v : zero;
    }
  };
  [[maybe_unused]] float sig_s = 1.0f;   // down: the scale of the lane's m-term row
  auto cvt_s = [&]() {
    if constexpr (CONV) {
      uint4 hi, lo;
      split8(sraw, sig_s, hi, lo);
      sv = sin ? (c16 < 8 ? hi : lo) : zero;
    }
  };
  if constexpr (Codes<F>::kHasM && (MODE == MODE_GATEUP || PRE)) load_s(u_beg);   // (CONV: after converting)
  load_chunk(u_beg);
  // nothing that uses a loaded value is scheduled among the loads above: no wait delays their issue
  __builtin_amdgcn_sched_barrier(0);
  // Every load of this wave is in flight.  Loads complete in issue order, so once no more than the
  // chunk's code and scale loads (issued last) are outstanding, the slices are in LDS and the m-term operands in registers; the codes
  // themselves are waited for where they are used.
  wait_vmem_at_most<CH * kNT * NM * 2>();
  // down: every row's scale from its block maxima, then this wave's range of each row converted in
  // place, four (row, pass) items per lane at a time: each item's values are read before any of
  // its pairs is written (a wave's LDS operations take effect in order)
  [[maybe_unused]] float sig = 1.0f;   // the scale of row lane / LPR
  if constexpr (CONV) {
    const int mr = lane / LPR;
    float hmx = 0.0f;
#pragma unroll
    for (int j = 0; j < HMJ; ++j) hmx = fmaxf(hmx, LPR * j + lane % LPR < nb ? hmv[j] : 0.0f);
    if (nb > 64)   // rows past 2048 values: the other maxima now (this waits for every load)
      for (int b = 64 + lane % LPR; b < nb; b += LPR)
        hmx = fmaxf(hmx, a.hmf[(int64_t)(p0 + (mr < rows ? mr : 0)) * a.nb32 + b]);
    if (mr >= rows) hmx = 0.0f;
#pragma unroll
    for (int o = 1; o < LPR; o <<= 1) hmx = fmaxf(hmx, __shfl_xor(hmx, o, kWave));
    sig = row_scale(hmx);
    constexpr int IB = 2;   // rows converted together
    for (int m0 = 0; m0 < rows; m0 += IB)
      for (int q0 = 0; q0 < k1 - k0; q0 += 4 * kWave) {
        const int hq = min(4 * kWave, k1 - k0 - q0) / 2, j = 4 * lane;
        const bool act = j < 2 * hq;
        // the lane's four values of the pass (row 0): the hi plane's bytes hold the first hq
        const float* src = j < hq ? reinterpret_cast<const float*>(st_hi + k0 + q0) + j
                                  : reinterpret_cast<const float*>(st_lo + k0 + q0) + (j - hq);
        float4 v[IB];
#pragma unroll
        for (int i = 0; i < IB; ++i)
          if (act) v[i] = *reinterpret_cast<const float4*>(src + (min(m0 + i, rows - 1) * K) / 2);
#pragma unroll
        for (int i = 0; i < IB; ++i) {
          const int m = m0 + i;
          const float sc =
              __uint_as_float((uint32_t)__builtin_amdgcn_readlane((int)__float_as_uint(sig), (m * LPR) % kWave)) * 64.0f;
          if (act && m < rows) {
            uint32_t h0, h1, h2, h3, l0, l1, l2, l3;
            split_f16(v[i].x * sc, h0, l0);
            split_f16(v[i].y * sc, h1, l1);
            split_f16(v[i].z * sc, h2, l2);
            split_f16(v[i].w * sc, h3, l3);
            *reinterpret_cast<uint2*>(st_hi + m * K + k0 + q0 + j) = make_uint2(h0 | (h1 << 16), h2 | (h3 << 16));
            *reinterpret_cast<uint2*>(st_lo + m * K + k0 + q0 + j) = make_uint2(l0 | (l1 << 16), l2 | (l3 << 16));
          }
        }
      }
    if constexpr (Codes<F>::kHasM) {
      // the first group's block sums, issued now (after the weights, which the main loop waits for
      // right away), so that they are not held in registers through the conversion
      sig_s = __shfl(sig, (slot_m < rows ? slot_m : 0) * LPR % kWave, kWave);
      load_s(u_beg);
      wait_vmem();
      cvt_s();
    }
  }
  f32x4_t acc[kNT][NM];
#pragma unroll
  for (int nt = 0; nt < kNT; ++nt)
#pragma unroll
    for (int mt = 0; mt < NM; ++mt) acc[nt][mt] = zero4;

  // m-term (2-bit blocks only): sum_b m_b (sigma S_b) over the wave's own units, four units (32
  // blocks) per product, the first group before the main loop
  // (one slot: on the vector units in fp32, sum_b m_b S_b for unit ug + g in lane group g, the
  // block sums read by lane index from sbl, in block order; the groups are added after the loop)
  [[maybe_unused]] float mtacc[kNT] = {};
  auto mterm = [&](int ug) {
    if constexpr (BSC) {
#pragma unroll
      for (int gg = 0; gg < 4; ++gg) {
        if (ug + gg >= u_end) break;
#pragma unroll
        for (int nt = 0; nt < kNT; ++nt) {
          const uint32_t mw[4] = {mv[nt][0].x, mv[nt][0].y, mv[nt][0].z, mv[nt][0].w};
          float t = 0.0f;
#pragma unroll
          for (int i = 0; i < UB; ++i) {
            const float sb = __uint_as_float(
                (uint32_t)__builtin_amdgcn_readlane((int)__float_as_uint(sbl), (ug + gg - u_beg) * UB + i));
            t = fmaf(half_bits_to_float((i & 1) ? (mw[i >> 1] >> 16) : (mw[i >> 1] & 0xFFFFu)), sb, t);
          }
          mtacc[nt] += g == gg ? t : 0.0f;
        }
      }
    } else {
#pragma unroll
      for (int nt = 0; nt < kNT; ++nt)
#pragma unroll
        for (int mt = 0; mt < NM; ++mt) acc[nt][mt] = mfma16(sv, mv[nt][mt], acc[nt][mt]);   // sigma * value units
    }
  };
  if constexpr (Codes<F>::kHasM) mterm(u_beg);

  // main loop over this wave's code units, a unit as soon as its codes are in; activations from LDS
  for (int u0 = u_beg; u0 < u_end; u0 += CH) {
    if (u0 != u_beg) load_chunk(u0);
#pragma unroll
    for (int j = 0; j < CH; ++j) {
      const int u = u0 + j;
      if (u >= u_end) break;
      if constexpr (HALF) {
        if (j > 0) {
          // the previous unit's operand reads are done; the next unit into the same window
          asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
          stage_unit(u);
          wait_vmem();
        }
      }
#pragma unroll
      for (int i = 0; i < UB; ++i) {
        const int b = u * UB + i;
        if (b >= nb) break;
        const uint4 av = *reinterpret_cast<const uint4*>(pa + 32 * (HALF ? i : b));
        // one slot: the block's inverse operand scale, folded into its weight scales
        [[maybe_unused]] float fb = 1.0f;
        if constexpr (BSC)
          fb = __uint_as_float((uint32_t)__builtin_amdgcn_readlane((int)__float_as_uint(fbl), (u - u_beg) * UB + i));
        // per output tile: the fragments of both matrices, both products, then both folds, so
        // that no fold waits on the product issued just before it
#pragma unroll
        for (int nt = 0; nt < kNT; ++nt) {
          uint4 bf[NM];
          f32x4_t p[NM];
#pragma unroll
          for (int mt = 0; mt < NM; ++mt) bf[mt] = Codes<F>::frag(cw[j][nt][mt], i, a.kc);
#pragma unroll
          for (int mt = 0; mt < NM; ++mt) p[mt] = mfma16(av, bf[mt], zero4);
#pragma unroll
          for (int mt = 0; mt < NM; ++mt) {
            float d = d_of<F>(dw[j][nt][mt], i);
            if constexpr (BSC) d *= fb;   // (a power of two: exact)
            // several slots: convert the scale once, then plain fp32 FMAs (one slot: a single
            // mixed-precision FMA is cheaper)
            if (!ONE) asm volatile("" : "+v"(d));
            acc[nt][mt][0] = fmaf(d, p[mt][0], acc[nt][mt][0]);
            if (!ONE) {
              acc[nt][mt][1] = fmaf(d, p[mt][1], acc[nt][mt][1]);
              acc[nt][mt][2] = fmaf(d, p[mt][2], acc[nt][mt][2]);
              acc[nt][mt][3] = fmaf(d, p[mt][3], acc[nt][mt][3]);
            }
          }
        }
      }
    }
  }
  if constexpr (MODE == MODE_GATEUP || PRE)
    if (tid < kStageRows) s_sig[tid] = sig_row;   // (read after the reduction's barrier)
  // m-term of the remaining groups (more than 4 units per wave)
  if constexpr (Codes<F>::kHasM) {
    for (int ug = u_beg + 4; ug < u_end; ug += 4) {
      load_m(ug);
      load_s(ug);
      cvt_s();
      mterm(ug);
    }
    if constexpr (BSC) {
      // the lane groups' sums of each column, added in group order, join row 0 (lanes 0 .. 15)
#pragma unroll
      for (int nt = 0; nt < kNT; ++nt) {
        float t = mtacc[nt] + __shfl_xor(mtacc[nt], 16, kWave);
        t += __shfl_xor(t, 32, kWave);
        if (lane < 16) acc[nt][0][0] += t;
      }
    }
  }
  if constexpr (ONE) {
    // One slot: its hi row is component 0 of lanes 0..15, its lo row component 0 of lanes 32..47.
    // Each wave adds the two (hi + lo, the lo half reaching lane l from lane l + 32) and leaves
    // the sums past the staging area; after one barrier wave 0 adds the waves in order (the same
    // additions as the general reduction below) and finishes the tile, lane 16 nt + l holding
    // column 16 nt + l.
    float* red1 = reinterpret_cast<float*>(smem + one_red_offset(SEL, a.stage_rows, K, LO));   // [wave][nt][mt][16]
#pragma unroll
    for (int nt = 0; nt < kNT; ++nt)
#pragma unroll
      for (int mt = 0; mt < NM; ++mt) {
        const float hi = acc[nt][mt][0];
        const float lo = __shfl_xor(hi, 32, kWave);
        if (lane < 16) red1[((wave * kNT + nt) * NM + mt) * 16 + lane] = hi + lo;
      }
    __syncthreads();
    if (wave != 0 || lane >= 16 * kNT) return;
    const int nt = lane >> 4, l = lane & 15;
    auto R1 = [&](int w, int mt) { return red1[((w * kNT + nt) * NM + mt) * 16 + l]; };
    if constexpr (MODE == MODE_DOWN) {
      float v = R1(0, 0);
#pragma unroll
      for (int w = 1; w < kFfnWaves; ++w) v += R1(w, 0);
      a.y[slot_out * a.N + n0 + 16 * nt + l] = v * (1.0f / sig);   // a power of two: exact
    } else {
      float gs = R1(0, 0), us = R1(0, 1);
#pragma unroll
      for (int w = 1; w < kFfnWaves; ++w) {
        gs += R1(w, 0);
        us += R1(w, 1);
      }
      const float inv = 1.0f / s_sig[0];   // a power of two: exact
      const float h = silu(gs * inv) * (us * inv);
      const int col = n0 + lane;
      const int blk = col >> 5, kk = col & 31, gg = kk >> 3;
      // block sum of h over the tile's 32 columns, in index order, and their largest |h|
      float sacc = 0.0f, smax = 0.0f;
#pragma unroll
      for (int i = 0; i < 16 * kNT; ++i) {
        const float hi = __uint_as_float((uint32_t)__builtin_amdgcn_readlane((int)__float_as_uint(h), i));
        sacc += hi;
        smax = fmaxf(smax, fabsf(hi));
      }
      // the down projection's operand of this block: h times 2^6 and the block's own scale, as an
      // fp16 hi + lo pair; with it the inverse of the scale and the block's unscaled sum
      const float sb = row_scale(smax);
      uint32_t hi, lo;
      split_f16(h * sb * 64.0f, hi, lo);
      const int64_t at = (int64_t)p0 * a.I + 32 * blk + 8 * gg + frag_val(kk & 7);
      a.hb_hi[at] = (uint16_t)hi;
      a.hb_lo[at] = (uint16_t)lo;
      if (lane == 0) {
        const int64_t at_s = (int64_t)p0 * a.nb32I + n0 / 32;
        a.hs[at_s] = sacc;
        a.hm[at_s] = 1.0f / sb;
      }
      if (blockIdx.x == 0) {
        const int nbI = a.I / 32;
        for (int bb = nbI + lane; bb < a.nb32I; bb += 16 * kNT) a.hs[(int64_t)p0 * a.nb32I + bb] = 0.0f;
      }
    }
    return;
  }
  // partial sums of the waves, added in wave order (the staging area is reused)
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
  // thread t < 128 owns output (slot m, column l) of each 16-column tile: the sum over the waves of
  // the hi row m (lane 16 (m / 4) + l, component m % 4) and the lo row 8 + m (lane
  // 16 (2 + m / 4) + l, the same component)
  const int m = tid >> 4, l = tid & 15;
  const bool owner = tid < 16 * kStageRows;
  const int lhi = 16 * ((m >> 2) & 1) + l, llo = lhi + 32, cm = m & 3;
  if constexpr (MODE == MODE_DOWN) {
    // the row's scale: converted here (CONV) or prepared (a power of two either way: exact)
    const float inv = PRE ? 1.0f / s_sig[m & 7] : 1.0f / __shfl(sig, (m & 7) * (kWave / kStageRows), kWave);
    if (owner && m < rows) {
#pragma unroll
      for (int nt = 0; nt < kNT; ++nt) {
        float v = R(0, nt, 0, cm, lhi) + R(0, nt, 0, cm, llo);
#pragma unroll
        for (int w = 1; w < kFfnWaves; ++w) v += R(w, nt, 0, cm, lhi) + R(w, nt, 0, cm, llo);
        a.y[slot_out * a.N + n0 + 16 * nt + l] = v * inv;
      }
    }
  } else {
    float* hbuf = red + kFfnWaves * kNT * NM * 4 * kWave;   // [8][33]
    const float inv = 1.0f / s_sig[m & 7];                   // a power of two: exact
#pragma unroll
    for (int nt = 0; nt < kNT; ++nt) {
      float gs = R(0, nt, 0, cm, lhi) + R(0, nt, 0, cm, llo), us = R(0, nt, 1, cm, lhi) + R(0, nt, 1, cm, llo);
#pragma unroll
      for (int w = 1; w < kFfnWaves; ++w) {
        gs += R(w, nt, 0, cm, lhi) + R(w, nt, 0, cm, llo);
        us += R(w, nt, 1, cm, lhi) + R(w, nt, 1, cm, llo);
      }
      const int cl = 16 * nt + l;
      float h = 0.0f;
      if (owner && m < rows) {
        h = silu(gs * inv) * (us * inv);
        const int col = n0 + cl;
        const int blk = col >> 5, kk = col & 31, gg = kk >> 3;
        a.h[(int64_t)(p0 + m) * a.I + 32 * blk + 8 * gg + frag_val(kk & 7)] = h;
      }
      if (owner) hbuf[m * 33 + cl] = h;
    }
    __syncthreads();
    // block sum of h over this tile's 32 columns (index order) and their largest |h|, and the
    // zero padding of the block sums
    if (tid < rows) {
      float sacc = 0.0f, smax = 0.0f;
      for (int i = 0; i < 32; ++i) {
        sacc += hbuf[tid * 33 + i];
        smax = fmaxf(smax, fabsf(hbuf[tid * 33 + i]));
      }
      const int64_t at = (int64_t)(p0 + tid) * a.nb32I + n0 / 32;
      a.hs[at] = sacc;
      a.hm[at] = smax;
    }
    if (blockIdx.x == 0) {
      const int nbI = a.I / 32;
      for (int j = tid; j < 16 * (a.nb32I - nbI); j += kFfnThreads) {
        const int mm = j % 16, bb = nbI + j / 16;
        if (mm < rows) a.hs[(int64_t)(p0 + mm) * a.nb32I + bb] = 0.0f;
      }
    }
  }
}

template <int F, int NM, bool LO, int MODE, bool ONE, bool SEL = false, bool PRE = false, bool HALF = false>
static hipError_t launch_small_t(const FfnTileArgs& t, int max_tiles, hipStream_t s) {
  const size_t stage = HALF ? half_stage_bytes(Codes<F>::kUnitBlocks)
                            : (size_t)t.stage_rows * t.K * 2 * (LO ? 2 : 1) + (size_t)t.K * 2;
  const size_t red = (size_t)kFfnWaves * kNT * NM * 4 * kWave * 4 + kStageRows * 33 * 4;
  size_t lds = stage > red ? stage : red;
  if (SEL && lds < kSelScratchBytes) lds = kSelScratchBytes;
  if (ONE) {   // selection candidates (with SEL) and the one-slot sums past the staging area
    const size_t one = one_red_offset(SEL, t.stage_rows, t.K, LO) + (size_t)kFfnWaves * kNT * NM * 16 * 4;
    if (lds < one) lds = one;
  }

  auto kern = ffn_small_kernel<F, NM, LO, MODE, ONE, SEL, PRE, HALF>;
  if (lds > 64 * 1024) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
  }
  return launch_stamped(kern, dim3(t.N / (16 * kNT), max_tiles), dim3(kFfnThreads), lds, s, t);
}

// (the staging area of 8 rows; the reduction area and the selection's LDS are smaller)
static size_t small_stage_bytes(int K, bool lo) { return (size_t)kSmallRowsMax * K * 2 * (lo ? 2 : 1) + (size_t)K * 2; }
constexpr size_t kTwoPerCu = 72 * 1024;

int small_tile_rows(int H, int I, bool f32_act) {
  return small_stage_bytes(H, f32_act) <= kTwoPerCu && small_stage_bytes(I, true) <= kTwoPerCu ? kSmallRowsMax : 4;
}

int small_down_tile_rows(int I) { return small_stage_bytes(I, true) <= kTwoPerCu ? kSmallRowsMax : 4; }

bool half_gateup_staging(int H, bool f32_act) {
  const int n_units = (H / 32 + Codes<FMT_Q2SM>::kUnitBlocks - 1) / Codes<FMT_Q2SM>::kUnitBlocks;
  return f32_act && small_stage_bytes(H, true) > kTwoPerCu && n_units <= 2 * kFfnWaves &&
         half_stage_bytes(Codes<FMT_Q2SM>::kUnitBlocks) <= kTwoPerCu;
}

hipError_t launch_ffn(const FfnArgs& a, hipStream_t s) {
  hipError_t err = hipSuccess;
  FfnTileArgs t{};
  t.slot_list = a.slot_list;
  t.k = a.k;
  t.stage_rows = a.T < a.bm_small ? a.T : a.bm_small;
  t.kc = frag_consts();
  // gate/up: activations (hi [+ lo]) x gate, up  ->  h
  t.a_hi = a.xq_hi; t.a_lo = a.xq_lo; t.s_hi = a.sq_hi; t.s_lo = a.sq_lo; t.sigma = a.sigma;
  t.K = a.H; t.N = a.I; t.nb32 = a.nb32H; t.w0 = a.gate; t.w1 = a.up;
  t.fd = a.fd; t.I = a.I; t.nb32I = a.nb32I;
  t.h = a.h; t.hs = a.hs; t.hm = a.hm; t.hb_hi = a.hq_hi; t.hb_lo = a.hq_lo;
  const bool lo = a.xq_lo != nullptr;
  const bool one = a.T == 1;
#define MOE_SMALL(F, NM, LO, MODE, S) \
  (one ? launch_small_t<F, NM, LO, MODE, true>(t, a.max_small, S) : launch_small_t<F, NM, LO, MODE, false>(t, a.max_small, S))
#define MOE_SMALL_SEL(F, LO)                                                                        \
  (one ? launch_small_t<F, 2, LO, MODE_GATEUP, true, true>(t, a.max_small, ss)                      \
       : launch_small_t<F, 2, LO, MODE_GATEUP, false, true>(t, a.max_small, ss))
  // The small tiles (their gate/up, the conversion of their rows of h, their down) and the large
  // tiles (the same three) touch disjoint rows of h and of y: with a second stream the two chains
  // run concurrently, the small tiles' streaming of the light experts' weights beside the large
  // tiles' matrix work.
  const bool fork = a.max_large > 0 && a.side;
  const hipStream_t ss = fork ? a.side : s;
  if (fork) {
    if ((err = hipEventRecord(a.fork, s)) != hipSuccess) return err;
    if ((err = hipStreamWaitEvent(ss, a.fork, 0)) != hipSuccess) return err;
  }
  // the rows of h as the down projection's prepared operand: the large tiles' rows, and for batches
  // of more than kSelMaxTokens tokens the small tiles' rows too (converted once per row instead of
  // in each of a tile's column workgroups)
  const bool pre = a.T > kSelMaxTokens;
  FfnTileArgs d = t;   // down: h (hi + lo) x down  ->  y_slot
  d.a_hi = a.hq_hi; d.a_lo = a.hq_lo; d.s_hi = a.hsq_hi; d.s_lo = a.hsq_lo; d.sigma = a.hsig;
  d.hf = a.h; d.hsf = a.hs; d.hmf = a.hm;
  d.K = a.I; d.N = a.H; d.nb32 = a.nb32I; d.w0 = a.down; d.w1 = a.down;
  d.y = a.y;

  // small tiles: gate/up, [conversion,] down (small tiles without the conversion scale and split
  // their rows of h themselves)
  auto small_chain = [&]() -> hipError_t {
    hipError_t e;
    t.tiles = a.small; t.tile_tok = a.small_tok; t.n_tiles = a.n_small;
    trace_pre("ffn_gateup", ss, true);
    if (a.sel) {
      t.sel = *a.sel;
      if (a.fg == FMT_Q2SM) e = lo ? MOE_SMALL_SEL(FMT_Q2SM, true) : MOE_SMALL_SEL(FMT_Q2SM, false);
      else e = lo ? MOE_SMALL_SEL(FMT_Q8_0, true) : MOE_SMALL_SEL(FMT_Q8_0, false);
    } else if (a.fg == FMT_Q2SM) {
      if (a.half_gateup && lo && !one)   // (tiles of 8 slots, staged unit by unit)
        e = launch_small_t<FMT_Q2SM, 2, true, MODE_GATEUP, false, false, false, true>(t, a.max_small, ss);
      else
        e = lo ? MOE_SMALL(FMT_Q2SM, 2, true, MODE_GATEUP, ss) : MOE_SMALL(FMT_Q2SM, 2, false, MODE_GATEUP, ss);
    } else {
      e = lo ? MOE_SMALL(FMT_Q8_0, 2, true, MODE_GATEUP, ss) : MOE_SMALL(FMT_Q8_0, 2, false, MODE_GATEUP, ss);
    }
    trace_post("ffn_gateup", ss);
    if (e != hipSuccess) return e;
    if (pre) {
      const HConvArgs c{a.h, a.hs, a.hm, a.hq_hi, a.hq_lo, a.hsq_hi, a.hsq_lo, a.hsig, a.small, a.n_small, a.I,
                        a.nb32I};
      trace_pre("hconv_small", ss);
      e = launch_hconv(c, a.max_small, a.bm_small, ss);
      trace_post("hconv_small", ss);
      if (e != hipSuccess) return e;
    }
    d.tiles = a.small; d.n_tiles = a.n_small;
    int max_dn = a.max_small;
    if (pre && a.down_small) {   // tiles of more slots where the down projection's staging holds them
      d.tiles = a.down_small; d.n_tiles = a.n_down_small;
      d.stage_rows = a.T < a.bm_down_small ? a.T : a.bm_down_small;
      max_dn = a.max_down_small;
    }
    const FfnTileArgs& t = d;   // (the launch macros take t)
    trace_pre("ffn_down", ss, true);
    if (pre)
      e = a.fd == FMT_Q2SM ? launch_small_t<FMT_Q2SM, 1, true, MODE_DOWN, false, false, true>(t, max_dn, ss)
                           : launch_small_t<FMT_Q8_0, 1, true, MODE_DOWN, false, false, true>(t, max_dn, ss);
    else
      e = a.fd == FMT_Q2SM ? MOE_SMALL(FMT_Q2SM, 1, true, MODE_DOWN, ss) : MOE_SMALL(FMT_Q8_0, 1, true, MODE_DOWN, ss);
    trace_post("ffn_down", ss);
    return e;
  };
  // large tiles: gate/up, conversion, down
  auto large_chain = [&]() -> hipError_t {
    if (a.max_large == 0) return hipSuccess;
    hipError_t e;
    t.tiles = a.large; t.n_tiles = a.n_large;
    trace_pre("ffn_gateup_large", s, true);
    e = launch_large(t, a.fg, MODE_GATEUP, lo, a.max_large, s);
    trace_post("ffn_gateup_large", s);
    if (e != hipSuccess) return e;
    const HConvArgs c{a.h, a.hs, a.hm, a.hq_hi, a.hq_lo, a.hsq_hi, a.hsq_lo, a.hsig, a.large, a.n_large, a.I,
                      a.nb32I};
    trace_pre("hconv", s);
    e = launch_hconv(c, a.max_large, kLargeTileRows, s);
    trace_post("hconv", s);
    if (e != hipSuccess) return e;
    d.tiles = a.large; d.n_tiles = a.n_large;
    trace_pre("ffn_down_large", s, true);
    e = launch_large(d, a.fd, MODE_DOWN, true, a.max_large, s);
    trace_post("ffn_down_large", s);
    return e;
  };
  err = small_chain();
  if (fork) {
    // the join, also after a failed launch: the caller's stream must not run ahead of what the
    // second stream already holds (if the join cannot be recorded, the host waits for that stream)
    hipError_t ej = hipEventRecord(a.join, ss);
    const hipError_t el = err == hipSuccess ? large_chain() : hipSuccess;
    if (ej == hipSuccess) ej = hipStreamWaitEvent(s, a.join, 0);
    if (ej != hipSuccess) (void)hipStreamSynchronize(ss);
    if (err == hipSuccess) err = el;
    if (err == hipSuccess) err = ej;
  } else if (err == hipSuccess) {
    err = large_chain();
  }
#undef MOE_SMALL_SEL
#undef MOE_SMALL
  return err;
}

}  // namespace moe
