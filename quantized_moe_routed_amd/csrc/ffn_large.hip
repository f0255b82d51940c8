// Expert FFN on fp16 matrix cores for tiles of up to 128 routed slots of one
// expert (the heavily loaded experts of a prefill batch).
//
// The arithmetic is the one of the small-tile kernel (fmt.h): every weight
// code enters the matrix cores as an exact small fp16 integer, the activation
// operand arrives prepared in the same element order, each 32-value block
// gives one fp32 product P_b that is folded in with its scale,
//     acc += (2^-6 d_b) * P_b,
// and the m-term of 2-bit blocks is one more product over the block index.
// Here the matrix instruction is v_mfma_f32_32x32x16_f16 (two per block and
// activation plane), and a workgroup of 8 waves owns 128 slots by 4 x 32 NT2
// output columns: 4 column groups by 2 row groups of 64 slots (a tile of at
// most 64 slots gives both row groups its rows, each half the contraction):
//   * The activation rows of the tile are shared by the 4 waves through LDS.
//     They are fetched by direct global->LDS loads, in stages of 8 blocks
//     (4 when the operand has a lo plane), double-buffered: the loads of stage
//     s+1 are in flight while stage s is multiplied.  Within a 64-byte row
//     block the four 16-byte groups are stored XOR-swizzled by (row / 4) mod 4,
//     so the 16-byte fragment reads of 16 consecutive lanes (16 rows) cover 16
//     distinct 16-byte bank groups: no bank conflicts (measured with the LDS
//     bank-conflict counter).
//   * Each wave reads the codes and scales of its own columns straight into
//     registers, one load group ahead (a 2-bit unit of 8 blocks, or a Q8_0 unit
//     of 2 blocks).
//   * Workgroups are numbered so that the column tiles of one slot tile are
//     consecutive on one XCD (workgroup i runs on XCD i mod 8): the tile's
//     activation rows are fetched from memory once per XCD L2.
// The epilogues are those of the small-tile kernel: h = silu(g) * u in fp32
// with its block sums and block maxima, or y_slot = acc / sigma of the row.
// The down projection's operand of the large tiles' rows is prepared between
// the two projections by hconv_kernel (below): each row of h scaled by the
// power of two of its largest |h| and split into fp16 hi and lo planes.
#include "device.h"
#include "fmt.h"
#include "launch.h"
#include "ffn.h"

namespace moe {

typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ f32x16_t mfma32(uint4 a, uint4 b, f32x16_t c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8_t, a), __builtin_bit_cast(f16x8_t, b), c, 0,
                                                0, 0);
}

constexpr int kLgRows = 128;      // slots per tile

// Value barriers: the computation of v stays ahead of every later volatile asm statement.
__device__ __forceinline__ void pin(uint4& v) {
  u32x4_t t = __builtin_bit_cast(u32x4_t, v);
  asm volatile("" : "+v"(t));
  v = __builtin_bit_cast(uint4, t);
}
__device__ __forceinline__ void pin(float& v) { asm volatile("" : "+v"(v)); }

template <int F, int NM, bool LO, int MODE, int NT2, int WM, int CG>
struct LargeCfg {
  static constexpr int UB = Codes<F>::kUnitBlocks;
  static constexpr int P = LO ? 2 : 1;                    // activation planes
  static constexpr int SB = (LO || F == FMT_Q8_0) ? 4 : 8;   // blocks per LDS stage
  static constexpr int GU = UB >= SB ? 1 : SB / UB;        // code units per weight-load group
  static constexpr int STAGE = P * SB * kLgRows * 64;     // LDS bytes per stage
  static constexpr int WC = 32 * NT2;                     // output columns per wave
  static constexpr int BN = CG * WC;                      // output columns per workgroup
  static constexpr int NW = CG * WM;                      // waves: CG column groups x WM row groups
  static constexpr int THREADS = 64 * NW;
  static constexpr int MIMAX = 4 / WM;                    // 32-row fragments per wave
  static constexpr int GPW = 8 / NW;                      // 16-row activation groups each wave fetches
};

// One wave of a workgroup: MI row fragments (0 .. MIMAX; so that the block
// loop carries no per-fragment branches) starting at tile row r0.  Every wave
// takes part in the activation loads and the barriers, also one with no rows.
// Past the contraction's end (K not a multiple of the stage) the loop runs on:
// the activation loads repeat the last block and the weight scales are zero,
// so those blocks add exact zeros.
// Columns past N (N not a multiple of the workgroup's width) are computed on
// a repeated column and not stored.
// ks (tiles of at most 64 rows, 8 waves in two row groups of 4): the two row
// groups take the same rows and split the contraction instead, so that no wave
// sits idle: row group g runs the stages from g * n_it on, its activation rows
// sit in LDS row slots 64 g .. 64 g + 63, and at the end row group 1 hands its
// sums to row group 0 through LDS, which adds them (a fixed order) and stores.
// A run-time switch, so that it adds no code path of its own.
template <int F, int NM, bool LO, int MODE, int NT2, int WM, int CG, int MI>
__device__ __forceinline__ void large_tile(const FfnTileArgs& a, int le, int p0, int rows, int ct, int r0, bool ks,
                                           const int32_t* s_slot, const float* s_inv) {
  using C = LargeCfg<F, NM, LO, MODE, NT2, WM, CG>;
  constexpr int UB = C::UB, P = C::P, SB = C::SB;
  extern __shared__ __align__(16) uint8_t lds[];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int c32 = lane & 31, g2 = lane >> 5;
  const int K = a.K, N = a.N, nb = K / 32;
  const int n_units = (nb + UB - 1) / UB;
  const int n_st = (nb + SB - 1) / SB;   // LDS stages over the contraction
  // stages this wave's row group runs, from s_base; with ks a half starts on a code unit
  const int kg = ks ? wave / CG : 0;
  const int n_it = ks ? (UB > SB ? (n_st + 3) / 4 * 2 : (n_st + 1) / 2) : n_st;
  const int s_base = kg * n_it;
  const int n0 = ct * C::BN + (wave % CG) * C::WC;
  const int64_t rbytes = Codes<F>::row_bytes(K);
  const int64_t sbytes = Codes<F>::scale_row_bytes(K);

  // the expert's matrices (uniform bases) and the lane's offsets in the row-group layout: column
  // n0 + 32 nt + c32 is row c32 % 16 of a group; unit u adds 1 KiB (codes) or the scale unit
  bool colv[NT2];
  const uint8_t* cb[NM];
  const uint8_t* sb[NM];
#pragma unroll
  for (int mt = 0; mt < NM; ++mt) {
    const QMat& w = mt ? a.w1 : a.w0;
    cb[mt] = reinterpret_cast<const uint8_t*>(w.codes) + (int64_t)le * N * rbytes;
    sb[mt] = reinterpret_cast<const uint8_t*>(w.scales) + (int64_t)le * N * sbytes;
  }
  uint32_t co[NT2], so[NT2];
#pragma unroll
  for (int nt = 0; nt < NT2; ++nt) {
    colv[nt] = n0 + 32 * nt < N;
    const int col = (colv[nt] ? n0 + 32 * nt : N - 32) + c32;
    co[nt] = (uint32_t)code_off(col, 0, n_units) + 16u * (uint32_t)g2;
    so[nt] = (uint32_t)Codes<F>::d_off(col, 0, n_units);
  }
  auto cp = [&](int nt, int mt, int u) { return cb[mt] + (co[nt] + 1024u * (uint32_t)u); };
  auto dp = [&](int nt, int mt, int u) { return sb[mt] + (so[nt] + (uint32_t)Codes<F>::kScaleUnit * (uint32_t)u); };
  // Weight registers.  A load group is what one stage consumes: one 2-bit unit (8 blocks, also
  // when a stage holds 4), or SB / 2 Q8_0 units.  For each unit: the codes of 16-byte groups g2
  // and g2 + 2 of the lane's column, and the unit's scales.
  constexpr int GU = C::GU;
  // Loaded values are first touched at the next stage (after its wait), never right after the
  // load: units past the row's end load the last unit again and get their scales zeroed then.
  uint4 cw[GU][NT2][NM][2], dw[GU][NT2][NM], cwn[GU][NT2][NM][2], dwn[GU][NT2][NM];
  bool inn[GU];
  auto load_group = [&](int g) {
#pragma unroll
    for (int j = 0; j < GU; ++j) {
      const int u = g * GU + j;
      inn[j] = u < n_units;
      const int uc = inn[j] ? u : n_units - 1;
#pragma unroll
      for (int nt = 0; nt < NT2; ++nt)
#pragma unroll
        for (int mt = 0; mt < NM; ++mt) {
          const uint8_t* c = cp(nt, mt, uc);
          cwn[j][nt][mt][0] = *reinterpret_cast<const uint4*>(c);
          cwn[j][nt][mt][1] = *reinterpret_cast<const uint4*>(c + 32);
          dwn[j][nt][mt] = load_d<F>(dp(nt, mt, uc));
        }
    }
  };
  auto next_group = [&](int g_next) {
#pragma unroll
    for (int j = 0; j < GU; ++j)
#pragma unroll
      for (int nt = 0; nt < NT2; ++nt)
#pragma unroll
        for (int mt = 0; mt < NM; ++mt) {
          cw[j][nt][mt][0] = cwn[j][nt][mt][0];
          cw[j][nt][mt][1] = cwn[j][nt][mt][1];
          dw[j][nt][mt] = inn[j] ? dwn[j][nt][mt] : make_uint4(0u, 0u, 0u, 0u);
          // every read of the previous group's loads happens here, before this stage's loads
          pin(cw[j][nt][mt][0]);
          pin(cw[j][nt][mt][1]);
          pin(dw[j][nt][mt]);
        }
    load_group(g_next);
  };
  if constexpr (MI > 0) load_group(UB > SB ? s_base * SB / UB : s_base);

  // activation rows this lane fetches: rows 16 (GPW wave + j) + lane / 4 of the tile, 16-byte
  // group (lane & 3) ^ swizzle of its LDS slot
  constexpr int GPW = C::GPW;
  const int rl = lane >> 2;
  const int grp = (lane & 3) ^ ((rl >> 2) & 3);
  const uint8_t* arow[GPW];
#pragma unroll
  for (int j = 0; j < GPW; ++j) {
    int r = 16 * (ks ? wave & 3 : GPW * wave + j) + rl;   // with ks slot group w holds rows 16 (w & 3) ..
    r = r < rows ? r : 0;
    const int64_t src = MODE == MODE_GATEUP ? a.slot_list[p0 + r] / a.k : p0 + r;
    arow[j] = reinterpret_cast<const uint8_t*>(a.a_hi) + (src * K + 8 * grp) * 2;
  }
  const int64_t lo_delta =
      LO ? (reinterpret_cast<const uint8_t*>(a.a_lo) - reinterpret_cast<const uint8_t*>(a.a_hi)) : 0;
  const uint32_t lds0 = (uint32_t)(uintptr_t)lds;
  auto issue_stage = [&](int it) {
    const uint32_t sbase = lds0 + (it & 1) * C::STAGE;
#pragma unroll
    for (int pl = 0; pl < P; ++pl)
#pragma unroll
      for (int sb = 0; sb < SB; ++sb) {
        const int b = min((s_base + it) * SB + sb, nb - 1);
#pragma unroll
        for (int j = 0; j < GPW; ++j) {
          const int rg = 16 * (GPW * wave + j);   // LDS row slot
          if (rg - 64 * kg < rows) {
            const uint32_t dst = sbase + (uint32_t)(((pl * SB + sb) * kLgRows + rg) * 64);
            dma16(arow[j] + pl * lo_delta + 64 * (int64_t)b, __builtin_amdgcn_readfirstlane(dst));
          }
        }
      }
  };
  issue_stage(0);

  // fragment reads: row 32 mi + c32, 16-byte group 2 h + g2 at its swizzled slot
  uint32_t aoff[2];
#pragma unroll
  for (int h = 0; h < 2; ++h) aoff[h] = (uint32_t)(c32 * 64 + (((2 * h + g2) ^ ((c32 >> 2) & 3)) * 16));

  f32x16_t acc[MI > 0 ? MI : 1][NT2][NM];
#pragma unroll
  for (int mi = 0; mi < MI; ++mi)
#pragma unroll
    for (int nt = 0; nt < NT2; ++nt)
#pragma unroll
      for (int mt = 0; mt < NM; ++mt)
#pragma unroll
        for (int e = 0; e < 16; ++e) acc[mi][nt][mt][e] = 0.0f;

  // The products of one block are taken pair by pair (row fragment, output matrix/tile); the
  // matrix instructions of pair q are issued between the fp32 scale-and-add of pair q - 1, so the
  // matrix cores and the vector ALUs work side by side and only two products are live at once.
  constexpr int QP = NT2 * NM;   // pairs per row fragment
  f32x16_t pprev = {};
  float dprev = 0.0f;
  auto fold = [&](int q, const f32x16_t& pv, float dv) {
    const int mi = q / QP, nt = (q / NM) % NT2, mt = q % NM;
#pragma unroll
    for (int e = 0; e < 16; ++e) acc[mi][nt][mt][e] = fmaf(dv, pv[e], acc[mi][nt][mt][e]);
  };
  uint4 afc[P][2], afn[P][2];
  // LDS addresses of this lane's fragment rows in the current stage buffer; recomputed behind an
  // opaque move at each stage, so every read is base + immediate offset (< 64 KiB)
  uint32_t rb[2];
  auto read_frags = [&](uint4 (&af)[P][2], int sb, int mi) {
#pragma unroll
    for (int pl = 0; pl < P; ++pl)
#pragma unroll
      for (int h = 0; h < 2; ++h)
        af[pl][h] = __builtin_bit_cast(uint4, *reinterpret_cast<const __attribute__((address_space(3))) u32x4_t*>(
                                                  (size_t)(rb[h] + ((pl * SB + sb) * kLgRows + 32 * mi) * 64)));
  };

  // One loop iteration = one LDS stage of SB blocks.  Order within an iteration: wait for this
  // stage's activations, switch weight groups and issue the next group's loads, unpack the first
  // block's codes, and only then issue the next stage's activation loads.  The compiler's own
  // waits for weight loads then all fall before the direct LDS loads, which it does not see;
  // a wait placed after them would also wait for them.
  for (int it = 0; it < n_it; ++it) {
    const int st = s_base + it, b0 = st * SB;
    wait_vmem();
    __syncthreads();   // stage st is in LDS; every wave is done with the buffer refilled next
    uint4 bf0[NT2][NM][2];
    float d0[NT2][NM];
    if constexpr (MI > 0) {
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        rb[h] = lds0 + (it & 1) * C::STAGE + (ks ? 64 * kg : r0) * 64 + aoff[h];
        asm volatile("" : "+v"(rb[h]));
      }
      read_frags(afn, 0, 0);
      if constexpr (UB > SB) {
        // a 2-bit unit spans two stages: switch on even stages, shift by half a unit on odd ones
        if ((st & 1) == 0) {
          next_group(b0 / UB + 1);
        } else {
#pragma unroll
          for (int nt = 0; nt < NT2; ++nt)
#pragma unroll
            for (int mt = 0; mt < NM; ++mt) {
#pragma unroll
              for (int h = 0; h < 2; ++h)
                cw[0][nt][mt][h] = make_uint4(cw[0][nt][mt][h].z, cw[0][nt][mt][h].w, 0u, 0u);
              dw[0][nt][mt] = make_uint4(dw[0][nt][mt].z, dw[0][nt][mt].w, 0u, 0u);
            }
        }
      } else {
        next_group(st + 1);
      }
#pragma unroll
      for (int nt = 0; nt < NT2; ++nt)
#pragma unroll
        for (int mt = 0; mt < NM; ++mt) {
          bf0[nt][mt][0] = Codes<F>::frag(cw[0][nt][mt][0], 0, a.kc);
          bf0[nt][mt][1] = Codes<F>::frag(cw[0][nt][mt][1], 0, a.kc);
          d0[nt][mt] = d_of<F>(dw[0][nt][mt], 0);
          // pinned here, ahead of the activation loads below
          pin(bf0[nt][mt][0]);
          pin(bf0[nt][mt][1]);
          pin(d0[nt][mt]);
        }
    }
    __builtin_amdgcn_sched_barrier(0);
    if (it + 1 < n_it) issue_stage(it + 1);
    __builtin_amdgcn_sched_barrier(0);
    if constexpr (MI > 0) {
#pragma unroll
      for (int i = 0; i < SB; ++i) {
        const int j = (i % (GU * UB)) / UB, ib = i % UB;   // unit within the group, block within the unit
        uint4 bf[NT2][NM][2];
        float d[NT2][NM];
#pragma unroll
        for (int nt = 0; nt < NT2; ++nt)
#pragma unroll
          for (int mt = 0; mt < NM; ++mt) {
            if (i == 0) {
              bf[nt][mt][0] = bf0[nt][mt][0];
              bf[nt][mt][1] = bf0[nt][mt][1];
              d[nt][mt] = d0[nt][mt];
            } else {
              bf[nt][mt][0] = Codes<F>::frag(cw[j][nt][mt][0], ib, a.kc);
              bf[nt][mt][1] = Codes<F>::frag(cw[j][nt][mt][1], ib, a.kc);
              d[nt][mt] = d_of<F>(dw[j][nt][mt], ib);
              pin(d[nt][mt]);   // converted once: the 16 folds are plain fp32 FMAs, not mixed-precision ones
            }
          }
#pragma unroll
        for (int q = 0; q < MI * QP; ++q) {
          const int mi = q / QP, nt = (q / NM) % NT2, mt = q % NM;
          if (q % QP == 0) {
#pragma unroll
            for (int pl = 0; pl < P; ++pl) {
              afc[pl][0] = afn[pl][0];
              afc[pl][1] = afn[pl][1];
            }
            if (mi + 1 < MI) read_frags(afn, i, mi + 1);
            else if (i + 1 < SB) read_frags(afn, i + 1, 0);   // next block, same stage
          }
          f32x16_t pc = {};
#pragma unroll
          for (int pl = 0; pl < P; ++pl) {
            pc = mfma32(afc[pl][0], bf[nt][mt][0], pc);
            pc = mfma32(afc[pl][1], bf[nt][mt][1], pc);
          }
          fold(q == 0 ? MI * QP - 1 : q - 1, pprev, dprev);   // the very first fold adds 0 * 0
          __builtin_amdgcn_sched_barrier(0);
          pprev = pc;
          dprev = d[nt][mt];
        }
      }
    }
  }
  if constexpr (MI > 0) fold(MI * QP - 1, pprev, dprev);

  if constexpr (Codes<F>::kHasM && MI > 0) if (kg == 0) {
    // sum_b m_b (sigma S_b): block index as the contraction, 32 blocks per step
    const int mlen = n_units * UB;   // blocks covered by the units (the rest of a step is zero)
    const uint4 zero = make_uint4(0u, 0u, 0u, 0u);
    for (int c = 0; c < (nb + 31) / 32; ++c) {
      uint4 bm[NT2][NM][2];
#pragma unroll
      for (int nt = 0; nt < NT2; ++nt)
#pragma unroll
        for (int mt = 0; mt < NM; ++mt)
#pragma unroll
          for (int h = 0; h < 2; ++h) {
            const int bb = 32 * c + 16 * h + 8 * g2;
            bm[nt][mt][h] = bb < mlen ? *reinterpret_cast<const uint4*>(dp(nt, mt, bb / UB) + 256u) : zero;
          }
#pragma unroll
      for (int mi = 0; mi < MI; ++mi) {
        int r = r0 + 32 * mi + c32;
        r = r < rows ? r : 0;
        const int64_t srow = MODE == MODE_GATEUP ? s_slot[r] / a.k : p0 + r;
        const int64_t so = srow * a.nb32 + 32 * c + 8 * g2;
        uint4 sh[2], sl[2];
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          sh[h] = *reinterpret_cast<const uint4*>(a.s_hi + so + 16 * h);
          sl[h] = *reinterpret_cast<const uint4*>(a.s_lo + so + 16 * h);
        }
#pragma unroll
        for (int nt = 0; nt < NT2; ++nt)
#pragma unroll
          for (int mt = 0; mt < NM; ++mt) {
            // a separate product, added in fp32, keeps acc out of the matrix-core registers
            f32x16_t t = {};
            t = mfma32(sh[0], bm[nt][mt][0], t);
            t = mfma32(sh[1], bm[nt][mt][1], t);
            t = mfma32(sl[0], bm[nt][mt][0], t);
            t = mfma32(sl[1], bm[nt][mt][1], t);
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[mi][nt][mt][e] += t[e];
          }
      }
    }
  }

  if (ks) {
    // row group 1's sums to row group 0, element by element through LDS (the stages are free once
    // every wave has passed the first barrier)
    float* red = reinterpret_cast<float*>(lds);
    const int cg = wave % CG;
    __syncthreads();
    if (kg == 1) {
#pragma unroll
      for (int mi = 0; mi < MI; ++mi)
#pragma unroll
        for (int nt = 0; nt < NT2; ++nt)
#pragma unroll
          for (int mt = 0; mt < NM; ++mt)
#pragma unroll
            for (int e = 0; e < 16; ++e) red[((((cg * MI + mi) * NT2 + nt) * NM + mt) * 16 + e) * 64 + lane] = acc[mi][nt][mt][e];
    }
    __syncthreads();
    if (kg == 1) return;
#pragma unroll
    for (int mi = 0; mi < MI; ++mi)
#pragma unroll
      for (int nt = 0; nt < NT2; ++nt)
#pragma unroll
        for (int mt = 0; mt < NM; ++mt)
#pragma unroll
          for (int e = 0; e < 16; ++e) acc[mi][nt][mt][e] += red[((((cg * MI + mi) * NT2 + nt) * NM + mt) * 16 + e) * 64 + lane];
  }

  // epilogue: acc[mi][nt][mt][e] is row r0 + 32 mi + 8 (e / 4) + 4 g2 + e % 4, column n0 + 32 nt + c32
#pragma unroll
  for (int mi = 0; mi < MI; ++mi) {
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const int row = r0 + 32 * mi + 8 * (e >> 2) + 4 * g2 + (e & 3);
      const bool valid = row < rows;
      if constexpr (MODE == MODE_DOWN) {
        if (valid) {
          const int64_t slot = s_slot[row];
#pragma unroll
          for (int nt = 0; nt < NT2; ++nt)
            if (colv[nt]) a.y[slot * N + n0 + 32 * nt + c32] = acc[mi][nt][0][e] * s_inv[row];
        }
      } else {
        // NT2 == 1: the wave's 32 columns are exactly block n0 / 32 of h
        float h = 0.0f;
        if (valid && colv[0]) {
          const float inv = s_inv[row];
          h = silu(acc[mi][0][0][e] * inv) * (acc[mi][0][1][e] * inv);
          a.h[(int64_t)(p0 + row) * a.I + n0 + 8 * (c32 >> 3) + frag_val(c32 & 7)] = h;
        }
        // block sum over the 32 lanes of this row (fixed order) and the block's largest |h|
        float hs = h, hm = fabsf(h);
#pragma unroll
        for (int m = 1; m < 32; m <<= 1) {
          hs += __shfl_xor(hs, m, kWave);
          hm = fmaxf(hm, __shfl_xor(hm, m, kWave));
        }
        if (valid && colv[0] && c32 == 0) {
          const int64_t at = (int64_t)(p0 + row) * a.nb32I + n0 / 32;
          a.hs[at] = hs;
          a.hm[at] = hm;
        }
      }
    }
  }
  if (MODE == MODE_GATEUP && ct == 0 && wave == 0) {
    const int nbI = a.I / 32, npad = a.nb32I - nbI;
    for (int j = lane; j < kLgRows * npad; j += kWave) {
      const int row = j % kLgRows, bb = nbI + j / kLgRows;
      if (row < rows) a.hs[(int64_t)(p0 + row) * a.nb32I + bb] = 0.0f;
    }
  }
}

template <int F, int NM, bool LO, int MODE, int NT2, int WM, int CG>
__global__ __launch_bounds__((LargeCfg<F, NM, LO, MODE, NT2, WM, CG>::THREADS), 1) void ffn_large_kernel(
    FfnTileArgs a, int n_ct) {
  using C = LargeCfg<F, NM, LO, MODE, NT2, WM, CG>;
  // workgroup i runs on XCD i mod 8: the column tiles of one slot tile are consecutive on one XCD
  const int id = blockIdx.x, q = id >> 3;
  const int tile = (id & 7) + 8 * (q / n_ct), ct = q % n_ct;
  if (tile >= *a.n_tiles) return;   // the whole workgroup
  const int4 tl = a.tiles[tile];
  // per-row slot and inverse row scale of the tile (the token's, or that of the row of h), for the
  // m-term and the epilogue; written by the first 128 threads, made visible by the first stage
  // barrier inside the tile loop
  __shared__ int32_t s_slot[kLgRows];
  __shared__ float s_inv[kLgRows];
  if (threadIdx.x < kLgRows) {
    const int r = (int)threadIdx.x < tl.z ? (int)threadIdx.x : 0;
    const int32_t sl = a.slot_list[tl.y + r];
    s_slot[threadIdx.x] = sl;
    // a power of two: exact
    s_inv[threadIdx.x] = 1.0f / (MODE == MODE_GATEUP ? a.sigma[sl / a.k] : a.sigma[tl.y + r]);
  }
  const int wm = __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6) / CG;
  int r0 = wm * 32 * C::MIMAX;
  const int mi = min(max((tl.z - r0 + 31) / 32, 0), C::MIMAX);
  bool ks = false;
#define MOE_TILE(M) large_tile<F, NM, LO, MODE, NT2, WM, CG, M>(a, tl.x, tl.y, tl.z, ct, r0, ks, s_slot, s_inv)
  if constexpr (C::MIMAX == 4) {
    switch (mi) {
      case 1: MOE_TILE(1); break;
      case 2: MOE_TILE(2); break;
      case 3: MOE_TILE(3); break;
      default: MOE_TILE(4); break;
    }
  } else {
    static_assert(C::MIMAX != 2 || (CG == 4 && C::GPW == 1), "the split contraction: 8 waves, one slot group each");
    static_assert(CG * C::MIMAX * NT2 * NM * 16 * 64 * 4 <= 2 * C::STAGE, "row group 1's sums fit the stages");
    // at most 64 rows: both row groups on them, each on half the contraction
    ks = tl.z <= 64;
    if (ks) r0 = 0;
    if ((ks ? tl.z : mi * 32) <= 32) MOE_TILE(1);
    else MOE_TILE(2);
  }
#undef MOE_TILE
}

template <int F, int NM, bool LO, int MODE, int NT2, int WM, int CG>
static hipError_t launch_large_t(const FfnTileArgs& t, int max_tiles, hipStream_t s) {
  using C = LargeCfg<F, NM, LO, MODE, NT2, WM, CG>;
  const size_t lds = 2 * (size_t)C::STAGE;
  // set on every launch (a host-side call): the attribute belongs to the kernel on the device that
  // launches it, and no state is kept between calls
  const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&ffn_large_kernel<F, NM, LO, MODE, NT2, WM, CG>),
                                           hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (e != hipSuccess) return e;
  const int n_ct = (t.N + C::BN - 1) / C::BN;
  const int grid = 8 * n_ct * ((max_tiles + 7) / 8);
  return launch_stamped(ffn_large_kernel<F, NM, LO, MODE, NT2, WM, CG>, dim3(grid), dim3(C::THREADS), lds, s, t, n_ct);
}

// The down projection's operand of the rows of a tile list (the large tiles; for batches of more
// than kSelMaxTokens tokens the small tiles too).  Workgroup (tile, q) takes rows
// 8 q .. 8 q + 7 of the tile, a wave per row: the row's scale from its block maxima (row_scale, the
// rule of the activation operand), then h times 2^6 sigma and the block sums times sigma as fp16
// hi + lo pairs.  Each row is read and written once.
constexpr int kConvWaves = 8;

__global__ __launch_bounds__(kConvWaves * kWave) void hconv_kernel(HConvArgs c) {
  const int tile = blockIdx.x;
  if (tile >= *c.n_tiles) return;
  const int4 tl = c.tiles[tile];
  const int r = blockIdx.y * kConvWaves + (int)(threadIdx.x / kWave), lane = threadIdx.x % kWave;
  if (r >= tl.z) return;   // the whole wave
  const int64_t p = tl.y + r;
  const int nb = c.I / 32;
  float m = 0.0f;
  for (int b = lane; b < nb; b += kWave) m = fmaxf(m, c.hm[p * c.nb32I + b]);
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) m = fmaxf(m, __shfl_xor(m, o, kWave));
  const float sg = row_scale(m);
  if (lane == 0) c.hsig[p] = sg;
  for (int ch = lane; ch < c.I / 8; ch += kWave) {
    const float4* src = reinterpret_cast<const float4*>(c.h + p * c.I + 8 * ch);
    const float4 v0 = src[0], v1 = src[1];
    const float v[8] = {v0.x, v0.y, v0.z, v0.w, v1.x, v1.y, v1.z, v1.w};
    uint4 hi, lo;
    split8(v, sg * 64.0f, hi, lo);
    *reinterpret_cast<uint4*>(c.hq_hi + p * c.I + 8 * ch) = hi;
    *reinterpret_cast<uint4*>(c.hq_lo + p * c.I + 8 * ch) = lo;
  }
  for (int b = lane; b < c.nb32I; b += kWave) {   // (the padding blocks hold zeros)
    uint32_t hi, lo;
    split_f16(c.hs[p * c.nb32I + b] * sg, hi, lo);
    c.hsq_hi[p * c.nb32I + b] = (uint16_t)hi;
    c.hsq_lo[p * c.nb32I + b] = (uint16_t)lo;
  }
}

hipError_t launch_hconv(const HConvArgs& c, int max_tiles, int max_rows, hipStream_t s) {
  hconv_kernel<<<dim3(max_tiles, (max_rows + kConvWaves - 1) / kConvWaves), kConvWaves * kWave, 0, s>>>(c);
  return hipGetLastError();
}

// Two row groups of waves (8 waves, two per SIMD): each wave holds half the accumulators, and
// one wave's matrix products run beside the other's vector work.
hipError_t launch_large(const FfnTileArgs& t, int fmt, int mode, bool lo, int max_tiles, hipStream_t s) {
  if (mode == MODE_GATEUP) {
    if (fmt == FMT_Q2SM)
      return lo ? launch_large_t<FMT_Q2SM, 2, true, MODE_GATEUP, 1, 2, 4>(t, max_tiles, s)
                : launch_large_t<FMT_Q2SM, 2, false, MODE_GATEUP, 1, 2, 4>(t, max_tiles, s);
    return lo ? launch_large_t<FMT_Q8_0, 2, true, MODE_GATEUP, 1, 2, 4>(t, max_tiles, s)
              : launch_large_t<FMT_Q8_0, 2, false, MODE_GATEUP, 1, 2, 4>(t, max_tiles, s);
  }
  return fmt == FMT_Q2SM ? launch_large_t<FMT_Q2SM, 1, true, MODE_DOWN, 2, 2, 4>(t, max_tiles, s)
                         : launch_large_t<FMT_Q8_0, 1, true, MODE_DOWN, 2, 2, 4>(t, max_tiles, s);
}

}  // namespace moe
