// Router scoring and top-k selection.
//
// Logits follow one fixed fp32 order so that expert ids are reproducible bit
// for bit (this file is compiled with -ffp-contract=off and every fused
// multiply-add is written out):
//   per 32-block b:  p = 0; p = fma(wq_i, x_i, p) for i = 0..31 in turn
//                    r_b = d_b * p            (Q8_0; an fp32 router has r_b = p)
//   z = balanced pairwise sum over b: (r0 + r1), (r2 + r3), ... level by level,
//       an odd last element carried up unchanged;  then z += bias.
// Three layouts take these sums.  fp32 router: a wave holds one expert row,
// lane l owns the C consecutive blocks l*C .. l*C+C-1, adds them pairwise in
// registers (the first log2 C levels of the tree) and the remaining levels are
// an xor butterfly across lanes, which adds adjacent subtrees exactly as the
// tree does (IEEE addition commutes).  Q8_0 router, batches below 16 tokens: a
// wave per 16 experts and four units, a workgroup per aligned range of 32
// blocks.  Q8_0 router, 16+ tokens: a token per lane, a workgroup per aligned
// range.  The last two write each range's subtree sum; the selection adds the
// ranges pairwise (the tree's top levels) and then the bias.  Blocks past the
// last contribute +0.0: padding the tree with zeros changes no value, so the
// result equals the carry-up tree for any block count.
#include <type_traits>

#include "device.h"
#include "fmt.h"
#include "launch.h"
#include "select.h"
#include "prep.h"

namespace moe {

// f(integral_constant<int, I>) for I = B .. E-1, unrolled at compile time
template <int B, int E, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (B < E) {
    f(std::integral_constant<int, B>{});
    static_for<B + 1, E>(f);
  }
}

constexpr int kRouteTokTile = 16;

// The 32 activations of one block as fp32 (fp32 or bf16 input).
template <int ACT>
__device__ __forceinline__ void load_x_block(const void* __restrict__ x, int64_t off, float (&xv)[32]) {
  if constexpr (ACT == ACT_F32) {
    const float4* x4 = reinterpret_cast<const float4*>(reinterpret_cast<const float*>(x) + off);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float4 v = x4[i];
      xv[4 * i] = v.x;
      xv[4 * i + 1] = v.y;
      xv[4 * i + 2] = v.z;
      xv[4 * i + 3] = v.w;
    }
  } else {
    const uint4* x4 = reinterpret_cast<const uint4*>(reinterpret_cast<const uint16_t*>(x) + off);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint4 v = x4[i];
      const uint32_t wds[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        xv[8 * i + 2 * q] = __uint_as_float(wds[q] << 16);
        xv[8 * i + 2 * q + 1] = __uint_as_float(wds[q] & 0xFFFF0000u);
      }
    }
  }
}

// The C blocks lane*C .. lane*C+C-1 of fp32 router row e; blocks past H/32 are zero.
template <int C>
__device__ __forceinline__ void load_router_blocks(const float* __restrict__ codes, int e, int H, int lane,
                                                   float (&wv)[C][32]) {
  const int nb = H / 32;
#pragma unroll
  for (int j = 0; j < C; ++j) {
    const int b = lane * C + j;
    if (b < nb) {
      const float4* w4 = reinterpret_cast<const float4*>(codes + (int64_t)e * H + b * 32);
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const float4 v = w4[i];
        wv[j][4 * i] = v.x;
        wv[j][4 * i + 1] = v.y;
        wv[j][4 * i + 2] = v.z;
        wv[j][4 * i + 3] = v.w;
      }
    } else {
#pragma unroll
      for (int i = 0; i < 32; ++i) wv[j][i] = 0.0f;
    }
  }
}

// z of one (token, expert) pair from the lane's block chains r[0..C-1]: the first log2 C levels of
// the pairwise tree in registers, the rest an xor butterfly across the wave (every lane ends with z).
template <int C>
__device__ __forceinline__ float tree_sum(float (&r)[C]) {
#pragma unroll
  for (int w = 1; w < C; w <<= 1) {
#pragma unroll
    for (int j = 0; j + w < C; j += 2 * w) r[j] = r[j] + r[j + w];
  }
  float v = r[0];
#pragma unroll
  for (int m = 1; m < kWave; m <<= 1) v = v + __shfl_xor(v, m, kWave);
  return v;
}


// fp32 router: one expert per wave, C blocks per lane; per token the block chains, then the tree
// (its first levels in the lane, the rest across the wave), plus the bias.
template <int ACT, int C>
__global__ __launch_bounds__(256) void route_logits_kernel(const void* __restrict__ x, int T, int H,
                                                           const void* __restrict__ codes,
                                                           const float* __restrict__ bias, int E,
                                                           float* __restrict__ z, PrepOut po) {
  // workgroups past the logits' ones (first row only) prepare one token's expert operand each
  const int n_logit_wg = (E + 3) / 4;
  if ((int)blockIdx.x >= n_logit_wg) {
    if (blockIdx.y == 0)
      prep_token<ACT, 256>(x, blockIdx.x - n_logit_wg, H, po.nb32, po.xq_hi, po.xq_lo, po.sq_hi, po.sq_lo, po.sigma);
    return;
  }
  const int lane = threadIdx.x % kWave;
  const int e = blockIdx.x * (blockDim.x / kWave) + threadIdx.x / kWave;
  if (e >= E) return;
  const int nb = H / 32;

  float wv[C][32];
  load_router_blocks<C>(reinterpret_cast<const float*>(codes), e, H, lane, wv);
  const float be = bias ? bias[e] : 0.0f;

  const int t0 = blockIdx.y * kRouteTokTile;
  const int t1 = min(T, t0 + kRouteTokTile);
  for (int t = t0; t < t1; ++t) {
    float r[C];
#pragma unroll
    for (int j = 0; j < C; ++j) {
      const int b = lane * C + j;
      r[j] = 0.0f;
      if (b < nb) {
        float xv[32];
        load_x_block<ACT>(x, (int64_t)t * H + b * 32, xv);
        float p = 0.0f;
#pragma unroll
        for (int i = 0; i < 32; ++i) p = __builtin_fmaf(wv[j][i], xv[i], p);
        r[j] = p;
      }
    }
    const float v = tree_sum<C>(r);
    if (lane == 0) z[(int64_t)t * E + e] = bias ? v + be : v;
  }
}

// ---- few tokens, Q8_0 router: a wave per 16 experts -----------------------------------------
// A wave takes one row group of the router (16 experts, whose rows lie side by side in each
// 1 KB unit) and kRgUnits consecutive units (two blocks each); lane (s, r) holds the 64 bytes
// of row r in unit s, read as four 16-byte loads, and the x blocks it needs are the same for the
// 16 lanes of a unit.  Per token and lane: the two blocks' chains in index order, times d; the
// two blocks added (tree level 1), then units in pairs across lanes (levels 2 and 3), then the
// waves of the workgroup in pairs through LDS.  A workgroup covers one aligned range of
// kRgBlocks blocks and writes its subtree sum zp[range][t][e]; the ranges' sums (the tree's top
// levels) and the bias are added by the selection.  Blocks past H/32 count as zero.
constexpr int kRgWaves = 4;
constexpr int kRgUnits = 4;
constexpr int kRgBlocks = 2 * kRgUnits * kRgWaves;

static int rg_ranges(int H) { return (H / 32 + kRgBlocks - 1) / kRgBlocks; }

template <int ACT>
__global__ __launch_bounds__(kRgWaves * kWave) void route_logits_rg_kernel(const void* __restrict__ x, int T, int H,
                                                                            const void* __restrict__ codes,
                                                                            const void* __restrict__ scales, int E,
                                                                            int S, float* __restrict__ zp,
                                                                            PrepOut po) {
  // workgroups past the S ranges (first row group and token tile only) prepare one token's
  // expert operand each
  if ((int)blockIdx.x >= S) {
    if (blockIdx.y == 0 && blockIdx.z == 0)
      prep_token<ACT, kRgWaves * kWave>(x, blockIdx.x - S, H, po.nb32, po.xq_hi, po.xq_lo, po.sq_hi, po.sq_lo,
                                        po.sigma);
    return;
  }
  __shared__ float part[kRouteTokTile][kRgWaves][16];
  const int tid = threadIdx.x, lane = tid % kWave, wave = tid / kWave;
  const int r = lane & 15, su = lane >> 4;
  const int nb = H / 32, nu = (nb + 1) / 2;
  const int e = blockIdx.y * 16 + r, ec = min(e, E - 1);
  const int u = ((int)blockIdx.x * kRgWaves + wave) * kRgUnits + su, uc = min(u, nu - 1);
  const int b0 = 2 * u, b1 = 2 * u + 1;
  // every load is issued (rows past E and units past the row read the last ones and are dropped)
  const uint8_t* cp = reinterpret_cast<const uint8_t*>(codes) + code_off(ec, uc, nu);
  uint4 c[4];
#pragma unroll
  for (int g = 0; g < 4; ++g) c[g] = *reinterpret_cast<const uint4*>(cp + 16 * g);
  const uint32_t dd = *reinterpret_cast<const uint32_t*>(reinterpret_cast<const uint8_t*>(scales) +
                                                         Codes<FMT_Q8_0>::d_off(ec, uc, nu));
  const float d0 = half_bits_to_float((uint16_t)(dd & 0xFFFFu)), d1 = half_bits_to_float((uint16_t)(dd >> 16));
  // group g holds values 8g..8g+7 of block b0 (words x, y) and of block b1 (words z, w)
  float w0[32], w1[32];
#pragma unroll
  for (int g = 0; g < 4; ++g) {
    const uint32_t a[4] = {c[g].x, c[g].y, c[g].z, c[g].w};
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      w0[8 * g + i] = (float)(int8_t)(a[i / 4] >> (8 * (i % 4)));
      w1[8 * g + i] = (float)(int8_t)(a[2 + i / 4] >> (8 * (i % 4)));
    }
  }
  const int t0 = blockIdx.z * kRouteTokTile;
  const int nt = min(T - t0, kRouteTokTile);
  for (int tl = 0; tl < nt; ++tl) {
    const int64_t row = (int64_t)(t0 + tl) * H;
    float x0[32], x1[32];
    load_x_block<ACT>(x, row + 32 * min(b0, nb - 1), x0);
    load_x_block<ACT>(x, row + 32 * min(b1, nb - 1), x1);
    float p0 = 0.0f, p1 = 0.0f;
#pragma unroll
    for (int i = 0; i < 32; ++i) {
      p0 = __builtin_fmaf(w0[i], x0[i], p0);
      p1 = __builtin_fmaf(w1[i], x1[i], p1);
    }
    const float r0 = b0 < nb ? d0 * p0 : 0.0f;
    const float r1 = b1 < nb ? d1 * p1 : 0.0f;
    float v = r0 + r1;
    v = v + __shfl_xor(v, 16, kWave);
    v = v + __shfl_xor(v, 32, kWave);
    if (su == 0) part[tl][wave][r] = v;
  }
  __syncthreads();
  static_assert(kRgWaves == 4, "the workgroup's tree below has two levels");
  if (tid < nt * 16 && e < E) {
    const int tl = tid >> 4;
    const float v = (part[tl][0][r] + part[tl][1][r]) + (part[tl][2][r] + part[tl][3][r]);
    zp[((int64_t)blockIdx.x * T + t0 + tl) * E + e] = v;
  }
}

// ---- many tokens: one token per lane ------------------------------------------------------
// For batches of kLanesMinTokens tokens or more (Q8_0 router) the logits are taken with one
// token per lane.  Each lane keeps its own chains and its own pairwise tree in registers (no
// cross-lane sums); the weight of a step is the same for every lane and reaches the lanes through
// the broadcast form of a fused multiply-add: v_fmac_f32_dpp with row_newbcast:n takes its weight
// from lane n of the lane's row of 16.  A register therefore carries 16 steps' weights of one
// expert (lane 16 r + n holds step n), and one 4-byte load per lane (4 consecutive codes) plus
// four conversions give the weights of 64 steps (a Q8_0 unit, two blocks): register k holds
// steps 4 n + k.
//
// Workgroup: 4 waves = 4 groups of 8 experts x 64 tokens x one of S equal ranges of the blocks.
// The tokens' activations pass through LDS in chunks of 4 blocks, stored transposed (lane t reads
// 16 bytes of its token at slot c * 64 + (t ^ (c & 15)): conflict-free for the reads and for
// the coalesced writes).  Each lane adds its blocks pairwise in registers: the 4 blocks of a
// chunk, then the chunks with a binary counter (level j holds a complete subtree of 2^j
// chunks).  A range of 2^n blocks therefore yields exactly the subtree of the canonical tree over
// those blocks; the S subtree sums are added pairwise (the tree's top levels) by the selection
// kernel, which then adds the bias.
constexpr int kLanesMinTokens = 16;
constexpr int kLaneGroup = 8;          // experts per wave
constexpr int kLanesWaves = 4;
constexpr int kChunkBlocks = 4;
constexpr int kMaxChunkLevels = 7;     // up to 128 chunks (512 blocks) per range

struct LanesPlan {
  bool use;
  int S;              // block ranges
  int groups;         // expert groups of 8
};

static LanesPlan lanes_plan(int T, int E, int H, int fmt) {
  LanesPlan p{};
  const int nb = H / 32;
  p.use = fmt == FMT_Q8_0 && T >= kLanesMinTokens && nb >= kChunkBlocks && (nb & (nb - 1)) == 0;
  if (!p.use) return p;
  p.groups = (E + kLaneGroup - 1) / kLaneGroup;
  const long wgs = (long)((T + 63) / 64) * ((p.groups + kLanesWaves - 1) / kLanesWaves);
  p.S = 1;
  while (nb / p.S > kChunkBlocks << kMaxChunkLevels) p.S <<= 1;
  while (wgs * p.S * 2 <= 512 && nb / (p.S * 2) >= kChunkBlocks && p.S * 2 <= kMaxRanges) p.S <<= 1;
  if (p.S > kMaxRanges) p.use = false;
  return p;
}

// partial sums per (token, expert) that the logits launch writes (0: finished logits)
int logit_ranges(int T, int E, int H, int fmt) {
  const LanesPlan p = lanes_plan(T, E, H, fmt);
  if (p.use) return p.S;
  return fmt == FMT_Q8_0 ? rg_ranges(H) : 0;
}

size_t route_ws_need(int T, int E, int H, int fmt) {
  return (size_t)std::max(1, logit_ranges(T, E, H, fmt)) * T * E * sizeof(float);
}

// p += w(lane 16 r + N) * x  (fused, one rounding).  A DPP operand must not have been written by
// a vector instruction in the two instructions before; the compiler does not look inside inline
// assembly, so the weights are produced by convert_codes (which ends with two wait states) and
// the library build scans the compiled code for any such write before a broadcast.
template <int N>
__device__ __forceinline__ void fmac_bcast(float& p, float w, float x) {
  asm("v_fmac_f32_dpp %0, %1, %2 row_newbcast:%3 row_mask:0xf bank_mask:0xf" : "+v"(p) : "v"(w), "v"(x), "n"(N));
}

// The four int8 codes of a word as fp32 (sign-extending byte selects), then two wait states.
__device__ __forceinline__ void convert_codes(uint32_t w, float (&o)[4]) {
  asm("v_cvt_f32_i32_sdwa %0, sext(%4) dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:BYTE_0\n\t"
      "v_cvt_f32_i32_sdwa %1, sext(%4) dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:BYTE_1\n\t"
      "v_cvt_f32_i32_sdwa %2, sext(%4) dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:BYTE_2\n\t"
      "v_cvt_f32_i32_sdwa %3, sext(%4) dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:BYTE_3\n\t"
      "s_nop 1"
      : "=&v"(o[0]), "=&v"(o[1]), "=&v"(o[2]), "=&v"(o[3])
      : "v"(w));
}

template <int ACT>
__global__ __launch_bounds__(kLanesWaves * 64) void route_logits_lanes_kernel(
    const void* __restrict__ x, int T, int H, const void* __restrict__ codes, const void* __restrict__ scales,
    int E, int groups, int S, float* __restrict__ zp) {
  __shared__ __align__(16) float4 xs[2][kChunkBlocks * 8 * 64];   // [buf][chunk slot * 64 + token]
  const int tid = threadIdx.x, lane = tid % kWave;
  const int g = blockIdx.y * kLanesWaves + __builtin_amdgcn_readfirstlane(tid / kWave);
  const bool active = g < groups;
  const int t0 = blockIdx.x * 64;
  const int nb = H / 32, nu = nb / 2;
  const int nbr = nb / S, b_beg = blockIdx.z * nbr;
  const int n_chunks = nbr / kChunkBlocks;
  // lane 16 r + n loads codes 4 n .. 4 n + 3 of a unit's 64 steps (block 2u: n < 8, then 2u + 1)
  const int n = lane & 15;
  const int woff = (n < 8 ? 0 : 8) + 16 * ((n & 7) >> 1) + 4 * (n & 1);
  const uint8_t* cbase[kLaneGroup];
  const uint8_t* sbase[kLaneGroup];
#pragma unroll
  for (int j = 0; j < kLaneGroup; ++j) {
    const int e = min(g * kLaneGroup + j, E - 1);   // rows past E: a valid row, never stored
    cbase[j] = reinterpret_cast<const uint8_t*>(codes) + code_off(e, 0, nu) + woff;
    sbase[j] = reinterpret_cast<const uint8_t*>(scales) + Codes<FMT_Q8_0>::d_off(e, 0, nu);
  }
  uint32_t wr[kLaneGroup], dr[kLaneGroup];
  auto load_unit = [&](int u) {
#pragma unroll
    for (int j = 0; j < kLaneGroup; ++j) {
      wr[j] = *reinterpret_cast<const uint32_t*>(cbase[j] + (int64_t)u * 1024);
      dr[j] = *reinterpret_cast<const uint32_t*>(sbase[j] + (int64_t)u * Codes<FMT_Q8_0>::kScaleUnit);
    }
  };

  // staging of chunk c (4 blocks = 128 values of 64 tokens): thread tid moves the 4 values q =
  // tid + 256 i; they are held as loaded (fp32, or bf16 bits) until stored, so that the wait for
  // them falls after the chunk's arithmetic
  using Raw = typename std::conditional<ACT == ACT_F32, float4, uint2>::type;
  Raw stg[8];
  auto fetch = [&](int c) {
    const int h0 = 32 * (b_beg + kChunkBlocks * c);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int q = tid + 256 * i, tl = q / 32, cp = q % 32;
      // every load is issued (tokens past T read the last token; their lanes store nothing), so
      // that none sits behind a branch that would wait for it on the spot
      const int64_t t = min(t0 + tl, T - 1);
      stg[i] = *reinterpret_cast<const Raw*>(reinterpret_cast<const uint8_t*>(x) +
                                             (t * H + h0 + 4 * cp) * (ACT == ACT_F32 ? 4 : 2));
    }
  };
  auto store = [&](int buf) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int q = tid + 256 * i, tl = q / 32, cp = q % 32;
      float4 v;
      if constexpr (ACT == ACT_F32) {
        v = stg[i];
      } else {
        v = make_float4(__uint_as_float(stg[i].x << 16), __uint_as_float(stg[i].x & 0xFFFF0000u),
                        __uint_as_float(stg[i].y << 16), __uint_as_float(stg[i].y & 0xFFFF0000u));
      }
      xs[buf][cp * 64 + (tl ^ (cp & 15))] = v;
    }
  };

  float lv[kMaxChunkLevels + 1][kLaneGroup];   // binary counter over the chunks
#pragma unroll
  for (int l = 0; l <= kMaxChunkLevels; ++l)
#pragma unroll
    for (int j = 0; j < kLaneGroup; ++j) lv[l][j] = 0.0f;
  if (n_chunks > 0) {
    fetch(0);
    store(0);
    load_unit(b_beg / 2);
  }
  for (int c = 0; c < n_chunks; ++c) {
    const int buf = c & 1;
    if (c + 1 < n_chunks) fetch(c + 1);
    __syncthreads();   // chunk c is in xs[buf]; nobody reads xs[buf ^ 1] any more
    float v[kLaneGroup];
    // the chunk's two units, their two blocks, their 32 steps: all unrolled at compile time, as
    // the broadcast lane of a step is an immediate of its instruction
    static_for<0, 2>([&](auto uu_) {
      constexpr int uu = decltype(uu_)::value;
      // the unit's weights (register k: steps 4 n + k) and its two block scales
      float W[kLaneGroup][4], d[kLaneGroup][2];
#pragma unroll
      for (int j = 0; j < kLaneGroup; ++j) {
        convert_codes(wr[j], W[j]);
        d[j][0] = half_bits_to_float(dr[j] & 0xFFFFu);
        d[j][1] = half_bits_to_float(dr[j] >> 16);
      }
      // next unit's codes and scales (the chunk's second unit, or the next chunk's first)
      if (uu == 0 || c + 1 < n_chunks) load_unit(b_beg / 2 + 2 * c + uu + 1);
      float half_sum[kLaneGroup];
      static_for<0, 2>([&](auto hb_) {
        constexpr int hb = decltype(hb_)::value;
        float p[kLaneGroup];
#pragma unroll
        for (int j = 0; j < kLaneGroup; ++j) p[j] = 0.0f;
        static_for<0, 8>([&](auto i4_) {
          constexpr int i4 = decltype(i4_)::value;
          constexpr int cp = 16 * uu + 8 * hb + i4;   // chunk slot: values 4 cp .. 4 cp + 3
          const float4 xv = xs[buf][cp * 64 + (lane ^ (cp & 15))];
          const float xq[4] = {xv.x, xv.y, xv.z, xv.w};
          // step 32 hb + 4 i4 + k of the unit: weight register k, broadcast lane 8 hb + i4
#pragma unroll
          for (int k = 0; k < 4; ++k)
#pragma unroll
            for (int j = 0; j < kLaneGroup; ++j) fmac_bcast<8 * hb + i4>(p[j], W[j][k], xq[k]);
        });
        // r_b = d_b * p_b, then the chunk's blocks pairwise: ((b0 + b1) + (b2 + b3))
#pragma unroll
        for (int j = 0; j < kLaneGroup; ++j) {
          const float r = d[j][hb] * p[j];
          half_sum[j] = hb == 0 ? r : half_sum[j] + r;
        }
      });
#pragma unroll
      for (int j = 0; j < kLaneGroup; ++j) v[j] = uu == 0 ? half_sum[j] : v[j] + half_sum[j];
    });
    if (active) {
      bool placed = false;
#pragma unroll
      for (int l = 0; l < kMaxChunkLevels; ++l) {
        if (!placed) {
          if (!((c >> l) & 1)) {
#pragma unroll
            for (int j = 0; j < kLaneGroup; ++j) lv[l][j] = v[j];
            placed = true;
          } else {
#pragma unroll
            for (int j = 0; j < kLaneGroup; ++j) v[j] = lv[l][j] + v[j];
          }
        }
      }
      if (!placed) {
#pragma unroll
        for (int j = 0; j < kLaneGroup; ++j) lv[kMaxChunkLevels][j] = v[j];
      }
    }
    if (c + 1 < n_chunks) store(buf ^ 1);
  }
  // n_chunks = 2^L: the range's sum is the subtree at level L
  const int t = t0 + lane;
  if (active && t < T && n_chunks > 0) {
    const int L = 31 - __builtin_clz(n_chunks);
    float r[kLaneGroup];
#pragma unroll
    for (int j = 0; j < kLaneGroup; ++j) r[j] = lv[0][j];
#pragma unroll
    for (int l = 1; l <= kMaxChunkLevels; ++l)
      if (L == l) {
#pragma unroll
        for (int j = 0; j < kLaneGroup; ++j) r[j] = lv[l][j];
      }
    float* dst = zp + ((int64_t)blockIdx.z * T + t) * E + g * kLaneGroup;
#pragma unroll
    for (int j = 0; j < kLaneGroup; ++j)
      if (g * kLaneGroup + j < E) dst[j] = r[j];
  }
}

template <int EPL>
__global__ __launch_bounds__(256) void route_topk_kernel(const float* __restrict__ z, int S,
                                                         const float* __restrict__ bias, int T, int E, int k,
                                                         int32_t* __restrict__ ids, float* __restrict__ w) {
  extern __shared__ uint64_t tk_cand[];   // E + kThrMaxK candidates per wave
  const int t = blockIdx.x * (blockDim.x / kWave) + threadIdx.x / kWave;
  if (t < T)
    topk_token<EPL>(z, S, bias, T, E, k, t, ids, w, nullptr, tk_cand + (size_t)(threadIdx.x / kWave) * (E + kThrMaxK));
}

// Many partial ranges (S >= 16): a workgroup of 4 waves per token.  Wave q adds its quarter of the
// M ranges (M the power of two that holds S) by the lower levels of the pairwise tree, exactly as
// logit_keys does for those indices, and leaves the quarter sums in LDS; wave 0 adds the quarters by
// the tree's two top levels, then the bias, and selects as topk_lanes.  The same additions in the
// same order: the same keys, and the loads of a token spread over four waves instead of one.
constexpr int kSplitWaves = 4;

template <int EPL, int M>
__global__ __launch_bounds__(kSplitWaves * kWave) void route_topk_split_kernel(const float* __restrict__ z, int S,
                                                                               const float* __restrict__ bias, int T,
                                                                               int E, int k, int32_t* __restrict__ ids,
                                                                               float* __restrict__ w) {
  static_assert(M % kSplitWaves == 0, "whole quarters");
  constexpr int G = M / kSplitWaves;   // ranges per wave
  __shared__ float qs[kSplitWaves][EPL * kWave];
  __shared__ uint64_t cand[EPL * kWave + kThrMaxK];
  const int t = blockIdx.x, lane = threadIdx.x % kWave;
  const int q = __builtin_amdgcn_readfirstlane((int)threadIdx.x / kWave);
  int ec[EPL];
#pragma unroll
  for (int i = 0; i < EPL; ++i) ec[i] = min(i * kWave + lane, E - 1);
  {
    float v[EPL][G];
#pragma unroll
    for (int jj = 0; jj < G; ++jj) {
      const float* zj = z + ((int64_t)min(q * G + jj, S - 1) * T + t) * E;
#pragma unroll
      for (int i = 0; i < EPL; ++i) v[i][jj] = zj[ec[i]];
    }
#pragma unroll
    for (int i = 0; i < EPL; ++i) {
#pragma unroll
      for (int wd = 1; wd < G; wd <<= 1)
#pragma unroll
        for (int jj = 0; jj + wd < G; jj += 2 * wd) {
          const int j = q * G + jj;   // the pair's left index in the whole tree
          v[i][jj] = j + wd < S ? v[i][jj] + v[i][jj + wd] : v[i][jj];
        }
      qs[q][i * kWave + lane] = v[i][0];
    }
  }
  __syncthreads();
  if (q != 0) return;
  uint32_t key[EPL];
  bool live[EPL];
#pragma unroll
  for (int i = 0; i < EPL; ++i) {
    live[i] = i * kWave + lane < E;
    const float bv = bias ? bias[ec[i]] : 0.0f;
    const float a0 = qs[0][i * kWave + lane], a1 = qs[1][i * kWave + lane];
    const float a2 = qs[2][i * kWave + lane], a3 = qs[3][i * kWave + lane];
    const float l = G < S ? a0 + a1 : a0;            // pair (0, G)
    const float r = 3 * G < S ? a2 + a3 : a2;        // pair (2G, 3G)
    const float zs = 2 * G < S ? l + r : l;          // pair (0, 2G)
    key[i] = live[i] ? float_key(bias ? zs + bv : zs) : 0u;
  }
  int my_id;
  uint32_t my_key;
  topk_of_keys<EPL>(key, live, E, k, lane, cand, my_id, my_key);
  if (w) topk_store(k, t, my_id, my_key, ids, w);
}

template <int ACT>
static hipError_t launch_logits_c(int C, const void* x, int T, int H, const QMat& r, const float* bias,
                                  float* z, const PrepOut& po, hipStream_t s) {
  const int E = r.rows;
  dim3 grid((E + 3) / 4 + (po.xq_hi ? T : 0), (T + kRouteTokTile - 1) / kRouteTokTile);
  switch (C) {
    case 1: route_logits_kernel<ACT, 1><<<grid, 256, 0, s>>>(x, T, H, r.codes, bias, E, z, po); break;
    case 2: route_logits_kernel<ACT, 2><<<grid, 256, 0, s>>>(x, T, H, r.codes, bias, E, z, po); break;
    case 4: route_logits_kernel<ACT, 4><<<grid, 256, 0, s>>>(x, T, H, r.codes, bias, E, z, po); break;
    case 8: route_logits_kernel<ACT, 8><<<grid, 256, 0, s>>>(x, T, H, r.codes, bias, E, z, po); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_logits(const void* x, int act, int T, int H, int fmt, const QMat& router, const float* bias,
                         void* ws, int* S_out, hipStream_t s, const PrepOut* prep) {
  const PrepOut po = prep ? *prep : PrepOut{};
  const int E = router.rows;
  const bool q8 = fmt == FMT_Q8_0;
  hipError_t err = hipSuccess;
  const LanesPlan lp = lanes_plan(T, E, H, fmt);
  float* z = reinterpret_cast<float*>(ws);
  int S = 0;
  if (lp.use && po.xq_hi) return hipErrorInvalidValue;   // operands ride only on the small-batch launch
  if (lp.use) {
    const dim3 grid((T + 63) / 64, (lp.groups + kLanesWaves - 1) / kLanesWaves, lp.S);
    trace_pre("route_logits", s);
    if (act == ACT_F32)
      route_logits_lanes_kernel<ACT_F32><<<grid, kLanesWaves * 64, 0, s>>>(x, T, H, router.codes, router.scales, E, lp.groups, lp.S, z);
    else
      route_logits_lanes_kernel<ACT_BF16><<<grid, kLanesWaves * 64, 0, s>>>(x, T, H, router.codes, router.scales, E, lp.groups, lp.S, z);
    trace_post("route_logits", s);
    err = hipGetLastError();
    S = lp.S;
  } else if (q8) {
    S = rg_ranges(H);
    if (S > kMaxRanges) return hipErrorInvalidValue;
    const dim3 grid(S + (po.xq_hi ? T : 0), (E + 15) / 16, (T + kRouteTokTile - 1) / kRouteTokTile);
    trace_pre("route_logits", s);
    if (act == ACT_F32)
      route_logits_rg_kernel<ACT_F32><<<grid, kRgWaves * kWave, 0, s>>>(x, T, H, router.codes, router.scales, E, S, z, po);
    else
      route_logits_rg_kernel<ACT_BF16><<<grid, kRgWaves * kWave, 0, s>>>(x, T, H, router.codes, router.scales, E, S, z, po);
    trace_post("route_logits", s);
    err = hipGetLastError();
  } else {   // fp32 router
    const int nb = H / 32;
    int C = 1;
    while (C * kWave < nb) C <<= 1;
    trace_pre("route_logits", s);
    err = act == ACT_F32 ? launch_logits_c<ACT_F32>(C, x, T, H, router, bias, z, po, s)
                         : launch_logits_c<ACT_BF16>(C, x, T, H, router, bias, z, po, s);
    trace_post("route_logits", s);
  }
  *S_out = S;
  return err;
}

// Table routing, one wave per token: lane j < k takes expert table[token_ids[t]][j] (both indices
// clamped into range, so no read leaves the arrays), its logit as the selection forms it (the S
// partial sums added pairwise, level by level, then the bias; S = 0: z holds the logit), and the
// weights by the top-k's rule, in the table row's order.
__global__ __launch_bounds__(256) void route_table_kernel(const float* __restrict__ z, int S,
                                                          const float* __restrict__ bias, int T, int E, int k,
                                                          const int32_t* __restrict__ token_ids,
                                                          const int32_t* __restrict__ table, int V,
                                                          int32_t* __restrict__ ids, float* __restrict__ w) {
  const int t = blockIdx.x * 4 + (int)threadIdx.x / kWave;
  if (t >= T) return;   // the whole wave
  const int lane = threadIdx.x % kWave;
  int e = 0;
  float zl = 0.0f;
  if (lane < k) {
    const int tok = min(max(token_ids[t], 0), V - 1);
    e = min(max(table[(int64_t)tok * k + lane], 0), E - 1);
    if (S == 0) {
      zl = z[(int64_t)t * E + e];
    } else {
      float v[kMaxRanges];
#pragma unroll
      for (int j = 0; j < kMaxRanges; ++j) v[j] = j < S ? z[((int64_t)j * T + t) * E + e] : 0.0f;
#pragma unroll
      for (int h = 1; h < kMaxRanges; h <<= 1)
#pragma unroll
        for (int j = 0; j + h < kMaxRanges; j += 2 * h) v[j] = j + h < S ? v[j] + v[j + h] : v[j];
      zl = bias ? v[0] + bias[e] : v[0];
    }
  }
  topk_store(k, t, e, float_key(zl), ids, w);
}

hipError_t launch_route_table(const void* x, int act, int T, int H, int fmt, const QMat& router, const float* bias,
                              const int32_t* token_ids, const int32_t* table, int V, int k, int32_t* ids, float* w,
                              void* ws, hipStream_t s) {
  int S = 0;
  hipError_t err = launch_logits(x, act, T, H, fmt, router, bias, ws, &S, s, nullptr);
  if (err != hipSuccess) return err;
  if (S > kMaxRanges) return hipErrorInvalidValue;
  trace_pre("route_table", s);
  route_table_kernel<<<(T + 3) / 4, 256, 0, s>>>(reinterpret_cast<const float*>(ws), S, bias, T, router.rows, k,
                                                  token_ids, table, V, ids, w);
  trace_post("route_table", s);
  return hipGetLastError();
}

hipError_t launch_route(const void* x, int act, int T, int H, int fmt, const QMat& router, const float* bias,
                        int k, int32_t* ids, float* w, void* ws, hipStream_t s) {
  const int E = router.rows;
  int S = 0;
  hipError_t err = launch_logits(x, act, T, H, fmt, router, bias, ws, &S, s, nullptr);
  if (err != hipSuccess) return err;
  const float* z = reinterpret_cast<const float*>(ws);
  if (S >= 16 && E <= 256) {   // the ranges of a token over four waves
    trace_pre("route_topk", s);
    if (S <= 16) route_topk_split_kernel<4, 16><<<T, kSplitWaves * kWave, 0, s>>>(z, S, bias, T, E, k, ids, w);
    else route_topk_split_kernel<4, 32><<<T, kSplitWaves * kWave, 0, s>>>(z, S, bias, T, E, k, ids, w);
    trace_post("route_topk", s);
    return hipGetLastError();
  }
  dim3 grid((T + 3) / 4);
  const size_t lds = (size_t)4 * (E + kThrMaxK) * sizeof(uint64_t);   // (at most 33 KiB: E <= 1024)
  trace_pre("route_topk", s);
  if (E <= 64) route_topk_kernel<1><<<grid, 256, lds, s>>>(z, S, bias, T, E, k, ids, w);
  else if (E <= 128) route_topk_kernel<2><<<grid, 256, lds, s>>>(z, S, bias, T, E, k, ids, w);
  else if (E <= 256) route_topk_kernel<4><<<grid, 256, lds, s>>>(z, S, bias, T, E, k, ids, w);
  else if (E <= 512) route_topk_kernel<8><<<grid, 256, lds, s>>>(z, S, bias, T, E, k, ids, w);
  else route_topk_kernel<16><<<grid, 256, lds, s>>>(z, S, bias, T, E, k, ids, w);
  trace_post("route_topk", s);
  return hipGetLastError();
}

}  // namespace moe
