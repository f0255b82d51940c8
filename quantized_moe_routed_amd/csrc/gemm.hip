// Grouped expert GEMM on bf16 matrix cores (bf16 activations): the expert FFN
// for prefill-size batches, the one place the layer is a dense contraction.
//
// Work is cut into tiles of BM routed slots of one expert (consecutive
// positions of the grouped slot list) by BN output columns.  A device-built
// tile list covers exactly the owned experts that received slots, so the grid
// is sized for the worst case and surplus workgroups exit at once; nothing is
// read back to the host.
//
// Exactness.  Weight codes enter the matrix cores as exact bf16 integers
// (2-bit codes 0..3, int8 codes -127..127), activations as the caller's bf16
// values, and one v_mfma_f32_16x16x32_bf16 covers exactly one 32-value block,
// so every block's partial dot product P is formed in fp32 before its scale is
// applied.  The block scale then enters in fp32:
//   2-bit gate/up:  acc += d * P + m * S,  S = the block's sum of x;
//   Q8_0 down:      acc += d * P.
// The intermediate h = silu(g) * u is handed to the down projection as a bf16
// pair hi + lo (hi = h rounded to bf16, lo = the remainder rounded to bf16),
// i.e. with 16 significant bits, and the down projection multiplies both.
//
// Inside one 32-block the order of the K index is free as long as activations
// and weights use the same order.  The 2-bit codes are unpacked into the order
// that a byte-table lookup (v_perm_b32) produces cheaply; the activation tile
// is written to LDS in that same order (a 4x4 transpose of 16-bit values per
// half block).  Each y_slot row is written by exactly one lane: no atomics, so
// results are bit-identical from run to run.
#include <algorithm>

#include "device.h"
#include "launch.h"

namespace moe {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

constexpr int kBM = 64;          // slots per tile
constexpr int kBN = 64;          // output columns per tile
constexpr int kBK = 64;          // contraction values per step (two 32-blocks)
constexpr int kLdsRow = kBK + 8; // bf16 per LDS row (16 bytes of padding)
constexpr int kGemmThreads = 256;

__device__ __forceinline__ f32x4_t mfma_bf16(uint4 a, uint4 b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a), __builtin_bit_cast(bf16x8_t, b),
                                                 c, 0, 0, 0);
}

// Round to the nearest bf16, ties to even (finite inputs).
__device__ __forceinline__ uint32_t bf16_rne_bits(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return u >> 16;
}

// Block sums of the activations: xs[t][b] = sum_{i<32} x[t][32b+i], summed in
// index order in fp32 (the m-term of the 2-bit blocks).
__global__ __launch_bounds__(256) void block_sums_bf16_kernel(const uint16_t* __restrict__ x, int T, int H,
                                                               float* __restrict__ xs) {
  const int nb = H / 32;
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= (int64_t)T * nb) return;
  const uint4* p = reinterpret_cast<const uint4*>(x + i * 32);
  float s = 0.0f;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const uint4 v = p[q];
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int h = 0; h < 4; ++h) {
      s += __uint_as_float(w[h] << 16);
      s += __uint_as_float(w[h] & 0xFFFF0000u);
    }
  }
  xs[i] = s;
}

// Tile list over the owned experts that received slots, in ascending global id:
// tile i covers grouped positions p0 .. p0+rows-1 of expert tile_e[i].
// Tiles past max_tiles, and rows past the n_slots grouped positions, are never
// produced, whatever the counts hold.
__global__ __launch_bounds__(1024) void gemm_tiles_kernel(const int32_t* __restrict__ counts,
                                                          const int32_t* __restrict__ offsets,
                                                          const int32_t* __restrict__ g2l, int E, int E_local,
                                                          int n_slots, int max_tiles, int4* __restrict__ tiles,
                                                          int32_t* __restrict__ n_tiles) {
  __shared__ int32_t wave_tot[16];
  const int tid = threadIdx.x, lane = tid % kWave, wave = tid / kWave;
  int n = 0, mt = 0;
  if (tid < E) {
    const int l = g2l ? g2l[tid] : tid;
    const int p = offsets[tid];
    n = (p >= 0 && p < n_slots) ? min(counts[tid], n_slots - p) : 0;
    if (n > 0 && l >= 0 && l < E_local) mt = (n + kBM - 1) / kBM;
  }
  int incl = mt;
#pragma unroll
  for (int d = 1; d < kWave; d <<= 1) {
    const int o = __shfl_up(incl, d, kWave);
    if (lane >= d) incl += o;
  }
  if (lane == kWave - 1) wave_tot[wave] = incl;
  __syncthreads();
  int base = 0;
  for (int w = 0; w < wave; ++w) base += wave_tot[w];
  base += incl - mt;
  if (mt > 0) {
    const int l = g2l ? g2l[tid] : tid;
    const int p = offsets[tid];
    for (int i = 0; i < mt && base + i < max_tiles; ++i)
      tiles[base + i] = make_int4(l, p + kBM * i, min(kBM, n - kBM * i), tid);
  }
  if (tid == 0) {
    int tot = 0;
    for (int w = 0; w < 16; ++w) tot += wave_tot[w];
    *n_tiles = min(tot, max_tiles);
  }
}

// 16 bf16 activations of a half block, natural order in w[0..7], rewritten in
// the order the 2-bit unpacking produces: value 4r+s goes to position 4s+r.
__device__ __forceinline__ void transpose_half_block(const uint32_t w[8], uint32_t o[8]) {
  o[0] = __builtin_amdgcn_perm(w[2], w[0], 0x05040100u);
  o[1] = __builtin_amdgcn_perm(w[6], w[4], 0x05040100u);
  o[2] = __builtin_amdgcn_perm(w[2], w[0], 0x07060302u);
  o[3] = __builtin_amdgcn_perm(w[6], w[4], 0x07060302u);
  o[4] = __builtin_amdgcn_perm(w[3], w[1], 0x05040100u);
  o[5] = __builtin_amdgcn_perm(w[7], w[5], 0x05040100u);
  o[6] = __builtin_amdgcn_perm(w[3], w[1], 0x07060302u);
  o[7] = __builtin_amdgcn_perm(w[7], w[5], 0x07060302u);
}

// 16 two-bit codes (one 32-bit word: value 4j+s at byte j, bits 2s) -> 16 bf16
// integers in the order value 4r+s at position 4s+r.  A byte table maps a
// code to the two bytes of its bf16 value (0, 1.0, 2.0, 3.0).
__device__ __forceinline__ void unpack_q2_half(uint32_t c, uint32_t o[8]) {
  constexpr uint32_t kLo = 0x40008000u;   // low bytes of bf16 0, 1, 2, 3
  constexpr uint32_t kHi = 0x40403F00u;   // high bytes
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    const uint32_t t = (c >> (2 * s)) & 0x03030303u;
    const uint32_t t4 = t | 0x04040404u;
    const uint32_t sa = __builtin_amdgcn_perm(t4, t, 0x05010400u);
    const uint32_t sb = __builtin_amdgcn_perm(t4, t, 0x07030602u);
    o[2 * s] = __builtin_amdgcn_perm(kHi, kLo, sa);
    o[2 * s + 1] = __builtin_amdgcn_perm(kHi, kLo, sb);
  }
}

// gate/up for one tile: h = silu(G x) * (U x), written as bf16 hi/lo planes at
// the tile's grouped positions.
__global__ __launch_bounds__(kGemmThreads) void gemm_gateup_kernel(
    const uint16_t* __restrict__ x, int H, int I, int k, QMat gate, QMat up, const int32_t* __restrict__ slot_list,
    const float* __restrict__ xs, const int4* __restrict__ tiles, const int32_t* __restrict__ n_tiles,
    uint16_t* __restrict__ h_hi, uint16_t* __restrict__ h_lo) {
  const int tile = blockIdx.y;
  if (tile >= *n_tiles) return;
  __shared__ __align__(16) uint16_t As[kBM][kLdsRow];
  __shared__ __align__(16) uint16_t Bs[2][kBN][kLdsRow];
  __shared__ float2 Sc[2][2][kBN];   // [matrix][block][column] = (d, m)
  __shared__ __align__(16) float Ss[2][kBM];   // [block][row] = block sum of x

  const int4 tl = tiles[tile];
  const int le = tl.x, p0 = tl.y, rows = tl.z;
  const int n0 = blockIdx.x * kBN;
  const int nb = H / 32;
  const int tid = threadIdx.x, lane = tid % kWave, wave = tid / kWave;
  const int wm = wave >> 1, wn = wave & 1;

  // staging roles
  const int xr = tid >> 2, xhb = tid & 3;                       // x: row, half block
  const int xtok = xr < rows ? slot_list[p0 + xr] / k : -1;
  const int cmat = tid >> 7, ccol = (tid >> 1) & 63, cblk = tid & 1;  // codes: matrix, column, block
  const QMat& cm = cmat ? up : gate;
  const int64_t crow = (int64_t)le * I + n0 + ccol;
  const uint8_t* cptr = reinterpret_cast<const uint8_t*>(cm.codes) + crow * (int64_t)(H / 4) + cblk * 8;
  const uint32_t* sptr = reinterpret_cast<const uint32_t*>(cm.scales) + crow * nb + cblk;
  const int sblk = tid >> 6, srow = tid & 63;                   // block sums (threads < 128)
  const int stok = (tid < 128 && srow < rows) ? slot_list[p0 + srow] / k : -1;

  f32x4_t ag[2][2], au[2][2];
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int b = 0; b < 2; ++b) {
      ag[a][b] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
      au[a][b] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
    }
  const f32x4_t zero4 = {0.0f, 0.0f, 0.0f, 0.0f};

  for (int kb = 0; kb < nb; kb += 2) {
    // global loads for this step
    uint32_t xw[8];
    if (xtok >= 0) {
      const uint4* xp = reinterpret_cast<const uint4*>(x + (int64_t)xtok * H + kb * 32 + xhb * 16);
      const uint4 v0 = xp[0], v1 = xp[1];
      xw[0] = v0.x; xw[1] = v0.y; xw[2] = v0.z; xw[3] = v0.w;
      xw[4] = v1.x; xw[5] = v1.y; xw[6] = v1.z; xw[7] = v1.w;
    } else {
#pragma unroll
      for (int i = 0; i < 8; ++i) xw[i] = 0u;
    }
    const uint2 cw = *reinterpret_cast<const uint2*>(cptr + kb * 8);
    const uint32_t dm = sptr[kb];
    const float ssum = stok >= 0 ? xs[(int64_t)stok * nb + kb + sblk] : 0.0f;

    __syncthreads();   // the previous step's LDS reads are done
    {
      uint32_t o[8];
      transpose_half_block(xw, o);
      uint4* dst = reinterpret_cast<uint4*>(&As[xr][xhb * 16]);
      dst[0] = make_uint4(o[0], o[1], o[2], o[3]);
      dst[1] = make_uint4(o[4], o[5], o[6], o[7]);
      uint32_t q0[8], q1[8];
      unpack_q2_half(cw.x, q0);
      unpack_q2_half(cw.y, q1);
      uint4* bd = reinterpret_cast<uint4*>(&Bs[cmat][ccol][cblk * 32]);
      bd[0] = make_uint4(q0[0], q0[1], q0[2], q0[3]);
      bd[1] = make_uint4(q0[4], q0[5], q0[6], q0[7]);
      bd[2] = make_uint4(q1[0], q1[1], q1[2], q1[3]);
      bd[3] = make_uint4(q1[4], q1[5], q1[6], q1[7]);
      Sc[cmat][cblk][ccol] = make_float2(half_bits_to_float(dm & 0xFFFFu), half_bits_to_float(dm >> 16));
      if (tid < 128) Ss[sblk][srow] = ssum;
    }
    __syncthreads();

#pragma unroll
    for (int blk = 0; blk < 2; ++blk) {
      const int kofs = blk * 32 + 8 * (lane / 16);
      uint4 bg[2], bu[2];
      float2 sg[2], su[2];
#pragma unroll
      for (int ni = 0; ni < 2; ++ni) {
        const int col = 32 * wn + 16 * ni + lane % 16;
        bg[ni] = *reinterpret_cast<const uint4*>(&Bs[0][col][kofs]);
        bu[ni] = *reinterpret_cast<const uint4*>(&Bs[1][col][kofs]);
        sg[ni] = Sc[0][blk][col];
        su[ni] = Sc[1][blk][col];
      }
#pragma unroll
      for (int mi = 0; mi < 2; ++mi) {
        const int r0 = 32 * wm + 16 * mi;
        if (r0 >= rows) break;
        const uint4 a = *reinterpret_cast<const uint4*>(&As[r0 + lane % 16][kofs]);
        const float4 s4 = *reinterpret_cast<const float4*>(&Ss[blk][r0 + 4 * (lane / 16)]);
        const float sv[4] = {s4.x, s4.y, s4.z, s4.w};
#pragma unroll
        for (int ni = 0; ni < 2; ++ni) {
          const f32x4_t pg = mfma_bf16(a, bg[ni], zero4);
          const f32x4_t pu = mfma_bf16(a, bu[ni], zero4);
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            ag[mi][ni][i] = fmaf(sg[ni].x, pg[i], ag[mi][ni][i]);
            ag[mi][ni][i] = fmaf(sg[ni].y, sv[i], ag[mi][ni][i]);
            au[mi][ni][i] = fmaf(su[ni].x, pu[i], au[mi][ni][i]);
            au[mi][ni][i] = fmaf(su[ni].y, sv[i], au[mi][ni][i]);
          }
        }
      }
    }
  }

  // h = silu(g) * u as a bf16 hi/lo pair
#pragma unroll
  for (int mi = 0; mi < 2; ++mi) {
#pragma unroll
    for (int ni = 0; ni < 2; ++ni) {
      const int col = n0 + 32 * wn + 16 * ni + lane % 16;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = 32 * wm + 16 * mi + 4 * (lane / 16) + i;
        if (r < rows) {
          const float h = silu(ag[mi][ni][i]) * au[mi][ni][i];
          const uint32_t hi = bf16_rne_bits(h);
          const uint32_t lo = bf16_rne_bits(h - __uint_as_float(hi << 16));
          const int64_t at = (int64_t)(p0 + r) * I + col;
          h_hi[at] = (uint16_t)hi;
          h_lo[at] = (uint16_t)lo;
        }
      }
    }
  }
}

// down for one tile: y_slot[slot] = D_e h, with h = hi + lo, Q8_0 weights.
__global__ __launch_bounds__(kGemmThreads) void gemm_down_kernel(
    const uint16_t* __restrict__ h_hi, const uint16_t* __restrict__ h_lo, int H, int I, QMat down,
    const int32_t* __restrict__ slot_list, const int4* __restrict__ tiles, const int32_t* __restrict__ n_tiles,
    float* __restrict__ y) {
  const int tile = blockIdx.y;
  if (tile >= *n_tiles) return;
  __shared__ __align__(16) uint16_t Ah[kBM][kLdsRow];
  __shared__ __align__(16) uint16_t Al[kBM][kLdsRow];
  __shared__ __align__(16) uint16_t Bs[kBN][kLdsRow];
  __shared__ float Sd[2][kBN];   // [block][column] = d

  const int4 tl = tiles[tile];
  const int le = tl.x, p0 = tl.y, rows = tl.z;
  const int n0 = blockIdx.x * kBN;
  const int nb = I / 32;
  const int tid = threadIdx.x, lane = tid % kWave, wave = tid / kWave;
  const int wm = wave >> 1, wn = wave & 1;

  // staging roles: h rows (two threads per 16 values of a row, hi and lo),
  // codes (16 int8 per thread), scales (threads < 128)
  const int hr = tid >> 2, hq = tid & 3;              // row, quarter (16 values)
  const bool hvalid = hr < rows;
  const int64_t hofs = (int64_t)(p0 + hr) * I + hq * 16;
  const int ccol = tid >> 2, cq = tid & 3;
  const int64_t crow = (int64_t)le * H + n0 + ccol;
  const int8_t* cptr = reinterpret_cast<const int8_t*>(down.codes) + crow * (int64_t)I + cq * 16;
  const int sblk = tid >> 6, scol = tid & 63;
  const uint16_t* sptr =
      reinterpret_cast<const uint16_t*>(down.scales) + ((int64_t)le * H + n0 + scol) * nb + sblk;

  f32x4_t acc[2][2];
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int b = 0; b < 2; ++b) acc[a][b] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
  const f32x4_t zero4 = {0.0f, 0.0f, 0.0f, 0.0f};

  for (int kb = 0; kb < nb; kb += 2) {
    uint4 vh0 = make_uint4(0, 0, 0, 0), vh1 = vh0, vl0 = vh0, vl1 = vh0;
    if (hvalid) {
      const uint4* ph = reinterpret_cast<const uint4*>(h_hi + hofs + kb * 32);
      const uint4* pl = reinterpret_cast<const uint4*>(h_lo + hofs + kb * 32);
      vh0 = ph[0]; vh1 = ph[1]; vl0 = pl[0]; vl1 = pl[1];
    }
    const uint4 cw = *reinterpret_cast<const uint4*>(cptr + kb * 32);
    const float dsc = tid < 128 ? half_bits_to_float(sptr[kb]) : 0.0f;

    __syncthreads();
    {
      uint4* dh = reinterpret_cast<uint4*>(&Ah[hr][hq * 16]);
      uint4* dl = reinterpret_cast<uint4*>(&Al[hr][hq * 16]);
      dh[0] = vh0; dh[1] = vh1; dl[0] = vl0; dl[1] = vl1;
      const uint32_t w[4] = {cw.x, cw.y, cw.z, cw.w};
      uint32_t o[8];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float f0 = (float)(int)(int8_t)(w[j] & 0xFFu);
        const float f1 = (float)(int)(int8_t)((w[j] >> 8) & 0xFFu);
        const float f2 = (float)(int)(int8_t)((w[j] >> 16) & 0xFFu);
        const float f3 = (float)(int)(int8_t)(w[j] >> 24);
        o[2 * j] = __builtin_amdgcn_perm(__float_as_uint(f1), __float_as_uint(f0), 0x07060302u);
        o[2 * j + 1] = __builtin_amdgcn_perm(__float_as_uint(f3), __float_as_uint(f2), 0x07060302u);
      }
      uint4* bd = reinterpret_cast<uint4*>(&Bs[ccol][cq * 16]);
      bd[0] = make_uint4(o[0], o[1], o[2], o[3]);
      bd[1] = make_uint4(o[4], o[5], o[6], o[7]);
      if (tid < 128) Sd[sblk][scol] = dsc;
    }
    __syncthreads();

#pragma unroll
    for (int blk = 0; blk < 2; ++blk) {
      const int kofs = blk * 32 + 8 * (lane / 16);
      uint4 b[2];
      float d[2];
#pragma unroll
      for (int ni = 0; ni < 2; ++ni) {
        const int col = 32 * wn + 16 * ni + lane % 16;
        b[ni] = *reinterpret_cast<const uint4*>(&Bs[col][kofs]);
        d[ni] = Sd[blk][col];
      }
#pragma unroll
      for (int mi = 0; mi < 2; ++mi) {
        const int r0 = 32 * wm + 16 * mi;
        if (r0 >= rows) break;
        const uint4 ahi = *reinterpret_cast<const uint4*>(&Ah[r0 + lane % 16][kofs]);
        const uint4 alo = *reinterpret_cast<const uint4*>(&Al[r0 + lane % 16][kofs]);
#pragma unroll
        for (int ni = 0; ni < 2; ++ni) {
          f32x4_t p = mfma_bf16(ahi, b[ni], zero4);
          p = mfma_bf16(alo, b[ni], p);
#pragma unroll
          for (int i = 0; i < 4; ++i) acc[mi][ni][i] = fmaf(d[ni], p[i], acc[mi][ni][i]);
        }
      }
    }
  }

#pragma unroll
  for (int mi = 0; mi < 2; ++mi) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = 32 * wm + 16 * mi + 4 * (lane / 16) + i;
      if (r < rows) {
        const int64_t slot = slot_list[p0 + r];
#pragma unroll
        for (int ni = 0; ni < 2; ++ni) {
          const int col = n0 + 32 * wn + 16 * ni + lane % 16;
          y[slot * H + col] = acc[mi][ni][i];
        }
      }
    }
  }
}

int gemm_max_tiles(int T, int k, int E_local) {
  const int64_t slots = (int64_t)T * k;
  return (int)((slots + kBM - 1) / kBM + std::min<int64_t>(E_local, slots));
}

hipError_t launch_gemm_forward(const uint16_t* x, int T, int H, int I, int k, const QMat& gate, const QMat& up,
                               const QMat& down, const int32_t* g2l, int E, int E_local, const int32_t* counts,
                               const int32_t* offsets, const int32_t* slot_list, float* xs, int4* tiles,
                               int32_t* n_tiles, uint16_t* h_hi, uint16_t* h_lo, float* y, hipStream_t s) {
  const int nb = H / 32;
  const int64_t n_sums = (int64_t)T * nb;
  trace_pre("block_sums", s);
  block_sums_bf16_kernel<<<(unsigned)((n_sums + 255) / 256), 256, 0, s>>>(x, T, H, xs);
  trace_post("block_sums", s);
  trace_pre("gemm_tiles", s);
  const int max_tiles = gemm_max_tiles(T, k, E_local);
  gemm_tiles_kernel<<<1, 1024, 0, s>>>(counts, offsets, g2l, E, E_local, T * k, max_tiles, tiles, n_tiles);
  trace_post("gemm_tiles", s);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  trace_pre("gemm_gateup", s);
  gemm_gateup_kernel<<<dim3(I / kBN, max_tiles), kGemmThreads, 0, s>>>(x, H, I, k, gate, up, slot_list, xs, tiles,
                                                                      n_tiles, h_hi, h_lo);
  trace_post("gemm_gateup", s);
  err = hipGetLastError();
  if (err != hipSuccess) return err;
  trace_pre("gemm_down", s);
  gemm_down_kernel<<<dim3(H / kBN, max_tiles), kGemmThreads, 0, s>>>(h_hi, h_lo, H, I, down, slot_list, tiles,
                                                                    n_tiles, y);
  trace_post("gemm_down", s);
  return hipGetLastError();
}

}  // namespace moe
