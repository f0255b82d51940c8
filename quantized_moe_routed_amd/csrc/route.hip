// Router scoring and top-k selection.
//
// Logits follow one fixed fp32 order so that expert ids are reproducible bit
// for bit (this file is compiled with -ffp-contract=off and every fused
// multiply-add is written out):
//   per 32-block b:  p = 0; p = fma(wq_i, x_i, p) for i = 0..31 in turn
//                    r_b = d_b * p            (Q8_0; an fp32 router has r_b = p)
//   z = balanced pairwise sum over b: (r0 + r1), (r2 + r3), ... level by level,
//       an odd last element carried up unchanged;  then z += bias.
// A wave holds one expert row: lane l owns the C consecutive blocks
// l*C .. l*C+C-1, adds them pairwise in registers (the first log2 C levels of
// the tree) and the remaining levels are an xor butterfly across lanes, which
// adds adjacent subtrees exactly as the tree does (IEEE addition commutes).
// Lanes past the last block contribute +0.0: padding the tree with zeros
// changes no value, so the result equals the carry-up tree for any block count.
#include "device.h"
#include "fmt.h"
#include "launch.h"

namespace moe {

constexpr int kRouteTokTile = 16;

template <int FMT, int ACT, int C>
__global__ __launch_bounds__(256) void route_logits_kernel(const void* __restrict__ x, int T, int H,
                                                           const void* __restrict__ codes,
                                                           const void* __restrict__ scales,
                                                           const float* __restrict__ bias, int E,
                                                           float* __restrict__ z) {
  const int lane = threadIdx.x % kWave;
  const int e = blockIdx.x * (blockDim.x / kWave) + threadIdx.x / kWave;
  if (e >= E) return;
  const int nb = H / 32;

  float wv[C][32];
  float dsc[C];
#pragma unroll
  for (int j = 0; j < C; ++j) {
    const int b = lane * C + j;
    dsc[j] = 0.0f;
    if (b < nb) {
      if constexpr (FMT == FMT_Q8_0) {
        // row-group layout: block b's values 8g..8g+7 in unit b/2 of row e, group g, half b%2
        const int nu = (nb + 1) / 2;
        const int8_t* q = reinterpret_cast<const int8_t*>(codes) + code_off(e, b >> 1, nu) + (b & 1) * 8;
        int words[8];
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int2 v = *reinterpret_cast<const int2*>(q + 16 * g);
          words[2 * g] = v.x;
          words[2 * g + 1] = v.y;
        }
#pragma unroll
        for (int i = 0; i < 32; ++i) wv[j][i] = (float)(int8_t)(words[i / 4] >> (8 * (i % 4)));
        dsc[j] = half_bits_to_float(*reinterpret_cast<const uint16_t*>(
            reinterpret_cast<const uint8_t*>(scales) + Codes<FMT_Q8_0>::d_off(e, b >> 1, nu) + 2 * (b & 1)));
      } else {
        const float4* w4 = reinterpret_cast<const float4*>(reinterpret_cast<const float*>(codes) +
                                                           (int64_t)e * H + b * 32);
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          float4 v = w4[i];
          wv[j][4 * i] = v.x;
          wv[j][4 * i + 1] = v.y;
          wv[j][4 * i + 2] = v.z;
          wv[j][4 * i + 3] = v.w;
        }
      }
    } else {
#pragma unroll
      for (int i = 0; i < 32; ++i) wv[j][i] = 0.0f;
    }
  }
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
        if constexpr (ACT == ACT_F32) {
          const float4* x4 = reinterpret_cast<const float4*>(reinterpret_cast<const float*>(x) +
                                                             (int64_t)t * H + b * 32);
#pragma unroll
          for (int i = 0; i < 8; ++i) {
            float4 v = x4[i];
            xv[4 * i] = v.x;
            xv[4 * i + 1] = v.y;
            xv[4 * i + 2] = v.z;
            xv[4 * i + 3] = v.w;
          }
        } else {
          const uint4* x4 = reinterpret_cast<const uint4*>(reinterpret_cast<const uint16_t*>(x) +
                                                           (int64_t)t * H + b * 32);
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            uint4 v = x4[i];
            uint32_t wds[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
            for (int q = 0; q < 4; ++q) {
              xv[8 * i + 2 * q] = __uint_as_float(wds[q] << 16);
              xv[8 * i + 2 * q + 1] = __uint_as_float(wds[q] & 0xFFFF0000u);
            }
          }
        }
        float p = 0.0f;
#pragma unroll
        for (int i = 0; i < 32; ++i) p = __builtin_fmaf(wv[j][i], xv[i], p);
        r[j] = (FMT == FMT_Q8_0) ? dsc[j] * p : p;
      }
    }
#pragma unroll
    for (int w = 1; w < C; w <<= 1) {
#pragma unroll
      for (int j = 0; j + w < C; j += 2 * w) r[j] = r[j] + r[j + w];
    }
    float v = r[0];
#pragma unroll
    for (int m = 1; m < kWave; m <<= 1) v = v + __shfl_xor(v, m, kWave);
    if (lane == 0) z[(int64_t)t * E + e] = bias ? v + be : v;
  }
}

// Order-preserving unsigned key of a logit: larger z -> larger key, -0 and +0
// equal, NaN -> 0 (below every number).  key_to_float inverts it (0 -> NaN).
__device__ __forceinline__ uint32_t float_key(float z) {
  if (z != z) return 0u;
  if (z == 0.0f) z = 0.0f;   // -0 -> +0
  const uint32_t b = __float_as_uint(z);
  return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}
__device__ __forceinline__ float key_to_float(uint32_t k) {
  return __uint_as_float((k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k);
}

// Wave-wide max / min of an unsigned value: quad and row permutes (DPP) reduce
// each row of 16 lanes, then the four row results are read out.
template <bool MAX>
__device__ __forceinline__ uint32_t wave_reduce_u32(uint32_t v) {
  auto op = [](uint32_t a, uint32_t b) { return MAX ? (a > b ? a : b) : (a < b ? a : b); };
  v = op(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0xB1, 0xF, 0xF, false));   // quad_perm [1,0,3,2]
  v = op(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x4E, 0xF, 0xF, false));   // quad_perm [2,3,0,1]
  v = op(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x141, 0xF, 0xF, false));  // row_half_mirror
  v = op(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x140, 0xF, 0xF, false));  // row_mirror
  const uint32_t r0 = (uint32_t)__builtin_amdgcn_readlane((int)v, 0);
  const uint32_t r1 = (uint32_t)__builtin_amdgcn_readlane((int)v, 16);
  const uint32_t r2 = (uint32_t)__builtin_amdgcn_readlane((int)v, 32);
  const uint32_t r3 = (uint32_t)__builtin_amdgcn_readlane((int)v, 48);
  return op(op(r0, r1), op(r2, r3));
}

// One wave per token: k rounds, each a wave max of the logit key over the
// untaken experts followed by a wave min of the expert index among those that
// hold it (ties go to the lower index).  Weights: s_j = sigmoid(z_j) in fp64
// on lane j, their sum taken in slot order by every lane, w_j = s_j / sum.
template <int EPL>  // experts per lane (E <= 64 * EPL)
__global__ __launch_bounds__(256) void route_topk_kernel(const float* __restrict__ z, int T, int E, int k,
                                                         int32_t* __restrict__ ids, float* __restrict__ w) {
  const int lane = threadIdx.x % kWave;
  const int t = blockIdx.x * (blockDim.x / kWave) + threadIdx.x / kWave;
  if (t >= T) return;
  uint32_t key[EPL];
  bool live[EPL];
#pragma unroll
  for (int i = 0; i < EPL; ++i) {
    const int e = i * kWave + lane;
    live[i] = e < E;
    key[i] = live[i] ? float_key(z[(int64_t)t * E + e]) : 0u;
  }
  int my_id = -1;
  uint32_t my_key = 0;
  for (int j = 0; j < k; ++j) {
    uint32_t lk = 0;
#pragma unroll
    for (int i = 0; i < EPL; ++i)
      if (live[i] && key[i] > lk) lk = key[i];
    const uint32_t mk = wave_reduce_u32<true>(lk);
    uint32_t li = 0xFFFFFFFFu;
#pragma unroll
    for (int i = 0; i < EPL; ++i) {
      const uint32_t e = (uint32_t)(i * kWave + lane);
      if (live[i] && key[i] == mk && e < li) li = e;
    }
    const uint32_t me = wave_reduce_u32<false>(li);
#pragma unroll
    for (int i = 0; i < EPL; ++i)
      if ((uint32_t)(i * kWave + lane) == me) live[i] = false;
    if (lane == j) {
      my_id = (int)me;
      my_key = mk;
    }
  }
  const double my_s = 1.0 / (1.0 + exp(-(double)key_to_float(my_key)));
  double ssum = 0.0;
  for (int j = 0; j < k; ++j) {
    const int lo = __builtin_amdgcn_readlane((int)(uint32_t)__double_as_longlong(my_s), j);
    const int hi = __builtin_amdgcn_readlane((int)(uint32_t)(__double_as_longlong(my_s) >> 32), j);
    ssum += __longlong_as_double(((long long)(uint32_t)hi << 32) | (uint32_t)lo);
  }
  if (lane < k) {
    ids[(int64_t)t * k + lane] = my_id;
    w[(int64_t)t * k + lane] = (float)(my_s / ssum);
  }
}

template <int FMT, int ACT>
static hipError_t launch_logits_c(int C, const void* x, int T, int H, const QMat& r, const float* bias,
                                  float* z, hipStream_t s) {
  const int E = r.rows;
  dim3 grid((E + 3) / 4, (T + kRouteTokTile - 1) / kRouteTokTile);
  switch (C) {
    case 1: route_logits_kernel<FMT, ACT, 1><<<grid, 256, 0, s>>>(x, T, H, r.codes, r.scales, bias, E, z); break;
    case 2: route_logits_kernel<FMT, ACT, 2><<<grid, 256, 0, s>>>(x, T, H, r.codes, r.scales, bias, E, z); break;
    case 4: route_logits_kernel<FMT, ACT, 4><<<grid, 256, 0, s>>>(x, T, H, r.codes, r.scales, bias, E, z); break;
    case 8: route_logits_kernel<FMT, ACT, 8><<<grid, 256, 0, s>>>(x, T, H, r.codes, r.scales, bias, E, z); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_route(const void* x, int act, int T, int H, int fmt, const QMat& router, const float* bias,
                        int k, int32_t* ids, float* w, float* z_ws, hipStream_t s) {
  const int nb = H / 32;
  int C = 1;
  while (C * kWave < nb) C <<= 1;
  hipError_t err;
  const bool q8 = fmt == FMT_Q8_0;
  trace_pre("route_logits", s);
  if (act == ACT_F32) {
    err = q8 ? launch_logits_c<FMT_Q8_0, ACT_F32>(C, x, T, H, router, bias, z_ws, s)
             : launch_logits_c<FMT_F32, ACT_F32>(C, x, T, H, router, bias, z_ws, s);
  } else {
    err = q8 ? launch_logits_c<FMT_Q8_0, ACT_BF16>(C, x, T, H, router, bias, z_ws, s)
             : launch_logits_c<FMT_F32, ACT_BF16>(C, x, T, H, router, bias, z_ws, s);
  }
  trace_post("route_logits", s);
  if (err != hipSuccess) return err;
  const int E = router.rows;
  dim3 grid((T + 3) / 4);
  trace_pre("route_topk", s);
  if (E <= 64) route_topk_kernel<1><<<grid, 256, 0, s>>>(z_ws, T, E, k, ids, w);
  else if (E <= 128) route_topk_kernel<2><<<grid, 256, 0, s>>>(z_ws, T, E, k, ids, w);
  else if (E <= 256) route_topk_kernel<4><<<grid, 256, 0, s>>>(z_ws, T, E, k, ids, w);
  else if (E <= 512) route_topk_kernel<8><<<grid, 256, 0, s>>>(z_ws, T, E, k, ids, w);
  else route_topk_kernel<16><<<grid, 256, 0, s>>>(z_ws, T, E, k, ids, w);
  trace_post("route_topk", s);
  return hipGetLastError();
}

}  // namespace moe
