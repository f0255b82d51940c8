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
        // unit layout: block b's values 8g..8g+7 at unit b/2, group g, half b%2
        const int8_t* q = reinterpret_cast<const int8_t*>(codes) + (int64_t)e * ((nb + 1) / 2) * 64 +
                          (b >> 1) * 64 + (b & 1) * 8;
        int words[8];
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int2 v = *reinterpret_cast<const int2*>(q + 16 * g);
          words[2 * g] = v.x;
          words[2 * g + 1] = v.y;
        }
#pragma unroll
        for (int i = 0; i < 32; ++i) wv[j][i] = (float)(int8_t)(words[i / 4] >> (8 * (i % 4)));
        dsc[j] = half_bits_to_float(reinterpret_cast<const uint16_t*>(scales)[(int64_t)e * ((nb + 1) / 2 * 2) + b]);
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

// a ranks before b: larger z, then lower index; NaN ranks last.
__device__ __forceinline__ bool ranks_before(float za, int a, float zb, int b) {
  const bool na = za != za, nb = zb != zb;
  if (na || nb) return (na != nb) ? nb : (a < b);
  if (za != zb) return za > zb;
  return a < b;
}

// One wave per token: k rounds of a wave-wide arg-max over the unselected experts.
template <int EPL>  // experts per lane (E <= 64 * EPL)
__global__ __launch_bounds__(256) void route_topk_kernel(const float* __restrict__ z, int T, int E, int k,
                                                         int32_t* __restrict__ ids, float* __restrict__ w) {
  const int lane = threadIdx.x % kWave;
  const int t = blockIdx.x * (blockDim.x / kWave) + threadIdx.x / kWave;
  if (t >= T) return;
  float zv[EPL];
  bool taken[EPL];
#pragma unroll
  for (int i = 0; i < EPL; ++i) {
    const int e = i * kWave + lane;
    taken[i] = e >= E;
    zv[i] = e < E ? z[(int64_t)t * E + e] : 0.0f;
  }
  // lane j keeps slot j's expert and sigmoid score; the sum is wave-uniform
  double my_s = 0.0, ssum = 0.0;
  int my_id = -1;
  for (int j = 0; j < k; ++j) {
    float bz = 0.0f;
    int be = -1;
#pragma unroll
    for (int i = 0; i < EPL; ++i) {
      const int e = i * kWave + lane;
      if (!taken[i] && (be < 0 || ranks_before(zv[i], e, bz, be))) {
        bz = zv[i];
        be = e;
      }
    }
#pragma unroll
    for (int m = 1; m < kWave; m <<= 1) {
      const float oz = __shfl_xor(bz, m, kWave);
      const int oe = __shfl_xor(be, m, kWave);
      if (oe >= 0 && (be < 0 || ranks_before(oz, oe, bz, be))) {
        bz = oz;
        be = oe;
      }
    }
#pragma unroll
    for (int i = 0; i < EPL; ++i)
      if (i * kWave + lane == be) taken[i] = true;
    const double sj = 1.0 / (1.0 + exp(-(double)bz));
    ssum += sj;
    if (lane == j) {
      my_s = sj;
      my_id = be;
    }
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
