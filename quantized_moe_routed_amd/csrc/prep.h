// Activation operand of one token for the expert kernels (internal to
// libmoe; used by the preparation launches and by the router launch of small
// batches).
//
// Activation operand of token t (see fmt.h):
//   sigma_t = 2^(9-E), E the smallest integer with max_i |x[t,i]| < 2^E
//             (1 for an all-zero token), so that |x| * sigma * 2^6 < 2^15;
//   A'[t][32b+8g+e] = x[t][32b+8g+frag_val(e)] * sigma_t * 2^6        (hi, lo)
//   S'[t][b]        = sigma_t * sum_{i<32} x[t][32b+i]               (hi, lo)
// The block sums are taken in index order in fp32; blocks past H/32 up to
// the padded count are zero.  One workgroup of NT threads per token.
#pragma once
#include "device.h"
#include "fmt.h"

namespace moe {

template <int ACT>
__device__ __forceinline__ float act_at(const void* x, int64_t i) {
  return load_act<ACT>(x, i);
}

template <int ACT, int NT>
__device__ void prep_token(const void* __restrict__ x, int t, int H, int nb32, uint16_t* __restrict__ xq_hi,
                           uint16_t* __restrict__ xq_lo, uint16_t* __restrict__ sq_hi, uint16_t* __restrict__ sq_lo,
                           float* __restrict__ sigma) {
  __shared__ float wmax[NT / kWave];
  __shared__ float s_sigma;
  const int tid = threadIdx.x, lane = tid % kWave, wave = tid / kWave;
  const int64_t row = (int64_t)t * H;
  float mx = 0.0f;
  for (int i = tid; i < H; i += NT) mx = fmaxf(mx, fabsf(act_at<ACT>(x, row + i)));
#pragma unroll
  for (int m = 1; m < kWave; m <<= 1) mx = fmaxf(mx, __shfl_xor(mx, m, kWave));
  if (lane == 0) wmax[wave] = mx;
  __syncthreads();
  if (tid == 0) {
    float m = 0.0f;
    for (int w = 0; w < NT / kWave; ++w) m = fmaxf(m, wmax[w]);
    int e = 0;
    if (m > 0.0f) (void)frexpf(m, &e);   // m = f * 2^e, f in [0.5, 1): m < 2^e
    const float sg = ldexpf(1.0f, 9 - e);
    s_sigma = sg;
    sigma[t] = sg;
  }
  __syncthreads();
  const float sg = s_sigma;
  const int nb = H / 32;
  // one thread per (block, K-group): 8 operand values
  for (int j = tid; j < nb * 4; j += NT) {
    const int b = j >> 2, g = j & 3;
    uint32_t hi[8], lo[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float v = act_at<ACT>(x, row + 32 * b + 8 * g + frag_val(e)) * sg * 64.0f;
      split_f16(v, hi[e], lo[e]);
    }
    const int64_t o = row + 32 * b + 8 * g;
    *reinterpret_cast<uint4*>(xq_hi + o) =
        make_uint4(hi[0] | (hi[1] << 16), hi[2] | (hi[3] << 16), hi[4] | (hi[5] << 16), hi[6] | (hi[7] << 16));
    if (xq_lo)
      *reinterpret_cast<uint4*>(xq_lo + o) =
          make_uint4(lo[0] | (lo[1] << 16), lo[2] | (lo[3] << 16), lo[4] | (lo[5] << 16), lo[6] | (lo[7] << 16));
  }
  for (int b = tid; b < nb32; b += NT) {
    uint32_t hi = 0, lo = 0;
    if (b < nb) {
      float s = 0.0f;
      for (int i = 0; i < 32; ++i) s += act_at<ACT>(x, row + 32 * b + i);
      split_f16(s * sg, hi, lo);
    }
    sq_hi[(int64_t)t * nb32 + b] = (uint16_t)hi;
    sq_lo[(int64_t)t * nb32 + b] = (uint16_t)lo;
  }
}

}  // namespace moe
