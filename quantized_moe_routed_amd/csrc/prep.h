// Activation operand of one token for the expert kernels (internal to
// libmoe; used by the preparation launches and by the router launch of small
// batches).
//
// Activation operand of token t (see fmt.h):
//   sigma_t = row_scale(max_i |x[t,i]|) = 2^(9-E), E the smallest integer with
//             max_i |x[t,i]| < 2^E (fmt.h), so that |x| * sigma * 2^6 < 2^15;
//   A'[t][32b+8g+e] = x[t][32b+8g+frag_val(e)] * sigma_t * 2^6        (hi, lo)
//   S'[t][b]        = sigma_t * sum_{i<32} x[t][32b+i]               (hi, lo)
// The block sums are taken in index order in fp32; blocks past H/32 up to
// the padded count are zero.  One workgroup of NT threads per token, one call
// per workgroup (its LDS is not guarded for a second call).
#pragma once
#include "device.h"
#include "fmt.h"

namespace moe {

constexpr int kPrepMaxH = 8192;   // longest row prep_token takes

// The 16 activations x[off .. off+15] as fp32 (fp32 or bf16 input, 16-byte aligned).
template <int ACT>
__device__ __forceinline__ void load_act16(const void* __restrict__ x, int64_t off, float (&v)[16]) {
  if constexpr (ACT == ACT_F32) {
    const float4* p = reinterpret_cast<const float4*>(reinterpret_cast<const float*>(x) + off);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float4 q = p[i];
      v[4 * i] = q.x;
      v[4 * i + 1] = q.y;
      v[4 * i + 2] = q.z;
      v[4 * i + 3] = q.w;
    }
  } else {
    const uint4* p = reinterpret_cast<const uint4*>(reinterpret_cast<const uint16_t*>(x) + off);
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const uint4 q = p[i];
      const uint32_t w[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        v[8 * i + 2 * j] = __uint_as_float(w[j] << 16);
        v[8 * i + 2 * j + 1] = __uint_as_float(w[j] & 0xFFFF0000u);
      }
    }
  }
}

// Thread i takes chunks i, i + NT, ... of 16 values (half a block): one load of the row, kept
// in registers.  The block sum of block b runs in index order: the even chunk's lane sums its 16
// values from +0.0, the odd chunk's lane (the next lane) continues from that partial.
template <int ACT, int NT>
__device__ void prep_token(const void* __restrict__ x, int t, int H, int nb32, uint16_t* __restrict__ xq_hi,
                           uint16_t* __restrict__ xq_lo, uint16_t* __restrict__ sq_hi, uint16_t* __restrict__ sq_lo,
                           float* __restrict__ sigma) {
  constexpr int MAXC = (kPrepMaxH / 16 + NT - 1) / NT;   // chunks per thread
  __shared__ float wmax[NT / kWave];
  const int tid = threadIdx.x, lane = tid % kWave, wave = tid / kWave;
  const int64_t row = (int64_t)t * H;
  const int nc = H / 16, nb = H / 32;
  float xv[MAXC][16];
  float mx = 0.0f;
#pragma unroll
  for (int c = 0; c < MAXC; ++c) {
    const int ch = tid + c * NT;
    load_act16<ACT>(x, row + 16 * min(ch, nc - 1), xv[c]);   // issued for every chunk, past nc dropped
  }
#pragma unroll
  for (int c = 0; c < MAXC; ++c)
    if (tid + c * NT < nc)
#pragma unroll
      for (int i = 0; i < 16; ++i) mx = fmaxf(mx, fabsf(xv[c][i]));
#pragma unroll
  for (int m = 1; m < kWave; m <<= 1) mx = fmaxf(mx, __shfl_xor(mx, m, kWave));
  if (lane == 0) wmax[wave] = mx;
  __syncthreads();
  float m = 0.0f;
#pragma unroll
  for (int w = 0; w < NT / kWave; ++w) m = fmaxf(m, wmax[w]);
  const float sg = row_scale(m);
  if (tid == 0) sigma[t] = sg;
#pragma unroll
  for (int c = 0; c < MAXC; ++c) {
    const int ch = tid + c * NT;
    // chunk ch: block ch / 2, K-groups 2 (ch % 2) and 2 (ch % 2) + 1
    float sa = 0.0f;
#pragma unroll
    for (int i = 0; i < 16; ++i) sa += xv[c][i];
    const float prev = __shfl_xor(sa, 1, kWave);   // NT is even: chunk ch ^ 1 sits in lane ^ 1
    if (ch < nc) {
      const int b = ch >> 1;
#pragma unroll
      for (int gg = 0; gg < 2; ++gg) {
        uint32_t hi[8], lo[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) split_f16(xv[c][8 * gg + frag_val(e)] * sg * 64.0f, hi[e], lo[e]);
        const int64_t o = row + 16 * ch + 8 * gg;
        *reinterpret_cast<uint4*>(xq_hi + o) =
            make_uint4(hi[0] | (hi[1] << 16), hi[2] | (hi[3] << 16), hi[4] | (hi[5] << 16), hi[6] | (hi[7] << 16));
        if (xq_lo)
          *reinterpret_cast<uint4*>(xq_lo + o) =
              make_uint4(lo[0] | (lo[1] << 16), lo[2] | (lo[3] << 16), lo[4] | (lo[5] << 16), lo[6] | (lo[7] << 16));
      }
      if (ch & 1) {
        float s = prev;
#pragma unroll
        for (int i = 0; i < 16; ++i) s += xv[c][i];
        uint32_t hi, lo;
        split_f16(s * sg, hi, lo);
        sq_hi[(int64_t)t * nb32 + b] = (uint16_t)hi;
        sq_lo[(int64_t)t * nb32 + b] = (uint16_t)lo;
      }
    }
  }
  for (int b = nb + tid; b < nb32; b += NT) {   // padding blocks
    sq_hi[(int64_t)t * nb32 + b] = 0;
    sq_lo[(int64_t)t * nb32 + b] = 0;
  }
}

}  // namespace moe
