// Top-k selection over router logits (internal to libmoe; shared by the
// selection kernel and the fused small-batch front kernel).
#pragma once
#include "device.h"

namespace moe {

constexpr int kMaxRanges = 32;   // partial logits per (token, expert): block ranges of the router

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

// Wave-wide maximum of an unsigned 64-bit value, in every lane: the two halves travel by DPP, the
// rows of 16 are reduced by quad and row permutes, then row 0's result is broadcast into row 1
// and rows 0-1's into rows 2-3, and lane 63 holds the maximum.
__device__ __forceinline__ uint64_t dpp_max_u64(uint64_t v, uint64_t o) { return o > v ? o : v; }
template <int CTRL, int ROWS>
__device__ __forceinline__ uint64_t dpp_step_u64(uint64_t v) {
  const int lo = (int)(uint32_t)v, hi = (int)(uint32_t)(v >> 32);
  const uint32_t olo = (uint32_t)__builtin_amdgcn_update_dpp(lo, lo, CTRL, ROWS, 0xF, false);
  const uint32_t ohi = (uint32_t)__builtin_amdgcn_update_dpp(hi, hi, CTRL, ROWS, 0xF, false);
  return dpp_max_u64(v, ((uint64_t)ohi << 32) | olo);
}
__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v) {
  v = dpp_step_u64<0xB1, 0xF>(v);    // quad_perm [1,0,3,2]
  v = dpp_step_u64<0x4E, 0xF>(v);    // quad_perm [2,3,0,1]
  v = dpp_step_u64<0x141, 0xF>(v);   // row_half_mirror
  v = dpp_step_u64<0x140, 0xF>(v);   // row_mirror: every lane of a row holds the row's maximum
  v = dpp_step_u64<0x142, 0xA>(v);   // row_bcast:15 into rows 1 and 3
  v = dpp_step_u64<0x143, 0xC>(v);   // row_bcast:31 into rows 2 and 3
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)v, 63);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(v >> 32), 63);
  return ((uint64_t)hi << 32) | lo;
}

// One wave per token: k rounds, each a wave max of the logit key over the
// untaken experts followed by a wave min of the expert index among those that
// hold it (ties go to the lower index).  Weights: s_j = sigmoid(z_j) in fp64
// on lane j, their sum taken in slot order by every lane, w_j = s_j / sum.
// With S > 0 the logits arrive as S partial sums per (token, expert) (block ranges, zp[s][t][e]),
// added here pairwise, level by level, and then the bias is added; with S == 0, z holds finished
// logits.
template <int EPL>  // experts per lane (E <= 64 * EPL)
__device__ __forceinline__ float logit_of(const float* __restrict__ z, int S, const float* __restrict__ bias,
                                          int T, int E, int t, int e) {
  if (S == 0) return z[(int64_t)t * E + e];
  // every load is issued (ranges past S read range S - 1 and are dropped): none behind a branch
  float v[kMaxRanges];
#pragma unroll
  for (int i = 0; i < kMaxRanges; ++i) {
    const float p = z[((int64_t)min(i, S - 1) * T + t) * E + e];
    v[i] = i < S ? p : 0.0f;
  }
#pragma unroll
  for (int w = 1; w < kMaxRanges; w <<= 1)
#pragma unroll
    for (int i = 0; i + w < kMaxRanges; i += 2 * w)
      if (i + w < S) v[i] = v[i] + v[i + w];
  return bias ? v[0] + bias[e] : v[0];
}

template <int EPL>  // experts per lane (E <= 64 * EPL)
__device__ __forceinline__ void topk_token(const float* __restrict__ z, int S, const float* __restrict__ bias, int T,
                                           int E, int k, int t, int32_t* __restrict__ ids, float* __restrict__ w,
                                           int32_t* ids_copy = nullptr) {
  const int lane = threadIdx.x % kWave;
  uint32_t key[EPL];
  bool live[EPL];
#pragma unroll
  for (int i = 0; i < EPL; ++i) {
    const int e = i * kWave + lane;
    live[i] = e < E;
    const uint32_t kv = float_key(logit_of<EPL>(z, S, bias, T, E, t, min(e, E - 1)));   // loaded unconditionally
    key[i] = live[i] ? kv : 0u;
  }
  // one wave maximum per round over (key, ~expert): the largest key, ties to the lower expert
  int my_id = -1;
  uint32_t my_key = 0;
  for (int j = 0; j < k; ++j) {
    uint64_t best = 0;
#pragma unroll
    for (int i = 0; i < EPL; ++i) {
      const uint64_t c = ((uint64_t)key[i] << 32) | (uint32_t)~(uint32_t)(i * kWave + lane);
      if (live[i] && c > best) best = c;
    }
    const uint64_t mx = wave_max_u64(best);
    const uint32_t me = ~(uint32_t)mx;
#pragma unroll
    for (int i = 0; i < EPL; ++i)
      if ((uint32_t)(i * kWave + lane) == me) live[i] = false;
    if (lane == j) {
      my_id = (int)me;
      my_key = (uint32_t)(mx >> 32);
    }
  }
  if (lane < k && ids_copy) ids_copy[t * k + lane] = my_id;
  if (!w) return;   // ids only (ids may be NULL too)
  const double my_s = 1.0 / (1.0 + exp(-(double)key_to_float(my_key)));
  double ssum = 0.0;
  for (int j = 0; j < k; ++j) {
    const int lo = __builtin_amdgcn_readlane((int)(uint32_t)__double_as_longlong(my_s), j);
    const int hi = __builtin_amdgcn_readlane((int)(uint32_t)(__double_as_longlong(my_s) >> 32), j);
    ssum += __longlong_as_double(((long long)(uint32_t)hi << 32) | (uint32_t)lo);
  }
  if (lane < k) {
    if (ids) ids[(int64_t)t * k + lane] = my_id;
    w[(int64_t)t * k + lane] = (float)(my_s / ssum);
  }
}

}  // namespace moe
