// Top-k selection over router logits (internal to libmoe; shared by the
// selection kernel and the fused small-batch front kernel).
#pragma once
#include "device.h"

namespace moe {

constexpr int kMaxRanges = 32;   // partial logits per (token, expert): block ranges of the router
constexpr int kSelMaxRanges = 8;  // ranges taken by the selections inside the small-batch launches

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

// Order-preserving keys of the lane's experts i * 64 + lane (0 and not live past E).  The logit
// of (t, e): with M == 0 z holds it (bias included); otherwise the S <= M partial sums are added
// pairwise, level by level, and then the bias.  Every load of every expert is issued before any
// is used: ranges past S read range S - 1 and experts past E read expert E - 1, both dropped, and
// with no bias the bias load reads z and is dropped.
template <int EPL, int M>
__device__ __forceinline__ void logit_keys(const float* __restrict__ z, int S, const float* __restrict__ bias,
                                           int T, int E, int t, int lane, uint32_t (&key)[EPL],
                                           bool (&live)[EPL]) {
  int ec[EPL];
#pragma unroll
  for (int i = 0; i < EPL; ++i) {
    live[i] = i * kWave + lane < E;
    ec[i] = min(i * kWave + lane, E - 1);
  }
  float zl[EPL];
  const int tu = __builtin_amdgcn_readfirstlane(t);   // (one token per wave: row bases stay scalar)
  if constexpr (M == 0) {
    const float* zt = z + (int64_t)tu * E;
#pragma unroll
    for (int i = 0; i < EPL; ++i) zl[i] = zt[ec[i]];
  } else {
    float v[EPL][M], bv[EPL];
    const float* bp = bias ? bias : z;
#pragma unroll
    for (int j = 0; j < M; ++j) {
      const float* zj = z + ((int64_t)min(j, S - 1) * T + tu) * E;
#pragma unroll
      for (int i = 0; i < EPL; ++i) v[i][j] = zj[ec[i]];
    }
#pragma unroll
    for (int i = 0; i < EPL; ++i) bv[i] = bp[ec[i]];
#pragma unroll
    for (int i = 0; i < EPL; ++i) {
#pragma unroll
      for (int w = 1; w < M; w <<= 1)
#pragma unroll
        for (int j = 0; j + w < M; j += 2 * w) v[i][j] = j + w < S ? v[i][j] + v[i][j + w] : v[i][j];
      zl[i] = bias ? v[i][0] + bv[i] : v[i][0];
    }
  }
#pragma unroll
  for (int i = 0; i < EPL; ++i) key[i] = live[i] ? float_key(zl[i]) : 0u;
}

// Keys from M partial ranges, M the first of M0, 2 M0, ... that holds S, at most MAXS.
template <int EPL, int M, int MAXS>
__device__ __forceinline__ void logit_keys_upto(const float* __restrict__ z, int S, const float* __restrict__ bias,
                                                int T, int E, int t, int lane, uint32_t (&key)[EPL],
                                                bool (&live)[EPL]) {
  if constexpr (M >= MAXS) {
    logit_keys<EPL, MAXS>(z, S, bias, T, E, t, lane, key, live);
  } else {
    if (S <= M) logit_keys<EPL, M>(z, S, bias, T, E, t, lane, key, live);
    else logit_keys_upto<EPL, 2 * M, MAXS>(z, S, bias, T, E, t, lane, key, live);
  }
}

// Top-k (k <= kThrMaxK) of one wave's keys by a threshold.  The row maxima (rows of 16 lanes, per
// key slot; 0 for a row without a live expert) go one per lane, and tau is the largest of them that
// at least k row maxima reach (0 when none does).  At least k distinct live experts then have a key
// >= tau, so the k-th largest key is >= tau and every expert of the top k is a candidate.  The
// candidates go to LDS as composites (key, complement of the expert index), which are all
// distinct, and a candidate's rank is the number of larger composites; the k of rank < k, in rank
// order, are exactly the k largest keys with ties to the lower index.  cand holds E + kThrMaxK
// entries.  Lanes j < k receive slot j's expert and key.
constexpr int kThrMaxK = 8;

__device__ __forceinline__ uint32_t row_max_u32(uint32_t v) {
  auto mx = [](uint32_t a, uint32_t b) { return a > b ? a : b; };
  v = mx(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0xB1, 0xF, 0xF, false));   // quad_perm [1,0,3,2]
  v = mx(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x4E, 0xF, 0xF, false));   // quad_perm [2,3,0,1]
  v = mx(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x141, 0xF, 0xF, false));  // row_half_mirror
  v = mx(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x140, 0xF, 0xF, false));  // row_mirror
  return v;
}

template <int EPL>
__device__ __forceinline__ void topk_threshold(const uint32_t (&key)[EPL], const bool (&live)[EPL], int E, int k,
                                               int lane, uint64_t* __restrict__ cand, int& my_id,
                                               uint32_t& my_key) {
  static_assert(EPL <= 16, "one row maximum per lane");
  // lane 16 r + i (i < EPL): the maximum of row r of key slot i (keys of experts past E are 0)
  uint32_t rm = 0;
#pragma unroll
  for (int i = 0; i < EPL; ++i) {
    const uint32_t g = row_max_u32(key[i]);
    rm = (lane & 15) == i ? g : rm;
  }
  // how many row maxima reach this lane's; tau: the largest that at least k of them reach
  int reach = 0;
#pragma unroll
  for (int q = 0; q < kWave; ++q)
    if ((q & 15) < EPL) reach += (uint32_t)__builtin_amdgcn_readlane((int)rm, q) >= rm ? 1 : 0;
  const uint32_t tau = wave_reduce_u32<true>((lane & 15) < EPL && reach >= k ? rm : 0u);
  int nc = 0;
#pragma unroll
  for (int i = 0; i < EPL; ++i) {
    const bool c = live[i] && key[i] >= tau;
    const uint64_t m = __ballot(c);
    if (c) {
      const int pos = nc + (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
      cand[pos] = ((uint64_t)key[i] << 32) | (uint32_t)~(uint32_t)(i * kWave + lane);
    }
    nc += __popcll(m);
  }
  uint64_t* top = cand + E;
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  for (int j0 = 0; j0 < nc; j0 += kWave) {
    const int j = j0 + lane;
    const uint64_t mine = cand[min(j, nc - 1)];
    int rank = 0;
#pragma unroll 4
    for (int q = 0; q < nc; ++q) rank += cand[q] > mine ? 1 : 0;
    if (j < nc && rank < k) top[rank] = mine;
  }
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  if (lane < k) {
    const uint64_t c = top[lane];
    my_id = (int)~(uint32_t)c;
    my_key = (uint32_t)(c >> 32);
  }
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");   // cand is free again for the next call
}

template <int EPL>
__device__ __forceinline__ void topk_of_keys(uint32_t (&key)[EPL], bool (&live)[EPL], int E, int k, int lane,
                                             uint64_t* cand, int& my_id, uint32_t& my_key);

// One wave per token: k rounds, each one wave maximum of (logit key, complement of the expert
// index) over the untaken experts, i.e. the largest logit with ties to the lower index.
// Weights: s_j = sigmoid(z_j) in fp64 on lane j, their sum taken in slot order by every lane,
// w_j = s_j / sum.  With S > 0 the logits arrive as S partial sums per (token, expert) over
// aligned block ranges (zp[s][t][e]); with S == 0, z holds finished logits.  Given LDS for
// E + kThrMaxK candidates (cand) and k <= kThrMaxK, the threshold selection above replaces the
// rounds (same result).
// The selection itself: lane j < k receives slot j's expert and its logit key.
template <int EPL, int MAXS = kMaxRanges>  // experts per lane (E <= 64 * EPL); S <= MAXS
__device__ __forceinline__ void topk_lanes(const float* __restrict__ z, int S, const float* __restrict__ bias, int T,
                                           int E, int k, int t, uint64_t* cand, int& my_id, uint32_t& my_key) {
  const int lane = threadIdx.x % kWave;
  uint32_t key[EPL];
  bool live[EPL];
  if (S == 0) logit_keys<EPL, 0>(z, S, bias, T, E, t, lane, key, live);
  else logit_keys_upto<EPL, 4, MAXS>(z, S, bias, T, E, t, lane, key, live);
  topk_of_keys<EPL>(key, live, E, k, lane, cand, my_id, my_key);
}

// The selection of topk_lanes from the lanes' keys (all lanes of the wave take part).
template <int EPL>
__device__ __forceinline__ void topk_of_keys(uint32_t (&key)[EPL], bool (&live)[EPL], int E, int k, int lane,
                                             uint64_t* cand, int& my_id, uint32_t& my_key) {
  my_id = -1;
  my_key = 0;
  if (cand && k <= kThrMaxK) {
    topk_threshold<EPL>(key, live, E, k, lane, cand, my_id, my_key);
    return;
  }
  // one wave maximum per round over (key, ~expert): the largest key, ties to the lower expert
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
}

// Routing outputs of token t from the lanes' slots (all lanes of the wave take part): the
// sigmoids in fp64, their sum in slot order by every lane, w_j = s_j / sum; ids (if given) beside.
__device__ __forceinline__ void topk_store(int k, int t, int my_id, uint32_t my_key, int32_t* __restrict__ ids,
                                           float* __restrict__ w) {
  const int lane = threadIdx.x % kWave;
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

template <int EPL, int MAXS = kMaxRanges>  // experts per lane (E <= 64 * EPL); S <= MAXS
__device__ __forceinline__ void topk_token(const float* __restrict__ z, int S, const float* __restrict__ bias, int T,
                                           int E, int k, int t, int32_t* __restrict__ ids, float* __restrict__ w,
                                           int32_t* ids_copy = nullptr, uint64_t* cand = nullptr) {
  const int lane = threadIdx.x % kWave;
  int my_id;
  uint32_t my_key;
  topk_lanes<EPL, MAXS>(z, S, bias, T, E, k, t, cand, my_id, my_key);
  if (lane < k && ids_copy) ids_copy[t * k + lane] = my_id;
  if (w) topk_store(k, t, my_id, my_key, ids, w);   // (without w nothing more is stored)
}

}  // namespace moe
