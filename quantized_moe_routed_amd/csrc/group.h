// Stable grouping of routing slots by expert (a counting sort), done by one
// workgroup (internal to libmoe; shared by the grouping kernel and the fused
// small-batch front kernel).
//
// Counts use LDS integer atomics (the total does not depend on their order).
// Placement walks the slots in chunks of 1024 in slot order; inside a wave the
// slots of one expert find each other with log2(E) ballots (a peer mask), their
// rank is the popcount of lower peers, and the per-wave counts of earlier
// waves plus a running per-expert cursor give the final position.  The result
// is the stable order, bit for bit.
#pragma once
#include "device.h"

namespace moe {

constexpr int kGroupThreads = 1024;
constexpr int kGroupWaves = kGroupThreads / kWave;

// The grouping done by one workgroup of kGroupThreads threads; sm: (2 + kGroupWaves) E ints of
// LDS.  counts and offsets may point to LDS as well as to global memory.
__device__ __forceinline__ void group_block(const int32_t* ids, int n, int E, int nbits, int32_t* counts,
                                            int32_t* offsets, int32_t* __restrict__ slot_list, int32_t* sm,
                                            int32_t* wave_tot) {
  int32_t* cnt = sm;                 // [E]
  int32_t* cur = sm + E;             // [E] running write cursor
  int32_t* wcnt = sm + 2 * E;        // [kGroupWaves][E]
  const int tid = threadIdx.x, lane = tid % kWave, wave = tid / kWave;

  for (int e = tid; e < E; e += kGroupThreads) cnt[e] = 0;
  for (int i = tid; i < kGroupWaves * E; i += kGroupThreads) wcnt[i] = 0;
  __syncthreads();
  for (int s = tid; s < n; s += kGroupThreads) {
    const int e = ids[s];
    if ((unsigned)e < (unsigned)E) atomicAdd(&cnt[e], 1);
  }
  __syncthreads();

  // exclusive scan of cnt (E <= 1024: one expert per thread)
  {
    const int c = tid < E ? cnt[tid] : 0;
    int incl = c;
#pragma unroll
    for (int d = 1; d < kWave; d <<= 1) {
      const int o = __shfl_up(incl, d, kWave);
      if (lane >= d) incl += o;
    }
    if (lane == kWave - 1) wave_tot[wave] = incl;
    __syncthreads();
    int before = 0;
    for (int w = 0; w < wave; ++w) before += wave_tot[w];
    if (tid < E) {
      const int ex = before + incl - c;
      counts[tid] = c;
      offsets[tid] = ex;
      cur[tid] = ex;
      if (tid == E - 1) offsets[E] = ex + c;
    }
  }
  __syncthreads();

  for (int base = 0; base < n; base += kGroupThreads) {
    const int s = base + tid;
    int e = s < n ? ids[s] : -1;
    const bool valid = (unsigned)e < (unsigned)E;
    uint64_t peers = __ballot(valid);
    for (int b = 0; b < nbits; ++b) {
      const uint64_t ones = __ballot(valid && ((e >> b) & 1));
      peers &= ((e >> b) & 1) ? ones : ~ones;
    }
    const int rank = __popcll(peers & lanemask_lt());
    if (valid && rank == 0) wcnt[wave * E + e] = __popcll(peers);
    __syncthreads();
    if (valid) {
      int pos = cur[e] + rank;
      for (int w = 0; w < wave; ++w) pos += wcnt[w * E + e];
      slot_list[pos] = s;
    }
    __syncthreads();
    for (int x = tid; x < E; x += kGroupThreads) {
      int add = 0;
      for (int w = 0; w < kGroupWaves; ++w) {
        add += wcnt[w * E + x];
        wcnt[w * E + x] = 0;
      }
      cur[x] += add;
    }
    __syncthreads();
  }
}

}  // namespace moe
