// Stable grouping of routing slots by expert (a counting sort), one workgroup
// per chunk of kGroupThreads slots (internal to libmoe).
//
// The workgroups do not communicate.  Each counts the expert of every slot
// itself (LDS integer atomics; the totals do not depend on their order), both
// over all slots and over the slots before its own chunk, so it knows every
// expert's offset and where its chunk's slots of each expert begin.  Inside its
// chunk, the slots of one expert within a wave find each other with log2(E)
// ballots (a peer mask); a slot's rank is the popcount of its lower peers, and
// the per-wave counts of the chunk's earlier waves are added.  Workgroup 0 also
// stores counts and offsets.  The result is the stable order, bit for bit, for
// any number of workgroups.
#pragma once
#include "device.h"

namespace moe {

constexpr int kGroupThreads = 1024;
constexpr int kGroupWaves = kGroupThreads / kWave;

// Chunk c of the n slots (c = blockIdx.x); sm: (2 + kGroupWaves) E ints of LDS.
__device__ __forceinline__ void group_chunk(const int32_t* __restrict__ ids, int n, int E, int nbits, int c,
                                            int32_t* __restrict__ counts, int32_t* __restrict__ offsets,
                                            int32_t* __restrict__ slot_list, int32_t* sm, int32_t* wave_tot) {
  int32_t* cnt = sm;                 // [E] slots of each expert
  int32_t* cur = sm + E;             // [E] slots of each expert before the chunk, then where they start
  int32_t* wcnt = sm + 2 * E;        // [kGroupWaves][E] the chunk's slots per wave
  const int tid = threadIdx.x, lane = tid % kWave, wave = tid / kWave;
  const int base = c * kGroupThreads;

  for (int e = tid; e < 2 * E; e += kGroupThreads) sm[e] = 0;
  for (int i = tid; i < kGroupWaves * E; i += kGroupThreads) wcnt[i] = 0;
  __syncthreads();
  for (int s = tid; s < n; s += kGroupThreads) {
    const int e = ids[s];
    if ((unsigned)e < (unsigned)E) {
      atomicAdd(&cnt[e], 1);
      if (s < base) atomicAdd(&cur[e], 1);
    }
  }
  __syncthreads();

  // exclusive scan of cnt (E <= 1024: one expert per thread)
  {
    const int ce = tid < E ? cnt[tid] : 0;
    int incl = ce;
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
      const int ex = before + incl - ce;
      if (c == 0) {
        counts[tid] = ce;
        offsets[tid] = ex;
        if (tid == E - 1) offsets[E] = ex + ce;
      }
      cur[tid] += ex;
    }
  }

  const int s = base + tid;
  const int e = s < n ? ids[s] : -1;
  const bool valid = (unsigned)e < (unsigned)E;
  uint64_t peers = __ballot(valid);
  for (int b = 0; b < nbits; ++b) {
    const uint64_t ones = __ballot(valid && ((e >> b) & 1));
    peers &= ((e >> b) & 1) ? ones : ~ones;
  }
  const int rank = __popcll(peers & lanemask_lt());
  if (valid && rank == 0) wcnt[wave * E + e] = __popcll(peers);
  __syncthreads();   // also: cur complete
  if (valid) {
    int pos = cur[e] + rank;
    for (int w = 0; w < wave; ++w) pos += wcnt[w * E + e];
    slot_list[pos] = s;
  }
}

}  // namespace moe
