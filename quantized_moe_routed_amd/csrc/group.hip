// Stable grouping of routing slots by expert (a counting sort).
//
// One workgroup of 16 waves.  Counts use LDS integer atomics (the total does
// not depend on their order).  Placement walks the slots in chunks of 1024 in
// slot order; inside a wave the slots of one expert find each other with
// log2(E) ballots (a peer mask), their rank is the popcount of lower peers,
// and the per-wave counts of earlier waves plus a running per-expert cursor
// give the final position.  The result is the stable order, bit for bit.
#include "device.h"
#include "launch.h"

namespace moe {

constexpr int kGroupThreads = 1024;
constexpr int kGroupWaves = kGroupThreads / kWave;

__global__ __launch_bounds__(kGroupThreads) void group_kernel(const int32_t* __restrict__ ids, int n, int E,
                                                              int nbits, int32_t* __restrict__ counts,
                                                              int32_t* __restrict__ offsets,
                                                              int32_t* __restrict__ slot_list) {
  extern __shared__ int32_t sm[];
  int32_t* cnt = sm;                 // [E]
  int32_t* cur = sm + E;             // [E] running write cursor
  int32_t* wcnt = sm + 2 * E;        // [kGroupWaves][E]
  __shared__ int32_t wave_tot[kGroupWaves];
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

hipError_t launch_group(const int32_t* ids, int T, int k, int E, int32_t* counts, int32_t* offsets,
                        int32_t* slot_list, hipStream_t s) {
  int nbits = 0;
  while ((1 << nbits) < E) ++nbits;
  const size_t lds = sizeof(int32_t) * (size_t)(2 + kGroupWaves) * E;
  trace_pre("group", s);
  group_kernel<<<1, kGroupThreads, lds, s>>>(ids, T * k, E, nbits, counts, offsets, slot_list);
  trace_post("group", s);
  return hipGetLastError();
}

size_t group_lds_bytes(int E) { return sizeof(int32_t) * (size_t)(2 + kGroupWaves) * E; }

hipError_t group_set_lds_limit(size_t bytes) {
  return hipFuncSetAttribute(reinterpret_cast<const void*>(&group_kernel),
                             hipFuncAttributeMaxDynamicSharedMemorySize, (int)bytes);
}

}  // namespace moe
