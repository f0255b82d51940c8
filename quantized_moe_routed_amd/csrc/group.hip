// Grouping of routing slots by expert: the counting sort of group.h, one
// workgroup per chunk of kGroupThreads slots.
#include "device.h"
#include "launch.h"
#include "group.h"

namespace moe {

__global__ __launch_bounds__(kGroupThreads) void group_kernel(const int32_t* __restrict__ ids, int n, int E,
                                                              int nbits, int32_t* __restrict__ counts,
                                                              int32_t* __restrict__ offsets,
                                                              int32_t* __restrict__ slot_list) {
  extern __shared__ int32_t sm[];
  __shared__ int32_t wave_tot[kGroupWaves];
  group_chunk(ids, n, E, nbits, blockIdx.x, counts, offsets, slot_list, sm, wave_tot);
}

hipError_t launch_group(const int32_t* ids, int T, int k, int E, int32_t* counts, int32_t* offsets,
                        int32_t* slot_list, hipStream_t s) {
  int nbits = 0;
  while ((1 << nbits) < E) ++nbits;
  const int n = T * k;
  const int chunks = n > 0 ? (n + kGroupThreads - 1) / kGroupThreads : 1;   // (no slots: zero counts and offsets)
  const size_t lds = sizeof(int32_t) * (size_t)(2 + kGroupWaves) * E;
  trace_pre("group", s);
  group_kernel<<<chunks, kGroupThreads, lds, s>>>(ids, n, E, nbits, counts, offsets, slot_list);
  trace_post("group", s);
  return hipGetLastError();
}

size_t group_lds_bytes(int E) { return sizeof(int32_t) * (size_t)(2 + kGroupWaves) * E; }

hipError_t group_set_lds_limit(size_t bytes) {
  return hipFuncSetAttribute(reinterpret_cast<const void*>(&group_kernel),
                             hipFuncAttributeMaxDynamicSharedMemorySize, (int)bytes);
}

}  // namespace moe
