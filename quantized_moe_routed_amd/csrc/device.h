// Device-side helpers shared by the gfx950 kernels of libmoe.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

constexpr int kWave = 64;

enum : int { FMT_F32 = 0, FMT_Q8_0 = 1, FMT_Q2SM = 2 };
enum : int { ACT_F32 = 0, ACT_BF16 = 1 };

// A stacked weight matrix in the planar layout (see include/moe.h).
struct QMat {
  const void* codes;
  const void* scales;
  int32_t rows;
  int32_t cols;
};

__device__ __forceinline__ float half_bits_to_float(uint32_t h16) {
  _Float16 h;
  uint16_t b = (uint16_t)h16;
  __builtin_memcpy(&h, &b, 2);
  return (float)h;
}

__device__ __forceinline__ float bf16_bits_to_float(uint32_t b16) {
  return __uint_as_float(b16 << 16);
}

// Load activation element i of a row (fp32 or bf16 bits), as fp32 (exact).
template <int ACT>
__device__ __forceinline__ float load_act(const void* x, int64_t i) {
  if constexpr (ACT == ACT_F32) {
    return reinterpret_cast<const float*>(x)[i];
  } else {
    return bf16_bits_to_float(reinterpret_cast<const uint16_t*>(x)[i]);
  }
}

// Sum over the 64 lanes of a wave; every lane receives the total.
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int m = 1; m < kWave; m <<= 1) v += __shfl_xor(v, m, kWave);
  return v;
}

__device__ __forceinline__ uint64_t lanemask_lt() {
  return (1ull << (threadIdx.x % kWave)) - 1ull;
}

__device__ __forceinline__ float silu(float g) { return g / (1.0f + expf(-g)); }

}  // namespace moe
