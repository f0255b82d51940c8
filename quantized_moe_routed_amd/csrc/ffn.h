// Shared pieces of the two expert-FFN kernels (internal to libmoe): the
// argument block of one projection launch and the block-scale accessors.
#pragma once
#include "device.h"
#include "fmt.h"
#include "smallsel.h"

namespace moe {

enum { MODE_GATEUP = 0, MODE_DOWN = 1 };

constexpr int kMaxFfnK = 8192;      // longest contraction (H or I) the expert kernels take

struct FfnTileArgs {
  const uint16_t *a_hi, *a_lo;      // prepared operand planes, row stride K (gate/up: x; large down: h)
  const uint16_t *s_hi, *s_lo;      // their block-sum planes, row stride nb32
  const float* sigma;               // their row scales: per token (gate/up), per grouped position (large down)
  const float *hf, *hsf, *hmf;      // small down: h, its block sums and block maxima, fp32 and unscaled
                                    // (row strides K, nb32, nb32), scaled per row while staged
  int K, N, nb32, k;
  QMat w0, w1;                      // gate, up (gate/up) or down (w0 only)
  const int32_t* slot_list;
  const int4* tiles;
  const int4* tile_tok;             // small gate/up tiles: the token of each row
  const int32_t* n_tiles;
  int fd, I, nb32I;                 // gate/up: down format, I, padded block count of h
  int stage_rows;                   // small tiles: rows of the LDS staging area (min(4, T))
  FragConsts kc;
  float *h, *hs, *hm;               // gate/up out: h = silu(g) * u (in the operand's K order), its block
                                    // sums (index order) and block maxima of |h|, row strides I, nb32I, nb32I;
                                    // one-slot tiles instead write the block-scaled planes below, and in
                                    // hm the inverse of each block's scale
  uint16_t *hb_hi, *hb_lo;          // gate/up of one-slot tiles: h as the down projection's fp16 hi + lo
                                    // operand, each 32-column block at its own power-of-two scale
  float* y;
  SelArgs sel;                      // SEL launches: selection inputs and routing outputs
};

// The d values of one row in one unit (at p): 8 fp16 (Q2SM) or 2 fp16 (Q8_0, in .x).
template <int F>
__device__ __forceinline__ uint4 load_d(const uint8_t* p) {
  if constexpr (F == FMT_Q2SM) {
    return *reinterpret_cast<const uint4*>(p);
  } else {
    return make_uint4(*reinterpret_cast<const uint32_t*>(p), 0u, 0u, 0u);
  }
}

template <int F>
__device__ __forceinline__ float d_of(const uint4& dw, int i) {
  uint32_t w;
  if constexpr (F == FMT_Q2SM) {
    w = (i >> 1) == 0 ? dw.x : (i >> 1) == 1 ? dw.y : (i >> 1) == 2 ? dw.z : dw.w;
  } else {
    w = dw.x;
  }
  return half_bits_to_float((i & 1) ? (w >> 16) : (w & 0xFFFFu)) * Codes<F>::kDScale;
}

// Direct load of 16 bytes per lane into LDS: lane l's bytes land at lds_base + 16 l (lanes off in
// EXEC load nothing).  Completion is tracked by vmcnt only; the compiler does not see these loads,
// so the caller waits for them explicitly before reading the LDS.
__device__ __forceinline__ void dma16(const void* src, uint32_t lds_base) {
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(src), "s"(lds_base)
               : "memory", "m0");
}
__device__ __forceinline__ void wait_vmem() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }
// Wait until at most N vector-memory loads of this wave are outstanding.
template <int N>
__device__ __forceinline__ void wait_vmem_at_most() {
  static_assert(N >= 0 && N <= 63, "vmcnt range");
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// Large-tile launch (ffn_large.hip): tiles of up to 128 slots of one expert.
hipError_t launch_large(const FfnTileArgs& t, int fmt, int mode, bool lo, int max_tiles, hipStream_t s);

// The down projection's operand of the rows of the large tiles (ffn_large.hip): each row's h and
// block sums scaled by the power of two of its largest |h| (row_scale), as fp16 hi + lo planes,
// and the scale itself.
struct HConvArgs {
  const float *h, *hs, *hm;
  uint16_t *hq_hi, *hq_lo, *hsq_hi, *hsq_lo;
  float* hsig;
  const int4* tiles;
  const int32_t* n_tiles;
  int I, nb32I;
};
hipError_t launch_hconv(const HConvArgs& c, int max_tiles, int max_rows, hipStream_t s);   // max_rows: per tile

}  // namespace moe
