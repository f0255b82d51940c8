// Device-side view of the quantised weight layouts and of the fp16 operands
// the expert kernels feed to the matrix cores (internal to libmoe).
//
// Every expert matrix product runs on v_mfma_f32_16x16x32_f16, one
// instruction per 32-value block, with the block's codes as the B operand.
// A code enters the matrix core as an exact small fp16 integer: OR-ing a 2-bit
// code q, shifted to bits p..p+1, into the mantissa of 1024.0 gives
// 1024 + q*2^p, and one packed fp16 subtraction of 1024 leaves q*2^p; an 8-bit
// code stored as u = q + 128 gives 1024 + u, and subtracting 1152 leaves q.
// (Codes placed directly as fp16 subnormals would need no subtraction, but the
// matrix cores then keep only about 17 significant bits of the block sum.)
// The activation operand is prepared to match: value i of a block sits at the
// K position its code occupies, multiplied by 2^(6-p) so that every product
// carries the same factor 2^6, and by a per-row power-of-two sigma that keeps
// it in fp16 range.  An fp32 activation is carried as two fp16 planes (hi + lo,
// 22 significant bits).  Hence, for each block b of 32 values,
//     P_b = sum_i A'_i B_i = 2^6 * sigma * sum_i q_i a_i
// and the layer's value  sum_b sum_i (d_b q_i + m_b) a_i  is assembled as
//     sigma * value = sum_b (2^-6 d_b) P_b  +  sum_b m_b (sigma S_b),
// the second sum (S_b = block sum of a; Q2SM only, Q8_0 has m = 0) being one
// more small matrix product over the block index.

// Planar layouts.  A row's codes are cut into 64-byte units (8 blocks of
// Q2SM, 2 blocks of Q8_0) in which the lane with K-group g of a 16x16x32
// fragment (values 8g..8g+7 of each block) finds its codes in the 16 bytes at
// 16g:
//   Q2SM: word i of those 16 bytes = [blk 2i byte 2g, blk 2i+1 byte 2g,
//         blk 2i byte 2g+1, blk 2i+1 byte 2g+1] (blk = block 8j+.. of unit j).
//   Q8_0: the 16 bytes are [blk 2j q[8g..8g+7], blk 2j+1 q[8g..8g+7]].
// Rows are taken in groups of 16, and a group stores unit by unit the 16
// rows' 64-byte units one after the other: a wave's load of one unit of 16
// rows reads 1 KiB of consecutive bytes.  Scales follow the same grouping:
// per (row group, unit), Q2SM the 16 rows' 8 fp16 d values (256 bytes) then
// their 8 fp16 m values (256 bytes); Q8_0 the 16 rows' 2 fp16 d values
// (64 bytes).  Missing blocks of a row's last unit, and the rows that pad the
// last group to 16, are zero.
#pragma once
#include "device.h"

namespace moe {

typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ f32x4_t mfma16(uint4 a, uint4 b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8_t, a), __builtin_bit_cast(f16x8_t, b), c,
                                                0, 0, 0);
}

__device__ __forceinline__ uint32_t f16_bits(float v) {
  _Float16 h = (_Float16)v;
  return (uint32_t)__builtin_bit_cast(uint16_t, h);
}

// hi = v rounded to fp16, lo = (v - hi) rounded to fp16
__device__ __forceinline__ void split_f16(float v, uint32_t& hi, uint32_t& lo) {
  const _Float16 h = (_Float16)v;
  hi = (uint32_t)__builtin_bit_cast(uint16_t, h);
  lo = f16_bits(v - (float)h);
}

constexpr float kScaleD = 0.015625f;  // 2^-6: the block scale's factor against P_b
constexpr float kSigmaH = 0.015625f;  // 2^-6: row scale of the intermediate h

template <int FMT>
struct Codes;

// Constants of the code unpacking, passed in from the host so that they live
// in registers: VOP3 instructions (v_and_or_b32, v_perm_b32) take no literals
// on this architecture.
struct FragConsts {
  uint32_t mask[4];      // 0x00030003 << 2s
  uint32_t k1024;        // fp16 1024.0 in both halves
  uint32_t neg1024;      // fp16 -1024.0 in both halves
  uint32_t x80;          // 0x80808080
  uint32_t k64;          // 0x64646464
  uint32_t neg1152;      // fp16 -1152.0 in both halves
  uint32_t sel_even;     // byte selectors {b0, 0x64, b2, 0x64} and {b1, 0x64, b3, 0x64}
  uint32_t sel_odd;
};

typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));

// 1024 + v in each half (v < 1024) -> v, exactly
__device__ __forceinline__ uint32_t sub_f16x2(uint32_t w, uint32_t neg_pair) {
  return __builtin_bit_cast(uint32_t, __builtin_bit_cast(f16x2_t, w) + __builtin_bit_cast(f16x2_t, neg_pair));
}

// A copy of a uniform value in a vector register, opaque to the optimiser.
__device__ __forceinline__ uint32_t to_vgpr(uint32_t v) {
  uint32_t r;
  asm volatile("v_mov_b32 %0, %1" : "=v"(r) : "s"(v));
  return r;
}

inline FragConsts frag_consts() {
  return FragConsts{{0x00030003u, 0x000C000Cu, 0x00300030u, 0x00C000C0u}, 0x64006400u, 0xE400E400u, 0x80808080u,
                    0x64646464u, 0xE480E480u, 0x04020400u, 0x04030401u};
}

// Byte offsets in the row-group layout (n_units units per row).
__host__ __device__ constexpr int64_t code_off(int row, int unit, int n_units) {
  return ((int64_t)(row >> 4) * n_units + unit) * 1024 + (row & 15) * 64;
}

template <>
struct Codes<FMT_Q2SM> {
  static constexpr int kUnitBlocks = 8;
  static constexpr bool kHasM = true;
  static constexpr int kDBytes = 16;      // d bytes of one row in one unit (8 fp16)
  static constexpr int kScaleUnit = 512;  // scale bytes of a (row group, unit): 16 rows of d, then of m
  static constexpr int kMOffset = 256;    // m values of a (row group, unit) after its d values
  __host__ __device__ static constexpr int64_t d_off(int row, int unit, int n_units) {
    return ((int64_t)(row >> 4) * n_units + unit) * kScaleUnit + (row & 15) * kDBytes;
  }
  // code and scale bytes per row (a matrix of 16 r rows takes r times 16 of these)
  __host__ __device__ static constexpr int64_t row_bytes(int cols) { return (int64_t)((cols / 32 + 7) / 8) * 64; }
  __host__ __device__ static constexpr int64_t scale_row_bytes(int cols) { return (int64_t)((cols / 32 + 7) / 8) * 32; }
  // B fragment of block i (0..7) of a unit from the lane's 16-byte chunk
  // k1024v: fp16 1024.0 pairs held in a vector register (a VALU instruction reads one scalar register)
  __device__ static __forceinline__ uint4 frag(const uint4& c, int i, const FragConsts& k, uint32_t k1024v) {
    const uint32_t w = (i >> 1) == 0 ? c.x : (i >> 1) == 1 ? c.y : (i >> 1) == 2 ? c.z : c.w;
    const uint32_t v = (i & 1) ? (w >> 8) : w;
    return make_uint4(sub_f16x2((v & k.mask[0]) | k1024v, k.neg1024), sub_f16x2((v & k.mask[1]) | k1024v, k.neg1024),
                      sub_f16x2((v & k.mask[2]) | k1024v, k.neg1024), sub_f16x2((v & k.mask[3]) | k1024v, k.neg1024));
  }
  // fragment element e (K position 8g+e) holds value 8g+val(e) at code bit position pos(e)
  __host__ __device__ static constexpr int val(int e) { return (e >> 1) + 4 * (e & 1); }
  __host__ __device__ static constexpr int pos(int e) { return 2 * (e >> 1); }
  __host__ __device__ static constexpr int elem_of(int r) { return 2 * (r & 3) + (r >> 2); }  // inverse of val
};

template <>
struct Codes<FMT_Q8_0> {
  static constexpr int kUnitBlocks = 2;
  static constexpr bool kHasM = false;
  static constexpr int kDBytes = 4;       // d bytes of one row in one unit (2 fp16)
  static constexpr int kScaleUnit = 64;   // scale bytes of a (row group, unit)
  __host__ __device__ static constexpr int64_t d_off(int row, int unit, int n_units) {
    return ((int64_t)(row >> 4) * n_units + unit) * kScaleUnit + (row & 15) * kDBytes;
  }
  __host__ __device__ static constexpr int64_t row_bytes(int cols) { return (int64_t)((cols / 32 + 1) / 2) * 64; }
  __host__ __device__ static constexpr int64_t scale_row_bytes(int cols) { return (int64_t)((cols / 32 + 1) / 2) * 4; }
  __device__ static __forceinline__ uint4 frag(const uint4& c, int i, const FragConsts& k, uint32_t) {
    const uint32_t a = (i ? c.z : c.x) ^ k.x80;   // u = q + 128
    const uint32_t b = (i ? c.w : c.y) ^ k.x80;
    return make_uint4(sub_f16x2(__builtin_amdgcn_perm(k.k64, a, k.sel_even), k.neg1152),
                      sub_f16x2(__builtin_amdgcn_perm(k.k64, a, k.sel_odd), k.neg1152),
                      sub_f16x2(__builtin_amdgcn_perm(k.k64, b, k.sel_even), k.neg1152),
                      sub_f16x2(__builtin_amdgcn_perm(k.k64, b, k.sel_odd), k.neg1152));
  }
  __host__ __device__ static constexpr int val(int e) { return (e == 1 || e == 5) ? e + 1 : (e == 2 || e == 6) ? e - 1 : e; }
  __host__ __device__ static constexpr int pos(int) { return 0; }
  __host__ __device__ static constexpr int elem_of(int r) { return val(r); }  // the order is an involution
};

// Runtime-format versions (the down projection's format decides how the
// intermediate h is laid out by the gate/up kernel).
__device__ __forceinline__ int elem_of_rt(int fmt, int r) {
  return fmt == FMT_Q2SM ? Codes<FMT_Q2SM>::elem_of(r) : Codes<FMT_Q8_0>::elem_of(r);
}
__device__ __forceinline__ int pos_rt(int fmt, int e) {
  return fmt == FMT_Q2SM ? Codes<FMT_Q2SM>::pos(e) : 0;
}

}  // namespace moe
