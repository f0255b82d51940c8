// Device-side view of the quantised weight layouts and of the fp16 operands
// the expert kernels feed to the matrix cores (internal to libmoe).
//
// Every expert matrix product runs on fp16 matrix cores with the weights'
// codes as the B operand, entering as exact small fp16 numbers:
//   2-bit codes: a code q placed alone in the low two bits of a 4-bit field is,
//     read as an FP4 (E2M1) number, exactly q/2; the gfx950 conversion
//     v_cvt_scalef32_pk_f16_fp4 turns two such fields into two fp16 values
//     times a scale, here 2^-5, so the operand is q * 2^-6 exactly;
//   8-bit codes stored as u = q + 128: OR-ing u into the mantissa of 1024.0
//     gives 1024 + u, and one packed fp16 subtraction of 1152 leaves q.
// The activation operand is prepared to match: value i of a block sits at the
// K position its code occupies, multiplied by 2^6 and by a per-row
// power-of-two sigma that keeps it in fp16 range.  An fp32 activation is
// carried as two fp16 planes (hi + lo, 22 significant bits).  Hence, for each
// block b of 32 values,
//     P_b = sum_i A'_i B_i = c * sigma * sum_i q_i a_i,  c = 1 (2-bit), 2^6 (8-bit)
// and the layer's value  sum_b sum_i (d_b q_i + m_b) a_i  is assembled as
//     sigma * value = sum_b (d_b / c) P_b  +  sum_b m_b (sigma S_b),
// the second sum (S_b = block sum of a; 2-bit only, Q8_0 has m = 0) being one
// more small matrix product over the block index.
// (Codes placed directly as fp16 subnormals would need no conversion at all,
// but the matrix cores then keep only about 17 significant bits of a block
// sum; normal fp16 operands keep the block sums exact to fp32 rounding.)

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

// Power-of-two scale of an operand row whose largest magnitude is m: sigma = 2^(9 - E), E the
// smallest integer with m < 2^E (E = 0 for an all-zero row), so that every value times
// sigma * 2^6 lies below 2^15 and its block sums times sigma below 2^14.  A value within 2^18 of
// the row's largest then keeps a normal fp16 lo half, i.e. 22 significant bits in its hi + lo
// pair; smaller ones keep an absolute error below 2^-25 in these units (2^-39 of the largest).  E
// is kept at -110 or above so that sigma stays a finite fp32 number for subnormal rows.
__device__ __forceinline__ float row_scale(float m) {
  int ex = 0;
  if (m > 0.0f) (void)frexpf(m, &ex);   // m = f * 2^ex, f in [0.5, 1): m < 2^ex
  return ldexpf(1.0f, 9 - max(ex, -110));
}

// hi + lo fp16 pairs of 8 values times sc, packed in the order given
__device__ __forceinline__ void split8(const float (&v)[8], float sc, uint4& hi, uint4& lo) {
  uint32_t h[8], l[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) split_f16(v[e] * sc, h[e], l[e]);
  hi = make_uint4(h[0] | (h[1] << 16), h[2] | (h[3] << 16), h[4] | (h[5] << 16), h[6] | (h[7] << 16));
  lo = make_uint4(l[0] | (l[1] << 16), l[2] | (l[3] << 16), l[4] | (l[5] << 16), l[6] | (l[7] << 16));
}

template <int FMT>
struct Codes;

// Two FP4 (E2M1) fields of byte SEL of t as fp16, times 2^-5: a field 00qq gives q * 2^-6.
template <int SEL>
__device__ __forceinline__ uint32_t fp4x2(uint32_t t) {
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(t, 0.03125f, SEL));
}

// Constants of the 8-bit code unpacking, passed in from the host so that they
// live in registers: VOP3 instructions (v_perm_b32) take no literals on this
// architecture.
struct FragConsts {
  uint32_t x80;          // 0x80808080
  uint32_t k64;          // 0x64646464
  uint32_t neg1152;      // fp16 -1152.0 in both halves
  uint32_t sel_even;     // byte selectors {b0, 0x64, b2, 0x64} and {b1, 0x64, b3, 0x64}
  uint32_t sel_odd;
};

typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));

// 1024 + v in each half plus a negative pair, exactly (v < 1024)
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
  return FragConsts{0x80808080u, 0x64646464u, 0xE480E480u, 0x04020400u, 0x04030401u};
}

// Fragment order shared by both formats: element e of a lane's 8 K positions (K position 8g+e of
// a block) holds value 8g+frag_val(e), bits 0 and 1 of e swapped; the map is its own inverse.
__host__ __device__ constexpr int frag_val(int e) { return (e & 4) | ((e & 1) << 1) | ((e >> 1) & 1); }

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
  static constexpr float kDScale = 1.0f;  // factor of d against P_b
  // B fragment of block i (0..7) of a unit from the lane's 16-byte chunk.  The word holding the
  // block's two bytes (values 8g..8g+3 and 8g+4..8g+7, value j of a byte at bits 2j) is masked
  // once into 4-bit fields holding codes 0 and 2 of each byte (t0) and codes 1 and 3 (t1); each
  // conversion reads one byte of t0 or t1.
  __device__ static __forceinline__ uint4 frag(const uint4& c, int i, const FragConsts&) {
    const uint32_t w = (i >> 1) == 0 ? c.x : (i >> 1) == 1 ? c.y : (i >> 1) == 2 ? c.z : c.w;
    const uint32_t t0 = w & 0x33333333u, t1 = (w >> 2) & 0x33333333u;
    if (i & 1) return make_uint4(fp4x2<1>(t0), fp4x2<1>(t1), fp4x2<3>(t0), fp4x2<3>(t1));
    return make_uint4(fp4x2<0>(t0), fp4x2<0>(t1), fp4x2<2>(t0), fp4x2<2>(t1));
  }
};

template <>
struct Codes<FMT_Q8_0> {
  static constexpr int kUnitBlocks = 2;
  static constexpr bool kHasM = false;
  static constexpr int kDBytes = 4;       // d bytes of one row in one unit (2 fp16)
  static constexpr int kScaleUnit = 64;   // scale bytes of a (row group, unit)
  static constexpr float kDScale = 0.015625f;   // 2^-6: factor of d against P_b
  __host__ __device__ static constexpr int64_t d_off(int row, int unit, int n_units) {
    return ((int64_t)(row >> 4) * n_units + unit) * kScaleUnit + (row & 15) * kDBytes;
  }
  __host__ __device__ static constexpr int64_t row_bytes(int cols) { return (int64_t)((cols / 32 + 1) / 2) * 64; }
  __host__ __device__ static constexpr int64_t scale_row_bytes(int cols) { return (int64_t)((cols / 32 + 1) / 2) * 4; }
  // B fragment of block i (0 or 1) of a unit: u = q + 128 in the mantissa of 1024.0, less 1152
  __device__ static __forceinline__ uint4 frag(const uint4& c, int i, const FragConsts& k) {
    const uint32_t a = (i ? c.z : c.x) ^ k.x80;   // u = q + 128
    const uint32_t b = (i ? c.w : c.y) ^ k.x80;
    return make_uint4(sub_f16x2(__builtin_amdgcn_perm(k.k64, a, k.sel_even), k.neg1152),
                      sub_f16x2(__builtin_amdgcn_perm(k.k64, a, k.sel_odd), k.neg1152),
                      sub_f16x2(__builtin_amdgcn_perm(k.k64, b, k.sel_even), k.neg1152),
                      sub_f16x2(__builtin_amdgcn_perm(k.k64, b, k.sel_odd), k.neg1152));
  }
};

}  // namespace moe
