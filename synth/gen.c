/*
 * Seeded synthetic inputs for the routed-expert MoE layer.
 *
 * This file generates inputs only: normal draws, permutations, and the
 * block encodings that turn a drawn fp32 matrix into the quantised bytes the
 * layer consumes.  It computes nothing of the layer itself (no routing, no
 * dequantisation, no projection, no combine).  Both the CPU oracle and the
 * GPU path read what it writes.
 *
 * Random numbers: SplitMix64 (Steele, Lea and Flood, "Fast splittable
 * pseudorandom number generators", OOPSLA 2014) used as a counter-based
 * generator: output i of stream s is mix64(key(seed, s) + (i + 1) * GAMMA).
 * Normals: Marsaglia's polar method (Marsaglia and Bray, 1964), one accepted
 * pair per counter index p giving normals 2p and 2p+1; each rejection redraws
 * from a sub-counter, so every index is independent of thread scheduling.
 *
 * Block formats written here (definition layout, array-of-structures):
 *   Q8_0 : { fp16 d; int8 q[32]; }              34 bytes per 32 values
 *   Q2SM : { fp16 d; fp16 m; uint8 qs[8]; }      12 bytes per 32 values
 *          value i of the block lives in byte i/4, bits 2*(i%4)..2*(i%4)+1
 * Blocks run along the contraction (column) axis; a matrix is row-major.
 */
#include <math.h>
#include <stdint.h>
#include <string.h>

#define GAMMA 0x9E3779B97F4A7C15ULL

static inline uint64_t mix64(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ULL;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBULL;
  return z ^ (z >> 31);
}

static inline uint64_t stream_key(uint64_t seed, uint64_t stream) {
  return mix64(mix64(seed * GAMMA + 0x632BE59BD9B4E019ULL) ^ (stream * 0xD1B54A32D192ED03ULL));
}

/* output i of a stream: SplitMix64 state after i+1 increments, mixed */
static inline uint64_t draw_u64(uint64_t key, uint64_t i) { return mix64(key + (i + 1) * GAMMA); }

/* uniform in the open interval (-1, 1), 53-bit resolution */
static inline double draw_sym(uint64_t key, uint64_t i) {
  return ((double)(draw_u64(key, i) >> 11) + 0.5) * (2.0 / 9007199254740992.0) - 1.0;
}

/* normal pair p of a stream (polar method) */
static void normal_pair(uint64_t key, uint64_t p, double* a, double* b) {
  for (uint64_t att = 0;; ++att) {
    /* sub-counter: 2 uniforms per attempt, attempts interleaved above all pairs */
    uint64_t base = (p << 8) + (att << 1);
    double u = draw_sym(key, base), v = draw_sym(key, base + 1);
    double s = u * u + v * v;
    if (s > 0.0 && s < 1.0) {
      double f = sqrt(-2.0 * log(s) / s);
      *a = u * f;
      *b = v * f;
      return;
    }
    if (att >= 120) { /* probability (1-pi/4)^120 ~ 1e-80: unreachable in practice */
      *a = 0.0;
      *b = 0.0;
      return;
    }
  }
}

/* float -> IEEE binary16 bits, round to nearest even (also subnormals, inf, nan) */
uint16_t synth_f32_to_f16_bits(float f) {
  uint32_t x;
  memcpy(&x, &f, 4);
  uint32_t sign = (x >> 16) & 0x8000u;
  uint32_t ax = x & 0x7FFFFFFFu;
  if (ax >= 0x7F800000u) return (uint16_t)(sign | (ax > 0x7F800000u ? 0x7E00u : 0x7C00u));
  if (ax >= 0x477FF000u) return (uint16_t)(sign | 0x7C00u); /* rounds to >= 65520 -> inf */
  if (ax < 0x38800000u) {                                     /* below 2^-14: subnormal half */
    if (ax < 0x33000000u) return (uint16_t)sign;              /* < 2^-25: rounds to zero */
    uint32_t mant = (ax & 0x7FFFFFu) | 0x800000u;
    int e = (int)(ax >> 23);                                  /* 102..112 */
    int shift = 126 - e;                                      /* value = mant * 2^(e-150); half ulp 2^-24 */
    uint32_t q = mant >> shift, rem = mant & ((1u << shift) - 1u), half = 1u << (shift - 1);
    if (rem > half || (rem == half && (q & 1u))) q++;
    return (uint16_t)(sign | q);
  }
  uint32_t e = (ax >> 23) - 112u; /* rebias 127 -> 15 */
  uint32_t mant = ax & 0x7FFFFFu;
  uint32_t h = (e << 10) | (mant >> 13);
  uint32_t rem = mant & 0x1FFFu;
  if (rem > 0x1000u || (rem == 0x1000u && (h & 1u))) h++;
  return (uint16_t)(sign | h);
}

double synth_f16_bits_to_f64(uint16_t h) {
  int e = (h >> 10) & 0x1F, m = h & 0x3FF;
  double v;
  if (e == 0) v = ldexp((double)m, -24);
  else if (e == 31) v = m ? NAN : INFINITY;
  else v = ldexp((double)(m | 0x400), e - 25);
  return (h & 0x8000) ? -v : v;
}

/* fp32 -> bfloat16 bits, round to nearest even (finite inputs) */
uint16_t synth_f32_to_bf16_bits(float f) {
  uint32_t x;
  memcpy(&x, &f, 4);
  if ((x & 0x7FFFFFFFu) > 0x7F800000u) return (uint16_t)((x >> 16) | 0x40u);
  x += 0x7FFFu + ((x >> 16) & 1u);
  return (uint16_t)(x >> 16);
}

/* n normals * sigma rounded to fp32 */
void synth_normal_f32(uint64_t seed, uint64_t stream, int64_t n, double sigma, float* out) {
  uint64_t key = stream_key(seed, stream);
  int64_t np = (n + 1) / 2;
#pragma omp parallel for schedule(static)
  for (int64_t p = 0; p < np; ++p) {
    double a, b;
    normal_pair(key, (uint64_t)p, &a, &b);
    out[2 * p] = (float)(a * sigma);
    if (2 * p + 1 < n) out[2 * p + 1] = (float)(b * sigma);
  }
}

/* n raw 64-bit draws */
void synth_u64(uint64_t seed, uint64_t stream, int64_t n, uint64_t* out) {
  uint64_t key = stream_key(seed, stream);
  for (int64_t i = 0; i < n; ++i) out[i] = draw_u64(key, (uint64_t)i);
}

/* seeded permutation of 0..n-1 (Fisher-Yates, Durstenfeld form, Lemire-free modulo
 * with 64-bit draws: bias below 2^-40 for n < 2^24) */
void synth_permutation(uint64_t seed, uint64_t stream, int32_t n, int32_t* out) {
  uint64_t key = stream_key(seed, stream);
  for (int32_t i = 0; i < n; ++i) out[i] = i;
  for (int32_t i = n - 1; i > 0; --i) {
    int32_t j = (int32_t)(draw_u64(key, (uint64_t)i) % (uint64_t)(i + 1));
    int32_t t = out[i];
    out[i] = out[j];
    out[j] = t;
  }
}

/* --- encoders: one 32-value block ------------------------------------------ */

static void encode_q8_0(const float* v, uint8_t* blk) {
  double amax = 0.0;
  for (int i = 0; i < 32; ++i) {
    double a = fabs((double)v[i]);
    if (a > amax) amax = a;
  }
  double d = amax / 127.0;
  uint16_t d16 = synth_f32_to_f16_bits((float)d);
  memcpy(blk, &d16, 2);
  int8_t* q = (int8_t*)(blk + 2);
  for (int i = 0; i < 32; ++i) {
    double r = d > 0.0 ? nearbyint((double)v[i] / d) : 0.0;
    if (r > 127.0) r = 127.0;
    if (r < -127.0) r = -127.0;
    q[i] = (int8_t)r;
  }
}

static void encode_q2sm(const float* v, uint8_t* blk) {
  double lo = v[0], hi = v[0];
  for (int i = 1; i < 32; ++i) {
    if (v[i] < lo) lo = v[i];
    if (v[i] > hi) hi = v[i];
  }
  uint16_t m16 = synth_f32_to_f16_bits((float)lo);
  uint16_t d16 = synth_f32_to_f16_bits((float)((hi - lo) / 3.0));
  double m = synth_f16_bits_to_f64(m16), d = synth_f16_bits_to_f64(d16);
  memcpy(blk, &d16, 2);
  memcpy(blk + 2, &m16, 2);
  uint8_t* qs = blk + 4;
  memset(qs, 0, 8);
  for (int i = 0; i < 32; ++i) {
    int q = 0;
    if (d > 0.0) {
      double r = nearbyint(((double)v[i] - m) / d);
      q = r < 0.0 ? 0 : (r > 3.0 ? 3 : (int)r);
    }
    qs[i >> 2] |= (uint8_t)(q << (2 * (i & 3)));
  }
}

/* fmt: 1 = Q8_0, 2 = Q2SM (0 = plain fp32 rows, copied) */
int64_t synth_block_bytes(int fmt) { return fmt == 1 ? 34 : (fmt == 2 ? 12 : 128); }

/* Draw n_mat matrices [rows x cols] of N(0, sigma) and encode them.  Matrix j
 * uses stream (stream0 + j), row r of it the normal indices r*cols .. r*cols+cols-1,
 * so any subset of matrices or rows can be regenerated identically. */
void synth_quant_matrices(uint64_t seed, uint64_t stream0, int32_t n_mat, int32_t rows, int32_t cols,
                          double sigma, int32_t fmt, uint8_t* out) {
  int64_t nb = cols / 32;
  int64_t row_bytes = fmt == 0 ? (int64_t)cols * 4 : nb * synth_block_bytes(fmt);
  int64_t total_rows = (int64_t)n_mat * rows;
#pragma omp parallel for schedule(dynamic, 16)
  for (int64_t gr = 0; gr < total_rows; ++gr) {
    int32_t j = (int32_t)(gr / rows), r = (int32_t)(gr % rows);
    uint64_t key = stream_key(seed, stream0 + (uint64_t)j);
    float v[32 * 512]; /* cols <= 16384 */
    for (int64_t c = 0; c < cols; c += 2) {
      double a, b;
      normal_pair(key, (uint64_t)(((int64_t)r * cols + c) / 2), &a, &b);
      v[c] = (float)(a * sigma);
      v[c + 1] = (float)(b * sigma);
    }
    uint8_t* dst = out + gr * row_bytes;
    if (fmt == 0) {
      memcpy(dst, v, (size_t)cols * 4);
    } else {
      for (int64_t b = 0; b < nb; ++b) {
        if (fmt == 1) encode_q8_0(v + 32 * b, dst + 34 * b);
        else encode_q2sm(v + 32 * b, dst + 12 * b);
      }
    }
  }
}

void synth_f32_to_bf16(const float* in, int64_t n, uint16_t* out) {
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; ++i) out[i] = synth_f32_to_bf16_bits(in[i]);
}

void synth_f32_to_f16(const float* in, int64_t n, uint16_t* out) {
  for (int64_t i = 0; i < n; ++i) out[i] = synth_f32_to_f16_bits(in[i]);
}
