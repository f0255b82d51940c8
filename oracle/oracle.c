/*
 * CPU oracle for the routed-expert MoE layer -- TEST INFRASTRUCTURE ONLY.
 *
 * Plain, slow, obviously correct.  Only the tests, the smoke check and the
 * benchmark's CPU-baseline leg may load this library; the product path never
 * does.  It shares no code with the GPU library.
 *
 * What it computes (the layer of a DeepSeek-V4-class model whose routed
 * experts the three pages split, slice and quantise):
 *
 *   z[t,e]   = x[t] . Wr[e] (+ bias[e])        router logit, canonical fp32 order (below)
 *   ids[t]   = the k experts with the largest z, ties to the lower index
 *   w[t,j]   = s_j / sum s,  s_j = sigmoid(z[t, ids[t,j]])     (fp64, rounded to fp32)
 *   y[t,j]   = D_e (silu(G_e x) * (U_e x)),  e = ids[t,j]      (fp64)
 *   out[t]   = sum over j ascending of owned slots: w[t,j] * y[t,j]   (fp64, rounded once)
 *
 * Expert ownership (aeonmindai/arc PR #89, "Stage 1 -- EP=2"): a share owns
 * a subset of experts, global ids map to local ids through a table (-1 =
 * unowned), and a share's partial is the sum over the slots it owns.  Every
 * slot is owned by exactly one share, so the partials over any partition add
 * up to the full output.
 *
 * Formats (definition layout, blocks of 32 along the contraction axis):
 *   Q8_0: {fp16 d; int8 q[32]}            value = d * q
 *   Q2SM: {fp16 d; fp16 m; uint8 qs[8]}   value = d * q + m, q = 2-bit code,
 *                                          value i in byte i/4 at bits 2*(i%4)
 *   F32 : plain fp32 rows
 * The routed gate/up/down roles of these formats follow antirez/ds4 PR #754,
 * "Supported paths and safety" (2-bit routed gate/up and down, Q8_0 dense
 * projections); the 2-bit layout above is a stand-in for the pages' IQ2_XXS /
 * Q2_K, whose codebooks the pages do not give.
 *
 * Canonical router order (fixed here so that expert ids are reproducible bit
 * for bit; the pages name no order):
 *   per block b of 32: p = 0.0f; p = fmaf(wq_i, x_i, p) for i = 0..31 in turn
 *                      (wq_i = int8 code as float for Q8_0, the fp32 weight for F32)
 *   r_b = d_b * p  (fp32 multiply; F32 router: r_b = p)
 *   z   = balanced pairwise tree over b: level 1 adds (r0+r1), (r2+r3), ...,
 *         an odd last element is carried up unchanged, repeat until one is left
 *   z  += bias[e] (fp32 add), when a bias is given.
 *
 * Build: gcc -O2 -ffp-contract=off -fopenmp (no contraction of the fp32
 * multiply and add, so every rounding is the one written here).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

enum { OR_F32 = 0, OR_Q8_0 = 1, OR_Q2SM = 2 };

/* IEEE binary16 bits -> double (exact) */
static double half_to_double(uint16_t h) {
  int e = (h >> 10) & 0x1F, m = h & 0x3FF;
  double v;
  if (e == 0) v = ldexp((double)m, -24);
  else if (e == 31) v = m ? NAN : INFINITY;
  else v = ldexp((double)(m | 0x400), e - 25);
  return (h & 0x8000) ? -v : v;
}

static uint16_t rd16(const uint8_t* p) { return (uint16_t)(p[0] | (p[1] << 8)); }

int64_t oracle_row_bytes(int fmt, int cols) {
  if (fmt == OR_Q8_0) return (int64_t)(cols / 32) * 34;
  if (fmt == OR_Q2SM) return (int64_t)(cols / 32) * 12;
  return (int64_t)cols * 4;
}

/* Dequantise one row of `cols` values from its definition bytes, exactly, in fp64. */
void oracle_dequant_row(int fmt, const uint8_t* row, int cols, double* out) {
  if (fmt == OR_F32) {
    for (int c = 0; c < cols; ++c) {
      float f;
      memcpy(&f, row + 4 * c, 4);
      out[c] = (double)f;
    }
    return;
  }
  for (int b = 0; b < cols / 32; ++b) {
    if (fmt == OR_Q8_0) {
      const uint8_t* blk = row + 34 * b;
      double d = half_to_double(rd16(blk));
      const int8_t* q = (const int8_t*)(blk + 2);
      for (int i = 0; i < 32; ++i) out[32 * b + i] = d * (double)q[i];
    } else {
      const uint8_t* blk = row + 12 * b;
      double d = half_to_double(rd16(blk)), m = half_to_double(rd16(blk + 2));
      for (int i = 0; i < 32; ++i) {
        int q = (blk[4 + i / 4] >> (2 * (i % 4))) & 3;
        out[32 * b + i] = d * (double)q + m;
      }
    }
  }
}

/* Router logit of one token against one router row, in the canonical fp32 order. */
float oracle_router_logit(int fmt, const uint8_t* wrow, const float* x, int H, const float* bias_e) {
  int nb = H / 32;
  float* r = (float*)malloc(sizeof(float) * (size_t)(nb > 0 ? nb : 1));
  for (int b = 0; b < nb; ++b) {
    float p = 0.0f;
    if (fmt == OR_Q8_0) {
      const uint8_t* blk = wrow + 34 * b;
      const int8_t* q = (const int8_t*)(blk + 2);
      for (int i = 0; i < 32; ++i) p = fmaf((float)q[i], x[32 * b + i], p);
      float d = (float)half_to_double(rd16(blk)); /* exact: every fp16 is an fp32 */
      r[b] = d * p;
    } else { /* F32 router */
      for (int i = 0; i < 32; ++i) {
        float wv;
        memcpy(&wv, wrow + 4 * (32 * b + i), 4);
        p = fmaf(wv, x[32 * b + i], p);
      }
      r[b] = p;
    }
  }
  int n = nb;
  while (n > 1) {
    int half = n / 2;
    for (int i = 0; i < half; ++i) r[i] = r[2 * i] + r[2 * i + 1];
    if (n & 1) r[half] = r[n - 1];
    n = half + (n & 1);
  }
  float z = nb > 0 ? r[0] : 0.0f;
  free(r);
  if (bias_e) z = z + *bias_e;
  return z;
}

/* a ranks before b: larger z first, equal z (including -0 == +0) to the lower index, NaN last */
static int ranks_before(float za, int a, float zb, int b) {
  int na = za != za, nb_ = zb != zb;
  if (na || nb_) return na != nb_ ? nb_ : a < b;
  if (za != zb) return za > zb;
  return a < b;
}

/* Route T tokens: ids [T,k] and weights [T,k]; z_out [T,E] optional. */
void oracle_route(const float* x, int T, int H, int E, int router_fmt, const uint8_t* router,
                  const float* bias, int k, int32_t* ids, float* w, float* z_out) {
  int64_t rb = oracle_row_bytes(router_fmt, H);
#pragma omp parallel for schedule(dynamic, 1)
  for (int t = 0; t < T; ++t) {
    float* z = (float*)malloc(sizeof(float) * (size_t)E);
    char* taken = (char*)calloc((size_t)E, 1);
    for (int e = 0; e < E; ++e)
      z[e] = oracle_router_logit(router_fmt, router + rb * e, x + (int64_t)t * H, H, bias ? bias + e : NULL);
    if (z_out) memcpy(z_out + (int64_t)t * E, z, sizeof(float) * (size_t)E);
    double* s = (double*)malloc(sizeof(double) * (size_t)(k > 0 ? k : 1));
    double ssum = 0.0;
    for (int j = 0; j < k; ++j) {
      int best = -1;
      for (int e = 0; e < E; ++e) {
        if (taken[e]) continue;
        if (best < 0 || ranks_before(z[e], e, z[best], best)) best = e;
      }
      taken[best] = 1;
      ids[(int64_t)t * k + j] = best;
      s[j] = 1.0 / (1.0 + exp(-(double)z[best]));
    }
    for (int j = 0; j < k; ++j) ssum += s[j];
    for (int j = 0; j < k; ++j) w[(int64_t)t * k + j] = (float)(s[j] / ssum);
    free(s);
    free(z);
    free(taken);
  }
}

/* Group slots s = t*k + j by expert: counts [E], offsets [E+1], slot_list [T*k]
 * (slots of one expert in ascending s). */
void oracle_group(const int32_t* ids, int T, int k, int E, int32_t* counts, int32_t* offsets,
                  int32_t* slot_list) {
  if (E <= 0) return;
  int64_t n = (int64_t)T * k;
  for (int e = 0; e < E; ++e) counts[e] = 0;
  for (int64_t s = 0; s < n; ++s) counts[ids[s]]++;
  offsets[0] = 0;
  for (int e = 0; e < E; ++e) offsets[e + 1] = offsets[e] + counts[e];
  int32_t* fill = (int32_t*)calloc((size_t)E, sizeof(int32_t));
  for (int64_t s = 0; s < n; ++s) {
    int e = ids[s];
    slot_list[offsets[e] + fill[e]++] = (int32_t)s;
  }
  free(fill);
}

/* One expert applied to one token, in fp64: y = D (silu(G x) * (U x)).
 * gate/up rows: I rows of H values; down rows: H rows of I values. */
void oracle_expert(int gate_fmt, const uint8_t* gate, int up_fmt, const uint8_t* up, int down_fmt,
                   const uint8_t* down, int H, int I, const double* x, double* y) {
  double* h = (double*)malloc(sizeof(double) * (size_t)I);
  int64_t grb = oracle_row_bytes(gate_fmt, H), urb = oracle_row_bytes(up_fmt, H);
  int64_t drb = oracle_row_bytes(down_fmt, I);
#pragma omp parallel
  {
    double* row = (double*)malloc(sizeof(double) * (size_t)(H > I ? H : I));
#pragma omp for schedule(static)
    for (int r = 0; r < I; ++r) {
      double g = 0.0, u = 0.0;
      oracle_dequant_row(gate_fmt, gate + grb * r, H, row);
      for (int c = 0; c < H; ++c) g += row[c] * x[c];
      oracle_dequant_row(up_fmt, up + urb * r, H, row);
      for (int c = 0; c < H; ++c) u += row[c] * x[c];
      h[r] = g / (1.0 + exp(-g)) * u;
    }
#pragma omp for schedule(static)
    for (int o = 0; o < H; ++o) {
      double acc = 0.0;
      oracle_dequant_row(down_fmt, down + drb * o, I, row);
      for (int r = 0; r < I; ++r) acc += row[r] * h[r];
      y[o] = acc;
    }
    free(row);
  }
  free(h);
}

/* Combine: out[t] = sum_j (owned) w[t,j] * y[t*k+j], j ascending from +0.0, fp64, rounded once.
 * g2l == NULL means every expert is owned. */
void oracle_combine(const double* y_slot, const float* w, const int32_t* ids, const int32_t* g2l, int T,
                    int k, int H, float* out) {
  for (int t = 0; t < T; ++t) {
    for (int c = 0; c < H; ++c) {
      double acc = 0.0;
      for (int j = 0; j < k; ++j) {
        int64_t s = (int64_t)t * k + j;
        if (g2l && g2l[ids[s]] < 0) continue;
        acc += (double)w[s] * y_slot[s * H + c];
      }
      out[(int64_t)t * H + c] = (float)acc;
    }
  }
}
