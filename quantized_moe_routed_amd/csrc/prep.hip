// Preparation launch of the expert forward: the tile list over the owned
// experts that received slots (workgroup 0) and the fp16 activation operand
// of every token (one workgroup per token).
//
// Activation operand of token t for a gate/up format F (see fmt.h):
//   sigma_t = 2^(9-E), E the smallest integer with max_i |x[t,i]| < 2^E
//             (1 for an all-zero token), so that |x| * sigma * 2^6 < 2^15;
//   A'[t][32b+8g+e] = x[t][32b+8g+frag_val(e)] * sigma_t * 2^6        (hi, lo)
//   S'[t][b]        = sigma_t * sum_{i<32} x[t][32b+i]               (hi, lo)
// The block sums are taken in index order in fp32; blocks past H/32 up to
// the padded count are zero.
#include "device.h"
#include "fmt.h"
#include "launch.h"

namespace moe {

constexpr int kPrepThreads = 1024;

template <int ACT>
__device__ __forceinline__ float act_at(const void* x, int64_t i) {
  return load_act<ACT>(x, i);
}

// Tiles of bm slots over the owned experts with lo_n <= slots < hi_n that
// received slots, in ascending global id: tile i covers grouped positions
// p0 .. p0+rows-1 of local expert .x.  Tiles past max_tiles, and rows past the
// n_slots grouped positions, are never produced, whatever the counts hold.
// With tok != NULL (tiles of up to 4 slots), tok[i] also receives the token of each row of tile i
// (slot / k; 0 for rows past the tile), so that the expert kernel can fetch the tile's activation
// rows without first reading the slot list.
__device__ void build_tiles(const int32_t* __restrict__ counts, const int32_t* __restrict__ offsets,
                            const int32_t* __restrict__ g2l, int E, int E_local, int n_slots, int bm, int lo_n,
                            int hi_n, int max_tiles, int4* __restrict__ tiles, int32_t* __restrict__ n_tiles,
                            int32_t* wave_tot, int4* __restrict__ tok = nullptr,
                            const int32_t* __restrict__ slot_list = nullptr, int k = 1) {
  const int tid = threadIdx.x, lane = tid % kWave, wave = tid / kWave;
  int n = 0, mt = 0, l = -1, p = 0;
  if (tid < E) {
    l = g2l ? g2l[tid] : tid;
    p = offsets[tid];
    n = (p >= 0 && p < n_slots) ? min(counts[tid], n_slots - p) : 0;
    if (n > 0 && n >= lo_n && n < hi_n && l >= 0 && l < E_local) mt = (n + bm - 1) / bm;
  }
  int incl = mt;
#pragma unroll
  for (int d = 1; d < kWave; d <<= 1) {
    const int o = __shfl_up(incl, d, kWave);
    if (lane >= d) incl += o;
  }
  __syncthreads();   // wave_tot may still be read by an earlier call
  if (lane == kWave - 1) wave_tot[wave] = incl;
  __syncthreads();
  int base = 0;
  for (int w = 0; w < wave; ++w) base += wave_tot[w];
  base += incl - mt;
  for (int i = 0; i < mt && base + i < max_tiles; ++i) {
    const int rows = min(bm, n - bm * i);
    tiles[base + i] = make_int4(l, p + bm * i, rows, tid);
    if (tok) {
      int r[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) r[j] = j < rows ? slot_list[p + bm * i + j] / k : 0;
      tok[base + i] = make_int4(r[0], r[1], r[2], r[3]);
    }
  }
  if (tid == 0) {
    int tot = 0;
    for (int w = 0; w < kPrepThreads / kWave; ++w) tot += wave_tot[w];
    *n_tiles = min(tot, max_tiles);
  }
}

template <int ACT, int FMT>
__device__ void prep_token(const void* __restrict__ x, int t, int H, int nb32, uint16_t* __restrict__ xq_hi,
                           uint16_t* __restrict__ xq_lo, uint16_t* __restrict__ sq_hi, uint16_t* __restrict__ sq_lo,
                           float* __restrict__ sigma) {
  __shared__ float wmax[kPrepThreads / kWave];
  __shared__ float s_sigma;
  const int tid = threadIdx.x, lane = tid % kWave, wave = tid / kWave;
  const int64_t row = (int64_t)t * H;
  float mx = 0.0f;
  for (int i = tid; i < H; i += kPrepThreads) mx = fmaxf(mx, fabsf(act_at<ACT>(x, row + i)));
#pragma unroll
  for (int m = 1; m < kWave; m <<= 1) mx = fmaxf(mx, __shfl_xor(mx, m, kWave));
  if (lane == 0) wmax[wave] = mx;
  __syncthreads();
  if (tid == 0) {
    float m = 0.0f;
    for (int w = 0; w < kPrepThreads / kWave; ++w) m = fmaxf(m, wmax[w]);
    int e = 0;
    if (m > 0.0f) (void)frexpf(m, &e);   // m = f * 2^e, f in [0.5, 1): m < 2^e
    const float sg = ldexpf(1.0f, 9 - e);
    s_sigma = sg;
    sigma[t] = sg;
  }
  __syncthreads();
  const float sg = s_sigma;
  const int nb = H / 32;
  // one thread per (block, K-group): 8 operand values
  for (int j = tid; j < nb * 4; j += kPrepThreads) {
    const int b = j >> 2, g = j & 3;
    uint32_t hi[8], lo[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float v = act_at<ACT>(x, row + 32 * b + 8 * g + frag_val(e)) * sg * 64.0f;
      split_f16(v, hi[e], lo[e]);
    }
    const int64_t o = row + 32 * b + 8 * g;
    *reinterpret_cast<uint4*>(xq_hi + o) =
        make_uint4(hi[0] | (hi[1] << 16), hi[2] | (hi[3] << 16), hi[4] | (hi[5] << 16), hi[6] | (hi[7] << 16));
    if (xq_lo)
      *reinterpret_cast<uint4*>(xq_lo + o) =
          make_uint4(lo[0] | (lo[1] << 16), lo[2] | (lo[3] << 16), lo[4] | (lo[5] << 16), lo[6] | (lo[7] << 16));
  }
  for (int b = tid; b < nb32; b += kPrepThreads) {
    uint32_t hi = 0, lo = 0;
    if (b < nb) {
      float s = 0.0f;
      for (int i = 0; i < 32; ++i) s += act_at<ACT>(x, row + 32 * b + i);
      split_f16(s * sg, hi, lo);
    }
    sq_hi[(int64_t)t * nb32 + b] = (uint16_t)hi;
    sq_lo[(int64_t)t * nb32 + b] = (uint16_t)lo;
  }
}

template <int ACT, int FMT>
__global__ __launch_bounds__(kPrepThreads) void prep_kernel(const void* __restrict__ x, int T, int H, int nb32,
                                                            uint16_t* __restrict__ xq_hi, uint16_t* __restrict__ xq_lo,
                                                            uint16_t* __restrict__ sq_hi, uint16_t* __restrict__ sq_lo,
                                                            float* __restrict__ sigma, TileLists tl) {
  __shared__ int32_t wave_tot[kPrepThreads / kWave];
  if (blockIdx.x == 0) {
    build_tiles(tl.counts, tl.offsets, tl.g2l, tl.E, tl.E_local, tl.n_slots, tl.bm_small, 1, tl.large_min,
                tl.max_small, tl.small, tl.n_small, wave_tot, tl.small_tok, tl.slot_list, tl.k);
    build_tiles(tl.counts, tl.offsets, tl.g2l, tl.E, tl.E_local, tl.n_slots, tl.bm_large, tl.large_min, 0x7FFFFFFF,
                tl.max_large, tl.large, tl.n_large, wave_tot);
  } else {
    const int t = blockIdx.x - 1;
    if (t < T) prep_token<ACT, FMT>(x, t, H, nb32, xq_hi, xq_lo, sq_hi, sq_lo, sigma);
  }
}

hipError_t launch_prep(const void* x, int act, int fmt, int T, int H, int nb32, uint16_t* xq_hi, uint16_t* xq_lo,
                       uint16_t* sq_hi, uint16_t* sq_lo, float* sigma, const TileLists& tl, hipStream_t s) {
  const dim3 grid(1 + T);
  trace_pre("prep", s);
#define MOE_PREP(A, F) \
  prep_kernel<A, F><<<grid, kPrepThreads, 0, s>>>(x, T, H, nb32, xq_hi, xq_lo, sq_hi, sq_lo, sigma, tl)
  if (act == ACT_F32) {
    if (fmt == FMT_Q2SM) MOE_PREP(ACT_F32, FMT_Q2SM);
    else MOE_PREP(ACT_F32, FMT_Q8_0);
  } else {
    if (fmt == FMT_Q2SM) MOE_PREP(ACT_BF16, FMT_Q2SM);
    else MOE_PREP(ACT_BF16, FMT_Q8_0);
  }
#undef MOE_PREP
  trace_post("prep", s);
  return hipGetLastError();
}

}  // namespace moe
