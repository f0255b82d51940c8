// Preparation launch of the expert forward: the tile list over the owned
// experts that received slots (workgroup 0) and the fp16 activation operand
// of every token (one workgroup per token, prep.h).
#include "device.h"
#include "fmt.h"
#include "launch.h"
#include "prep.h"
#include "select.h"

namespace moe {

constexpr int kPrepThreads = 1024;

// Tiles of bm slots over the owned experts with lo_n <= slots < hi_n that
// received slots, in ascending global id: tile i covers grouped positions
// p0 .. p0+rows-1 of local expert .x.  Tiles past max_tiles, and rows past the
// n_slots grouped positions, are never produced, whatever the counts hold.
// With tok != NULL (small tiles, bm <= kSmallRowsMax), tok[2 i] and tok[2 i + 1] also receive the
// token of each row of tile i (slot / k; 0 for rows past the tile), so that the expert kernel can
// fetch the tile's activation rows without first reading the slot list.
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
    if (tok) {   // (bm <= kSmallRowsMax)
      int r[kSmallRowsMax];
#pragma unroll
      for (int j = 0; j < kSmallRowsMax; ++j) r[j] = j < rows ? slot_list[p + bm * i + j] / k : 0;
      tok[2 * (base + i)] = make_int4(r[0], r[1], r[2], r[3]);
      tok[2 * (base + i) + 1] = make_int4(r[4], r[5], r[6], r[7]);
    }
  }
  if (tid == 0) {
    int tot = 0;
    for (int w = 0; w < kPrepThreads / kWave; ++w) tot += wave_tot[w];
    *n_tiles = min(tot, max_tiles);
  }
}

template <int ACT>
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
    if (tl.down)   // the down projection's small tiles: the same experts and rows, bm_down slots each
      build_tiles(tl.counts, tl.offsets, tl.g2l, tl.E, tl.E_local, tl.n_slots, tl.bm_down, 1, tl.large_min,
                  tl.max_down, tl.down, tl.n_down, wave_tot);
  } else {
    const int t = blockIdx.x - 1;
    if (t < T) prep_token<ACT, kPrepThreads>(x, t, H, nb32, xq_hi, xq_lo, sq_hi, sq_lo, sigma);
  }
}

hipError_t launch_prep(const void* x, int act, int fmt, int T, int H, int nb32, uint16_t* xq_hi, uint16_t* xq_lo,
                       uint16_t* sq_hi, uint16_t* sq_lo, float* sigma, const TileLists& tl, hipStream_t s) {
  (void)fmt;   // the operand layout is the same for both weight formats
  const dim3 grid(1 + T);
  trace_pre("prep", s);
  if (act == ACT_F32)
    prep_kernel<ACT_F32><<<grid, kPrepThreads, 0, s>>>(x, T, H, nb32, xq_hi, xq_lo, sq_hi, sq_lo, sigma, tl);
  else
    prep_kernel<ACT_BF16><<<grid, kPrepThreads, 0, s>>>(x, T, H, nb32, xq_hi, xq_lo, sq_hi, sq_lo, sigma, tl);
  trace_post("prep", s);
  return hipGetLastError();
}

// ---- small batches: selection, grouping, tile lists and operands in one launch ----------------
// Workgroup 0 takes the top-k of every token (wave w: tokens w, w + 16, ...), groups the slots by
// expert (a direct stable counting sort of at most 8 k slots) and builds the tile lists, keeping
// ids, counts, offsets and the slot list in LDS between the steps (each step reads what other
// threads wrote); the other workgroups prepare one token's operand each, which does not depend on
// the routing (when the router's launch has not prepared them already).
template <int EPL, int ACT>
__global__ __launch_bounds__(kPrepThreads) void front_kernel(const float* __restrict__ z, int S,
                                                             const float* __restrict__ bias, int T, int E, int k,
                                                             int32_t* __restrict__ ids,
                                                             float* __restrict__ w, int32_t* __restrict__ counts,
                                                             int32_t* __restrict__ offsets,
                                                             int32_t* __restrict__ slot_list, const void* __restrict__ x,
                                                             int H, int nb32, uint16_t* __restrict__ xq_hi,
                                                             uint16_t* __restrict__ xq_lo, uint16_t* __restrict__ sq_hi,
                                                             uint16_t* __restrict__ sq_lo, float* __restrict__ sigma,
                                                             TileLists tl) {
  // counts [E], offsets [E + 1], ids [T k], slots [T k], g2l [E], then (8-byte aligned) the
  // selection's candidates, E + kThrMaxK per token
  extern __shared__ __align__(8) int32_t fsm[];
  __shared__ int32_t wave_tot[kPrepThreads / kWave];
  if (blockIdx.x == 0) {
    const int tid = threadIdx.x, wave = tid / kWave, n = T * k;
    int32_t* s_cnt = fsm;
    int32_t* s_off = s_cnt + E;
    int32_t* s_ids = s_off + E + 1;
    int32_t* s_slot = s_ids + n;
    int32_t* s_g2l = s_slot + n;
    // the ownership table is fetched now and lands in LDS after the selection
    const int g2l_e = tid < E ? (tl.g2l ? tl.g2l[tid] : tid) : 0;
    uint64_t* s_cand = reinterpret_cast<uint64_t*>(fsm + ((3 * E + 1 + 2 * n + 1) & ~1));
    for (int t = wave; t < T; t += kPrepThreads / kWave)
      topk_token<EPL, kSelMaxRanges>(z, S, bias, T, E, k, t, ids, w, s_ids, s_cand + (size_t)t * (E + kThrMaxK));
    if (tid < E) s_g2l[tid] = g2l_e;
    __syncthreads();
    // the stable counting sort of a few slots, directly: expert e's count and offset are the slots
    // with id e and with a smaller id; slot i goes to (slots with a smaller id) + (earlier slots
    // with its id).  Ids outside [0, E) take part in nothing.
    for (int e = tid; e < E; e += kPrepThreads) {
      int c = 0, o = 0;
      for (int i = 0; i < n; ++i) {
        const int v = s_ids[i];
        c += v == e;
        o += (unsigned)v < (unsigned)e;
      }
      s_cnt[e] = c;
      s_off[e] = o;
    }
    if (tid == 0) {
      int c = 0;
      for (int i = 0; i < n; ++i) c += (unsigned)s_ids[i] < (unsigned)E;
      s_off[E] = c;
    }
    for (int i = tid; i < n; i += kPrepThreads) {
      const int v = s_ids[i];
      if ((unsigned)v < (unsigned)E) {
        int r = 0;
        for (int j = 0; j < n; ++j) {
          const int u = s_ids[j];
          r += (unsigned)u < (unsigned)v || (u == v && j < i);
        }
        s_slot[r] = i;
      }
    }
    __syncthreads();
    for (int i = tid; i < n; i += kPrepThreads) slot_list[i] = s_slot[i];
    for (int e = tid; e <= E; e += kPrepThreads) {
      if (e < E) counts[e] = s_cnt[e];
      offsets[e] = s_off[e];
    }
    build_tiles(s_cnt, s_off, s_g2l, E, tl.E_local, tl.n_slots, tl.bm_small, 1, tl.large_min, tl.max_small,
                tl.small, tl.n_small, wave_tot, tl.small_tok, s_slot, k);
    if (tl.max_large > 0)   // (batches this small have no large tiles; their count is never read)
      build_tiles(s_cnt, s_off, s_g2l, E, tl.E_local, tl.n_slots, tl.bm_large, tl.large_min, 0x7FFFFFFF,
                  tl.max_large, tl.large, tl.n_large, wave_tot);
  } else {
    const int t = blockIdx.x - 1;
    if (t < T) prep_token<ACT, kPrepThreads>(x, t, H, nb32, xq_hi, xq_lo, sq_hi, sq_lo, sigma);
  }
}

size_t front_lds_bytes(int T, int E, int k) {
  const size_t words = (3 * (size_t)E + 1 + 2 * (size_t)T * k + 1) & ~(size_t)1;
  return sizeof(int32_t) * words + sizeof(uint64_t) * (size_t)T * (E + kThrMaxK);
}

hipError_t launch_front(const float* z, int S, const float* bias, int T, int E, int k, int32_t* ids, float* w,
                        int32_t* counts, int32_t* offsets, int32_t* slot_list, const void* x, int act, int H,
                        const PrepOut* prep, const TileLists& tl, hipStream_t s) {
  const PrepOut po = prep ? *prep : PrepOut{};
  const int nb32 = po.nb32;
  uint16_t *xq_hi = po.xq_hi, *xq_lo = po.xq_lo, *sq_hi = po.sq_hi, *sq_lo = po.sq_lo;
  float* sigma = po.sigma;
  const size_t lds = front_lds_bytes(T, E, k);
  const dim3 grid(1 + (prep ? T : 0));
#define MOE_FRONT(EPL, A)                                                                                       \
  do {                                                                                                          \
    auto kern = front_kernel<EPL, A>;                                                                           \
    if (lds > 64 * 1024) {                                                                                      \
      const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),                            \
                                               hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);          \
      if (e != hipSuccess) return e;                                                                            \
    }                                                                                                           \
    kern<<<grid, kPrepThreads, lds, s>>>(z, S, bias, T, E, k, ids, w, counts, offsets, slot_list, x, H,  \
                                         nb32, xq_hi, xq_lo, sq_hi, sq_lo, sigma, tl);                          \
  } while (0)
#define MOE_FRONT_E(A)                  \
  if (E <= 64) MOE_FRONT(1, A);         \
  else if (E <= 128) MOE_FRONT(2, A);   \
  else if (E <= 256) MOE_FRONT(4, A);   \
  else if (E <= 512) MOE_FRONT(8, A);   \
  else MOE_FRONT(16, A);
  trace_pre("front", s);
  if (act == ACT_F32) { MOE_FRONT_E(ACT_F32) } else { MOE_FRONT_E(ACT_BF16) }
  trace_post("front", s);
#undef MOE_FRONT_E
#undef MOE_FRONT
  return hipGetLastError();
}

}  // namespace moe
