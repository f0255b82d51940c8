// Selection, grouping and small-tile list of a batch of at most kSelMaxTokens
// tokens, computed by one workgroup entirely in LDS (internal to libmoe).
//
// Every workgroup of the gate/up launch of such a batch runs it on the finished
// logits, so that no launch of its own stands between the router and the
// expert kernel; the workgroup that is marked as the writer also stores the
// results (ids, weights, counts, offsets, slot list, tile list) for the later
// launches.  The results equal those of the separate kernels: the same top-k
// (select.h), the stable counting sort of the slots by expert, and tiles of up
// to bm slots over the owned experts that received slots, in ascending global
// id, capped at max_tiles.
#pragma once
#include "device.h"
#include "launch.h"
#include "select.h"

namespace moe {

constexpr int kSelMaxTokens = 8;
constexpr int kSelMaxE = 256;    // experts: 4 per lane of a wave

struct SelArgs {
  const float* z;                // [S][T][E] partial logits over aligned block ranges ([T][E] finished ones if S == 0)
  int S;
  const float* bias;
  int T, E, k, E_local;
  const int32_t* g2l;            // NULL: every expert owned, local = global
  int max_tiles, bm;             // small tiles: at most max_tiles of at most bm slots
  int32_t *ids, *counts, *offsets, *slot_list, *n_tiles;
  float* w;
  int4 *tiles, *tile_tok;
};

struct SelLds {
  int32_t ids[kSelMaxTokens * 32];
  int32_t slot[kSelMaxTokens * 32];
  int32_t cnt[kSelMaxE], off[kSelMaxE + 1], g2l[kSelMaxE];
  int32_t wave_tot[16];
  int4 tile, tok[2];
  int32_t n_tiles;
};

// LDS for the threshold selection: E + kThrMaxK candidates per token
constexpr size_t kSelScratchBytes = (size_t)kSelMaxTokens * (kSelMaxE + kThrMaxK) * sizeof(uint64_t);

// want: the tile whose description lands in L.tile / L.tok[2] (when want < L.n_tiles).  scratch:
// kSelScratchBytes of LDS, free again when the call returns.
template <int NT>
__device__ __forceinline__ void small_select(const SelArgs& a, SelLds& L, bool writer, int want,
                                             uint64_t* scratch) {
  static_assert(NT >= kSelMaxE && NT % kWave == 0, "one thread per expert");
  const int tid = threadIdx.x, lane = tid % kWave, wave = tid / kWave;
  const int E = a.E, k = a.k, n = a.T * a.k;
  const int g2l_e = tid < E ? (a.g2l ? a.g2l[tid] : tid) : -1;   // lands in LDS after the selection
  for (int t = wave; t < a.T; t += NT / kWave)
    topk_token<4, kSelMaxRanges>(a.z, a.S, a.bias, a.T, E, k, t, writer ? a.ids : nullptr, writer ? a.w : nullptr, L.ids,
                                 scratch + (size_t)t * (E + kThrMaxK));
  if (tid < E) L.g2l[tid] = g2l_e;
  __syncthreads();
  // stable counting sort of the n slots: expert e's count and offset are the slots with id e and
  // with a smaller id; slot i goes to (slots with a smaller id) + (earlier slots with its id)
  int c = 0, o = 0;
  if (tid < E) {
    for (int i = 0; i < n; ++i) {
      const int v = L.ids[i];
      c += v == tid;
      o += (unsigned)v < (unsigned)tid;
    }
    L.cnt[tid] = c;
    L.off[tid] = o;
    if (tid == E - 1) L.off[E] = o + c;
  }
  if (tid < n) {
    const int v = L.ids[tid];
    if ((unsigned)v < (unsigned)E) {
      int r = 0;
      for (int j = 0; j < n; ++j) {
        const int u = L.ids[j];
        r += (unsigned)u < (unsigned)v || (u == v && j < tid);
      }
      L.slot[r] = tid;
    }
  }
  // tiles of up to bm slots per owned expert that received slots, numbered in ascending id
  const int le = tid < E ? g2l_e : -1;
  const int bm = a.bm;
  const int mt = (c > 0 && le >= 0 && le < a.E_local) ? (c + bm - 1) / bm : 0;
  int incl = mt;
#pragma unroll
  for (int d = 1; d < kWave; d <<= 1) {
    const int u = __shfl_up(incl, d, kWave);
    if (lane >= d) incl += u;
  }
  if (lane == kWave - 1) L.wave_tot[wave] = incl;
  __syncthreads();   // also: slot list, counts and offsets complete
  int base = incl - mt;
  for (int w = 0; w < wave; ++w) base += L.wave_tot[w];
  if (tid == 0) {
    int tot = 0;
    for (int w = 0; w < NT / kWave; ++w) tot += L.wave_tot[w];
    L.n_tiles = min(tot, a.max_tiles);
    if (writer) *a.n_tiles = min(tot, a.max_tiles);
  }
  for (int i = 0; i < mt; ++i) {
    const int ti = base + i;
    if (ti >= a.max_tiles) break;
    const int rows = min(bm, c - bm * i), p0 = o + bm * i;
    int r[kSmallRowsMax];
#pragma unroll
    for (int j = 0; j < kSmallRowsMax; ++j) r[j] = j < rows ? L.slot[p0 + j] / k : 0;
    const int4 tl = make_int4(le, p0, rows, tid), tk0 = make_int4(r[0], r[1], r[2], r[3]),
               tk1 = make_int4(r[4], r[5], r[6], r[7]);
    if (ti == want) {
      L.tile = tl;
      L.tok[0] = tk0;
      L.tok[1] = tk1;
    }
    if (writer) {
      a.tiles[ti] = tl;
      a.tile_tok[2 * ti] = tk0;
      a.tile_tok[2 * ti + 1] = tk1;
    }
  }
  if (writer) {
    for (int i = tid; i < n; i += NT) a.slot_list[i] = L.slot[i];
    for (int e = tid; e <= E; e += NT) {
      if (e < E) a.counts[e] = L.cnt[e];
      a.offsets[e] = L.off[e];
    }
  }
  __syncthreads();
}

// One token: its k experts are distinct, so every selected expert holds one slot and, when owned,
// one tile, and the stable counting sort reduces to ranks.  One wave selects (cand: E + kThrMaxK
// entries of LDS) and finds tile want with no LDS exchange: slot j's position is the number of
// selected ids below id_j, its tile number the number of owned selected ids below id_j (tiles in
// ascending expert id, as in small_select).  Wave 0 of the writer stores what small_select stores
// for one token.  Returns the tile count; tl receives tile want when want is below it (its one row
// is token 0).
__device__ __forceinline__ int one_token_select(const SelArgs& a, bool writer, int want, uint64_t* cand,
                                                int4& tl) {
  const int lane = threadIdx.x % kWave, wave = threadIdx.x / kWave;
  const int E = a.E, k = a.k;
  // ownership table in registers, fetched ahead of the selection: expert i * 64 + lane in slot i
  // (without a table the load reads the logits and is dropped)
  const int32_t* gp = a.g2l ? a.g2l : reinterpret_cast<const int32_t*>(a.z);
  int g2l_r[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int e = i * kWave + lane;
    const int v = gp[min(e, E - 1)];
    g2l_r[i] = a.g2l ? v : e;
  }
  int my_id;
  uint32_t my_key;
  topk_lanes<4, kSelMaxRanges>(a.z, a.S, a.bias, 1, E, k, 0, cand, my_id, my_key);
  // local id of lane j's expert: lane id_j % 64 holds it in slot id_j / 64 (without a table it is id_j)
  int le = my_id;
  if (a.g2l) {
    const int src = my_id < 0 ? 0 : my_id % kWave;
    le = -1;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int v = __shfl(g2l_r[i], src, kWave);
      if (my_id >= 0 && my_id / kWave == i) le = v;
    }
  }
  const bool owned = lane < k && le >= 0 && le < a.E_local;
  const uint64_t om = __ballot(owned);
  int rank = 0, trank = 0;
  for (int j = 0; j < k; ++j) {
    const int idj = __builtin_amdgcn_readlane(my_id, j);
    const bool below = idj < my_id;
    rank += below ? 1 : 0;
    trank += below && ((om >> j) & 1) ? 1 : 0;
  }
  const int n_tiles = min((int)__popcll(om), a.max_tiles);
  const uint64_t hit = __ballot(owned && trank == want);
  if (hit) {
    const int sl = __builtin_ctzll(hit);
    tl = make_int4(__builtin_amdgcn_readlane(le, sl), __builtin_amdgcn_readlane(rank, sl), 1,
                   __builtin_amdgcn_readlane(my_id, sl));
  }
  if (writer && wave == 0) {
    topk_store(k, 0, my_id, my_key, a.ids, a.w);
    if (lane < k) a.slot_list[rank] = lane;
    if (owned && trank < a.max_tiles) {
      a.tiles[trank] = make_int4(le, rank, 1, my_id);
      a.tile_tok[2 * trank] = make_int4(0, 0, 0, 0);
      a.tile_tok[2 * trank + 1] = make_int4(0, 0, 0, 0);
    }
    if (lane == 0) *a.n_tiles = n_tiles;
    // every expert's count (its slots) and offset (the slots of smaller ids); offsets[E] = k
    for (int e = lane; e <= E; e += kWave) {
      int c = 0, o = 0;
      for (int j = 0; j < k; ++j) {
        const int idj = __builtin_amdgcn_readlane(my_id, j);
        c += idj == e ? 1 : 0;
        o += idj < e ? 1 : 0;
      }
      if (e < E) a.counts[e] = c;
      a.offsets[e] = o;
    }
  }
  return n_tiles;
}

}  // namespace moe
