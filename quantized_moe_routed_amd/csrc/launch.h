// Host-side launchers of the gfx950 kernels (internal to libmoe).
#pragma once
#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace moe {

struct QMat;
struct SelArgs;   // smallsel.h

// Optional event tracing of one kernel (see moe_trace_kernel): record an event
// on the stream before and after the launch of kernel `name`.  With stamped,
// the launch in between goes through launch_stamped, which hands the events
// to the runtime instead: they then carry the kernel's own start and end, the
// interval a profiler reports, without the stream's dispatch gaps around it.
void trace_pre(const char* name, hipStream_t s, bool stamped = false);
void trace_post(const char* name, hipStream_t s);

// Events for the next launch_stamped (both null unless trace_pre armed them).
struct StampEvents {
  hipEvent_t start = nullptr, stop = nullptr;
};
StampEvents& stamp_events();

template <typename... KArgs, typename... Args>
hipError_t launch_stamped(void (*kern)(KArgs...), dim3 grid, dim3 block, size_t lds, hipStream_t s, Args... args) {
  StampEvents& ev = stamp_events();
  hipExtLaunchKernelGGL(kern, grid, block, (uint32_t)lds, s, ev.start, ev.stop, 0u, args...);
  ev = StampEvents{};
  return hipGetLastError();
}

// Table routing: the experts of token t are row token_ids[t] of table [V, k]; logits and weights
// as launch_route's (ws the same size).
hipError_t launch_route_table(const void* x, int act, int T, int H, int fmt, const QMat& router, const float* bias,
                              const int32_t* token_ids, const int32_t* table, int V, int k, int32_t* ids, float* w,
                              void* ws, hipStream_t s);
hipError_t launch_route(const void* x, int act, int T, int H, int fmt, const QMat& router, const float* bias,
                        int k, int32_t* ids, float* w, void* ws, hipStream_t s);
size_t route_ws_need(int T, int E, int H, int fmt);   // workspace bytes of launch_route
int logit_ranges(int T, int E, int H, int fmt);       // partial sums per (token, expert) of the logits launch
// Outputs of the expert operand preparation (prep.h) of every token.
struct PrepOut {
  int nb32;
  uint16_t *xq_hi, *xq_lo, *sq_hi, *sq_lo;
  float* sigma;
};
// The logits alone, into ws: finished logits (*S = 0) or S partial sums per (token, expert) whose
// pairwise sum plus the bias is the logit (*S > 0); the selection kernels take either.  With prep,
// the same launch also prepares every token's expert operand (only where the logits are finished:
// batches below the token-per-lane router's size).
hipError_t launch_logits(const void* x, int act, int T, int H, int fmt, const QMat& router, const float* bias,
                         void* ws, int* S, hipStream_t s, const PrepOut* prep);

hipError_t launch_group(const int32_t* ids, int T, int k, int E, int32_t* counts, int32_t* offsets,
                        int32_t* slot_list, hipStream_t s);
size_t group_lds_bytes(int E);
hipError_t group_set_lds_limit(size_t bytes);

// Two tile lists over the owned experts that received slots: experts with
// fewer than large_min slots in tiles of bm_small, the others in tiles of
// bm_large.  A tile is {local expert, first grouped position, rows, global id}.
struct TileLists {
  const int32_t *counts, *offsets, *g2l;
  int E, E_local, n_slots, large_min;
  int bm_small, max_small, bm_large, max_large;
  int4 *small, *large;
  int32_t *n_small, *n_large;
  int4* small_tok;              // tokens of the rows of each small tile: two int4 per tile (bm_small <= 8)
  const int32_t* slot_list;
  int k;
  // non-NULL: the down projection's own small tiles, of bm_down slots (the same experts and rows)
  int4* down;
  int32_t* n_down;
  int bm_down, max_down;
};

// Batches of up to kFrontMaxTokens tokens: top-k selection, grouping, tile lists and the
// activation operands in one launch (prep.hip), after launch_logits.
constexpr int kFrontMaxTokens = 8;
size_t front_lds_bytes(int T, int E, int k);
// prep: also prepare the operands (NULL: the router's launch did).
hipError_t launch_front(const float* z, int S, const float* bias, int T, int E, int k, int32_t* ids, float* w,
                        int32_t* counts, int32_t* offsets, int32_t* slot_list, const void* x, int act, int H,
                        const PrepOut* prep, const TileLists& tl, hipStream_t s);

// Arguments of the expert FFN launches (workspace pointers included).
struct FfnArgs {
  int T, H, I, k, fg, fd, nb32H, nb32I;
  QMat gate, up, down;
  const int32_t* slot_list;
  const int4 *small, *large;
  const int4* small_tok;
  const int32_t *n_small, *n_large;
  int max_small, max_large;   // max_large = 0: no large tiles can exist
  int bm_small;               // slots per small tile (4 or 8)
  const uint16_t *xq_hi, *xq_lo, *sq_hi, *sq_lo;
  const float* sigma;
  float *h, *hs, *hm;           // h = silu(g) * u, its block sums and block maxima (fp32, unscaled)
  uint16_t *hq_hi, *hq_lo, *hsq_hi, *hsq_lo;   // large tiles: the down projection's operand of their rows
  float* hsig;                  //   and its row scales (NULL when no large tiles can exist)
  float* y;
  // non-NULL: the gate/up launch selects, groups and numbers the small tiles itself from finished
  // logits (batches of at most kSelMaxTokens tokens, no large tiles) and stores the routing
  // results; small, small_tok and n_small are then its outputs
  const SelArgs* sel;
  // non-NULL with large tiles: the small tiles' launches run on this second stream of the device,
  // concurrently with the large tiles' (fork: recorded on the caller's stream before them, join:
  // recorded on the second stream after them and waited for by the caller's stream)
  hipStream_t side;
  hipEvent_t fork, join;
  // non-NULL (batches of more than kSelMaxTokens tokens where the down projection's staging holds
  // more slots than the gate/up's): the down projection's own small tiles, of bm_down slots
  const int4* down_small;
  const int32_t* n_down_small;
  int max_down_small, bm_down_small;
  // the 2-bit gate/up of several slots stages its rows one code unit at a time (tiles of 8 slots
  // where staging whole rows would take 4)
  bool half_gateup;
};

// Tile lists + fp16 activation operand (fmt.h) in one launch.
hipError_t launch_prep(const void* x, int act, int fmt, int T, int H, int nb32, uint16_t* xq_hi, uint16_t* xq_lo,
                       uint16_t* sq_hi, uint16_t* sq_lo, float* sigma, const TileLists& tl, hipStream_t s);

// gate/up then down: small tiles (up to 8 slots, 32 output columns per
// workgroup) and large tiles (up to 128 slots, 64 columns per workgroup).
hipError_t launch_ffn(const FfnArgs& a, hipStream_t s);

// Slots per small tile: 8 when the activation rows of 8 slots stay within the LDS that lets two
// workgroups share a compute unit, for gate/up (K = H; hi and lo planes for fp32 activations) and
// for down (K = I, hi and lo planes), else 4.
constexpr int kSmallRowsMax = 8;
constexpr int kLargeTileRows = 128;   // slots per large tile
int small_tile_rows(int H, int I, bool f32_act);
// Slots per small tile of the down projection alone (its staging: K = I, hi and lo planes).
int small_down_tile_rows(int I);
// Whether the 2-bit gate/up of several slots (batches past kSelMaxTokens tokens, fp32 activations)
// stages its rows one code unit at a time: where 8 whole rows would not let two workgroups share a
// compute unit and a wave takes at most two code units (K = H <= 4096).
bool half_gateup_staging(int H, bool f32_act);

hipError_t launch_combine(const float* y, const float* w, const int32_t* ids, const int32_t* g2l, int T, int k,
                          int H, int E, float* out, hipStream_t s);

}  // namespace moe
