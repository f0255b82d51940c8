// The C ABI of libmoe: argument checks, workspace layout and kernel dispatch.
// Every check runs before the first launch; a failing call launches nothing.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdarg>
#include <mutex>
#include <cstdio>
#include <cstring>
#include <string>
#include <vector>

#include "../../include/moe.h"
#include "device.h"
#include "launch.h"
#include "smallsel.h"
#include "status.h"

namespace {

// set while a call runs on the library's own scratch array (its address is the library's, so the
// caller-pointer check on the workspace is skipped)
thread_local bool g_ws_is_scratch = false;

using moe::fail;
using moe::ok;

constexpr size_t kAlign = 256;
size_t align_up(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }

constexpr int kMaxE = 1024;
constexpr int kMaxK = 32;
constexpr int kMaxRouteH = 16384;
constexpr int kMaxFfnDim = 8192;

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Device of a stream (NULL stream: the current device).
moe_status stream_device(hipStream_t s, int* dev) {
  hipError_t e = s ? hipStreamGetDevice(s, dev) : hipGetDevice(dev);
  if (e != hipSuccess) {
    (void)hipGetLastError();
    return fail(MOE_ERR_HIP, "cannot query the stream's device: %s", hipGetErrorString(e));
  }
  return MOE_OK;
}

// The pointer must be device (or managed) memory of device `dev` (the ordinal,
// not only the kind: arc PR #89, Stage 0).
moe_status check_dev(const void* p, int dev, const char* name) {
  if (!p) return MOE_OK;
  hipPointerAttribute_t a;
  hipError_t e = hipPointerGetAttributes(&a, p);
  if (e != hipSuccess) {
    (void)hipGetLastError();
    return fail(MOE_ERR_DEVICE, "%s is not HIP device memory", name);
  }
  if (a.type != hipMemoryTypeDevice && a.type != hipMemoryTypeManaged)
    return fail(MOE_ERR_DEVICE, "%s is not device memory (memory type %d)", name, (int)a.type);
  if (a.device != dev)
    return fail(MOE_ERR_DEVICE, "%s lives on device %d but the stream runs on device %d", name, a.device, dev);
  return MOE_OK;
}

struct DevCheck {
  int dev = 0;
  moe_status st = MOE_OK;
  void operator()(const void* p, const char* name) {
    if (st == MOE_OK) st = check_dev(p, dev, name);
  }
};

moe_status hip_fail(hipError_t e, const char* what) {
  (void)hipGetLastError();
  return fail(MOE_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

// ---- kernel event tracing (thread-local; off unless moe_trace_kernel set it) ----
struct Trace {
  std::string name;
  hipEvent_t* start = nullptr;
  hipEvent_t* stop = nullptr;
  int n = 0;
  int every = 1;       // record launches 0, every, 2 every, ...
  int seen = 0;        // launches of the kernel since tracing was set
  bool armed = false;  // the current launch is being recorded
  bool stamped = false;  // ... by the launch itself (launch_stamped)
  int32_t* count = nullptr;
};
thread_local Trace g_trace;

moe::QMat qm(const moe_qmat& m) { return moe::QMat{m.codes, m.scales, m.rows, m.cols}; }

// ---- workspace layouts -------------------------------------------------------
// (the size query does not know the router's format: it reports the larger, Q8_0, need)
size_t route_ws_bytes(int T, int E, int H, int fmt = MOE_W_Q8_0) { return align_up(moe::route_ws_need(T, E, H, fmt)); }

// Expert-forward workspace: tile list, per-token row scales, the fp16
// activation operand (hi plane; lo plane for fp32 activations) with its block
// sums, the intermediate h in fp32 with its block sums and block maxima, and,
// where large tiles can occur or the batch has more than kSelMaxTokens tokens,
// the down projection's fp16 hi + lo operand of the tiles' rows with its block
// sums and row scales (single tokens: the block-scaled planes of h).  Block
// rows are padded to a multiple of 32 blocks.
constexpr int kLargeTile = moe::kLargeTileRows;   // slots per large tile

// Fewest slots of an expert that go to large tiles in a batch of T tokens, 0 = small tiles only.
// Up to 32 tokens an expert fills at most 4 small tiles of 8 and the large-tile launches would run
// all but empty; up to 255 tokens the few large tiles form a short, latency-bound launch, so
// only experts of more than 4 small tiles take one; from 256 tokens the large-tile launches are
// full, and an expert of 12 or more slots costs less there than on 2 or more small tiles.
int large_tile_min(int64_t T) { return T <= 32 ? 0 : T < 256 ? 33 : 12; }

int64_t max_tiles(int64_t slots, int64_t experts, int bm) { return (slots + bm - 1) / bm + experts; }

// Tile-list bounds for T tokens (an expert receives at most T slots).
struct TilePlan {
  int large_min, bm_small, max_small, max_large;
  int bm_down, max_down;   // max_down > 0: the down projection's own small tiles of bm_down slots
};

// half: the 2-bit gate/up stages its rows one code unit at a time (moe::half_gateup_staging), which
// lets its small tiles take 8 slots
TilePlan tile_plan(int T, int H, int I, int k, int E_local, int xt, bool half = false) {
  const int64_t slots = (int64_t)T * k;
  TilePlan p{};
  const int lmin = large_tile_min(T);
  const bool large = lmin > 0;
  p.large_min = large ? lmin : 0x7FFFFFFF;
  p.bm_small = half ? moe::kSmallRowsMax : moe::small_tile_rows(H, I, xt == MOE_ACT_F32);
  // (one token: each of its k experts is a tile of one slot, so at most min(k, E_local) tiles; the
  // launches' grids hold exactly the tiles that can occur)
  p.max_small = T == 1 ? std::min(k, E_local) : (int)max_tiles(slots, std::min<int64_t>(E_local, slots), p.bm_small);
  // with large tiles, small tiles take only experts of fewer than large_min slots: at most
  // ceil((large_min - 1) / bm_small) tiles each (the launches' grids hold max_small tiles, and a
  // workgroup past the tile count only reads the count and ends)
  if (large)
    p.max_small = (int)std::min<int64_t>(p.max_small, std::min<int64_t>(E_local, slots) *
                                                          ((lmin - 1 + p.bm_small - 1) / p.bm_small));
  p.max_large = large ? (int)max_tiles(slots, std::min<int64_t>(E_local, slots / lmin), kLargeTile) : 0;
  // past kSelMaxTokens tokens the down projection stages prepared rows, and where its staging (K = I)
  // holds another number of slots than the gate/up's (K = H, fp32 activations), its small tiles take
  // that many: an expert of 5-8 slots then streams its down weights once instead of on two tiles
  p.bm_down = p.bm_small;
  p.max_down = 0;
  const int bmd = moe::small_down_tile_rows(I);
  if (T > moe::kSelMaxTokens && bmd != p.bm_small) {
    p.bm_down = bmd;
    p.max_down = (int)max_tiles(slots, std::min<int64_t>(E_local, slots), bmd);
    if (large)
      p.max_down = (int)std::min<int64_t>(p.max_down, std::min<int64_t>(E_local, slots) * ((lmin - 1 + bmd - 1) / bmd));
  }
  return p;
}

int pad32(int nb) { return (nb + 31) / 32 * 32; }

struct FwdLayout {
  size_t n_small, n_large, n_down, small, small_tok, down, large, sigma, xq_hi, xq_lo, sq_hi, sq_lo, h, hs, hm;
  size_t hq_hi, hq_lo, hsq_hi, hsq_lo, hsig, total;
};

FwdLayout fwd_layout(int T, int H, int I, int k, int E_local, int xt) {
  FwdLayout L{};
  const size_t TK = (size_t)T * k;
  const size_t nb32H = pad32(H / 32), nb32I = pad32(I / 32);
  // the weight format is not known here: room for the tile lists of either gate/up staging
  TilePlan tp = tile_plan(T, H, I, k, E_local, xt);
  if (T > moe::kSelMaxTokens && moe::half_gateup_staging(H, xt == MOE_ACT_F32)) {
    const TilePlan th = tile_plan(T, H, I, k, E_local, xt, true);
    tp.max_small = std::max(tp.max_small, th.max_small);
    tp.max_down = std::max(tp.max_down, th.max_down);
  }
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t at = off;
    off += align_up(bytes);
    return at;
  };
  L.n_small = take(sizeof(int32_t));
  L.n_large = take(sizeof(int32_t));
  L.small = take((size_t)tp.max_small * 4 * sizeof(int32_t));
  L.small_tok = take((size_t)tp.max_small * moe::kSmallRowsMax * sizeof(int32_t));
  L.n_down = take(tp.max_down > 0 ? sizeof(int32_t) : 0);
  L.down = take((size_t)tp.max_down * 4 * sizeof(int32_t));
  L.large = take((size_t)tp.max_large * 4 * sizeof(int32_t));
  L.sigma = take((size_t)T * sizeof(float));
  L.xq_hi = take((size_t)T * H * 2);
  L.xq_lo = xt == MOE_ACT_F32 ? take((size_t)T * H * 2) : 0;
  L.sq_hi = take((size_t)T * nb32H * 2);
  L.sq_lo = take((size_t)T * nb32H * 2);
  L.h = take(TK * I * 4);
  L.hs = take(TK * nb32I * 4);
  L.hm = take(TK * nb32I * 4);
  // the down projection's prepared operand: of the large tiles' rows and, past kSelMaxTokens
  // tokens, of the small tiles' rows (one-slot tiles: their block-scaled planes)
  const bool prep = tp.max_large > 0 || T > moe::kSelMaxTokens;
  if (prep || T == 1) {
    L.hq_hi = take(TK * I * 2);
    L.hq_lo = take(TK * I * 2);
  }
  if (prep) {
    L.hsq_hi = take(TK * nb32I * 2);
    L.hsq_lo = take(TK * nb32I * 2);
    L.hsig = take(TK * sizeof(float));
  }
  L.total = off;
  return L;
}

moe_status check_qmat(const moe_qmat& m, const char* name, int rows, int cols, bool allow_q2sm, bool allow_f32) {
  if (m.fmt != MOE_W_F32 && m.fmt != MOE_W_Q8_0 && m.fmt != MOE_W_Q2SM)
    return fail(MOE_ERR_UNSUPPORTED, "%s: unknown weight format %d", name, m.fmt);
  if ((m.fmt == MOE_W_Q2SM && !allow_q2sm) || (m.fmt == MOE_W_F32 && !allow_f32))
    return fail(MOE_ERR_UNSUPPORTED, "%s: format %s is not supported here", name,
                m.fmt == MOE_W_F32 ? "F32" : "Q2SM");
  if (m.rows != rows || m.cols != cols)
    return fail(MOE_ERR_ARG, "%s: shape %dx%d, expected %dx%d", name, m.rows, m.cols, rows, cols);
  if (!m.codes) return fail(MOE_ERR_ARG, "%s: codes is NULL", name);
  if (m.fmt != MOE_W_F32 && !m.scales) return fail(MOE_ERR_ARG, "%s: scales is NULL", name);
  if (!aligned16(m.codes) || (m.scales && !aligned16(m.scales)))
    return fail(MOE_ERR_ARG, "%s: code and scale planes must be 16-byte aligned", name);
  return MOE_OK;
}

}  // namespace

namespace moe {
thread_local StampEvents g_stamp;
StampEvents& stamp_events() { return g_stamp; }

void trace_pre(const char* name, hipStream_t s, bool stamped) {
  Trace& t = g_trace;
  if (t.n > 0 && t.name == name) {
    t.armed = t.seen % t.every == 0 && *t.count < t.n;
    t.stamped = stamped;
    if (t.armed) {
      if (stamped) g_stamp = StampEvents{t.start[*t.count], t.stop[*t.count]};
      else (void)hipEventRecord(t.start[*t.count], s);
    }
  }
}
void trace_post(const char* name, hipStream_t s) {
  Trace& t = g_trace;
  if (t.n > 0 && t.name == name) {
    if (t.armed) {
      // a stamped launch consumes its events; ones still here belong to a launch that never
      // happened (an error before it), and are not counted
      const bool recorded = !t.stamped || g_stamp.start == nullptr;
      if (!t.stamped) (void)hipEventRecord(t.stop[*t.count], s);
      g_stamp = StampEvents{};
      if (recorded) ++*t.count;
      t.armed = false;
    }
    ++t.seen;
  }
}
}  // namespace moe

extern "C" {

moe_status moe_trace_kernel_every(const char* name, hipEvent_t* start, hipEvent_t* stop, int32_t n, int32_t every,
                                  int32_t* count) {
  if (n <= 0) {
    g_trace = Trace{};
    return ok();
  }
  if (!name || !start || !stop || !count) return fail(MOE_ERR_ARG, "moe_trace_kernel: NULL argument");
  if (every < 1) return fail(MOE_ERR_ARG, "moe_trace_kernel_every: every = %d", every);
  g_trace = Trace{};
  g_trace.name = name;
  g_trace.start = start;
  g_trace.stop = stop;
  g_trace.n = n;
  g_trace.every = every;
  g_trace.count = count;
  *count = 0;
  return ok();
}

moe_status moe_trace_kernel(const char* name, hipEvent_t* start, hipEvent_t* stop, int32_t n, int32_t* count) {
  return moe_trace_kernel_every(name, start, stop, n, 1, count);
}


int32_t moe_large_tile_min(int32_t T) { return large_tile_min(T); }

moe_status moe_workspace_size(int32_t T, int32_t H, int32_t I, int32_t k, int32_t E, int32_t E_local, int32_t xt,
                              size_t* route_ws, size_t* group_ws, size_t* forward_ws) {
  if (T < 0 || H <= 0 || I <= 0 || k <= 0 || E <= 0 || E_local < 0 || E_local > E)
    return fail(MOE_ERR_ARG, "moe_workspace_size: bad sizes");
  if (xt != MOE_ACT_F32 && xt != MOE_ACT_BF16) return fail(MOE_ERR_ARG, "moe_workspace_size: unknown activation type");
  if (route_ws) *route_ws = route_ws_bytes(T, E, H);
  if (group_ws) *group_ws = 0;
  if (forward_ws) *forward_ws = fwd_layout(T, H, I, k, E_local, xt).total;
  return ok();
}

}  // extern "C"

namespace {

// ---- argument checks and launch setup (shared by the four calls and the whole-layer call) ----
// Each returns MOE_OK when every argument is valid (and, for T > 0, every pointer is memory of
// the stream's device); nothing is launched by them.

moe_status route_check(const char* fn, const void* x, int32_t xt, int32_t T, int32_t H, const moe_qmat* router,
                       const float* bias, int32_t k, const int32_t* ids, const float* w, const void* ws,
                       size_t ws_bytes, hipStream_t s) {
  if (T < 0) return fail(MOE_ERR_ARG, "%s: T < 0", fn);
  if (xt != MOE_ACT_F32 && xt != MOE_ACT_BF16) return fail(MOE_ERR_ARG, "%s: unknown activation type %d", fn, xt);
  if (!router) return fail(MOE_ERR_ARG, "%s: router is NULL", fn);
  if (H <= 0 || H % 32) return fail(MOE_ERR_ARG, "%s: H = %d is not a positive multiple of 32", fn, H);
  if (H > kMaxRouteH) return fail(MOE_ERR_UNSUPPORTED, "%s: H = %d exceeds %d", fn, H, kMaxRouteH);
  const int E = router->rows;
  if (E < 1) return fail(MOE_ERR_ARG, "%s: router has %d rows", fn, E);
  if (E > kMaxE) return fail(MOE_ERR_UNSUPPORTED, "%s: E = %d exceeds %d", fn, E, kMaxE);
  moe_status st = check_qmat(*router, "router", E, H, false, true);
  if (st) return st;
  if (k < 1 || k > E) return fail(MOE_ERR_ARG, "%s: k = %d outside 1..E (E = %d)", fn, k, E);
  if (k > kMaxK) return fail(MOE_ERR_UNSUPPORTED, "%s: k = %d exceeds %d", fn, k, kMaxK);
  if (T > 0 && (!x || !ids || !w)) return fail(MOE_ERR_ARG, "%s: x, ids and w must not be NULL", fn);
  if (!aligned16(x)) return fail(MOE_ERR_ARG, "%s: x must be 16-byte aligned", fn);
  const size_t need = route_ws_bytes(T, E, H, router->fmt);
  if (ws_bytes < need || (need && !ws))
    return fail(MOE_ERR_WORKSPACE, "%s: router workspace %zu bytes, need %zu", fn, ws_bytes, need);
  if (!aligned16(ws)) return fail(MOE_ERR_ARG, "%s: workspace must be 16-byte aligned", fn);
  if (T == 0) return MOE_OK;
  DevCheck dc;
  if ((st = stream_device(s, &dc.dev))) return st;
  dc(x, "x");
  dc(router->codes, "router codes");
  dc(router->scales, "router scales");
  dc(bias, "bias");
  dc(ids, "ids");
  dc(w, "w");
  if (!g_ws_is_scratch) dc(ws, "workspace");
  return dc.st;
}

moe_status group_check(const char* fn, const int32_t* ids, int32_t T, int32_t k, int32_t E, const int32_t* counts,
                       const int32_t* offsets, const int32_t* slot_list, hipStream_t s) {
  if (T < 0 || k < 1) return fail(MOE_ERR_ARG, "%s: T = %d, k = %d", fn, T, k);
  if (E < 1) return fail(MOE_ERR_ARG, "%s: E = %d", fn, E);
  if (E > kMaxE) return fail(MOE_ERR_UNSUPPORTED, "%s: E = %d exceeds %d", fn, E, kMaxE);
  if ((int64_t)T * k > (int64_t)0x7FFFFFFF) return fail(MOE_ERR_ARG, "%s: T*k overflows int32", fn);
  if (!counts || !offsets || (T > 0 && (!ids || !slot_list))) return fail(MOE_ERR_ARG, "%s: NULL output or ids", fn);
  moe_status st;
  DevCheck dc;
  if ((st = stream_device(s, &dc.dev))) return st;
  dc(ids, "ids");
  dc(counts, "counts");
  dc(offsets, "offsets");
  dc(slot_list, "slot_list");
  if (dc.st) return dc.st;
  const size_t lds = moe::group_lds_bytes(E);
  if (lds > 64 * 1024) {
    // more than the default dynamic LDS for large expert counts (set per call: cheap, per device)
    hipError_t e = moe::group_set_lds_limit(lds);
    if (e != hipSuccess) return hip_fail(e, "group LDS attribute");
  }
  return MOE_OK;
}

// Checks of moe_expert_forward's arguments and the launch arguments (FFN launches and tile lists)
// over the workspace.
struct FwdSetup {
  moe::FfnArgs a;
  moe::TileLists tl;
  FwdLayout L;
  int dev = 0;   // the stream's device (T > 0)
};

moe_status forward_setup(const char* fn, const void* x, int32_t xt, int32_t T, int32_t H, int32_t I, int32_t k,
                         const moe_experts* local, const int32_t* g2l, int32_t E, int32_t E_local,
                         const int32_t* counts, const int32_t* offsets, const int32_t* slot_list, float* y_slot,
                         void* ws, size_t ws_bytes, hipStream_t s, FwdSetup& f) {
  if (T < 0) return fail(MOE_ERR_ARG, "%s: T < 0", fn);
  if (xt != MOE_ACT_F32 && xt != MOE_ACT_BF16) return fail(MOE_ERR_ARG, "%s: unknown activation type %d", fn, xt);
  if (H <= 0 || H % 32 || I <= 0 || I % 32)
    return fail(MOE_ERR_ARG, "%s: H = %d, I = %d must be positive multiples of 32", fn, H, I);
  if (H > kMaxFfnDim || I > kMaxFfnDim) return fail(MOE_ERR_UNSUPPORTED, "%s: H and I are limited to %d", fn, kMaxFfnDim);
  if (k < 1 || k > kMaxK) return fail(MOE_ERR_ARG, "%s: k = %d", fn, k);
  if (E < 1 || k > E) return fail(MOE_ERR_ARG, "%s: E = %d, k = %d", fn, E, k);
  if (E > kMaxE) return fail(MOE_ERR_UNSUPPORTED, "%s: E = %d exceeds %d", fn, E, kMaxE);
  if (!local) return fail(MOE_ERR_ARG, "%s: local experts is NULL", fn);
  if (local->n_experts != E_local || E_local < 1 || E_local > E)
    return fail(MOE_ERR_ARG, "%s: E_local = %d but the owned stack holds %d experts (E = %d)", fn, E_local,
                local->n_experts, E);
  if (!g2l && E_local != E) return fail(MOE_ERR_ARG, "%s: no g2l table but only %d of %d experts owned", fn, E_local, E);
  moe_status st;
  if ((st = check_qmat(local->gate, "gate", I, H, true, false))) return st;
  if ((st = check_qmat(local->up, "up", I, H, true, false))) return st;
  if ((st = check_qmat(local->down, "down", H, I, true, false))) return st;
  if (local->gate.fmt != local->up.fmt) return fail(MOE_ERR_UNSUPPORTED, "%s: gate and up must share a format", fn);
  if (T > 0 && (!x || !counts || !offsets || !slot_list || !y_slot))
    return fail(MOE_ERR_ARG, "%s: NULL x, counts, offsets, slot_list or y_slot", fn);
  if (!aligned16(x) || !aligned16(y_slot)) return fail(MOE_ERR_ARG, "%s: x and y_slot must be 16-byte aligned", fn);
  f.L = fwd_layout(T, H, I, k, E_local, xt);
  const FwdLayout& L = f.L;
  if (ws_bytes < L.total || !ws)
    return fail(MOE_ERR_WORKSPACE, "%s: expert workspace %zu bytes, need %zu", fn, ws_bytes, L.total);
  if (T == 0) return MOE_OK;
  DevCheck dc;
  if ((st = stream_device(s, &dc.dev))) return st;
  f.dev = dc.dev;
  dc(x, "x");
  dc(local->gate.codes, "gate codes");
  dc(local->gate.scales, "gate scales");
  dc(local->up.codes, "up codes");
  dc(local->up.scales, "up scales");
  dc(local->down.codes, "down codes");
  dc(local->down.scales, "down scales");
  dc(g2l, "g2l");
  dc(counts, "counts");
  dc(offsets, "offsets");
  dc(slot_list, "slot_list");
  dc(y_slot, "y_slot");
  if (!g_ws_is_scratch) dc(ws, "workspace");
  if (dc.st) return dc.st;

  char* wsb = reinterpret_cast<char*>(ws);
  auto at16 = [&](size_t o) { return reinterpret_cast<uint16_t*>(wsb + o); };
  moe::FfnArgs& a = f.a;
  a = moe::FfnArgs{};
  // 2-bit gate/up past kSelMaxTokens tokens: its rows staged one code unit at a time where whole
  // rows of 8 slots would not fit (tiles of 8 slots instead of 4)
  const bool half = T > moe::kSelMaxTokens && local->gate.fmt == MOE_W_Q2SM &&
                    moe::half_gateup_staging(H, xt == MOE_ACT_F32);
  const TilePlan tp = tile_plan(T, H, I, k, E_local, xt, half);
  a.half_gateup = half;
  a.T = T; a.H = H; a.I = I; a.k = k;
  a.fg = local->gate.fmt;
  a.fd = local->down.fmt;
  a.nb32H = pad32(H / 32);
  a.nb32I = pad32(I / 32);
  a.gate = qm(local->gate);
  a.up = qm(local->up);
  a.down = qm(local->down);
  a.slot_list = slot_list;
  a.small = reinterpret_cast<const int4*>(wsb + L.small);
  a.small_tok = reinterpret_cast<const int4*>(wsb + L.small_tok);
  a.large = reinterpret_cast<const int4*>(wsb + L.large);
  a.n_small = reinterpret_cast<const int32_t*>(wsb + L.n_small);
  a.n_large = reinterpret_cast<const int32_t*>(wsb + L.n_large);
  a.max_small = tp.max_small;
  a.bm_small = tp.bm_small;
  if (tp.max_down > 0) {
    a.down_small = reinterpret_cast<const int4*>(wsb + L.down);
    a.n_down_small = reinterpret_cast<const int32_t*>(wsb + L.n_down);
    a.max_down_small = tp.max_down;
    a.bm_down_small = tp.bm_down;
  }
  a.max_large = tp.max_large;
  a.xq_hi = at16(L.xq_hi);
  a.xq_lo = xt == MOE_ACT_F32 ? at16(L.xq_lo) : nullptr;
  a.sq_hi = at16(L.sq_hi);
  a.sq_lo = at16(L.sq_lo);
  a.sigma = reinterpret_cast<const float*>(wsb + L.sigma);
  auto atf = [&](size_t o) { return reinterpret_cast<float*>(wsb + o); };
  a.h = atf(L.h);
  a.hs = atf(L.hs);
  a.hm = atf(L.hm);
  const bool prep = tp.max_large > 0 || T > moe::kSelMaxTokens;   // (as fwd_layout)
  if (prep || T == 1) {
    a.hq_hi = at16(L.hq_hi);
    a.hq_lo = at16(L.hq_lo);
  }
  if (prep) {
    a.hsq_hi = at16(L.hsq_hi);
    a.hsq_lo = at16(L.hsq_lo);
    a.hsig = atf(L.hsig);
  }
  a.y = y_slot;
  moe::TileLists& tl = f.tl;
  tl = moe::TileLists{};
  tl.counts = counts;
  tl.offsets = offsets;
  tl.g2l = g2l;
  tl.E = E;
  tl.E_local = E_local;
  tl.n_slots = T * k;
  tl.large_min = tp.large_min;
  tl.bm_small = tp.bm_small;
  tl.max_small = tp.max_small;
  tl.bm_large = kLargeTile;
  tl.max_large = tp.max_large;
  tl.small = reinterpret_cast<int4*>(wsb + L.small);
  tl.small_tok = reinterpret_cast<int4*>(wsb + L.small_tok);
  tl.slot_list = slot_list;
  tl.k = k;
  tl.large = reinterpret_cast<int4*>(wsb + L.large);
  tl.n_small = reinterpret_cast<int32_t*>(wsb + L.n_small);
  tl.n_large = reinterpret_cast<int32_t*>(wsb + L.n_large);
  if (tp.max_down > 0) {
    tl.down = reinterpret_cast<int4*>(wsb + L.down);
    tl.n_down = reinterpret_cast<int32_t*>(wsb + L.n_down);
    tl.bm_down = tp.bm_down;
    tl.max_down = tp.max_down;
  }
  return MOE_OK;
}

moe_status combine_check(const char* fn, const float* y_slot, const float* w, const int32_t* ids, const int32_t* g2l,
                         int32_t T, int32_t k, int32_t H, int32_t E, const float* out, hipStream_t s) {
  if (T < 0 || k < 1 || E < 1) return fail(MOE_ERR_ARG, "%s: T = %d, k = %d, E = %d", fn, T, k, E);
  if (H <= 0 || H % 4) return fail(MOE_ERR_ARG, "%s: H = %d must be a positive multiple of 4", fn, H);
  if (T > 0 && (!y_slot || !w || !ids || !out)) return fail(MOE_ERR_ARG, "%s: NULL pointer", fn);
  if (!aligned16(y_slot) || !aligned16(out)) return fail(MOE_ERR_ARG, "%s: y_slot and out must be 16-byte aligned", fn);
  if (T == 0) return MOE_OK;
  moe_status st;
  DevCheck dc;
  if ((st = stream_device(s, &dc.dev))) return st;
  dc(y_slot, "y_slot");
  dc(w, "w");
  dc(ids, "ids");
  dc(g2l, "g2l");
  dc(out, "out");
  return dc.st;
}

hipError_t launch_prep_of(const FwdSetup& f, const void* x, int xt, hipStream_t s) {
  return moe::launch_prep(x, xt, f.a.fg, f.a.T, f.a.H, f.a.nb32H, const_cast<uint16_t*>(f.a.xq_hi),
                          const_cast<uint16_t*>(f.a.xq_lo), const_cast<uint16_t*>(f.a.sq_hi),
                          const_cast<uint16_t*>(f.a.sq_lo), const_cast<float*>(f.a.sigma), f.tl, s);
}

// ---- the second stream of batches with large tiles ----
// Per device: a stream (default priority) and two events, created by the device's first call
// with large tiles and held until the process ends.  The calls on a device share them: a mutex
// keeps each call's fork, launches and join together, and the small-tile launches of concurrent
// calls queue on the one stream.
constexpr int kMaxSideDevices = 64;
struct SideStream {
  std::mutex mu;
  bool tried = false;
  hipStream_t s = nullptr;
  hipEvent_t fork = nullptr, join = nullptr;
};
SideStream g_side[kMaxSideDevices];
std::mutex g_side_init_mu;

// The device's side stream, NULL where there is none: not created while the caller's stream is
// being captured into a graph (creation is no stream operation), nor by the call without
// allocation (creating a stream allocates), or failed to be created.
SideStream* side_of(int dev, hipStream_t s) {
  if (dev < 0 || dev >= kMaxSideDevices) return nullptr;
  SideStream& sd = g_side[dev];
  std::lock_guard<std::mutex> lk(g_side_init_mu);
  if (sd.tried) return sd.s ? &sd : nullptr;
  if (g_ws_is_scratch) return nullptr;   // (a stream created by an earlier call is used)
  hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
  if (hipStreamIsCapturing(s, &cs) != hipSuccess || cs != hipStreamCaptureStatusNone) {
    (void)hipGetLastError();
    return nullptr;
  }
  sd.tried = true;
  int cur = 0;
  if (hipGetDevice(&cur) != hipSuccess) return nullptr;
  if (cur != dev && hipSetDevice(dev) != hipSuccess) return nullptr;
  hipStream_t st = nullptr;
  hipEvent_t e0 = nullptr, e1 = nullptr;
  bool okc = hipStreamCreateWithFlags(&st, hipStreamNonBlocking) == hipSuccess &&
             hipEventCreateWithFlags(&e0, hipEventDisableTiming) == hipSuccess &&
             hipEventCreateWithFlags(&e1, hipEventDisableTiming) == hipSuccess;
  if (cur != dev) okc = hipSetDevice(cur) == hipSuccess && okc;
  (void)hipGetLastError();
  if (!okc) return nullptr;   // (whatever was created stays unused)
  sd.s = st;
  sd.fork = e0;
  sd.join = e1;
  return &sd;
}

// The FFN launches of a prepared call: with large tiles in a batch of at least kForkMinTokens
// tokens, the small tiles' chain on the device's side stream (when there is one), joined back into
// s before the call's later launches.  Below that the large-tile launches are short and themselves
// bound by memory, and sharing the compute units with the small tiles' launches slows the pair
// (128 tokens on 128 owned experts: 0.563 -> 0.578 ms per call; 2048 tokens: 2.374 -> 2.336 ms).
constexpr int kForkMinTokens = 256;
hipError_t run_ffn(FwdSetup& f, hipStream_t s) {
  SideStream* sd = f.a.max_large > 0 && f.a.T >= kForkMinTokens ? side_of(f.dev, s) : nullptr;
  if (!sd) return moe::launch_ffn(f.a, s);
  std::lock_guard<std::mutex> lk(sd->mu);
  f.a.side = sd->s;
  f.a.fork = sd->fork;
  f.a.join = sd->join;
  const hipError_t e = moe::launch_ffn(f.a, s);
  f.a.side = nullptr;
  return e;
}

}  // namespace

namespace moe {   // combine.hip
hipError_t launch_shared_group(int T, int32_t* counts, int32_t* offsets, int32_t* slot_list, hipStream_t s);
hipError_t launch_add_rows(const float* y, float* out, int64_t n, hipStream_t s);
}  // namespace moe

// Shared expert workspace: counts [1], offsets [2], slot_list [T], y [T, H] fp32, then the expert
// forward's own workspace (one expert, one slot per token).
struct SharedLayout {
  size_t counts, offsets, slots, y, fwd, total;
};
static SharedLayout shared_layout(int T, int H, int I, int xt) {
  SharedLayout L{};
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t at = off;
    off += align_up(bytes);
    return at;
  };
  L.counts = take(sizeof(int32_t));
  L.offsets = take(2 * sizeof(int32_t));
  L.slots = take((size_t)T * sizeof(int32_t));
  L.y = take((size_t)T * H * sizeof(float));
  L.fwd = take(fwd_layout(T, H, I, 1, 1, xt).total);
  L.total = off;
  return L;
}

extern "C" {

moe_status moe_route(const void* x, int32_t xt, int32_t T, int32_t H, const moe_qmat* router, const float* bias,
                     int32_t k, int32_t* ids, float* w, void* ws, size_t ws_bytes, hipStream_t s) {
  moe_status st = route_check("moe_route", x, xt, T, H, router, bias, k, ids, w, ws, ws_bytes, s);
  if (st) return st;
  if (T == 0) return ok();
  hipError_t e = moe::launch_route(x, xt, T, H, router->fmt, qm(*router), bias, k, ids, w, ws, s);
  if (e != hipSuccess) return hip_fail(e, "moe_route launch");
  return ok();
}

moe_status moe_route_table(const void* x, int32_t xt, int32_t T, int32_t H, const moe_qmat* router, const float* bias,
                           const int32_t* token_ids, const int32_t* table, int32_t V, int32_t k, int32_t* ids,
                           float* w, void* ws, size_t ws_bytes, hipStream_t s) {
  const char* fn = "moe_route_table";
  if (V < 1) return fail(MOE_ERR_ARG, "%s: V = %d, the table needs a row", fn, V);
  if (T > 0 && (!token_ids || !table)) return fail(MOE_ERR_ARG, "%s: token_ids and table must not be NULL", fn);
  moe_status st = route_check(fn, x, xt, T, H, router, bias, k, ids, w, ws, ws_bytes, s);
  if (st) return st;
  if (T == 0) return ok();
  DevCheck dc;
  if ((st = stream_device(s, &dc.dev))) return st;
  dc(token_ids, "token_ids");
  dc(table, "table");
  if (dc.st) return dc.st;
  hipError_t e = moe::launch_route_table(x, xt, T, H, router->fmt, qm(*router), bias, token_ids, table, V, k, ids, w,
                                         ws, s);
  if (e != hipSuccess) return hip_fail(e, "moe_route_table launch");
  return ok();
}

moe_status moe_group_tokens(const int32_t* ids, int32_t T, int32_t k, int32_t E, int32_t* counts, int32_t* offsets,
                            int32_t* slot_list, void* ws, size_t ws_bytes, hipStream_t s) {
  (void)ws;
  (void)ws_bytes;
  moe_status st = group_check("moe_group_tokens", ids, T, k, E, counts, offsets, slot_list, s);
  if (st) return st;
  hipError_t e = moe::launch_group(ids, T, k, E, counts, offsets, slot_list, s);
  if (e != hipSuccess) return hip_fail(e, "moe_group_tokens launch");
  return ok();
}

moe_status moe_expert_forward(const void* x, int32_t xt, int32_t T, int32_t H, int32_t I, int32_t k,
                              const moe_experts* local, const int32_t* g2l, int32_t E, int32_t E_local,
                              const int32_t* counts, const int32_t* offsets, const int32_t* slot_list, float* y_slot,
                              void* ws, size_t ws_bytes, hipStream_t s) {
  FwdSetup f;
  moe_status st = forward_setup("moe_expert_forward", x, xt, T, H, I, k, local, g2l, E, E_local, counts, offsets,
                                slot_list, y_slot, ws, ws_bytes, s, f);
  if (st) return st;
  if (T == 0) return ok();
  hipError_t e = launch_prep_of(f, x, xt, s);
  if (e != hipSuccess) return hip_fail(e, "moe_expert_forward: prep launch");
  e = run_ffn(f, s);
  if (e != hipSuccess) return hip_fail(e, "moe_expert_forward: FFN launch");
  return ok();
}

moe_status moe_combine(const float* y_slot, const float* w, const int32_t* ids, const int32_t* g2l, int32_t T,
                       int32_t k, int32_t H, int32_t E, float* out, hipStream_t s) {
  moe_status st = combine_check("moe_combine", y_slot, w, ids, g2l, T, k, H, E, out, s);
  if (st) return st;
  if (T == 0) return ok();
  hipError_t e = moe::launch_combine(y_slot, w, ids, g2l, T, k, H, E, out, s);
  if (e != hipSuccess) return hip_fail(e, "moe_combine launch");
  return ok();
}

moe_status moe_layer_forward(const void* x, int32_t xt, int32_t T, int32_t H, int32_t I, int32_t k,
                             const moe_qmat* router, const float* bias, const moe_experts* local, const int32_t* g2l,
                             int32_t E, int32_t E_local, int32_t* ids, float* w, int32_t* counts, int32_t* offsets,
                             int32_t* slot_list, float* y_slot, float* out, void* ws, size_t ws_bytes, hipStream_t s) {
  const char* fn = "moe_layer_forward";
  if (!router) return fail(MOE_ERR_ARG, "%s: router is NULL", fn);
  if (router->rows != E) return fail(MOE_ERR_ARG, "%s: router has %d rows but E = %d", fn, router->rows, E);
  if (H <= 0 || H % 32 || E < 1 || E > kMaxE) return fail(MOE_ERR_ARG, "%s: H = %d, E = %d", fn, H, E);
  if (T < 0) return fail(MOE_ERR_ARG, "%s: T < 0", fn);
  // the router's part of the workspace first, then the expert part
  const size_t rws = route_ws_bytes(T, E, H);
  if (ws_bytes < rws) return fail(MOE_ERR_WORKSPACE, "%s: workspace %zu bytes, need more than %zu", fn, ws_bytes, rws);
  char* wsb = reinterpret_cast<char*>(ws);
  moe_status st = route_check(fn, x, xt, T, H, router, bias, k, ids, w, ws, rws, s);
  if (st) return st;
  if ((st = group_check(fn, ids, T, k, E, counts, offsets, slot_list, s))) return st;
  FwdSetup f;
  if ((st = forward_setup(fn, x, xt, T, H, I, k, local, g2l, E, E_local, counts, offsets, slot_list, y_slot,
                          wsb ? wsb + rws : nullptr, ws_bytes - rws, s, f)))
    return st;
  if ((st = combine_check(fn, y_slot, w, ids, g2l, T, k, H, E, out, s))) return st;
  hipError_t e;
  if (T == 0) {
    // as the four calls: only the grouping writes anything (zero counts and offsets)
    e = moe::launch_group(ids, T, k, E, counts, offsets, slot_list, s);
    if (e != hipSuccess) return hip_fail(e, "moe_layer_forward: group launch");
    return ok();
  }
  moe::SelArgs sel{};
  if (T <= moe::kSelMaxTokens && E <= moe::kSelMaxE && f.a.max_large == 0 &&
      moe::logit_ranges(T, E, H, router->fmt) <= moe::kSelMaxRanges) {
    // router launch (with the operands), then the gate/up launch selects and groups by itself
    int S = 0;
    const moe::PrepOut po{f.a.nb32H, const_cast<uint16_t*>(f.a.xq_hi), const_cast<uint16_t*>(f.a.xq_lo),
                          const_cast<uint16_t*>(f.a.sq_hi), const_cast<uint16_t*>(f.a.sq_lo),
                          const_cast<float*>(f.a.sigma)};
    e = moe::launch_logits(x, xt, T, H, router->fmt, qm(*router), bias, ws, &S, s, &po);
    if (e != hipSuccess) return hip_fail(e, "moe_layer_forward: logits launch");
    sel.z = reinterpret_cast<const float*>(ws);
    sel.S = S;
    sel.bias = bias;
    sel.T = T;
    sel.E = E;
    sel.k = k;
    sel.E_local = E_local;
    sel.g2l = g2l;
    sel.max_tiles = f.tl.max_small;
    sel.bm = f.tl.bm_small;
    sel.ids = ids;
    sel.w = w;
    sel.counts = counts;
    sel.offsets = offsets;
    sel.slot_list = slot_list;
    sel.n_tiles = f.tl.n_small;
    sel.tiles = f.tl.small;
    sel.tile_tok = f.tl.small_tok;
    f.a.sel = &sel;
  } else if (T <= moe::kFrontMaxTokens && moe::logit_ranges(T, E, H, router->fmt) <= moe::kSelMaxRanges) {
    const size_t lds = moe::front_lds_bytes(T, E, k);
    if (lds > 160 * 1024) return fail(MOE_ERR_UNSUPPORTED, "%s: E = %d needs %zu bytes of LDS", fn, E, lds);
    int S = 0;
    const moe::PrepOut po{f.a.nb32H, const_cast<uint16_t*>(f.a.xq_hi), const_cast<uint16_t*>(f.a.xq_lo),
                          const_cast<uint16_t*>(f.a.sq_hi), const_cast<uint16_t*>(f.a.sq_lo),
                          const_cast<float*>(f.a.sigma)};
    // the operands ride on the router's launch (batches this small take the small-batch logits
    // kernels)
    e = moe::launch_logits(x, xt, T, H, router->fmt, qm(*router), bias, ws, &S, s, &po);
    if (e != hipSuccess) return hip_fail(e, "moe_layer_forward: logits launch");
    e = moe::launch_front(reinterpret_cast<const float*>(ws), S, bias, T, E, k, ids, w, counts, offsets, slot_list, x,
                          xt, H, nullptr, f.tl, s);
    if (e != hipSuccess) return hip_fail(e, "moe_layer_forward: selection launch");
  } else {
    e = moe::launch_route(x, xt, T, H, router->fmt, qm(*router), bias, k, ids, w, ws, s);
    if (e != hipSuccess) return hip_fail(e, "moe_layer_forward: route launch");
    e = moe::launch_group(ids, T, k, E, counts, offsets, slot_list, s);
    if (e != hipSuccess) return hip_fail(e, "moe_layer_forward: group launch");
    e = launch_prep_of(f, x, xt, s);
    if (e != hipSuccess) return hip_fail(e, "moe_layer_forward: prep launch");
  }
  e = run_ffn(f, s);
  if (e != hipSuccess) return hip_fail(e, "moe_layer_forward: FFN launch");
  e = moe::launch_combine(y_slot, w, ids, g2l, T, k, H, E, out, s);
  if (e != hipSuccess) return hip_fail(e, "moe_layer_forward: combine launch");
  return ok();
}

// ---- the layer call without allocation: a workspace the library holds ---------------------
// One array per device, of kScratchBytes, reserved when the library is loaded onto the device and
// held until the process ends; its device address comes from hipGetSymbolAddress, once per
// device with that device current, and every call on the device shares it.
constexpr size_t kScratchBytes = (size_t)32 << 20;
static __device__ __align__(256) uint8_t scratch[kScratchBytes];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// The device address of device dev's scratch array (looked up on the first call for the device).
moe_status scratch_of(int dev, void** p) {
  if (dev < 0 || dev >= kMaxDevices) return fail(MOE_ERR_DEVICE, "device %d: no scratch slot", dev);
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    int cur = 0;
    hipError_t e = hipGetDevice(&cur);
    if (e != hipSuccess) return hip_fail(e, "scratch: current device");
    if (cur != dev && (e = hipSetDevice(dev)) != hipSuccess) return hip_fail(e, "scratch: set device");
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    const hipError_t e2 = cur != dev ? hipSetDevice(cur) : hipSuccess;
    if (e != hipSuccess) return hip_fail(e, "scratch: hipGetSymbolAddress");
    if (e2 != hipSuccess) return hip_fail(e2, "scratch: restore device");
    if (!ptr) return fail(MOE_ERR_HIP, "scratch: no device address");
    g_scratch_ptr[dev] = ptr;
  }
  *p = g_scratch_ptr[dev];
  return MOE_OK;
}
}  // namespace

extern "C" moe_status moe_layer_forward_noalloc(const void* x, int32_t xt, int32_t T, int32_t H, int32_t I,
                                                int32_t k, const moe_qmat* router, const float* bias,
                                                const moe_experts* local, const int32_t* g2l, int32_t E,
                                                int32_t E_local, int32_t* ids, float* w, int32_t* counts,
                                                int32_t* offsets, int32_t* slot_list, float* y_slot, float* out,
                                                hipStream_t s) {
  const char* fn = "moe_layer_forward_noalloc";
  if (T < 0 || H <= 0 || I <= 0 || k <= 0 || E <= 0 || E_local < 0 || E_local > E || E > kMaxE)
    return fail(MOE_ERR_ARG, "%s: bad sizes", fn);
  if (xt != MOE_ACT_F32 && xt != MOE_ACT_BF16) return fail(MOE_ERR_ARG, "%s: unknown activation type %d", fn, xt);
  const size_t need = route_ws_bytes(T, E, H) + fwd_layout(T, H, I, k, E_local, xt).total;
  if (need > kScratchBytes)
    return fail(MOE_ERR_UNSUPPORTED, "%s: this batch needs %zu bytes of workspace; the library's scratch holds %zu "
                "(use moe_layer_forward with a caller workspace)", fn, need, kScratchBytes);
  int dev = 0;
  moe_status st = stream_device(s, &dev);
  if (st) return st;
  void* ws = nullptr;
  if ((st = scratch_of(dev, &ws))) return st;
  g_ws_is_scratch = true;
  st = moe_layer_forward(x, xt, T, H, I, k, router, bias, local, g2l, E, E_local, ids, w, counts, offsets,
                         slot_list, y_slot, out, ws, kScratchBytes, s);
  g_ws_is_scratch = false;
  if (st) return st;
  return ok();
}

moe_status moe_shared_expert_workspace(int32_t T, int32_t H, int32_t I, int32_t xt, size_t* ws_bytes) {
  if (T < 0 || H <= 0 || I <= 0 || !ws_bytes) return fail(MOE_ERR_ARG, "moe_shared_expert_workspace: bad arguments");
  *ws_bytes = shared_layout(T, H, I, xt).total;
  return ok();
}

moe_status moe_shared_expert_forward(const void* x, int32_t xt, int32_t T, int32_t H, int32_t I,
                                     const moe_experts* shared, float* out, void* ws, size_t ws_bytes, hipStream_t s) {
  const char* fn = "moe_shared_expert_forward";
  if (!shared || shared->n_experts != 1) return fail(MOE_ERR_ARG, "%s: shared must hold exactly one expert", fn);
  if (T < 0 || H <= 0 || I <= 0) return fail(MOE_ERR_ARG, "%s: bad sizes", fn);
  if (T > 0 && !out) return fail(MOE_ERR_ARG, "%s: out must not be NULL", fn);
  const SharedLayout L = shared_layout(T, H, I, xt);
  if (ws_bytes < L.total || (L.total && !ws))
    return fail(MOE_ERR_WORKSPACE, "%s: workspace %zu bytes, need %zu", fn, ws_bytes, L.total);
  if (!aligned16(ws) || !aligned16(out)) return fail(MOE_ERR_ARG, "%s: workspace and out must be 16-byte aligned", fn);
  if (T == 0) return ok();
  uint8_t* b = static_cast<uint8_t*>(ws);
  int32_t* counts = reinterpret_cast<int32_t*>(b + L.counts);
  int32_t* offsets = reinterpret_cast<int32_t*>(b + L.offsets);
  int32_t* slots = reinterpret_cast<int32_t*>(b + L.slots);
  float* y = reinterpret_cast<float*>(b + L.y);
  // the argument and device checks of the expert call come first: nothing is launched on failure
  FwdSetup f;
  moe_status st = forward_setup(fn, x, xt, T, H, I, 1, shared, nullptr, 1, 1, counts, offsets, slots, y, b + L.fwd,
                                ws_bytes - L.fwd, s, f);
  if (st) return st;
  DevCheck dc;
  if ((st = stream_device(s, &dc.dev))) return st;
  dc(out, "out");
  if (dc.st) return dc.st;
  hipError_t e = moe::launch_shared_group(T, counts, offsets, slots, s);
  if (e != hipSuccess) return hip_fail(e, "moe_shared_expert_forward: group launch");
  e = launch_prep_of(f, x, xt, s);
  if (e != hipSuccess) return hip_fail(e, "moe_shared_expert_forward: prep launch");
  e = run_ffn(f, s);
  if (e != hipSuccess) return hip_fail(e, "moe_shared_expert_forward: FFN launch");
  e = moe::launch_add_rows(y, out, (int64_t)T * H, s);
  if (e != hipSuccess) return hip_fail(e, "moe_shared_expert_forward: add launch");
  return ok();
}

}  // extern "C"
