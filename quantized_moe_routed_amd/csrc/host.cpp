// Host-only entry points of libmoe (no device access, no HIP calls): the error
// state behind moe_last_error, the planar weight packer and its size query,
// LPT placement, share tables and the load-time checks of placement and routing
// tables.  Plain C++, so that it also builds with the host compiler's
// sanitizers on a machine without a GPU.
#include <algorithm>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <string>
#include <vector>

#include "../../include/moe.h"
#include "status.h"

namespace {
thread_local std::string g_err;
}  // namespace

namespace moe {
moe_status fail(moe_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_err = buf;
  return st;
}

moe_status ok() {
  g_err.clear();
  return MOE_OK;
}
}  // namespace moe

using moe::fail;
using moe::ok;

extern "C" {

const char* moe_last_error(void) { return g_err.c_str(); }

const char* moe_version(void) { return "moe-gfx950 0.1"; }

static size_t groups16(int64_t rows) { return (size_t)((rows + 15) / 16); }

moe_status moe_planar_bytes(int32_t fmt, int32_t rows, int32_t cols, size_t* codes_bytes, size_t* scales_bytes) {
  if (rows < 0 || cols <= 0 || cols % 32) return fail(MOE_ERR_ARG, "moe_planar_bytes: bad shape %dx%d", rows, cols);
  size_t c, sc;
  const size_t nb = (size_t)(cols / 32);
  switch (fmt) {
    case MOE_W_F32: c = (size_t)rows * cols * 4; sc = 0; break;
    case MOE_W_Q8_0: c = groups16(rows) * ((nb + 1) / 2) * 1024; sc = groups16(rows) * ((nb + 1) / 2) * 64; break;
    case MOE_W_Q2SM: c = groups16(rows) * ((nb + 7) / 8) * 1024; sc = groups16(rows) * ((nb + 7) / 8) * 512; break;
    default: return fail(MOE_ERR_UNSUPPORTED, "moe_planar_bytes: unknown format %d", fmt);
  }
  if (codes_bytes) *codes_bytes = c;
  if (scales_bytes) *scales_bytes = sc;
  return ok();
}

// Re-lay definition blocks into the unit layout documented in moe.h.
moe_status moe_pack_planar(int32_t fmt, int32_t n, int32_t rows, int32_t cols, const void* aos, void* codes,
                           void* scales) {
  if (n < 0 || rows < 0 || cols <= 0 || cols % 32) return fail(MOE_ERR_ARG, "moe_pack_planar: bad shape");
  if (!aos || !codes || (fmt != MOE_W_F32 && !scales)) return fail(MOE_ERR_ARG, "moe_pack_planar: NULL pointer");
  const int64_t nb = cols / 32;
  const int64_t nrows = (int64_t)n * rows;
  const uint8_t* src = static_cast<const uint8_t*>(aos);
  uint8_t* dc = static_cast<uint8_t*>(codes);
  uint8_t* ds = static_cast<uint8_t*>(scales);
  switch (fmt) {
    case MOE_W_F32:
      std::memcpy(dc, src, (size_t)nrows * cols * 4);
      break;
    case MOE_W_Q8_0: {
      // row groups of 16 rows; per (group, unit of 2 blocks): 16 rows x 64 code bytes, and
      // 16 rows x 2 fp16 d
      const int64_t nu = (nb + 1) / 2, rg = (int64_t)groups16(rows);
      const int64_t mc = rg * nu * 1024, ms = rg * nu * 64;   // bytes per matrix
      std::memset(dc, 0, (size_t)(n * mc));
      std::memset(ds, 0, (size_t)(n * ms));
      for (int64_t r = 0; r < nrows; ++r) {
        const int64_t mat = r / rows, row = r % rows;
        uint8_t* mcodes = dc + mat * mc;
        uint8_t* mscales = ds + mat * ms;
        for (int64_t b = 0; b < nb; ++b) {
          const uint8_t* blk = src + (r * nb + b) * 34;
          const int64_t u = b / 2, h = b % 2;
          std::memcpy(mscales + ((row / 16) * nu + u) * 64 + (row % 16) * 4 + 2 * h, blk, 2);
          for (int g = 0; g < 4; ++g)
            std::memcpy(mcodes + ((row / 16) * nu + u) * 1024 + (row % 16) * 64 + g * 16 + h * 8, blk + 2 + 8 * g, 8);
        }
      }
      break;
    }
    case MOE_W_Q2SM: {
      // row groups of 16 rows; per (group, unit of 8 blocks): 16 rows x 64 code bytes, and
      // 16 rows x 8 fp16 d followed by 16 rows x 8 fp16 m
      const int64_t nu = (nb + 7) / 8, rg = (int64_t)groups16(rows);
      const int64_t mc = rg * nu * 1024, ms = rg * nu * 512;
      std::memset(dc, 0, (size_t)(n * mc));
      std::memset(ds, 0, (size_t)(n * ms));
      for (int64_t r = 0; r < nrows; ++r) {
        const int64_t mat = r / rows, row = r % rows;
        uint8_t* mcodes = dc + mat * mc;
        uint8_t* mscales = ds + mat * ms;
        for (int64_t b = 0; b < nb; ++b) {
          const uint8_t* blk = src + (r * nb + b) * 12;
          const int64_t u = b / 8, k = b % 8;
          uint8_t* su = mscales + ((row / 16) * nu + u) * 512;
          std::memcpy(su + (row % 16) * 16 + 2 * k, blk, 2);         // d
          std::memcpy(su + 256 + (row % 16) * 16 + 2 * k, blk + 2, 2);  // m
          const int64_t i = k / 2, h = k % 2;
          for (int g = 0; g < 4; ++g) {
            uint8_t* w = mcodes + ((row / 16) * nu + u) * 1024 + (row % 16) * 64 + g * 16 + i * 4;
            w[h] = blk[4 + 2 * g];
            w[2 + h] = blk[4 + 2 * g + 1];
          }
        }
      }
      break;
    }
    default:
      return fail(MOE_ERR_UNSUPPORTED, "moe_pack_planar: unknown format %d", fmt);
  }
  return ok();
}

moe_status moe_place_lpt(const int64_t* load, int32_t E, int32_t n_shares, int32_t* owner) {
  if (!load || !owner) return fail(MOE_ERR_ARG, "moe_place_lpt: NULL pointer");
  if (E < 1 || n_shares < 1 || E % n_shares)
    return fail(MOE_ERR_ARG, "moe_place_lpt: E = %d is not a positive multiple of n_shares = %d", E, n_shares);
  std::vector<int> order(E);
  for (int e = 0; e < E; ++e) order[e] = e;
  std::stable_sort(order.begin(), order.end(), [&](int a, int b) { return load[a] > load[b]; });
  const int cap = E / n_shares;
  std::vector<int64_t> sl(n_shares, 0);
  std::vector<int> sn(n_shares, 0);
  for (int e : order) {
    int best = -1;
    for (int sh = 0; sh < n_shares; ++sh) {
      if (sn[sh] >= cap) continue;
      if (best < 0 || sl[sh] < sl[best]) best = sh;
    }
    owner[e] = best;
    sl[best] += load[e];
    sn[best] += 1;
  }
  return ok();
}

moe_status moe_share_tables(const int32_t* owner, int32_t E, int32_t share, const int32_t* local_order, int32_t* g2l,
                            int32_t* l2g, int32_t* E_local) {
  if (!owner || !g2l || !l2g || !E_local || E < 1) return fail(MOE_ERR_ARG, "moe_share_tables: bad arguments");
  std::vector<int> owned;
  for (int e = 0; e < E; ++e)
    if (owner[e] == share) owned.push_back(e);
  if (local_order)
    std::stable_sort(owned.begin(), owned.end(), [&](int a, int b) { return local_order[a] < local_order[b]; });
  for (int e = 0; e < E; ++e) g2l[e] = -1;
  for (size_t l = 0; l < owned.size(); ++l) {
    g2l[owned[l]] = (int32_t)l;
    l2g[l] = owned[l];
  }
  *E_local = (int32_t)owned.size();
  return ok();
}

moe_status moe_table_check(const int32_t* table, int32_t V, int32_t k, int32_t E) {
  if (!table || V < 1 || k < 1 || E < 1 || k > E) return fail(MOE_ERR_ARG, "moe_table_check: bad arguments");
  std::vector<int> row_of(E, -1);   // the last row that named each expert
  for (int v = 0; v < V; ++v)
    for (int j = 0; j < k; ++j) {
      const int e = table[(int64_t)v * k + j];
      if (e < 0 || e >= E) return fail(MOE_ERR_ARG, "moe_table_check: table[%d][%d] = %d outside 0..%d", v, j, e, E - 1);
      if (row_of[e] == v) return fail(MOE_ERR_ARG, "moe_table_check: expert %d twice in row %d", e, v);
      row_of[e] = v;
    }
  return ok();
}

moe_status moe_plan_check(const int32_t* g2l, int32_t E, int32_t E_local) {
  if (!g2l || E < 1 || E_local < 0 || E_local > E) return fail(MOE_ERR_ARG, "moe_plan_check: bad arguments");
  std::vector<char> seen(E_local, 0);
  int owned = 0;
  for (int e = 0; e < E; ++e) {
    const int l = g2l[e];
    if (l == -1) continue;
    if (l < 0 || l >= E_local) return fail(MOE_ERR_ARG, "moe_plan_check: g2l[%d] = %d outside -1..%d", e, l, E_local - 1);
    if (seen[l]) return fail(MOE_ERR_ARG, "moe_plan_check: local id %d owned twice", l);
    seen[l] = 1;
    ++owned;
  }
  if (owned != E_local)
    return fail(MOE_ERR_ARG, "moe_plan_check: %d experts owned but E_local = %d", owned, E_local);
  return ok();
}

}  // extern "C"
