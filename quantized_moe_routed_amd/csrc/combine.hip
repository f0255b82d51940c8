// Fixed-order weighted combine: out[t] = sum_{j ascending, owned} w[t,j] * y[t*k+j].
// One thread per (token, 4 columns); each output element is accumulated by a
// single thread in slot order from +0.0, so the result never depends on
// scheduling (no atomics anywhere).
#include <algorithm>

#include "device.h"
#include "launch.h"

namespace moe {

__global__ __launch_bounds__(256) void combine_kernel(const float* __restrict__ y, const float* __restrict__ w,
                                                      const int32_t* __restrict__ ids,
                                                      const int32_t* __restrict__ g2l, int T, int k, int H, int E,
                                                      float* __restrict__ out) {
  const int t = blockIdx.y;
  const int c4 = blockIdx.x * blockDim.x + threadIdx.x;  // index of a 4-column group
  if (c4 * 4 >= H) return;
  float4 acc = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
  for (int j = 0; j < k; ++j) {
    const int64_t s = (int64_t)t * k + j;
    const int e = ids[s];
    if (g2l && ((unsigned)e >= (unsigned)E || g2l[e] < 0)) continue;
    const float ws = w[s];
    const float4 v = *reinterpret_cast<const float4*>(y + s * H + c4 * 4);
    acc.x = fmaf(ws, v.x, acc.x);
    acc.y = fmaf(ws, v.y, acc.y);
    acc.z = fmaf(ws, v.z, acc.z);
    acc.w = fmaf(ws, v.w, acc.w);
  }
  *reinterpret_cast<float4*>(out + (int64_t)t * H + c4 * 4) = acc;
}

// k <= KM: every slot's y, id and weight are loaded before any is used (slots past k repeat the
// last one and are dropped), then the owner table; the fused multiply-adds run in slot order over
// the owned slots exactly as in the loop above, so the two kernels agree bit for bit.
template <int KM>
__global__ __launch_bounds__(256) void combine_kernel_k(const float* __restrict__ y, const float* __restrict__ w,
                                                        const int32_t* __restrict__ ids,
                                                        const int32_t* __restrict__ g2l, int T, int k, int H,
                                                        int E, float* __restrict__ out) {
  const int t = blockIdx.y;
  const int c4 = blockIdx.x * blockDim.x + threadIdx.x;  // index of a 4-column group
  if (c4 * 4 >= H) return;
  float4 v[KM];
  int e[KM];
  float ws[KM];
#pragma unroll
  for (int j = 0; j < KM; ++j) {
    const int64_t s = (int64_t)t * k + min(j, k - 1);
    v[j] = *reinterpret_cast<const float4*>(y + s * H + c4 * 4);
    e[j] = ids[s];
    ws[j] = w[s];
  }
  bool own[KM];
#pragma unroll
  for (int j = 0; j < KM; ++j) {
    own[j] = j < k;
    if (g2l) {
      const bool in = (unsigned)e[j] < (unsigned)E;
      own[j] = own[j] && in && g2l[in ? e[j] : 0] >= 0;
    }
  }
  float4 acc = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
#pragma unroll
  for (int j = 0; j < KM; ++j) {
    if (own[j]) {
      acc.x = fmaf(ws[j], v[j].x, acc.x);
      acc.y = fmaf(ws[j], v[j].y, acc.y);
      acc.z = fmaf(ws[j], v[j].z, acc.z);
      acc.w = fmaf(ws[j], v[j].w, acc.w);
    }
  }
  *reinterpret_cast<float4*>(out + (int64_t)t * H + c4 * 4) = acc;
}

hipError_t launch_combine(const float* y, const float* w, const int32_t* ids, const int32_t* g2l, int T, int k,
                          int H, int E, float* out, hipStream_t s) {
  // small batches: workgroups of one wave, so that the few rows spread over more compute units
  const int nt = T <= 16 ? 64 : 256;
  dim3 grid((H / 4 + nt - 1) / nt, T);
  trace_pre("combine", s);
  if (k <= 8)
    combine_kernel_k<8><<<grid, nt, 0, s>>>(y, w, ids, g2l, T, k, H, E, out);
  else
    combine_kernel<<<grid, nt, 0, s>>>(y, w, ids, g2l, T, k, H, E, out);
  trace_post("combine", s);
  return hipGetLastError();
}

// The shared expert takes every token: one expert with counts = {T}, offsets = {0, T} and the
// slots in order.
__global__ __launch_bounds__(256) void shared_group_kernel(int T, int32_t* __restrict__ counts,
                                                           int32_t* __restrict__ offsets,
                                                           int32_t* __restrict__ slot_list) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < T) slot_list[i] = i;
  if (i == 0) {
    counts[0] = T;
    offsets[0] = 0;
    offsets[1] = T;
  }
}

// out[i] += y[i], one fp32 addition per element (n a multiple of 4).
__global__ __launch_bounds__(256) void add_rows_kernel(const float4* __restrict__ y, float4* __restrict__ out,
                                                       int64_t n4) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n4; i += (int64_t)gridDim.x * blockDim.x) {
    const float4 a = out[i], b = y[i];
    out[i] = make_float4(a.x + b.x, a.y + b.y, a.z + b.z, a.w + b.w);
  }
}

hipError_t launch_shared_group(int T, int32_t* counts, int32_t* offsets, int32_t* slot_list, hipStream_t s) {
  shared_group_kernel<<<(T + 255) / 256, 256, 0, s>>>(T, counts, offsets, slot_list);
  return hipGetLastError();
}

hipError_t launch_add_rows(const float* y, float* out, int64_t n, hipStream_t s) {
  const int64_t n4 = n / 4;
  const int64_t blocks = std::min<int64_t>((n4 + 255) / 256, 2048);
  trace_pre("add_shared", s);
  add_rows_kernel<<<(int)blocks, 256, 0, s>>>(reinterpret_cast<const float4*>(y), reinterpret_cast<float4*>(out), n4);
  trace_post("add_shared", s);
  return hipGetLastError();
}

}  // namespace moe
