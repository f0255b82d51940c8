// Fixed-order weighted combine: out[t] = sum_{j ascending, owned} w[t,j] * y[t*k+j].
// One thread per (token, 4 columns); each output element is accumulated by a
// single thread in slot order from +0.0, so the result never depends on
// scheduling (no atomics anywhere).
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

}  // namespace moe
