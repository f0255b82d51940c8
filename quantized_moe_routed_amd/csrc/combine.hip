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

hipError_t launch_combine(const float* y, const float* w, const int32_t* ids, const int32_t* g2l, int T, int k,
                          int H, int E, float* out, hipStream_t s) {
  dim3 grid((H / 4 + 255) / 256, T);
  trace_pre("combine", s);
  combine_kernel<<<grid, 256, 0, s>>>(y, w, ids, g2l, T, k, H, E, out);
  trace_post("combine", s);
  return hipGetLastError();
}

}  // namespace moe
