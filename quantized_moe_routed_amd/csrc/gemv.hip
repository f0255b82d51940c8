// Dequant-GEMV family (fp32 activations): the expert FFN for decode-size
// batches.  The work is bound by streaming the quantised expert weights from
// HBM, so the kernels are shaped for coalesced wide loads: a wave owns whole
// weight rows, lane l owns the NBL consecutive 32-blocks l*NBL.. of a row
// (one 16-byte load of 2-bit codes for NBL = 2), dequantises in registers and
// reduces across the wave.  The activation chunk of a lane stays in registers
// while the wave walks its rows.
//
// Q2SM blocks use the factorisation  sum_i (d q_i + m) x_i = d sum_i q_i x_i + m sum_i x_i,
// with the block sums of x computed once per token.
#include "device.h"
#include "launch.h"

namespace moe {

constexpr int kGemvWaves = 4;
constexpr int kRowsPerWave = 4;

// Active owned experts in ascending global id: act[0..n_act).
__global__ __launch_bounds__(1024) void active_experts_kernel(const int32_t* __restrict__ counts,
                                                              const int32_t* __restrict__ g2l, int E,
                                                              int E_local, int32_t* __restrict__ act,
                                                              int32_t* __restrict__ n_act) {
  __shared__ int32_t wave_tot[16];
  const int tid = threadIdx.x, lane = tid % kWave, wave = tid / kWave;
  bool on = false;
  if (tid < E) {
    const int l = g2l ? g2l[tid] : tid;
    on = counts[tid] > 0 && l >= 0 && l < E_local;
  }
  const uint64_t m = __ballot(on);
  if (lane == 0) wave_tot[wave] = __popcll(m);
  __syncthreads();
  int before = 0;
  for (int w = 0; w < wave; ++w) before += wave_tot[w];
  if (on) act[before + __popcll(m & lanemask_lt())] = tid;
  if (tid == 0) {
    int tot = 0;
    for (int w = 0; w < 16; ++w) tot += wave_tot[w];
    *n_act = tot;
  }
}

// Activation chunk of one lane: NBL blocks of 32 fp32 values and their block sums.
template <int NBL>
struct XChunk {
  float v[NBL][32];
  float sum[NBL];
};

template <int NBL>
__device__ __forceinline__ void load_chunk(const float* __restrict__ row, int nb, int lane, XChunk<NBL>& c) {
#pragma unroll
  for (int j = 0; j < NBL; ++j) {
    const int b = lane * NBL + j;
    float s = 0.0f;
    if (b < nb) {
      const float4* p = reinterpret_cast<const float4*>(row + b * 32);
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const float4 q = p[i];
        c.v[j][4 * i] = q.x;
        c.v[j][4 * i + 1] = q.y;
        c.v[j][4 * i + 2] = q.z;
        c.v[j][4 * i + 3] = q.w;
      }
#pragma unroll
      for (int i = 0; i < 32; ++i) s += c.v[j][i];
    } else {
#pragma unroll
      for (int i = 0; i < 32; ++i) c.v[j][i] = 0.0f;
    }
    c.sum[j] = s;
  }
}

// Partial dot product of one quantised row with the lane's chunk.
template <int FMT, int NBL>
__device__ __forceinline__ float row_dot(const QMat& m, int64_t row, int nb, int lane, const XChunk<NBL>& c) {
  float acc = 0.0f;
  const int b0 = lane * NBL;
  if (b0 >= nb) return 0.0f;
  if constexpr (FMT == FMT_Q2SM) {
    const uint8_t* codes = reinterpret_cast<const uint8_t*>(m.codes) + row * (int64_t)(nb * 8) + b0 * 8;
    const uint32_t* sc = reinterpret_cast<const uint32_t*>(m.scales) + row * nb + b0;
    uint32_t w[NBL][2];
    uint32_t dm[NBL];
    if (NBL % 2 == 0 && (nb & 1) == 0) {
      // rows hold an even number of blocks: 16-byte code loads stay in the row
#pragma unroll
      for (int j = 0; j < NBL; j += 2) {
        const uint4 q = *reinterpret_cast<const uint4*>(codes + j * 8);
        w[j][0] = q.x; w[j][1] = q.y; w[j + 1][0] = q.z; w[j + 1][1] = q.w;
        const uint2 d2 = *reinterpret_cast<const uint2*>(sc + j);
        dm[j] = d2.x; dm[j + 1] = d2.y;
      }
    } else {
#pragma unroll
      for (int j = 0; j < NBL; ++j) {
        w[j][0] = w[j][1] = dm[j] = 0u;
        if (b0 + j < nb) {
          const uint2 q = *reinterpret_cast<const uint2*>(codes + j * 8);
          w[j][0] = q.x; w[j][1] = q.y;
          dm[j] = sc[j];
        }
      }
    }
#pragma unroll
    for (int j = 0; j < NBL; ++j) {
      if (b0 + j >= nb) break;
      float p = 0.0f;
#pragma unroll
      for (int h = 0; h < 2; ++h) {
#pragma unroll
        for (int sft = 0; sft < 4; ++sft) {
          // bytes of t hold the codes of values 4*byte + sft (of this dword)
          const uint32_t t = (w[j][h] >> (2 * sft)) & 0x03030303u;
#pragma unroll
          for (int by = 0; by < 4; ++by) {
            const float q = (float)((t >> (8 * by)) & 0xFFu);
            p = fmaf(q, c.v[j][16 * h + 4 * by + sft], p);
          }
        }
      }
      const float d = half_bits_to_float(dm[j] & 0xFFFFu);
      const float mn = half_bits_to_float(dm[j] >> 16);
      acc = fmaf(d, p, acc);
      acc = fmaf(mn, c.sum[j], acc);
    }
  } else {  // Q8_0
    const int8_t* codes = reinterpret_cast<const int8_t*>(m.codes) + row * (int64_t)(nb * 32) + b0 * 32;
    const uint16_t* sc = reinterpret_cast<const uint16_t*>(m.scales) + row * nb + b0;
#pragma unroll
    for (int j = 0; j < NBL; ++j) {
      if (b0 + j >= nb) break;
      const int4* q4 = reinterpret_cast<const int4*>(codes + j * 32);
      const int4 a0 = q4[0], a1 = q4[1];
      const int wd[8] = {a0.x, a0.y, a0.z, a0.w, a1.x, a1.y, a1.z, a1.w};
      float p = 0.0f;
#pragma unroll
      for (int i = 0; i < 32; ++i) p = fmaf((float)(int8_t)(wd[i / 4] >> (8 * (i % 4))), c.v[j][i], p);
      acc = fmaf(half_bits_to_float(sc[j]), p, acc);
    }
  }
  return acc;
}

// h[s, r] = silu(G_e x_t)[r] * (U_e x_t)[r] for every slot s of every active expert.
template <int FMT, int NBL>
__global__ __launch_bounds__(kGemvWaves * kWave) void gemv_gateup_kernel(
    const float* __restrict__ x, int H, int I, int k, QMat gate, QMat up, const int32_t* __restrict__ act,
    const int32_t* __restrict__ n_act, const int32_t* __restrict__ g2l, const int32_t* __restrict__ offsets,
    const int32_t* __restrict__ slot_list, float* __restrict__ h) {
  const int a = blockIdx.y;
  if (a >= *n_act) return;
  const int lane = threadIdx.x % kWave;
  const int r0 = (blockIdx.x * kGemvWaves + threadIdx.x / kWave) * kRowsPerWave;
  if (r0 >= I) return;
  const int g = act[a];
  const int le = g2l ? g2l[g] : g;
  const int nb = H / 32;
  const int s0 = offsets[g], s1 = offsets[g + 1];
  XChunk<NBL> c;
  for (int si = s0; si < s1; ++si) {
    const int slot = slot_list[si];
    load_chunk<NBL>(x + (int64_t)(slot / k) * H, nb, lane, c);
    float res = 0.0f;
#pragma unroll
    for (int rr = 0; rr < kRowsPerWave; ++rr) {
      const int r = r0 + rr;
      if (r >= I) break;
      const int64_t row = (int64_t)le * I + r;
      const float gv = wave_sum(row_dot<FMT, NBL>(gate, row, nb, lane, c));
      const float uv = wave_sum(row_dot<FMT, NBL>(up, row, nb, lane, c));
      if (lane == rr) res = silu(gv) * uv;
    }
    if (lane < kRowsPerWave && r0 + lane < I) h[(int64_t)slot * I + r0 + lane] = res;
  }
}

// y_slot[s, o] = (D_e h_s)[o] for every slot s of every active expert.
template <int FMT, int NBL>
__global__ __launch_bounds__(kGemvWaves * kWave) void gemv_down_kernel(
    const float* __restrict__ h, int H, int I, QMat down, const int32_t* __restrict__ act,
    const int32_t* __restrict__ n_act, const int32_t* __restrict__ g2l, const int32_t* __restrict__ offsets,
    const int32_t* __restrict__ slot_list, float* __restrict__ y) {
  const int a = blockIdx.y;
  if (a >= *n_act) return;
  const int lane = threadIdx.x % kWave;
  const int r0 = (blockIdx.x * kGemvWaves + threadIdx.x / kWave) * kRowsPerWave;
  if (r0 >= H) return;
  const int g = act[a];
  const int le = g2l ? g2l[g] : g;
  const int nb = I / 32;
  const int s0 = offsets[g], s1 = offsets[g + 1];
  XChunk<NBL> c;
  for (int si = s0; si < s1; ++si) {
    const int slot = slot_list[si];
    load_chunk<NBL>(h + (int64_t)slot * I, nb, lane, c);
    float res = 0.0f;
#pragma unroll
    for (int rr = 0; rr < kRowsPerWave; ++rr) {
      const int r = r0 + rr;
      if (r >= H) break;
      const float v = wave_sum(row_dot<FMT, NBL>(down, (int64_t)le * H + r, nb, lane, c));
      if (lane == rr) res = v;
    }
    if (lane < kRowsPerWave && r0 + lane < H) y[(int64_t)slot * H + r0 + lane] = res;
  }
}

static int nbl_for(int cols) {
  const int nb = cols / 32;
  int n = 1;
  while (n * kWave < nb) n <<= 1;
  return n;
}

template <int FMT>
static hipError_t launch_gateup_f(int nbl, dim3 grid, const float* x, int H, int I, int k, const QMat& g,
                                  const QMat& u, const int32_t* act, const int32_t* n_act, const int32_t* g2l,
                                  const int32_t* off, const int32_t* sl, float* h, hipStream_t s) {
  const dim3 blk(kGemvWaves * kWave);
  switch (nbl) {
    case 1: gemv_gateup_kernel<FMT, 1><<<grid, blk, 0, s>>>(x, H, I, k, g, u, act, n_act, g2l, off, sl, h); break;
    case 2: gemv_gateup_kernel<FMT, 2><<<grid, blk, 0, s>>>(x, H, I, k, g, u, act, n_act, g2l, off, sl, h); break;
    case 4: gemv_gateup_kernel<FMT, 4><<<grid, blk, 0, s>>>(x, H, I, k, g, u, act, n_act, g2l, off, sl, h); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <int FMT>
static hipError_t launch_down_f(int nbl, dim3 grid, const float* h, int H, int I, const QMat& d,
                                const int32_t* act, const int32_t* n_act, const int32_t* g2l,
                                const int32_t* off, const int32_t* sl, float* y, hipStream_t s) {
  const dim3 blk(kGemvWaves * kWave);
  switch (nbl) {
    case 1: gemv_down_kernel<FMT, 1><<<grid, blk, 0, s>>>(h, H, I, d, act, n_act, g2l, off, sl, y); break;
    case 2: gemv_down_kernel<FMT, 2><<<grid, blk, 0, s>>>(h, H, I, d, act, n_act, g2l, off, sl, y); break;
    case 4: gemv_down_kernel<FMT, 4><<<grid, blk, 0, s>>>(h, H, I, d, act, n_act, g2l, off, sl, y); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_active(const int32_t* counts, const int32_t* g2l, int E, int E_local, int32_t* act,
                         int32_t* n_act, hipStream_t s) {
  trace_pre("active", s);
  active_experts_kernel<<<1, 1024, 0, s>>>(counts, g2l, E, E_local, act, n_act);
  trace_post("active", s);
  return hipGetLastError();
}

hipError_t launch_gemv_forward(const float* x, int T, int H, int I, int k, const QMat& gate, const QMat& up,
                               int gate_fmt, const QMat& down, int down_fmt, const int32_t* g2l,
                               const int32_t* offsets, const int32_t* slot_list, const int32_t* act,
                               const int32_t* n_act, int max_active, float* h_ws, float* y, hipStream_t s) {
  const int rows_per_block = kGemvWaves * kRowsPerWave;
  dim3 g1((I + rows_per_block - 1) / rows_per_block, max_active);
  hipError_t err;
  trace_pre("gemv_gateup", s);
  if (gate_fmt == FMT_Q2SM)
    err = launch_gateup_f<FMT_Q2SM>(nbl_for(H), g1, x, H, I, k, gate, up, act, n_act, g2l, offsets, slot_list, h_ws, s);
  else
    err = launch_gateup_f<FMT_Q8_0>(nbl_for(H), g1, x, H, I, k, gate, up, act, n_act, g2l, offsets, slot_list, h_ws, s);
  trace_post("gemv_gateup", s);
  if (err != hipSuccess) return err;
  dim3 g2((H + rows_per_block - 1) / rows_per_block, max_active);
  trace_pre("gemv_down", s);
  if (down_fmt == FMT_Q2SM)
    err = launch_down_f<FMT_Q2SM>(nbl_for(I), g2, h_ws, H, I, down, act, n_act, g2l, offsets, slot_list, y, s);
  else
    err = launch_down_f<FMT_Q8_0>(nbl_for(I), g2, h_ws, H, I, down, act, n_act, g2l, offsets, slot_list, y, s);
  trace_post("gemv_down", s);
  return err;
}

}  // namespace moe
