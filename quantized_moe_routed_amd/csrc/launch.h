// Host-side launchers of the gfx950 kernels (internal to libmoe).
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace moe {

struct QMat;

// Optional event tracing of one kernel (see moe_trace_kernel): record an event
// on the stream before and after the launch of kernel `name`.
void trace_pre(const char* name, hipStream_t s);
void trace_post(const char* name, hipStream_t s);

hipError_t launch_route(const void* x, int act, int T, int H, int fmt, const QMat& router, const float* bias,
                        int k, int32_t* ids, float* w, float* z_ws, hipStream_t s);

hipError_t launch_group(const int32_t* ids, int T, int k, int E, int32_t* counts, int32_t* offsets,
                        int32_t* slot_list, hipStream_t s);
size_t group_lds_bytes(int E);
hipError_t group_set_lds_limit(size_t bytes);

hipError_t launch_active(const int32_t* counts, const int32_t* g2l, int E, int E_local, int32_t* act,
                         int32_t* n_act, hipStream_t s);

hipError_t launch_gemv_forward(const float* x, int T, int H, int I, int k, const QMat& gate, const QMat& up,
                               int gate_fmt, const QMat& down, int down_fmt, const int32_t* g2l,
                               const int32_t* offsets, const int32_t* slot_list, const int32_t* act,
                               const int32_t* n_act, int max_active, float* h_ws, float* y, hipStream_t s);

// Grouped MFMA GEMM (bf16 activations).  H and I must be multiples of 64.
int gemm_max_tiles(int T, int k, int E_local);
hipError_t launch_gemm_forward(const uint16_t* x, int T, int H, int I, int k, const QMat& gate, const QMat& up,
                               const QMat& down, const int32_t* g2l, int E, int E_local, const int32_t* counts,
                               const int32_t* offsets, const int32_t* slot_list, float* xs, int4* tiles,
                               int32_t* n_tiles, uint16_t* h_hi, uint16_t* h_lo, float* y, hipStream_t s);

hipError_t launch_combine(const float* y, const float* w, const int32_t* ids, const int32_t* g2l, int T, int k,
                          int H, int E, float* out, hipStream_t s);

}  // namespace moe
