/*
 * moe.h -- C ABI of libmoe.so, the routed-expert mixture-of-experts layer
 * for AMD Instinct MI355X (gfx950).
 *
 * The layer (one DeepSeek-V4-class MoE layer, routed experts only):
 *
 *   z[t,e]  = x[t] . Wr[e] + bias[e]                      router logits
 *   ids[t]  = the k experts with the largest z, ties to the lower expert index
 *   w[t,j]  = sigmoid(z[t,ids[t,j]]) / sum_j' sigmoid(z[t,ids[t,j']])
 *   y[t,j]  = D_e (silu(G_e x[t]) * (U_e x[t])),  e = ids[t,j]
 *   out[t]  = sum_{j = 0..k-1, ids[t,j] owned} w[t,j] * y[t,j]
 *
 * The pages this layer comes from:
 *  - aeonmindai/arc PR #89, "Stage 1 -- EP=2": experts are split into shares,
 *    global ids are remapped to share-local ids through device tables built
 *    once at load, unowned slots are masked, and a share's partial is the sum
 *    over the slots it owns, so the partials over any partition add up to the
 *    full output.  The same section: placements are contiguous, explicit or
 *    LPT-balanced; the expert axis is sliced at load and unsupported formats
 *    are refused by name; a size that disagrees with the placement is an
 *    error, never a silent fallback.
 *  - arc PR #89, "Stage 0": pointers are checked against the device ordinal,
 *    not only the device kind; the per-share load counter is a device-side
 *    array read back outside any captured region.
 *  - TrevorS/ds4 PR #13, "Tested": accumulating the routed down projection
 *    with float atomics makes runs drift; here every reduction has a fixed
 *    order and the library uses no floating-point atomics, so repeated calls
 *    give bit-identical results.
 *  - antirez/ds4 PR #754, "Supported paths and safety": 2-bit routed gate/up
 *    and down projections, Q8_0 dense projections (here: the router, and the
 *    routed down projection of the batched workloads).
 *
 * Conventions for every entry point:
 *  - Device pointers are caller-allocated HIP device memory on the device of
 *    the stream `s` (NULL stream = the current device).  The library
 *    allocates nothing and keeps no pointer after a call returns.
 *  - Calls are asynchronous on `s`; they never synchronise and never copy to
 *    the host, so they may be captured in a HIP graph.  Results are visible
 *    after the stream is synchronised.
 *  - All arguments are checked before anything is launched.  On an error the
 *    call returns a non-zero moe_status, launches nothing, leaves every output
 *    unmodified, and moe_last_error() describes the problem (thread-local).
 *  - T = 0 is a successful no-op.  There are no environment switches and no
 *    fallback paths: every expert runs on the fp16 matrix cores, on tiles of up
 *    to 8 slots (4 where the activation rows of 8 slots would not fit the LDS
 *    of two workgroups per compute unit), or of up to 128 slots for experts with
 *    at least moe_large_tile_min(T) slots.
 *  - Calls that overlap on one stream are ordered; calls sharing a workspace
 *    on different streams race.
 */
#ifndef MOE_H_
#define MOE_H_

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MOE_OK = 0,
  MOE_ERR_ARG = 1,          /* bad size, null pointer, k > E, inconsistent shapes */
  MOE_ERR_UNSUPPORTED = 2,  /* format / size outside what the kernels implement */
  MOE_ERR_DEVICE = 3,       /* a pointer is not device memory of the stream's device */
  MOE_ERR_WORKSPACE = 4,    /* workspace missing or smaller than moe_workspace_size() */
  MOE_ERR_HIP = 5           /* a HIP runtime call failed (launch, attribute query) */
} moe_status;

/* Weight formats.  Blocks of 32 values run along the contraction axis.
 *   MOE_W_F32  : plain fp32.
 *   MOE_W_Q8_0 : 32 int8 codes q and one fp16 scale d; value = d*q.
 *   MOE_W_Q2SM : 32 two-bit codes q in {0..3}, fp16 scale d and fp16 min m;
 *                value = d*q + m.  A stand-in for the pages' 2-bit routed
 *                formats (IQ2_XXS / Q2_K), whose codebooks are not given. */
typedef enum { MOE_W_F32 = 0, MOE_W_Q8_0 = 1, MOE_W_Q2SM = 2 } moe_wfmt;

typedef enum { MOE_ACT_F32 = 0, MOE_ACT_BF16 = 1 } moe_act;

/* A stack of n matrices, each `rows` outputs x `cols` inputs, in the planar
 * device layout written by moe_pack_planar() (sizes from moe_planar_bytes()).
 * nb = cols/32 blocks per row.  A row's codes are cut into 64-byte units so
 * that the lane that owns values 8g..8g+7 of a block (g = 0..3, the K-group of
 * a 16x16x32 matrix-core fragment) reads exactly its codes with one 16-byte
 * load:
 *   Q8_0 : units of 2 blocks; in unit j the 16 bytes at 16g are
 *          {block 2j q[8g..8g+7], block 2j+1 q[8g..8g+7]}.
 *   Q2SM : units of 8 blocks; in unit j the 16 bytes at 16g are 4 words,
 *          word i = {block 8j+2i byte 2g, block 8j+2i+1 byte 2g, block 8j+2i
 *          byte 2g+1, block 8j+2i+1 byte 2g+1}, where byte r of a block holds
 *          its values 4r..4r+3 (2 bits each, value 4r+s at bits 2s..2s+1).
 * Rows are taken in groups of 16 (the last group padded with zero rows); with
 * U = units per row, each matrix is
 *   codes  = [ceil(rows/16)][U][16 rows][64 bytes]: one unit of 16 rows is
 *            1 KiB of consecutive bytes;
 *   scales = Q8_0: [ceil(rows/16)][U][16 rows][2 fp16 d];
 *            Q2SM: [ceil(rows/16)][U] { [16 rows][8 fp16 d], [16 rows][8 fp16 m] }.
 *   F32  : codes = float [n][rows][cols];  scales = NULL.
 * Blocks past nb (padding of a row's last unit) have zero codes and scales.
 * cols must be a multiple of 32. */
typedef struct {
  int32_t fmt;
  int32_t rows;
  int32_t cols;
  const void* codes;
  const void* scales;
} moe_qmat;

/* The experts a caller owns, indexed by LOCAL id 0..n_experts-1.
 * gate, up: rows = I, cols = H.  down: rows = H, cols = I. */
typedef struct {
  moe_qmat gate;
  moe_qmat up;
  moe_qmat down;
  int32_t n_experts;
} moe_experts;

/* Message describing the last error on the calling thread ("" after success). */
const char* moe_last_error(void);

/* Library version string. */
const char* moe_version(void);

/* Bytes of workspace each call needs for the given shapes.  Any output may be
 * NULL.  xt selects the expert kernels (their workspace differs).  */
moe_status moe_workspace_size(int32_t T, int32_t H, int32_t I, int32_t k, int32_t E, int32_t E_local,
                              int32_t xt, size_t* route_ws, size_t* group_ws, size_t* forward_ws);

/* Fewest slots of one expert that moe_expert_forward and moe_layer_forward put
 * on tiles of up to 128 slots in a batch of T tokens; experts with fewer slots
 * take tiles of up to 8.  0 = small tiles only (T <= 32); 33 for 33 <= T < 256
 * (experts of more than 4 small tiles); 12 from 256 tokens.  Host only, no GPU
 * work; the choice changes speed only, never results. */
int32_t moe_large_tile_min(int32_t T);

/* Router scoring and top-k selection (one token per row of x): the routing
 * step of the layer above, which the pages assume rather than write out (the
 * expert-parallel page, "Stage 1 -- EP=2", partitions exactly these routed
 * slots).
 *   x      : [T, H] fp32 or bf16 (xt), row-major.
 *   router : rows = E, cols = H, n = 1; format F32 or Q8_0.
 *   bias   : [E] fp32 added to every logit (used for selection and weights), or NULL.
 *   ids    : [T, k] int32 out, experts by decreasing logit, ties to the lower index.
 *   w      : [T, k] fp32 out, sigmoid scores of the selected experts renormalised to sum 1.
 * Logits are computed in one fixed fp32 order (per 32-block a chain of fused
 * multiply-adds from 0, times the block scale, then a balanced pairwise sum
 * over blocks, then + bias), so ids are reproducible bit for bit and equal to
 * any implementation of that order.  Weights are evaluated in fp64 and rounded.
 * Limits: 1 <= k <= min(E, 32), E <= 1024, H <= 16384.  */
moe_status moe_route(const void* x, int32_t xt, int32_t T, int32_t H, const moe_qmat* router,
                     const float* bias, int32_t k, int32_t* ids, float* w, void* ws, size_t ws_bytes,
                     hipStream_t s);

/* Table (hash) routing: the experts of token t are row token_ids[t] of a fixed
 * [V, k] token-id table, in the row's order, in place of the top k (the
 * expert-parallel page, "Stage 0": the model's first layers route by a fixed
 * token-id table).  The pages give no weight rule for such routes; the
 * reading taken is the learned routes' own: w[t,j] = sigmoid(z) of expert
 * ids[t,j] renormalised over the row, z the logit of moe_route (bias
 * included), in fp64 and rounded.  A table row equal to a token's top k gives
 * moe_route's ids and weights bit for bit.
 *   token_ids : [T] int32 device; values outside 0..V-1 are clamped.
 *   table     : [V, k] int32 device; entries must lie in 0..E-1 and be
 *               distinct within a row (check once on the host with
 *               moe_table_check); entries outside are clamped, so no read
 *               leaves the arrays.
 * Other arguments, workspace and limits as moe_route. */
moe_status moe_route_table(const void* x, int32_t xt, int32_t T, int32_t H, const moe_qmat* router,
                           const float* bias, const int32_t* token_ids, const int32_t* table, int32_t V,
                           int32_t k, int32_t* ids, float* w, void* ws, size_t ws_bytes, hipStream_t s);

/* Shared expert beside the routed sum: out[t] += D(silu(G x_t) * U x_t) for
 * every token, one fp32 addition per element after the expert's own result
 * (the pages name a Q8_0 shared expert next to the routed ones but give no
 * shapes; any format and intermediate size the expert calls take are
 * accepted).  shared holds exactly one expert (gate/up I x H, down H x I);
 * out [T, H] fp32 is read and written (call after moe_combine or
 * moe_layer_forward to add the shared expert to the routed output).  The
 * expert runs on the same kernels as the routed ones, every token a slot of
 * the one expert.  Workspace: moe_shared_expert_workspace. */
moe_status moe_shared_expert_workspace(int32_t T, int32_t H, int32_t I, int32_t xt, size_t* ws_bytes);
moe_status moe_shared_expert_forward(const void* x, int32_t xt, int32_t T, int32_t H, int32_t I,
                                     const moe_experts* shared, float* out, void* ws, size_t ws_bytes,
                                     hipStream_t s);

/* Host check of a routing table [V, k] (host memory): every entry in 0..E-1,
 * no expert twice in a row.  MOE_ERR_ARG names the first offending entry. */
moe_status moe_table_check(const int32_t* table, int32_t V, int32_t k, int32_t E);

/* Group the T*k routing slots (slot s = t*k + j) by expert: per-expert token
 * lists and loads, the quantities the expert-parallel page weighs ("Stage 0":
 * tokens are compute, distinct experts are bytes; the load counter is a device
 * array read outside captured work).
 *   counts    : [E] int32 out, slots routed to each expert (the per-expert token
 *               load; the number of non-zero entries is the count of distinct
 *               experts the batch touches).
 *   offsets   : [E+1] int32 out, exclusive prefix sum of counts.
 *   slot_list : [T*k] int32 out, slots of expert e at offsets[e]..offsets[e+1]-1,
 *               in ascending slot order (a stable sort; bit-reproducible).
 * ids outside [0, E) are left out of the grouping.  Limits: E <= 1024. */
moe_status moe_group_tokens(const int32_t* ids, int32_t T, int32_t k, int32_t E, int32_t* counts,
                            int32_t* offsets, int32_t* slot_list, void* ws, size_t ws_bytes,
                            hipStream_t s);

/* The owned experts' FFN for every routed slot they own.
 *   x       : [T, H] fp32 or bf16 (xt), the same tensor given to moe_route.
 *   local   : the owned expert stack, local-indexed (gate/up Q8_0 or Q2SM,
 *             down Q8_0 or Q2SM; F32 expert weights are not supported).
 *   g2l     : [E] int32 device table, global id -> local id, -1 = unowned (the
 *             owned-expert mask); NULL = every expert owned with local = global.
 *   counts, offsets, slot_list : from moe_group_tokens.
 *   y_slot  : [T*k, H] fp32 out; row s = D_e(silu(G_e x) * U_e x) for owned
 *             slots, rows of unowned slots are left untouched.
 * E_local must equal local->n_experts; the table's consistency is checked once
 * on the host with moe_plan_check().  Every product runs on the fp16 matrix
 * cores: weight codes enter them as exact small integers, block scales are
 * applied in fp32 per 32-block.  The activations enter as an fp16 hi + lo
 * pair (fp32 x) or one fp16 plane (bf16 x), and the intermediate silu(g)*u
 * as an fp16 hi + lo pair, each row of either scaled by the power of two that
 * brings its largest magnitude to [2^14, 2^15) (single-token batches: each
 * 32-value block of silu(g)*u by its own): a value within 2^18 of its row's
 * (block's) largest keeps 22 significant bits, smaller ones an absolute error
 * below 2^-39 of that largest, and any finite input is in range.  No path
 * uses floating-point atomics; results do not depend on scheduling.
 * From 256 tokens, when some expert takes large tiles, the launches of the
 * small tiles run on a second stream of the device, created by the library on
 * the device's first such call (not while s is being captured) and held until
 * the process ends; they are forked from s and joined back into s with events,
 * so the call stays ordered on s as a whole, and a graph captured from s holds
 * both branches.  The calls on one device share that stream.
 * Limits: H and I multiples of 32, H <= 8192, I <= 8192. */
moe_status moe_expert_forward(const void* x, int32_t xt, int32_t T, int32_t H, int32_t I, int32_t k,
                              const moe_experts* local, const int32_t* g2l, int32_t E, int32_t E_local,
                              const int32_t* counts, const int32_t* offsets, const int32_t* slot_list,
                              float* y_slot, void* ws, size_t ws_bytes, hipStream_t s);

/* Weighted combine (the expert-parallel page, "Stage 1 -- EP=2": a share's
 * partial is the sum over the slots it owns; TrevorS/ds4 PR #13, "Tested": no
 * float atomics, so runs are bit-identical):
 * out[t] = sum over j = 0..k-1 in that order, of owned slots,
 * of w[t,j] * y_slot[t*k+j], starting from +0.0, in fp32, with no atomics.
 * g2l NULL = every slot owned.  out: [T, H] fp32. */
moe_status moe_combine(const float* y_slot, const float* w, const int32_t* ids, const int32_t* g2l,
                       int32_t T, int32_t k, int32_t H, int32_t E, float* out, hipStream_t s);

/* The whole layer in one call: moe_route, moe_group_tokens, moe_expert_forward
 * and moe_combine in turn on stream s, with their arguments and outputs (ids,
 * w, counts, offsets, slot_list, y_slot, out) and the same results bit for bit;
 * router->rows must equal E.  For batches of up to 8 tokens the logits launch
 * also prepares the activation operand, and the gate/up launch itself takes
 * the top-k, groups the slots and numbers the tiles (more than 256 experts:
 * one launch between the two does so).
 *   ws : route_ws + forward_ws bytes from moe_workspace_size, the router's part
 *        first (route_ws is a multiple of 256), 16-byte aligned.
 * All arguments are checked before the first launch; errors as for the four
 * calls. */
moe_status moe_layer_forward(const void* x, int32_t xt, int32_t T, int32_t H, int32_t I, int32_t k,
                             const moe_qmat* router, const float* bias, const moe_experts* local,
                             const int32_t* g2l, int32_t E, int32_t E_local, int32_t* ids, float* w,
                             int32_t* counts, int32_t* offsets, int32_t* slot_list, float* y_slot,
                             float* out, void* ws, size_t ws_bytes, hipStream_t s);

/* The whole layer as moe_layer_forward, with the same arguments and results
 * bit for bit, but without a workspace argument: for callers that cannot
 * allocate device memory (code being captured into a HIP graph, tight serving
 * loops, harnesses that forbid allocation).  The workspace is a 32 MiB array
 * the library holds on each device from the moment it is loaded there until
 * the process ends; this call allocates nothing (it forks onto the second
 * stream of large batches, see moe_expert_forward, only where an earlier call
 * created that stream, and otherwise runs on s alone).  Every call on a device uses
 * that device's one array, so calls that overlap on one device (on different
 * streams, or from different threads) race; the array keeps the last call's
 * contents, none of which a later call reads before writing it.  A batch whose
 * workspace (moe_workspace_size: route_ws + forward_ws) exceeds 32 MiB is
 * refused with MOE_ERR_UNSUPPORTED (at H = 4096, I = 2048, E = 256, k = 8: up
 * to 128 tokens fit).  Errors as for moe_layer_forward. */
moe_status moe_layer_forward_noalloc(const void* x, int32_t xt, int32_t T, int32_t H, int32_t I, int32_t k,
                                     const moe_qmat* router, const float* bias, const moe_experts* local,
                                     const int32_t* g2l, int32_t E, int32_t E_local, int32_t* ids, float* w,
                                     int32_t* counts, int32_t* offsets, int32_t* slot_list, float* y_slot,
                                     float* out, hipStream_t s);

/* ---- profiling ------------------------------------------------------------ */

/* Record HIP events around launches of one kernel, for live per-kernel timing.
 * While set (on the calling thread), the i-th launch of the kernel called
 * `name` gets hipEventRecord(start[i]) before and hipEventRecord(stop[i])
 * after it on the call's stream, for i < n; *count holds how many launches
 * were recorded.  The expert kernels (ffn_*) instead hand start[i] and stop[i]
 * to the launch itself (hipExtLaunchKernel), so that they hold the kernel's
 * own start and end, the interval a profiler reports.  Kernel names:
 * route_logits, route_topk, route_table, group, prep, front (selection to operands in one
 * launch, small batches), ffn_gateup, ffn_down (small tiles),
 * ffn_gateup_large, ffn_down_large, combine, add_shared.  The caller owns
 * the events and must keep them, and count, alive while tracing; n <= 0
 * switches tracing off. */
moe_status moe_trace_kernel(const char* name, hipEvent_t* start, hipEvent_t* stop, int32_t n, int32_t* count);

/* As moe_trace_kernel, recording only launches 0, every, 2 every, ... of the
 * kernel (every >= 1), so that the events disturb few of the traced steps. */
moe_status moe_trace_kernel_every(const char* name, hipEvent_t* start, hipEvent_t* stop, int32_t n,
                                  int32_t every, int32_t* count);

/* ---- host helpers (no device access) ---------------------------------- */

/* Sizes of the planar code and scale planes for one rows x cols matrix. */
moe_status moe_planar_bytes(int32_t fmt, int32_t rows, int32_t cols, size_t* codes_bytes,
                            size_t* scales_bytes);

/* Re-lay n matrices from the definition layout (array of blocks: Q8_0
 * {fp16 d; int8 q[32]}, Q2SM {fp16 d; fp16 m; uint8 qs[8]}, F32 plain rows)
 * into the planar layout above.  Host memory in and out; a byte permutation of
 * the definition bytes plus zero padding. */
moe_status moe_pack_planar(int32_t fmt, int32_t n, int32_t rows, int32_t cols, const void* aos,
                           void* codes, void* scales);

/* LPT-balanced placement of E experts onto n_shares shares of E/n_shares
 * experts each (arc PR #89, "Stage 1"): experts by load descending (ties to
 * the lower id), each to the least-loaded share with room (ties to the lower
 * share).  owner: [E] out. */
moe_status moe_place_lpt(const int64_t* load, int32_t E, int32_t n_shares, int32_t* owner);

/* Tables of one share: g2l [E] (-1 = unowned) and l2g [E] (first *E_local
 * entries used).  Local ids ascend with global id, or with local_order[e]
 * when local_order is not NULL (a permuted placement). */
moe_status moe_share_tables(const int32_t* owner, int32_t E, int32_t share, const int32_t* local_order,
                            int32_t* g2l, int32_t* l2g, int32_t* E_local);

/* Check a global->local table once at load: every entry is -1 or a local id,
 * the owned ids are a bijection onto 0..E_local-1. */
moe_status moe_plan_check(const int32_t* g2l, int32_t E, int32_t E_local);

#ifdef __cplusplus
}
#endif

#endif /* MOE_H_ */
