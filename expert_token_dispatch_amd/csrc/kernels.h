// Host-side interface between the C ABI (api.hip) and the kernel files.
// Arguments reaching these launchers have been validated by api.hip.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "moe.h"

namespace moe {

// ---- error and profiling plumbing (defined in api.hip) --------------------
moe_status set_error(moe_status st, const char* fmt, ...);
void prof_before(const char* name, hipStream_t s);
moe_status prof_after(const char* name, hipStream_t s);

#define MOE_LAUNCH(name, kernel, grid, block, lds, stream, ...)                 \
  do {                                                                          \
    ::moe::prof_before(name, stream);                                           \
    hipLaunchKernelGGL(kernel, grid, block, lds, stream, __VA_ARGS__);          \
    const moe_status _moe_st = ::moe::prof_after(name, stream);                 \
    if (_moe_st != MOE_OK) return _moe_st;                                      \
  } while (0)

// ---- sizes ------------------------------------------------------------------
inline size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }
inline size_t dtype_bytes(int32_t dt) { return dt == MOE_BF16 ? 2 : 4; }

// Dispatch works on chunks of kDispatchTokens consecutive tokens (their
// k pairs each): per-chunk expert histograms, per-chunk segment bases.
constexpr int kDispatchThreads = 256;
constexpr int kDispatchTokens = 64;
inline int64_t dispatch_blocks(int64_t num_tokens) { return (num_tokens + kDispatchTokens - 1) / kDispatchTokens; }

// ---- stage launchers --------------------------------------------------------
struct RouteArgs {
  const moe_layer_desc* d;
  const void* x;
  const void* w_router;
  const float* b_router;
  const float* logits_in;
  float* logits_out;
  int32_t* topk_ids;
  float* topk_w;
  float* topk_logit;
  float* partial;       // route scratch: per-slice partial logits
  int32_t* blk_counts;  // optional [dispatch_blocks(T), E]: per-chunk expert histogram for dispatch
  hipStream_t s;
  const float* sel_bias = nullptr;  // optional [E]: added to the logits for choosing experts only
  int group_size = 0;               // experts per group when the groups per token are limited, else 0
  int max_groups = 0;               // groups a token may use (with group_size)
};
size_t route_scratch_bytes(const moe_layer_desc* d);
moe_status launch_route(const RouteArgs& a);
moe_status launch_selection_bias_update(const moe_layer_desc* d, const int32_t* counts, float* bias, float gamma,
                                        hipStream_t s);

// Dispatch scratch, carved from the caller's workspace.
struct DispatchScratch {
  int32_t* blk_all;    // [nblk, E]   per-block counts over all experts
  int32_t* blk_base;   // [nblk, L]   first (pre-capacity) row of each block's pairs
  int32_t* tmp_sorted; // [T*k]       pre-capacity permutation (capacity only)
  uint32_t* tmp_key;   // [T*k]       logit keys beside it (capacity only)
  int32_t* tmp_final;  // [T*k]       final row of each pre-capacity row, -1 if cut (capacity only)
  int32_t* slice_off;  // [L+1]       first capacity slice of each local expert (capacity only)
  int32_t* slice_desc; // [slices, 4] per capacity slice: its expert's first slice, pre-capacity segment
                       //             start and length, and first kept row (capacity only)
  uint32_t* slice_hist; // [slices, 4096] leading-digit histogram of each slice of an expert over
                        //             capacity (capacity only)
};
size_t dispatch_scratch_bytes(const moe_layer_desc* d);
DispatchScratch carve_dispatch_scratch(const moe_layer_desc* d, void* ws);

struct DispatchArgs {
  const moe_layer_desc* d;
  const void* x;
  const int32_t* topk_ids;
  const float* topk_logit;
  int32_t* counts;
  int32_t* offsets;
  int32_t* sorted_pairs;
  int32_t* pair_row;
  void* x_sorted;
  int64_t* num_dropped;
  DispatchScratch scr;
  int64_t capacity;     // -1: none
  bool counts_ready;    // scr.blk_all already holds the per-chunk histograms (written by the router)
  hipStream_t s;
};
moe_status launch_dispatch(const DispatchArgs& a);

struct FfnArgs {
  const moe_layer_desc* d;
  const void* x_sorted;
  const int32_t* offsets;
  const void* w_gate;
  const void* w_up;
  const void* w_down;
  void* y_sorted;
  void* h;         // [P_max, I]
  void* scratch;   // ffn_scratch_bytes: the large-tile path's tile plan and split-K pieces
  int64_t max_pairs;
  hipStream_t s;
  void* g_out = nullptr;  // optional [P_max, I] each: the gate and up pre-activations (training forward)
  void* u_out = nullptr;
};
// Scratch of the large-tile path (tile plan; split-K pieces when K is long), else 0.
size_t ffn_scratch_bytes(const moe_layer_desc* d, int64_t max_pairs);
moe_status launch_grouped_ffn(const FfnArgs& a);
// the kernels launch_grouped_ffn picks from (skinny_gemm.hip, general_gemm.hip)
bool skinny_ffn_fits(const moe_layer_desc* d, int64_t max_pairs);
moe_status launch_skinny_ffn(const FfnArgs& a);
moe_status launch_general_ffn(const FfnArgs& a);

struct CombineArgs {
  const moe_layer_desc* d;
  const void* y_sorted;
  const int32_t* pair_row;
  const float* topk_w;
  void* y;
  hipStream_t s;
};
moe_status launch_combine(const CombineArgs& a);

// ---- backward ----------------------------------------------------------------
struct CombineBwdArgs {
  const moe_layer_desc* d;
  const void* dy;        // [T, H]
  const void* y_sorted;  // [P_max, H]
  const int32_t* pair_row;
  const float* topk_w;
  void* dy_sorted;       // [P_max, H]
  float* dl;             // [T, k]: gradient of the chosen logits
  hipStream_t s;
};
moe_status launch_combine_backward(const CombineBwdArgs& a);

struct FfnBwdArgs {
  const moe_layer_desc* d;
  const void* x_sorted;
  const int32_t* offsets;
  const void* w_gate;
  const void* w_up;
  const void* w_down;
  const void* gate;      // [P_max, I] saved pre-activations
  const void* up;
  const void* h;         // [P_max, I] saved silu(gate) * up
  const void* dy_sorted; // [P_max, H]
  void* dx_sorted;       // [P_max, H]
  void* dw_gate;         // [L, I, H]
  void* dw_up;
  void* dw_down;         // [L, H, I]
  void* scratch;         // ffn_bwd_scratch_bytes
  int64_t max_pairs;
  hipStream_t s;
};
// dg | du [P_max, 2I]; on the large-tile path also the transposed expert
// weights, the tile plan and the split-K pieces.
size_t ffn_bwd_scratch_bytes(const moe_layer_desc* d, int64_t max_pairs);
moe_status launch_grouped_ffn_backward(const FfnBwdArgs& a);
// the large-tile kernel's part of it (grouped_gemm.hip)
bool big_backward_supported(const moe_layer_desc* d, int64_t max_pairs);
size_t big_backward_scratch_bytes(const moe_layer_desc* d);
moe_status launch_big_backward_dgrad(const moe_layer_desc* d, const uint16_t* dy_sorted, const int32_t* offsets,
                                     const uint16_t* w_down, const uint16_t* w_gate, const uint16_t* w_up,
                                     const uint16_t* gate, const uint16_t* up, uint16_t* dgu, uint16_t* dx_sorted,
                                     int64_t max_pairs, void* scratch, hipStream_t s);
// dW_e = A_e^T B_e over each local expert's rows on the large tile, both operands read
// in place (row p of A and B is k = p; rows of lda, ldb elements); Z outputs C0, C1,
// the z-th reading A and B at column offsets z * a_zoff, z * b_zoff.
bool big_wgrad_supported(const moe_layer_desc* d, int64_t max_pairs);
moe_status launch_big_backward_wgrad(const char* name, const moe_layer_desc* d, const int32_t* offsets,
                                     const uint16_t* A, int lda, int a_zoff, const uint16_t* B, int ldb, int b_zoff,
                                     uint16_t* C0, uint16_t* C1, int M, int N, int Z, int64_t max_pairs,
                                     hipStream_t s);

struct RouteBwdScratch {
  void* dlogits;     // [T, Ep] in the layer's type (Ep = E rounded up to 8)
  float* dlogits32;  // [T, Ep] float32 (bias gradient)
  float* part;       // column sums per token chunk
  float* pieces;     // split-K pieces of dW (NULL when one piece)
};
size_t route_bwd_scratch_bytes(const moe_layer_desc* d);
RouteBwdScratch carve_route_bwd_scratch(const moe_layer_desc* d, void* ws);

struct RouteBwdArgs {
  const moe_layer_desc* d;
  const void* x;
  const int32_t* topk_ids;
  const float* dl;
  void* dw_router;   // [E, H]
  float* db_router;  // [E] or NULL
  void* ws;          // route_bwd_scratch_bytes
  hipStream_t s;
};
moe_status launch_route_backward(const RouteBwdArgs& a);

struct DispatchBwdArgs {
  const moe_layer_desc* d;
  const void* dx_sorted;
  const int32_t* pair_row;
  const int32_t* topk_ids;
  const float* dl;
  const void* w_router;
  void* dx;          // [T, H]
  hipStream_t s;
};
moe_status launch_dispatch_backward(const DispatchBwdArgs& a);
// Zero `bytes` (a multiple of 4) at a 16-byte aligned device pointer, by a kernel.
moe_status launch_zero(const char* name, void* p, size_t bytes, hipStream_t s);

}  // namespace moe
