/*
 * moe.h -- C ABI of libmoe: the forward pass of one mixture-of-experts layer
 * on one GPU's share of the experts, for AMD Instinct MI355X (gfx950).
 *
 * The layer follows the four steps named on the Ultralytics glossary page
 * "Expert Parallelism", section "How tokens move between GPUs": route every
 * token to its k best experts, dispatch each (token, expert) pair to the
 * expert, run the experts, and combine the results weighted by the router
 * scores.  The Hugging Face Transformers page "Expert parallelism", section
 * "Token dispatch", fixes what one rank does with its share: it runs only
 * its local experts on the pairs routed to them, and the router yields
 * global expert ids so that the owner of every expert can be found.  The
 * collectives that move pairs between GPUs are outside this library: the
 * calls below are the single-GPU core (permute -> compute -> un-permute).
 *
 * Conventions shared by every call
 * --------------------------------
 *  - Pointers marked "device" are GPU memory on the current HIP device;
 *    "host" pointers are CPU memory.  The caller owns every buffer; the
 *    library allocates no memory and keeps no state between calls apart from
 *    a thread-local error message, the optional profiling events and the
 *    static device buffer of moe_dispatch_noalloc.
 *  - Tensors are dense and row-major.  Device pointers to activations,
 *    weights and outputs must be 16-byte aligned; index arrays 4-byte aligned.
 *  - Activations and weights share one element type, desc->dtype: MOE_BF16
 *    (bfloat16 storage, float32 accumulation) or MOE_F32.  Router bias,
 *    logits and routing weights are always float32; ids and rows int32.
 *  - The router weight is stored as a linear layer stores it, [out, in]:
 *    w_router [E, H].  The expert weights are stacked along the expert
 *    dimension (Transformers "Expert parallelism": the grouped_gemm style
 *    splits them along that dimension) in one of two layouts, chosen by
 *    desc->weight_layout:
 *      MOE_WEIGHTS_OUT_IN (0)  w_gate, w_up [L, I, H], w_down [L, H, I]
 *                              (each matrix [out, in], as a linear layer
 *                              stores it): y = (silu(v Wg^T) * (v Wu^T)) Wd^T
 *      MOE_WEIGHTS_IN_OUT (1)  w_gate, w_up [L, H, I], w_down [L, I, H]
 *                              (the math form):  y = (silu(v Wg) * (v Wu)) Wd
 *    Both describe the same layer; the weight gradients of the backward take
 *    the layout of the weights.
 *  - Work is enqueued on `stream` (a hipStream_t; NULL = the null stream)
 *    and runs asynchronously; no call synchronises or copies device data to
 *    the host.  Device-side data produced by an earlier call (ids, offsets,
 *    rows) is trusted.
 *  - Every argument is validated on the host before anything is enqueued; a
 *    non-OK status means nothing was enqueued, except MOE_ERR_HIP, which
 *    reports a failed launch.  moe_last_error() describes the failure.
 *  - Calls on one stream may share a workspace; concurrent calls need
 *    distinct workspaces.
 */
#ifndef MOE_H_
#define MOE_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MOE_OK = 0,
  MOE_ERR_INVALID_ARG = -1, /* a size, range or pointer is not acceptable */
  MOE_ERR_UNSUPPORTED = -2, /* a valid request the library does not handle */
  MOE_ERR_WORKSPACE = -3,   /* workspace missing or smaller than required */
  MOE_ERR_HIP = -4          /* the HIP runtime reported an error          */
} moe_status;

typedef enum { MOE_F32 = 0, MOE_BF16 = 1 } moe_dtype;

/* Layout of the stacked expert weights (see the conventions above). */
typedef enum { MOE_WEIGHTS_OUT_IN = 0, MOE_WEIGHTS_IN_OUT = 1 } moe_weight_layout;

/* Problem statement of one layer on one GPU.
 *   num_tokens       T >= 0 tokens held by this GPU (T == 0: every call is a
 *                    successful no-op).
 *   hidden           H > 0, multiple of 8.
 *   intermediate     I > 0, multiple of 8 (expert FFN width).
 *   num_experts      E >= 1 experts in the whole layer (global ids 0..E-1).
 *   top_k            1 <= k <= E experts per token.
 *   local_begin,     this GPU holds experts [local_begin, local_begin +
 *   local_count      local_count), 1 <= local_count, local_begin >= 0,
 *                    local_begin + local_count <= E.
 *   capacity_factor  <= 0: no limit.  > 0: each local expert keeps at most
 *                    C = floor(capacity_factor * T * k / E) pairs (the even
 *                    share T*k/E scaled, glossary section "Load balancing and
 *                    capacity"); the pairs with the largest router logit are
 *                    kept, ties to the lower token index.
 *   dtype            a moe_dtype value.
 *   weight_layout    a moe_weight_layout value (0, the zero-initialised
 *                    default, is MOE_WEIGHTS_OUT_IN).
 */
typedef struct {
  int64_t num_tokens;
  int32_t hidden;
  int32_t intermediate;
  int32_t num_experts;
  int32_t top_k;
  int32_t local_begin;
  int32_t local_count;
  float capacity_factor;
  int32_t dtype;
  int32_t weight_layout;
} moe_layer_desc;

/* Stages whose workspace size can be queried. */
typedef enum {
  MOE_STAGE_ROUTE = 0,
  MOE_STAGE_DISPATCH = 1,
  MOE_STAGE_FFN = 2,
  MOE_STAGE_COMBINE = 3,
  MOE_STAGE_LAYER = 4, /* moe_layer_forward: all intermediates of the layer */
  MOE_STAGE_FFN_BACKWARD = 5,   /* moe_grouped_ffn_backward: dg, du [P_max, I] each */
  MOE_STAGE_ROUTE_BACKWARD = 6, /* moe_route_backward: the logit gradients [T, E] */
  MOE_STAGE_LAYER_BACKWARD = 7  /* moe_layer_backward: all backward intermediates */
} moe_stage;

/* ------------------------------------------------------------------------ */
/* Host helpers (no GPU work)                                                */
/* ------------------------------------------------------------------------ */

/* Message for the last non-OK status returned on this thread ("" if none). */
const char* moe_last_error(void);

/* Library version string. */
const char* moe_version(void);

/* Experts held by `rank` when ep_size ranks split E experts.  Transformers
 * "Expert parallelism", section "How the sizes combine": ep_size splits the
 * expert list into ep_size contiguous blocks and ep_size consecutive ranks
 * hold one full set, so rank r holds block (r mod ep_size).
 *   begin, count: host outputs.  INVALID_ARG unless E >= 1, ep_size >= 1,
 *   ep_size divides E and rank >= 0. */
moe_status moe_ep_local_range(int32_t num_experts, int32_t ep_size, int32_t rank,
                              int32_t* begin, int32_t* count);

/* Per-expert capacity C (see moe_layer_desc), or -1 when there is no limit.
 * Returns -1 for an invalid descriptor too (moe_last_error says why). */
int64_t moe_capacity(const moe_layer_desc* d);

/* Rows that the permuted buffers (sorted_pairs, x_sorted, y_sorted) must
 * hold: P_max = T*k without capacity, min(T*k, local_count*C) with it. */
int64_t moe_max_pairs(const moe_layer_desc* d);

/* Workspace bytes the given stage needs (0 is a valid answer). */
moe_status moe_workspace_size(const moe_layer_desc* d, int32_t stage, size_t* bytes);

/* Optional kernel timing, for benchmarks.  While set (events != NULL), every
 * library call on this thread records events[2i] on its stream just before
 * its i-th kernel launch and events[2i+1] just after it, for i < count/2.
 * events are hipEvent_t handles created by the caller; a NULL pair skips
 * kernel i (give both of a pair or neither).  count must be even and at most
 * 64.  count == 0 or events == NULL switches timing off. */
moe_status moe_profile_events(void* const* events, int32_t count);

/* Name of the i-th kernel launched by the last library call on this thread,
 * or NULL if there was none. */
const char* moe_profile_kernel_name(int32_t i);

/* Number of kernels launched by the last library call on this thread. */
int32_t moe_profile_kernel_count(void);

/* ------------------------------------------------------------------------ */
/* Stage 1: route.  Glossary, "How tokens move between GPUs", step 1: score  */
/* every token against every expert with a linear router and keep the k     */
/* best.  Ties go to the lower expert id; slot j holds the j-th best.  The  */
/* routing weights are a softmax over the k chosen logits.  Ids are global  */
/* (Transformers, "Expert parallelism": dispatch needs global expert ids).  */
/* ------------------------------------------------------------------------ */
/*   x           device [T, H] dtype      hidden states
 *   w_router    device [E, H] dtype      router weight
 *   b_router    device [E] float32 or NULL
 *   logits_in   device [T, E] float32 or NULL: if given, x/w_router/b_router
 *               are ignored and top-k runs on these logits
 *   logits_out  device [T, E] float32 or NULL: the logits routed on
 *   topk_ids    device [T, k] int32      global expert ids, best first
 *   topk_w      device [T, k] float32    softmax over the k chosen logits
 *   topk_logit  device [T, k] float32 or NULL: the chosen logits (needed by
 *               moe_dispatch when capacity_factor > 0)
 *   ws          device workspace of MOE_STAGE_ROUTE bytes (partial logits of
 *               the H slices); not used, and may be NULL, when logits_in is given */
moe_status moe_route(const moe_layer_desc* d, const void* x, const void* w_router,
                     const float* b_router, const float* logits_in, float* logits_out,
                     int32_t* topk_ids, float* topk_w, float* topk_logit,
                     void* ws, size_t ws_bytes, void* stream);

/* Routing options.  Ultralytics glossary "Expert Parallelism", section "Load
 * balancing and capacity":
 *  - bias-based balancing: a per-expert bias is added to the router scores
 *    for choosing experts only.  Here experts are chosen by logit + bias (a
 *    float32 sum), in that order, ties to the lower id; topk_logit, the
 *    weights (softmax over the k chosen) and the capacity ranking use the
 *    logits without the bias.
 *  - node-limited routing: each token's experts lie on at most a few nodes.
 *    Here the E experts form num_groups contiguous groups of E/num_groups;
 *    a group scores its best expert's selection score, a token keeps the
 *    max_groups best groups (equal scores to the lower group) and takes its
 *    k experts from them.
 * selection_bias: [E] float32 on the device, or NULL for none.
 * num_groups: 0 or 1 for no limit, else 2..16 dividing E; max_groups: 1..num_groups,
 * with max_groups * (E / num_groups) >= top_k.  Options are read at the call. */
typedef struct moe_route_opts {
  const float* selection_bias;
  int32_t num_groups;
  int32_t max_groups;
} moe_route_opts;

/* moe_route with options (NULL opts: same as moe_route).  Errors as moe_route,
 * plus MOE_ERR_INVALID_ARG for group settings outside the ranges above. */
moe_status moe_route_ex(const moe_layer_desc* d, const moe_route_opts* opts, const void* x, const void* w_router,
                        const float* b_router, const float* logits_in, float* logits_out,
                        int32_t* topk_ids, float* topk_w, float* topk_logit,
                        void* ws, size_t ws_bytes, void* stream);

/* One balancing step on the selection bias from a batch's expert loads (same
 * section: after each step the bias goes down for overloaded experts and up
 * for idle ones).  counts: [E] int32 device (moe_dispatch's counts, or
 * moe_layer_forward's counts_out); bias: [E] float32 device, updated in
 * place: bias[e] -= gamma where counts[e] * E > sum(counts), += gamma where
 * counts[e] * E < sum(counts), unchanged at the mean.  One kernel on stream,
 * no workspace.  MOE_ERR_INVALID_ARG for NULL pointers or a non-finite gamma. */
moe_status moe_selection_bias_update(const moe_layer_desc* d, const int32_t* counts, float* bias, float gamma,
                                     void* stream);

/* ------------------------------------------------------------------------ */
/* Stage 2: dispatch.  Transformers, "Token dispatch": every (token, expert) */
/* pair goes to the owner of its expert.  On one GPU this is a histogram of  */
/* pairs per expert (the glossary snippet's bincount), an exclusive scan    */
/* into per-expert segment offsets, an optional capacity cut, and a stable  */
/* permutation that gathers the token rows into expert-sorted order.       */
/* Pair p = t*k + j.  Within a segment pairs appear in ascending p.          */
/* ------------------------------------------------------------------------ */
/*   x             device [T, H] dtype
 *   topk_ids      device [T, k] int32 (from moe_route)
 *   topk_logit    device [T, k] float32; required iff capacity_factor > 0
 *   counts        device [E] int32 out: pairs routed to each expert, all E,
 *                 before any capacity cut
 *   offsets       device [L+1] int32 out: local segment i is rows
 *                 [offsets[i], offsets[i+1]); offsets[L] = P kept pairs
 *   sorted_pairs  device [P_max] int32 out: pair id at each sorted row
 *                 (rows >= P are left untouched)
 *   pair_row      device [T*k] int32 out: sorted row of each pair, -1 if its
 *                 expert is not local or the pair was dropped
 *   x_sorted      device [P_max, H] dtype out: row q = x[sorted_pairs[q] / k]
 *   num_dropped   device int64 out (may be NULL): pairs cut by capacity
 *   ws            device workspace of MOE_STAGE_DISPATCH bytes */
moe_status moe_dispatch(const moe_layer_desc* d, const void* x, const int32_t* topk_ids,
                        const float* topk_logit, int32_t* counts, int32_t* offsets,
                        int32_t* sorted_pairs, int32_t* pair_row, void* x_sorted,
                        int64_t* num_dropped, void* ws, size_t ws_bytes, void* stream);

/* moe_dispatch for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc):
 * the same kernels and outputs as moe_dispatch, bit for bit, but the
 * dispatch scratch (per-chunk expert histograms, per-chunk segment bases,
 * the pre-capacity permutation and its slice tables) lives in a static
 * 16 MiB device buffer of the library instead of a caller workspace.  Each
 * GPU the library runs on holds its own buffer until the process ends; its
 * address is resolved on the first call on each device.  The call allocates
 * nothing.
 * Arguments as moe_dispatch, without ws / ws_bytes.  Every call on one GPU
 * shares that GPU's buffer: calls that overlap in time on one GPU (other
 * streams, other host threads) race and must be serialised by the caller.
 * Each call writes every scratch entry it reads, so nothing carries over
 * from the previous call.  MOE_ERR_UNSUPPORTED (nothing enqueued) when the
 * layer needs more scratch than the buffer holds (the MOE_STAGE_DISPATCH
 * size, moe_workspace_size, above 16 MiB: roughly T * (E + L) / 16 bytes,
 * plus 16 T k + 16 KiB * L with a capacity factor); other errors as
 * moe_dispatch. */
moe_status moe_dispatch_noalloc(const moe_layer_desc* d, const void* x, const int32_t* topk_ids,
                                const float* topk_logit, int32_t* counts, int32_t* offsets,
                                int32_t* sorted_pairs, int32_t* pair_row, void* x_sorted,
                                int64_t* num_dropped, void* stream);

/* ------------------------------------------------------------------------ */
/* Stage 3: local experts as one grouped GEMM.  Glossary, step 3: each GPU  */
/* runs its local experts on the tokens it received; Transformers names the */
/* expert kernel style "grouped_gemm".  Segment i of x_sorted goes through  */
/* expert local_begin + i:  y = (silu(x Wg) * (x Wu)) Wd (in the math     */
/* form; see the weight layouts above), with                               */
/* silu(z) = z / (1 + exp(-z)), float32 accumulation, the gate/up product   */
/* rounded to dtype once.  Offsets are read on the device (no host sync).   */
/* ------------------------------------------------------------------------ */
/*   x_sorted  device [P_max, H] dtype
 *   offsets   device [L+1] int32 (from moe_dispatch)
 *   w_gate, w_up  device dtype, [L, I, H] (MOE_WEIGHTS_OUT_IN) or [L, H, I]
 *                 (MOE_WEIGHTS_IN_OUT);  w_down [L, H, I] or [L, I, H]
 *   y_sorted  device [P_max, H] dtype out (rows >= P untouched)
 *   ws        device workspace of MOE_STAGE_FFN bytes: h [P_max, I], and on
 *             the large-tile path its tile plan and (K >= 2048) the float32
 *             K pieces of tiles in each XCD's last, partly filled round */
moe_status moe_grouped_ffn(const moe_layer_desc* d, const void* x_sorted, const int32_t* offsets,
                           const void* w_gate, const void* w_up, const void* w_down,
                           void* y_sorted, void* ws, size_t ws_bytes, void* stream);

/* ------------------------------------------------------------------------ */
/* Stage 4: combine.  Glossary, step 4: results return to their token and   */
/* are weighted by the router scores and summed.  y[t] = sum over slots j   */
/* in order 0..k-1 with pair_row[t*k+j] >= 0 of topk_w[t,j] *              */
/* y_sorted[pair_row[t*k+j]], accumulated in float32 and rounded once; a    */
/* token with no kept local pair gets 0.  The residual branch is not added. */
/* ------------------------------------------------------------------------ */
/*   y_sorted  device [P_max, H] dtype;  pair_row device [T*k] int32
 *   topk_w    device [T, k] float32;    y device [T, H] dtype out */
moe_status moe_combine(const moe_layer_desc* d, const void* y_sorted, const int32_t* pair_row,
                       const float* topk_w, void* y, void* stream);

/* ------------------------------------------------------------------------ */
/* All four stages in one call.  The intermediates live in ws (size from    */
/* MOE_STAGE_LAYER); the optional outputs (NULL to skip) receive copies:    */
/*   topk_ids_out [T,k] int32, topk_w_out [T,k] float32, counts_out [E]      */
/*   int32, num_dropped_out int64 -- all device pointers.                    */
/* ------------------------------------------------------------------------ */
moe_status moe_layer_forward(const moe_layer_desc* d, const void* x, const void* w_router,
                             const float* b_router, const void* w_gate, const void* w_up,
                             const void* w_down, void* y, int32_t* topk_ids_out,
                             float* topk_w_out, int32_t* counts_out, int64_t* num_dropped_out,
                             void* ws, size_t ws_bytes, void* stream);

/* moe_layer_forward with routing options (see moe_route_opts); NULL opts is
 * moe_layer_forward.  The same workspace. */
moe_status moe_layer_forward_ex(const moe_layer_desc* d, const moe_route_opts* opts, const void* x,
                                const void* w_router, const float* b_router, const void* w_gate, const void* w_up,
                                const void* w_down, void* y, int32_t* topk_ids_out, float* topk_w_out,
                                int32_t* counts_out, int64_t* num_dropped_out, void* ws, size_t ws_bytes,
                                void* stream);

/* ======================================================================== */
/* Training: the backward pass.                                              */
/*                                                                           */
/* Transformers "Expert parallelism", section "Token dispatch": every rank   */
/* trains on its own share of the batch, and an expert's weight gradient is  */
/* the sum over the pairs that reached it; an expert that received no       */
/* tokens still takes part (its gradient is zero).  The gradients are the   */
/* chain rule through the forward above, given dy = dLoss/dy for the layer   */
/* output y (no residual).  Which experts a token uses (top-k, selection     */
/* bias, group limit, capacity) is a discrete choice and carries no          */
/* gradient; the router receives it through the softmax over the k chosen   */
/* logits (all k slots take part; a slot with no kept local pair has a zero  */
/* weight gradient).  Rounding: every stored gradient is accumulated in      */
/* float32 and rounded to dtype once; dl and db are float32.                 */
/* ======================================================================== */

/* What the training forward keeps for the backward (all device, caller-owned).
 * The index arrays and rows are the forward's own (see moe_route,
 * moe_dispatch, moe_grouped_ffn). */
typedef struct moe_saved {
  int32_t* topk_ids;  /* [T, k] int32 global expert ids */
  float* topk_w;      /* [T, k] float32 routing weights */
  int32_t* offsets;   /* [L+1] int32 segment offsets */
  int32_t* pair_row;  /* [T*k] int32 sorted row of each pair, -1 = not local or dropped */
  void* x_sorted;     /* [P_max, H] dtype */
  void* gate;         /* [P_max, I] dtype: x_sorted Wg^T (rounded once) */
  void* up;           /* [P_max, I] dtype: x_sorted Wu^T */
  void* h;            /* [P_max, I] dtype: silu(gate) * up from the float32 products */
  void* y_sorted;     /* [P_max, H] dtype */
} moe_saved;

/* moe_grouped_ffn that also keeps the gate and up pre-activations (and h in
 * the caller's buffer instead of the workspace).  y_sorted and h are the
 * values moe_grouped_ffn produces (the same kernels, with the extra stores).
 *   h, gate, up  device [P_max, I] dtype out
 *   ws           device workspace of MOE_STAGE_FFN bytes */
moe_status moe_grouped_ffn_train(const moe_layer_desc* d, const void* x_sorted, const int32_t* offsets,
                                 const void* w_gate, const void* w_up, const void* w_down, void* y_sorted,
                                 void* h, void* gate, void* up, void* ws, size_t ws_bytes, void* stream);

/* moe_layer_forward_ex that writes every intermediate the backward needs
 * into `saved` (all nine pointers required).  counts_out and
 * num_dropped_out are optional.  Workspace: MOE_STAGE_LAYER bytes. */
moe_status moe_layer_forward_train(const moe_layer_desc* d, const moe_route_opts* opts, const void* x,
                                   const void* w_router, const float* b_router, const void* w_gate,
                                   const void* w_up, const void* w_down, void* y, const moe_saved* saved,
                                   int32_t* counts_out, int64_t* num_dropped_out, void* ws, size_t ws_bytes,
                                   void* stream);

/* Combine backward with the softmax over k.  For each kept local pair
 * (t, j) at row q: dy_sorted[q] = topk_w[t,j] * dy[t] (rounded once), and
 * dw[t,j] = <dy[t], y_sorted[q]> (float32; 0 for slots without a row); then
 * dl[t,j] = topk_w[t,j] * (dw[t,j] - sum_i topk_w[t,i] dw[t,i]).
 *   dy         device [T, H] dtype;  y_sorted device [P_max, H] dtype
 *   pair_row   device [T*k] int32;   topk_w device [T, k] float32
 *   dy_sorted  device [P_max, H] dtype out (rows >= P untouched)
 *   dl         device [T, k] float32 out: gradient of the chosen logits */
moe_status moe_combine_backward(const moe_layer_desc* d, const void* dy, const void* y_sorted,
                                const int32_t* pair_row, const float* topk_w, void* dy_sorted, float* dl,
                                void* stream);

/* The local experts' backward.  Per expert e with rows [o_e, o_{e+1}), with
 * the weights in the math form (MOE_WEIGHTS_IN_OUT; the other layout stores
 * the transposes):
 *   dh = dy_sorted Wd_e^T;  dg = dh * up * silu'(gate);  du = dh * silu(gate)
 *   dx_sorted = dg Wg_e^T + du Wu_e^T
 *   dWd_e = h^T dy_sorted,  dWg_e = x_sorted^T dg,  dWu_e = x_sorted^T du
 * summed over the expert's rows (an empty expert gets zeros).
 *   gate, up, h          device [P_max, I] dtype (from moe_grouped_ffn_train)
 *   dy_sorted            device [P_max, H] dtype (from moe_combine_backward)
 *   dx_sorted            device [P_max, H] dtype out
 *   dw_gate, dw_up, dw_down  device dtype out, in the layout of w_gate, w_up, w_down
 *   ws                   device workspace of MOE_STAGE_FFN_BACKWARD bytes */
moe_status moe_grouped_ffn_backward(const moe_layer_desc* d, const void* x_sorted, const int32_t* offsets,
                                    const void* w_gate, const void* w_up, const void* w_down, const void* gate,
                                    const void* up, const void* h, const void* dy_sorted, void* dx_sorted,
                                    void* dw_gate, void* dw_up, void* dw_down, void* ws, size_t ws_bytes,
                                    void* stream);

/* The router's parameter gradients: dlogits[t, e] = sum of dl[t, j] over the
 * slots with topk_ids[t, j] = e (0 elsewhere); dw_router = dlogits^T x and
 * db_router = sum over tokens of dlogits.
 *   x          device [T, H] dtype;  topk_ids device [T, k] int32
 *   dl         device [T, k] float32 (from moe_combine_backward)
 *   dw_router  device [E, H] dtype out
 *   db_router  device [E] float32 out, or NULL when the router has no bias
 *   ws         device workspace of MOE_STAGE_ROUTE_BACKWARD bytes */
moe_status moe_route_backward(const moe_layer_desc* d, const void* x, const int32_t* topk_ids, const float* dl,
                              void* dw_router, float* db_router, void* ws, size_t ws_bytes, void* stream);

/* Gradient of the layer input: dx[t] = sum_j dx_sorted[pair_row[t*k+j]]
 * (kept local pairs, slot order) + sum_j dl[t,j] w_router[topk_ids[t,j]],
 * accumulated in float32 and rounded once.
 *   dx_sorted  device [P_max, H] dtype;  pair_row device [T*k] int32
 *   topk_ids   device [T, k] int32;      dl device [T, k] float32
 *   w_router   device [E, H] dtype;      dx device [T, H] dtype out */
moe_status moe_dispatch_backward(const moe_layer_desc* d, const void* dx_sorted, const int32_t* pair_row,
                                 const int32_t* topk_ids, const float* dl, const void* w_router, void* dx,
                                 void* stream);

/* The four backward stages in one call, from the training forward's saved
 * intermediates.  db_router may be NULL (no router bias).  Workspace:
 * MOE_STAGE_LAYER_BACKWARD bytes.
 *   dy  device [T, H] dtype;  dx device [T, H] dtype out
 *   dw_router [E, H] dtype out; dw_gate, dw_up, dw_down dtype out in the layout of the weights */
moe_status moe_layer_backward(const moe_layer_desc* d, const void* x, const void* w_router, const void* w_gate,
                              const void* w_up, const void* w_down, const moe_saved* saved, const void* dy,
                              void* dx, void* dw_router, float* db_router, void* dw_gate, void* dw_up,
                              void* dw_down, void* ws, size_t ws_bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* MOE_H_ */
