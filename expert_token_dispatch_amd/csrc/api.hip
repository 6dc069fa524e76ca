// libmoe C ABI: host-side validation, workspace layout and stage orchestration.
// The operations are defined in moe.h; every check below runs before any
// work is enqueued, following the Transformers "Expert parallelism" page's
// convention of rejecting a bad configuration before anything is sharded.
#include <cmath>
#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <algorithm>
#include <mutex>

#include "kernels.h"

namespace moe {

namespace {
thread_local char g_err[1024] = "";
thread_local hipEvent_t g_prof_events[64];
thread_local int g_prof_count = 0;
thread_local int g_kernel_idx = 0;
thread_local int g_last_kernel_count = 0;
thread_local const char* g_kernel_names[64];

// Resets the per-call kernel counter; on exit records how many kernels ran.
struct CallScope {
  CallScope() { g_kernel_idx = 0; }
  ~CallScope() { g_last_kernel_count = g_kernel_idx; }
};
}  // namespace

moe_status set_error(moe_status st, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return st;
}

void prof_before(const char* name, hipStream_t s) {
  if (g_kernel_idx < 64) g_kernel_names[g_kernel_idx] = name;
  if (2 * g_kernel_idx + 1 < g_prof_count && g_prof_events[2 * g_kernel_idx] != nullptr)
    (void)hipEventRecord(g_prof_events[2 * g_kernel_idx], s);
}

moe_status prof_after(const char* name, hipStream_t s) {
  const hipError_t e = hipGetLastError();
  if (2 * g_kernel_idx + 1 < g_prof_count && g_prof_events[2 * g_kernel_idx + 1] != nullptr)
    (void)hipEventRecord(g_prof_events[2 * g_kernel_idx + 1], s);
  ++g_kernel_idx;
  if (e != hipSuccess) return set_error(MOE_ERR_HIP, "%s: launch failed: %s", name, hipGetErrorString(e));
  return MOE_OK;
}

namespace {

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

moe_status check_desc(const moe_layer_desc* d) {
  if (d == nullptr) return set_error(MOE_ERR_INVALID_ARG, "descriptor is NULL");
  if (d->num_tokens < 0) return set_error(MOE_ERR_INVALID_ARG, "num_tokens must be >= 0 (got %lld)", (long long)d->num_tokens);
  if (d->hidden <= 0 || d->hidden % 8 != 0)
    return set_error(MOE_ERR_INVALID_ARG, "hidden must be a positive multiple of 8 (got %d)", d->hidden);
  if (d->intermediate <= 0 || d->intermediate % 8 != 0)
    return set_error(MOE_ERR_INVALID_ARG, "intermediate must be a positive multiple of 8 (got %d)", d->intermediate);
  if (d->num_experts < 1) return set_error(MOE_ERR_INVALID_ARG, "num_experts must be >= 1 (got %d)", d->num_experts);
  if (d->top_k < 1 || d->top_k > d->num_experts)
    return set_error(MOE_ERR_INVALID_ARG, "top_k must be in [1, num_experts] (got %d, E=%d)", d->top_k, d->num_experts);
  if (d->local_begin < 0 || d->local_count < 1 || int64_t(d->local_begin) + d->local_count > d->num_experts)
    return set_error(MOE_ERR_INVALID_ARG, "local experts [%d, %d+%d) do not fit in [0, %d)", d->local_begin,
                     d->local_begin, d->local_count, d->num_experts);
  if (d->dtype != MOE_F32 && d->dtype != MOE_BF16) return set_error(MOE_ERR_INVALID_ARG, "unknown dtype %d", d->dtype);
  if (d->weight_layout != MOE_WEIGHTS_OUT_IN && d->weight_layout != MOE_WEIGHTS_IN_OUT)
    return set_error(MOE_ERR_INVALID_ARG, "unknown weight_layout %d", d->weight_layout);
  if (isnan(d->capacity_factor) || isinf(d->capacity_factor))
    return set_error(MOE_ERR_INVALID_ARG, "capacity_factor must be finite");
  if (d->num_tokens * int64_t(d->top_k) > INT32_MAX)
    return set_error(MOE_ERR_UNSUPPORTED, "num_tokens * top_k must be below 2^31");
  if (d->top_k > 32) return set_error(MOE_ERR_UNSUPPORTED, "top_k above 32 is not supported (got %d)", d->top_k);
  if (d->num_experts > 4096) return set_error(MOE_ERR_UNSUPPORTED, "num_experts above 4096 is not supported");
  return MOE_OK;
}

int64_t capacity_of(const moe_layer_desc* d) {
  if (d->capacity_factor <= 0.0f) return -1;
  const double c = floor(double(d->capacity_factor) * double(d->num_tokens) * double(d->top_k) / double(d->num_experts));
  return c > double(INT32_MAX) ? int64_t(INT32_MAX) : int64_t(c);
}

int64_t max_pairs_of(const moe_layer_desc* d) {
  const int64_t n = d->num_tokens * d->top_k;
  const int64_t c = capacity_of(d);
  return c < 0 ? n : std::min<int64_t>(n, int64_t(d->local_count) * c);
}

// moe_grouped_ffn's workspace: h [P_max, I], then the split-K pieces
size_t ffn_h_bytes(const moe_layer_desc* d) {
  return align_up(size_t(max_pairs_of(d)) * d->intermediate * dtype_bytes(d->dtype), 256);
}

// Layout of the moe_layer_forward workspace.
struct LayerWs {
  int32_t* topk_ids;
  float* topk_w;
  float* topk_logit;
  int32_t* counts;
  int32_t* offsets;
  int32_t* sorted_pairs;
  int32_t* pair_row;
  int64_t* num_dropped;
  void* route;
  void* dispatch;
  void* x_sorted;
  void* h;
  void* ffn_scratch;
  void* y_sorted;
  size_t bytes;
};

LayerWs layer_layout(const moe_layer_desc* d, void* base) {
  const int64_t n = d->num_tokens * d->top_k;
  const int64_t pm = max_pairs_of(d);
  const size_t dt = dtype_bytes(d->dtype);
  char* p = static_cast<char*>(base);
  size_t o = 0;
  LayerWs w{};
  auto take = [&](size_t bytes) -> void* {
    void* r = p ? p + o : nullptr;
    o += align_up(bytes, 256);
    return r;
  };
  w.topk_ids = static_cast<int32_t*>(take(size_t(n) * 4));
  w.topk_w = static_cast<float*>(take(size_t(n) * 4));
  w.topk_logit = static_cast<float*>(take(size_t(n) * 4));
  w.counts = static_cast<int32_t*>(take(size_t(d->num_experts) * 4));
  w.offsets = static_cast<int32_t*>(take(size_t(d->local_count + 1) * 4));
  w.sorted_pairs = static_cast<int32_t*>(take(size_t(pm) * 4));
  w.pair_row = static_cast<int32_t*>(take(size_t(n) * 4));
  w.num_dropped = static_cast<int64_t*>(take(8));
  w.route = take(route_scratch_bytes(d));
  w.dispatch = take(dispatch_scratch_bytes(d));
  w.x_sorted = take(size_t(pm) * d->hidden * dt);
  w.h = take(size_t(pm) * d->intermediate * dt);
  const size_t fb = ffn_scratch_bytes(d, pm);
  w.ffn_scratch = fb ? take(fb) : nullptr;
  w.y_sorted = take(size_t(pm) * d->hidden * dt);
  w.bytes = o;
  return w;
}

// moe_grouped_ffn_backward's workspace: dg | du [P_max, 2I] and the large-tile path's scratch
size_t ffn_bwd_bytes(const moe_layer_desc* d) { return ffn_bwd_scratch_bytes(d, max_pairs_of(d)); }

// Layout of the moe_layer_backward workspace.
struct LayerBwdWs {
  void* dy_sorted;
  float* dl;
  void* dx_sorted;
  void* ffn;    // dg, du
  void* route;  // logit gradients
  size_t bytes;
};

LayerBwdWs layer_bwd_layout(const moe_layer_desc* d, void* base) {
  const int64_t pm = max_pairs_of(d);
  const size_t dt = dtype_bytes(d->dtype);
  char* p = static_cast<char*>(base);
  size_t o = 0;
  LayerBwdWs w{};
  auto take = [&](size_t bytes) -> void* {
    void* r = p ? p + o : nullptr;
    o += align_up(bytes, 256);
    return r;
  };
  w.dy_sorted = take(size_t(pm) * d->hidden * dt);
  w.dl = static_cast<float*>(take(size_t(d->num_tokens) * d->top_k * 4));
  w.dx_sorted = take(size_t(pm) * d->hidden * dt);
  w.ffn = take(ffn_bwd_bytes(d));
  w.route = take(route_bwd_scratch_bytes(d));
  w.bytes = o;
  return w;
}

size_t stage_bytes(const moe_layer_desc* d, int32_t stage) {
  switch (stage) {
    case MOE_STAGE_ROUTE:
      return route_scratch_bytes(d);
    case MOE_STAGE_COMBINE:
      return 0;
    case MOE_STAGE_DISPATCH:
      return dispatch_scratch_bytes(d);
    case MOE_STAGE_FFN:
      return ffn_h_bytes(d) + align_up(ffn_scratch_bytes(d, max_pairs_of(d)), 256);
    case MOE_STAGE_LAYER:
      return layer_layout(d, nullptr).bytes;
    case MOE_STAGE_FFN_BACKWARD:
      return ffn_bwd_bytes(d);
    case MOE_STAGE_ROUTE_BACKWARD:
      return route_bwd_scratch_bytes(d);
    case MOE_STAGE_LAYER_BACKWARD:
      return layer_bwd_layout(d, nullptr).bytes;
    default:
      return 0;
  }
}

#define TRY_ZERO(expr)                 \
  do {                                 \
    const moe_status _z = (expr);      \
    if (_z != MOE_OK) return _z;       \
  } while (0)

#define REQUIRE_PTR(p, a)                                                                                  \
  do {                                                                                                     \
    if ((p) == nullptr) return set_error(MOE_ERR_INVALID_ARG, "%s is NULL", #p);                           \
    if (!aligned((p), (a))) return set_error(MOE_ERR_INVALID_ARG, "%s is not %d-byte aligned", #p, int(a)); \
  } while (0)
#define OPTIONAL_PTR(p, a)                                                                                  \
  do {                                                                                                     \
    if ((p) != nullptr && !aligned((p), (a)))                                                              \
      return set_error(MOE_ERR_INVALID_ARG, "%s is not %d-byte aligned", #p, int(a));                       \
  } while (0)

moe_status check_ws(const moe_layer_desc* d, int32_t stage, const void* ws, size_t ws_bytes) {
  const size_t need = stage_bytes(d, stage);
  if (need == 0) return MOE_OK;
  if (ws == nullptr || ws_bytes < need)
    return set_error(MOE_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given%s", need, ws_bytes,
                     ws == nullptr ? " (NULL)" : "");
  if (!aligned(ws, 256)) return set_error(MOE_ERR_INVALID_ARG, "workspace must be 256-byte aligned");
  return MOE_OK;
}

moe_status route_checks(const moe_layer_desc* d, const void* x, const void* w_router, const float* b_router,
                        const float* logits_in, const float* logits_out, const int32_t* topk_ids, const float* topk_w,
                        const float* topk_logit) {
  if (d->num_experts > 256) return set_error(MOE_ERR_UNSUPPORTED, "route: num_experts above 256 is not supported");
  if (logits_in == nullptr) {
    REQUIRE_PTR(x, 16);
    REQUIRE_PTR(w_router, 16);
    OPTIONAL_PTR(b_router, 4);
  } else {
    REQUIRE_PTR(logits_in, 4);
  }
  OPTIONAL_PTR(logits_out, 4);
  REQUIRE_PTR(topk_ids, 4);
  REQUIRE_PTR(topk_w, 4);
  OPTIONAL_PTR(topk_logit, 4);
  return MOE_OK;
}

moe_status dispatch_checks(const moe_layer_desc* d, const void* x, const int32_t* topk_ids, const float* topk_logit,
                           const int32_t* counts, const int32_t* offsets, const int32_t* sorted_pairs,
                           const int32_t* pair_row, const void* x_sorted, const int64_t* num_dropped) {
  if (d->local_count > 3000) return set_error(MOE_ERR_UNSUPPORTED, "dispatch: local_count above 3000 is not supported");
  REQUIRE_PTR(x, 16);
  REQUIRE_PTR(topk_ids, 4);
  if (d->capacity_factor > 0) {
    REQUIRE_PTR(topk_logit, 4);
  }
  REQUIRE_PTR(counts, 4);
  REQUIRE_PTR(offsets, 4);
  REQUIRE_PTR(sorted_pairs, 4);
  REQUIRE_PTR(pair_row, 4);
  REQUIRE_PTR(x_sorted, 16);
  OPTIONAL_PTR(num_dropped, 8);
  // the capacity cut holds an expert's pairs (at most one per token) in registers
  if (d->capacity_factor > 0 && d->num_tokens > 32768)
    return set_error(MOE_ERR_UNSUPPORTED, "capacity_factor > 0 supports at most 32768 tokens per call");
  return MOE_OK;
}

moe_status ffn_checks(const void* x_sorted, const int32_t* offsets, const void* w_gate, const void* w_up,
                      const void* w_down, const void* y_sorted) {
  REQUIRE_PTR(x_sorted, 16);
  REQUIRE_PTR(offsets, 4);
  REQUIRE_PTR(w_gate, 16);
  REQUIRE_PTR(w_up, 16);
  REQUIRE_PTR(w_down, 16);
  REQUIRE_PTR(y_sorted, 16);
  return MOE_OK;
}

moe_status combine_checks(const void* y_sorted, const int32_t* pair_row, const float* topk_w, const void* y) {
  REQUIRE_PTR(y_sorted, 16);
  REQUIRE_PTR(pair_row, 4);
  REQUIRE_PTR(topk_w, 4);
  REQUIRE_PTR(y, 16);
  return MOE_OK;
}

moe_status saved_checks(const moe_saved* v) {
  if (v == nullptr) return set_error(MOE_ERR_INVALID_ARG, "saved is NULL");
  REQUIRE_PTR(v->topk_ids, 4);
  REQUIRE_PTR(v->topk_w, 4);
  REQUIRE_PTR(v->offsets, 4);
  REQUIRE_PTR(v->pair_row, 4);
  REQUIRE_PTR(v->x_sorted, 16);
  REQUIRE_PTR(v->gate, 16);
  REQUIRE_PTR(v->up, 16);
  REQUIRE_PTR(v->h, 16);
  REQUIRE_PTR(v->y_sorted, 16);
  return MOE_OK;
}

moe_status combine_bwd_checks(const void* dy, const void* y_sorted, const int32_t* pair_row, const float* topk_w,
                              const void* dy_sorted, const float* dl) {
  REQUIRE_PTR(dy, 16);
  REQUIRE_PTR(y_sorted, 16);
  REQUIRE_PTR(pair_row, 4);
  REQUIRE_PTR(topk_w, 4);
  REQUIRE_PTR(dy_sorted, 16);
  REQUIRE_PTR(dl, 4);
  return MOE_OK;
}

moe_status ffn_bwd_checks(const void* x_sorted, const int32_t* offsets, const void* w_gate, const void* w_up,
                          const void* w_down, const void* gate, const void* up, const void* h, const void* dy_sorted,
                          const void* dx_sorted, const void* dw_gate, const void* dw_up, const void* dw_down) {
  REQUIRE_PTR(x_sorted, 16);
  REQUIRE_PTR(offsets, 4);
  REQUIRE_PTR(w_gate, 16);
  REQUIRE_PTR(w_up, 16);
  REQUIRE_PTR(w_down, 16);
  REQUIRE_PTR(gate, 16);
  REQUIRE_PTR(up, 16);
  REQUIRE_PTR(h, 16);
  REQUIRE_PTR(dy_sorted, 16);
  REQUIRE_PTR(dx_sorted, 16);
  REQUIRE_PTR(dw_gate, 16);
  REQUIRE_PTR(dw_up, 16);
  REQUIRE_PTR(dw_down, 16);
  return MOE_OK;
}

moe_status route_bwd_checks(const void* x, const int32_t* topk_ids, const float* dl, const void* dw_router,
                            const float* db_router) {
  REQUIRE_PTR(x, 16);
  REQUIRE_PTR(topk_ids, 4);
  REQUIRE_PTR(dl, 4);
  REQUIRE_PTR(dw_router, 16);
  OPTIONAL_PTR(db_router, 16);
  return MOE_OK;
}

moe_status dispatch_bwd_checks(const void* dx_sorted, const int32_t* pair_row, const int32_t* topk_ids,
                               const float* dl, const void* w_router, const void* dx) {
  REQUIRE_PTR(dx_sorted, 16);
  REQUIRE_PTR(pair_row, 4);
  REQUIRE_PTR(topk_ids, 4);
  REQUIRE_PTR(dl, 4);
  REQUIRE_PTR(w_router, 16);
  REQUIRE_PTR(dx, 16);
  return MOE_OK;
}

// Zero weight gradients of a layer that saw no tokens (no expert received any).
moe_status zero_ffn_grads(const moe_layer_desc* d, void* dw_gate, void* dw_up, void* dw_down, hipStream_t s) {
  const size_t n = size_t(d->local_count) * d->intermediate * d->hidden * dtype_bytes(d->dtype);
  TRY_ZERO(launch_zero("ffn_bwd_zero", dw_gate, n, s));
  TRY_ZERO(launch_zero("ffn_bwd_zero", dw_up, n, s));
  return launch_zero("ffn_bwd_zero", dw_down, n, s);
}

moe_status zero_route_grads(const moe_layer_desc* d, void* dw_router, float* db_router, hipStream_t s) {
  TRY_ZERO(launch_zero("route_bwd_zero", dw_router, size_t(d->num_experts) * d->hidden * dtype_bytes(d->dtype), s));
  return launch_zero("route_bwd_zero", db_router, size_t(d->num_experts) * 4, s);
}

#define TRY(expr)                          \
  do {                                     \
    const moe_status _s = (expr);          \
    if (_s != MOE_OK) return _s;           \
  } while (0)

}  // namespace
}  // namespace moe

using namespace moe;

namespace moe {
namespace {
// Routing options: glossary "Load balancing and capacity" (selection bias, groups per token).
moe_status opts_checks(const moe_layer_desc* d, const moe_route_opts* o) {
  if (o == nullptr || o->num_groups <= 1) return MOE_OK;
  const int E = d->num_experts, G = o->num_groups;
  if (G > 16) return set_error(MOE_ERR_UNSUPPORTED, "route options: num_groups above 16 is not supported (got %d)", G);
  if (E % G != 0) return set_error(MOE_ERR_INVALID_ARG, "route options: num_groups %d does not divide E=%d", G, E);
  if (o->max_groups < 1 || o->max_groups > G)
    return set_error(MOE_ERR_INVALID_ARG, "route options: max_groups must be in [1, %d] (got %d)", G, o->max_groups);
  if (int64_t(o->max_groups) * (E / G) < d->top_k)
    return set_error(MOE_ERR_INVALID_ARG, "route options: %d groups of %d experts hold fewer than k=%d", o->max_groups,
                     E / G, d->top_k);
  return MOE_OK;
}

void apply_opts(RouteArgs& a, const moe_layer_desc* d, const moe_route_opts* o) {
  if (o == nullptr) return;
  a.sel_bias = o->selection_bias;
  if (o->num_groups > 1 && o->max_groups < o->num_groups) {
    a.group_size = d->num_experts / o->num_groups;
    a.max_groups = o->max_groups;
  }
}
}  // namespace
}  // namespace moe

// ---- the dispatch scratch of moe_dispatch_noalloc -----------------------------
// For callers that cannot allocate device memory (code under graph capture,
// tight serving loops, harnesses that forbid hipMalloc): the dispatch kernels'
// scratch (per-chunk histograms, per-chunk segment bases, pre-capacity
// offsets and permutation) lives in this file-scope device array instead of a
// caller workspace.  Each GPU holds its own copy for the life of the process.
// Host code never passes the array's name to a kernel (on the host it only
// names a stand-in): it resolves the device address once per device with
// hipGetSymbolAddress and passes that.
namespace moe {
namespace {
constexpr size_t kNoAllocScratchBytes = size_t(16) << 20;
constexpr int kMaxDevices = 64;
static __device__ __align__(256) char scratch[kNoAllocScratchBytes];

std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];

// The current device's address of `scratch` (resolved on the first call per device).
moe_status noalloc_scratch(void** out) {
  int dev = -1;
  const hipError_t ge = hipGetDevice(&dev);
  if (ge != hipSuccess) return set_error(MOE_ERR_HIP, "hipGetDevice: %s", hipGetErrorString(ge));
  if (dev < 0 || dev >= kMaxDevices) return set_error(MOE_ERR_UNSUPPORTED, "device %d: at most %d devices", dev, kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* ptr = nullptr;
    const hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess || ptr == nullptr)
      return set_error(MOE_ERR_HIP, "hipGetSymbolAddress(scratch) on device %d: %s", dev, hipGetErrorString(e));
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return MOE_OK;
}
}  // namespace
}  // namespace moe

extern "C" {

const char* moe_last_error(void) { return g_err; }

const char* moe_version(void) { return "libmoe 0.1 (gfx950)"; }

moe_status moe_ep_local_range(int32_t num_experts, int32_t ep_size, int32_t rank, int32_t* begin, int32_t* count) {
  if (begin == nullptr || count == nullptr) return set_error(MOE_ERR_INVALID_ARG, "begin/count are NULL");
  if (num_experts < 1) return set_error(MOE_ERR_INVALID_ARG, "num_experts must be >= 1");
  if (ep_size < 1) return set_error(MOE_ERR_INVALID_ARG, "ep_size must be >= 1");
  if (rank < 0) return set_error(MOE_ERR_INVALID_ARG, "rank must be >= 0");
  if (num_experts % ep_size != 0)
    return set_error(MOE_ERR_INVALID_ARG, "ep_size %d does not divide num_experts %d", ep_size, num_experts);
  const int32_t per = num_experts / ep_size;
  *begin = (rank % ep_size) * per;
  *count = per;
  return MOE_OK;
}

int64_t moe_capacity(const moe_layer_desc* d) {
  if (check_desc(d) != MOE_OK) return -1;
  return capacity_of(d);
}

int64_t moe_max_pairs(const moe_layer_desc* d) {
  if (check_desc(d) != MOE_OK) return -1;
  return max_pairs_of(d);
}

moe_status moe_workspace_size(const moe_layer_desc* d, int32_t stage, size_t* bytes) {
  TRY(check_desc(d));
  if (bytes == nullptr) return set_error(MOE_ERR_INVALID_ARG, "bytes is NULL");
  if (stage < MOE_STAGE_ROUTE || stage > MOE_STAGE_LAYER_BACKWARD)
    return set_error(MOE_ERR_INVALID_ARG, "unknown stage %d", stage);
  *bytes = stage_bytes(d, stage);
  return MOE_OK;
}

moe_status moe_profile_events(void* const* events, int32_t count) {
  if (events == nullptr || count <= 0) {
    g_prof_count = 0;
    return MOE_OK;
  }
  if (count > 64 || count % 2 != 0)
    return set_error(MOE_ERR_INVALID_ARG, "profiling events: an even count of at most 64 (got %d)", count);
  for (int i = 0; i < count; ++i) {
    if ((events[i] == nullptr) != (events[i ^ 1] == nullptr))
      return set_error(MOE_ERR_INVALID_ARG, "profiling events %d and %d: give both or neither", i & ~1, i | 1);
    g_prof_events[i] = static_cast<hipEvent_t>(events[i]);
  }
  g_prof_count = count;
  return MOE_OK;
}

const char* moe_profile_kernel_name(int32_t i) {
  if (i < 0 || i >= g_last_kernel_count || i >= 64) return nullptr;
  return g_kernel_names[i];
}

int32_t moe_profile_kernel_count(void) { return g_last_kernel_count; }

moe_status moe_route_ex(const moe_layer_desc* d, const moe_route_opts* opts, const void* x, const void* w_router,
                        const float* b_router, const float* logits_in, float* logits_out, int32_t* topk_ids,
                        float* topk_w, float* topk_logit, void* ws, size_t ws_bytes, void* stream) {
  CallScope scope;
  TRY(check_desc(d));
  if (d->num_tokens == 0) return MOE_OK;
  TRY(route_checks(d, x, w_router, b_router, logits_in, logits_out, topk_ids, topk_w, topk_logit));
  TRY(opts_checks(d, opts));
  if (logits_in == nullptr) TRY(check_ws(d, MOE_STAGE_ROUTE, ws, ws_bytes));
  RouteArgs a{d, x, w_router, b_router, logits_in, logits_out, topk_ids, topk_w, topk_logit,
              static_cast<float*>(ws), nullptr, static_cast<hipStream_t>(stream)};
  apply_opts(a, d, opts);
  return launch_route(a);
}

moe_status moe_route(const moe_layer_desc* d, const void* x, const void* w_router, const float* b_router,
                     const float* logits_in, float* logits_out, int32_t* topk_ids, float* topk_w, float* topk_logit,
                     void* ws, size_t ws_bytes, void* stream) {
  return moe_route_ex(d, nullptr, x, w_router, b_router, logits_in, logits_out, topk_ids, topk_w, topk_logit, ws,
                      ws_bytes, stream);
}

moe_status moe_selection_bias_update(const moe_layer_desc* d, const int32_t* counts, float* bias, float gamma,
                                     void* stream) {
  CallScope scope;
  TRY(check_desc(d));
  if (counts == nullptr || bias == nullptr)
    return set_error(MOE_ERR_INVALID_ARG, "selection bias update: counts and bias are required");
  if (!std::isfinite(gamma)) return set_error(MOE_ERR_INVALID_ARG, "selection bias update: gamma must be finite");
  return launch_selection_bias_update(d, counts, bias, gamma, static_cast<hipStream_t>(stream));
}

moe_status moe_dispatch(const moe_layer_desc* d, const void* x, const int32_t* topk_ids, const float* topk_logit,
                        int32_t* counts, int32_t* offsets, int32_t* sorted_pairs, int32_t* pair_row, void* x_sorted,
                        int64_t* num_dropped, void* ws, size_t ws_bytes, void* stream) {
  CallScope scope;
  TRY(check_desc(d));
  if (d->num_tokens == 0) return MOE_OK;
  TRY(dispatch_checks(d, x, topk_ids, topk_logit, counts, offsets, sorted_pairs, pair_row, x_sorted, num_dropped));
  TRY(check_ws(d, MOE_STAGE_DISPATCH, ws, ws_bytes));
  DispatchArgs a{d, x, topk_ids, topk_logit, counts, offsets, sorted_pairs, pair_row, x_sorted, num_dropped,
                 carve_dispatch_scratch(d, ws), capacity_of(d), false, static_cast<hipStream_t>(stream)};
  return launch_dispatch(a);
}

moe_status moe_dispatch_noalloc(const moe_layer_desc* d, const void* x, const int32_t* topk_ids,
                                const float* topk_logit, int32_t* counts, int32_t* offsets, int32_t* sorted_pairs,
                                int32_t* pair_row, void* x_sorted, int64_t* num_dropped, void* stream) {
  CallScope scope;
  TRY(check_desc(d));
  if (d->num_tokens == 0) return MOE_OK;
  TRY(dispatch_checks(d, x, topk_ids, topk_logit, counts, offsets, sorted_pairs, pair_row, x_sorted, num_dropped));
  const size_t need = dispatch_scratch_bytes(d);
  if (need > kNoAllocScratchBytes)
    return set_error(MOE_ERR_UNSUPPORTED, "dispatch_noalloc: %zu bytes of scratch needed, the static buffer holds %zu",
                     need, kNoAllocScratchBytes);
  void* scr = nullptr;
  TRY(noalloc_scratch(&scr));
  // every scratch entry the kernels read is written earlier in the same call, so
  // nothing needs clearing between calls
  DispatchArgs a{d, x, topk_ids, topk_logit, counts, offsets, sorted_pairs, pair_row, x_sorted, num_dropped,
                 carve_dispatch_scratch(d, scr), capacity_of(d), false, static_cast<hipStream_t>(stream)};
  return launch_dispatch(a);
}

moe_status moe_grouped_ffn(const moe_layer_desc* d, const void* x_sorted, const int32_t* offsets, const void* w_gate,
                           const void* w_up, const void* w_down, void* y_sorted, void* ws, size_t ws_bytes,
                           void* stream) {
  CallScope scope;
  TRY(check_desc(d));
  if (d->num_tokens == 0) return MOE_OK;
  TRY(ffn_checks(x_sorted, offsets, w_gate, w_up, w_down, y_sorted));
  TRY(check_ws(d, MOE_STAGE_FFN, ws, ws_bytes));
  void* scratch = ffn_scratch_bytes(d, max_pairs_of(d)) ? static_cast<char*>(ws) + ffn_h_bytes(d) : nullptr;
  FfnArgs a{d, x_sorted, offsets, w_gate, w_up, w_down, y_sorted, ws, scratch, max_pairs_of(d),
            static_cast<hipStream_t>(stream)};
  return launch_grouped_ffn(a);
}

moe_status moe_combine(const moe_layer_desc* d, const void* y_sorted, const int32_t* pair_row, const float* topk_w,
                       void* y, void* stream) {
  CallScope scope;
  TRY(check_desc(d));
  if (d->num_tokens == 0) return MOE_OK;
  TRY(combine_checks(y_sorted, pair_row, topk_w, y));
  CombineArgs a{d, y_sorted, pair_row, topk_w, y, static_cast<hipStream_t>(stream)};
  return launch_combine(a);
}

moe_status moe_layer_forward(const moe_layer_desc* d, const void* x, const void* w_router, const float* b_router,
                             const void* w_gate, const void* w_up, const void* w_down, void* y, int32_t* topk_ids_out,
                             float* topk_w_out, int32_t* counts_out, int64_t* num_dropped_out, void* ws,
                             size_t ws_bytes, void* stream) {
  return moe_layer_forward_ex(d, nullptr, x, w_router, b_router, w_gate, w_up, w_down, y, topk_ids_out, topk_w_out,
                              counts_out, num_dropped_out, ws, ws_bytes, stream);
}

moe_status moe_layer_forward_ex(const moe_layer_desc* d, const moe_route_opts* opts, const void* x,
                                const void* w_router, const float* b_router, const void* w_gate, const void* w_up,
                                const void* w_down, void* y, int32_t* topk_ids_out, float* topk_w_out,
                                int32_t* counts_out, int64_t* num_dropped_out, void* ws, size_t ws_bytes,
                                void* stream) {
  CallScope scope;
  TRY(check_desc(d));
  if (d->num_tokens == 0) return MOE_OK;
  TRY(check_ws(d, MOE_STAGE_LAYER, ws, ws_bytes));
  LayerWs w = layer_layout(d, ws);
  int32_t* ids = topk_ids_out ? topk_ids_out : w.topk_ids;
  float* tw = topk_w_out ? topk_w_out : w.topk_w;
  int32_t* counts = counts_out ? counts_out : w.counts;
  int64_t* dropped = num_dropped_out ? num_dropped_out : w.num_dropped;
  const bool cap = capacity_of(d) >= 0;
  TRY(route_checks(d, x, w_router, b_router, nullptr, nullptr, ids, tw, w.topk_logit));
  TRY(dispatch_checks(d, x, ids, w.topk_logit, counts, w.offsets, w.sorted_pairs, w.pair_row, w.x_sorted, dropped));
  TRY(ffn_checks(w.x_sorted, w.offsets, w_gate, w_up, w_down, w.y_sorted));
  TRY(combine_checks(w.y_sorted, w.pair_row, tw, y));
  TRY(opts_checks(d, opts));
  const hipStream_t s = static_cast<hipStream_t>(stream);

  const DispatchScratch scr = carve_dispatch_scratch(d, w.dispatch);
  // the router's top-k kernel also writes the per-chunk expert histograms
  RouteArgs ra{d, x, w_router, b_router, nullptr, nullptr, ids, tw, cap ? w.topk_logit : nullptr,
               static_cast<float*>(w.route), scr.blk_all, s};
  apply_opts(ra, d, opts);
  TRY(launch_route(ra));
  DispatchArgs da{d, x, ids, w.topk_logit, counts, w.offsets, w.sorted_pairs, w.pair_row, w.x_sorted, dropped,
                  scr, capacity_of(d), true, s};
  TRY(launch_dispatch(da));
  FfnArgs fa{d, w.x_sorted, w.offsets, w_gate, w_up, w_down, w.y_sorted, w.h, w.ffn_scratch, max_pairs_of(d), s};
  TRY(launch_grouped_ffn(fa));
  CombineArgs ca{d, w.y_sorted, w.pair_row, tw, y, s};
  return launch_combine(ca);
}

moe_status moe_grouped_ffn_train(const moe_layer_desc* d, const void* x_sorted, const int32_t* offsets,
                                 const void* w_gate, const void* w_up, const void* w_down, void* y_sorted, void* h,
                                 void* gate, void* up, void* ws, size_t ws_bytes, void* stream) {
  CallScope scope;
  TRY(check_desc(d));
  if (d->num_tokens == 0) return MOE_OK;
  TRY(ffn_checks(x_sorted, offsets, w_gate, w_up, w_down, y_sorted));
  REQUIRE_PTR(h, 16);
  REQUIRE_PTR(gate, 16);
  REQUIRE_PTR(up, 16);
  TRY(check_ws(d, MOE_STAGE_FFN, ws, ws_bytes));
  void* scratch = ffn_scratch_bytes(d, max_pairs_of(d)) ? static_cast<char*>(ws) + ffn_h_bytes(d) : nullptr;
  FfnArgs a{d, x_sorted, offsets, w_gate, w_up, w_down, y_sorted, h, scratch, max_pairs_of(d),
            static_cast<hipStream_t>(stream), gate, up};
  return launch_grouped_ffn(a);
}

moe_status moe_layer_forward_train(const moe_layer_desc* d, const moe_route_opts* opts, const void* x,
                                   const void* w_router, const float* b_router, const void* w_gate, const void* w_up,
                                   const void* w_down, void* y, const moe_saved* saved, int32_t* counts_out,
                                   int64_t* num_dropped_out, void* ws, size_t ws_bytes, void* stream) {
  CallScope scope;
  TRY(check_desc(d));
  if (d->num_tokens == 0) return MOE_OK;
  TRY(saved_checks(saved));
  TRY(check_ws(d, MOE_STAGE_LAYER, ws, ws_bytes));
  LayerWs w = layer_layout(d, ws);
  const moe_saved& v = *saved;
  int32_t* counts = counts_out ? counts_out : w.counts;
  int64_t* dropped = num_dropped_out ? num_dropped_out : w.num_dropped;
  const bool cap = capacity_of(d) >= 0;
  TRY(route_checks(d, x, w_router, b_router, nullptr, nullptr, v.topk_ids, v.topk_w, w.topk_logit));
  TRY(dispatch_checks(d, x, v.topk_ids, w.topk_logit, counts, v.offsets, w.sorted_pairs, v.pair_row, v.x_sorted,
                      dropped));
  TRY(ffn_checks(v.x_sorted, v.offsets, w_gate, w_up, w_down, v.y_sorted));
  TRY(combine_checks(v.y_sorted, v.pair_row, v.topk_w, y));
  TRY(opts_checks(d, opts));
  const hipStream_t s = static_cast<hipStream_t>(stream);
  const DispatchScratch scr = carve_dispatch_scratch(d, w.dispatch);
  RouteArgs ra{d, x, w_router, b_router, nullptr, nullptr, v.topk_ids, v.topk_w, cap ? w.topk_logit : nullptr,
               static_cast<float*>(w.route), scr.blk_all, s};
  apply_opts(ra, d, opts);
  TRY(launch_route(ra));
  DispatchArgs da{d, x, v.topk_ids, w.topk_logit, counts, v.offsets, w.sorted_pairs, v.pair_row, v.x_sorted,
                  dropped, scr, capacity_of(d), true, s};
  TRY(launch_dispatch(da));
  FfnArgs fa{d, v.x_sorted, v.offsets, w_gate, w_up, w_down, v.y_sorted, v.h, w.ffn_scratch, max_pairs_of(d), s,
             v.gate, v.up};
  TRY(launch_grouped_ffn(fa));
  CombineArgs ca{d, v.y_sorted, v.pair_row, v.topk_w, y, s};
  return launch_combine(ca);
}

moe_status moe_combine_backward(const moe_layer_desc* d, const void* dy, const void* y_sorted,
                                const int32_t* pair_row, const float* topk_w, void* dy_sorted, float* dl,
                                void* stream) {
  CallScope scope;
  TRY(check_desc(d));
  if (d->num_tokens == 0) return MOE_OK;
  TRY(combine_bwd_checks(dy, y_sorted, pair_row, topk_w, dy_sorted, dl));
  CombineBwdArgs a{d, dy, y_sorted, pair_row, topk_w, dy_sorted, dl, static_cast<hipStream_t>(stream)};
  return launch_combine_backward(a);
}

moe_status moe_grouped_ffn_backward(const moe_layer_desc* d, const void* x_sorted, const int32_t* offsets,
                                    const void* w_gate, const void* w_up, const void* w_down, const void* gate,
                                    const void* up, const void* h, const void* dy_sorted, void* dx_sorted,
                                    void* dw_gate, void* dw_up, void* dw_down, void* ws, size_t ws_bytes,
                                    void* stream) {
  CallScope scope;
  TRY(check_desc(d));
  const hipStream_t s = static_cast<hipStream_t>(stream);
  if (d->num_tokens == 0) {
    REQUIRE_PTR(dw_gate, 16);
    REQUIRE_PTR(dw_up, 16);
    REQUIRE_PTR(dw_down, 16);
    return zero_ffn_grads(d, dw_gate, dw_up, dw_down, s);
  }
  TRY(ffn_bwd_checks(x_sorted, offsets, w_gate, w_up, w_down, gate, up, h, dy_sorted, dx_sorted, dw_gate, dw_up,
                     dw_down));
  TRY(check_ws(d, MOE_STAGE_FFN_BACKWARD, ws, ws_bytes));
  FfnBwdArgs a{d, x_sorted, offsets, w_gate, w_up, w_down, gate, up, h, dy_sorted, dx_sorted, dw_gate, dw_up,
               dw_down, ws, max_pairs_of(d), s};
  return launch_grouped_ffn_backward(a);
}

moe_status moe_route_backward(const moe_layer_desc* d, const void* x, const int32_t* topk_ids, const float* dl,
                              void* dw_router, float* db_router, void* ws, size_t ws_bytes, void* stream) {
  CallScope scope;
  TRY(check_desc(d));
  const hipStream_t s = static_cast<hipStream_t>(stream);
  if (d->num_tokens == 0) {
    REQUIRE_PTR(dw_router, 16);
    OPTIONAL_PTR(db_router, 16);
    return zero_route_grads(d, dw_router, db_router, s);
  }
  TRY(route_bwd_checks(x, topk_ids, dl, dw_router, db_router));
  TRY(check_ws(d, MOE_STAGE_ROUTE_BACKWARD, ws, ws_bytes));
  RouteBwdArgs a{d, x, topk_ids, dl, dw_router, db_router, ws, s};
  return launch_route_backward(a);
}

moe_status moe_dispatch_backward(const moe_layer_desc* d, const void* dx_sorted, const int32_t* pair_row,
                                 const int32_t* topk_ids, const float* dl, const void* w_router, void* dx,
                                 void* stream) {
  CallScope scope;
  TRY(check_desc(d));
  if (d->num_tokens == 0) return MOE_OK;
  TRY(dispatch_bwd_checks(dx_sorted, pair_row, topk_ids, dl, w_router, dx));
  DispatchBwdArgs a{d, dx_sorted, pair_row, topk_ids, dl, w_router, dx, static_cast<hipStream_t>(stream)};
  return launch_dispatch_backward(a);
}

moe_status moe_layer_backward(const moe_layer_desc* d, const void* x, const void* w_router, const void* w_gate,
                              const void* w_up, const void* w_down, const moe_saved* saved, const void* dy,
                              void* dx, void* dw_router, float* db_router, void* dw_gate, void* dw_up,
                              void* dw_down, void* ws, size_t ws_bytes, void* stream) {
  CallScope scope;
  TRY(check_desc(d));
  const hipStream_t s = static_cast<hipStream_t>(stream);
  if (d->num_tokens == 0) {
    REQUIRE_PTR(dw_router, 16);
    OPTIONAL_PTR(db_router, 16);
    REQUIRE_PTR(dw_gate, 16);
    REQUIRE_PTR(dw_up, 16);
    REQUIRE_PTR(dw_down, 16);
    TRY(zero_route_grads(d, dw_router, db_router, s));
    return zero_ffn_grads(d, dw_gate, dw_up, dw_down, s);
  }
  TRY(saved_checks(saved));
  TRY(check_ws(d, MOE_STAGE_LAYER_BACKWARD, ws, ws_bytes));
  const moe_saved& v = *saved;
  LayerBwdWs w = layer_bwd_layout(d, ws);
  TRY(combine_bwd_checks(dy, v.y_sorted, v.pair_row, v.topk_w, w.dy_sorted, w.dl));
  TRY(ffn_bwd_checks(v.x_sorted, v.offsets, w_gate, w_up, w_down, v.gate, v.up, v.h, w.dy_sorted, w.dx_sorted,
                     dw_gate, dw_up, dw_down));
  TRY(route_bwd_checks(x, v.topk_ids, w.dl, dw_router, db_router));
  TRY(dispatch_bwd_checks(w.dx_sorted, v.pair_row, v.topk_ids, w.dl, w_router, dx));
  CombineBwdArgs ca{d, dy, v.y_sorted, v.pair_row, v.topk_w, w.dy_sorted, w.dl, s};
  TRY(launch_combine_backward(ca));
  FfnBwdArgs fa{d, v.x_sorted, v.offsets, w_gate, w_up, w_down, v.gate, v.up, v.h, w.dy_sorted, w.dx_sorted,
                dw_gate, dw_up, dw_down, w.ffn, max_pairs_of(d), s};
  TRY(launch_grouped_ffn_backward(fa));
  RouteBwdArgs ra{d, x, v.topk_ids, w.dl, dw_router, db_router, w.route, s};
  TRY(launch_route_backward(ra));
  DispatchBwdArgs da{d, w.dx_sorted, v.pair_row, v.topk_ids, w.dl, w_router, dx, s};
  return launch_dispatch_backward(da);
}

}  // extern "C"
