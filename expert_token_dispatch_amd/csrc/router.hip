// Stage 1: router logits, top-k and routing weights.
//
// Ultralytics glossary "Expert Parallelism", section "How tokens move between
// GPUs", step 1: the router scores every token against every expert and keeps
// the k best.  Here the scores are a linear layer, logits = x Wr^T + b, with
// float32 accumulation; the k best are taken in descending order with ties to
// the lower expert id, and the routing weights are a softmax over the k chosen
// logits.
//
// One block handles 64 tokens with four waves.  Each wave computes a 16-token
// by E-expert logit tile with MFMA (bf16: 16x16x32, f32: 16x16x4), streaming
// its 16 rows of x straight from HBM into registers (every x element is used
// by exactly one wave, so LDS staging would buy nothing) and reading the small
// router matrix through the caches.  The logits go to LDS, and one thread per
// token then keeps a sorted list of its k best with a strict compare while
// walking the experts in ascending id order, which gives lowest-id ties.
#include <math.h>

#include "common.h"
#include "kernels.h"

namespace moe {
namespace {

constexpr int kRouteTokens = 64;   // tokens per block
constexpr int kRouteThreads = 256;

template <typename T> struct RouterMma;
template <> struct RouterMma<bf16_t> {
  static constexpr int kStep = 32;   // k consumed per MFMA step: 4 lane groups x 8
  static constexpr int kLaneK = 8;   // k values one lane supplies per step
  __device__ static void mma(const uint4& a, const uint4& b, f32x4_t& c) {
    c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
  }
};
template <> struct RouterMma<float> {
  static constexpr int kStep = 16;   // 4 lane groups x 4
  static constexpr int kLaneK = 4;
  __device__ static void mma(const uint4& a, const uint4& b, f32x4_t& c) {
    c = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a.x), __uint_as_float(b.x), c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a.y), __uint_as_float(b.y), c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a.z), __uint_as_float(b.z), c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a.w), __uint_as_float(b.w), c, 0, 0, 0);
  }
};

// NEB: 16-expert column blocks (E <= 16*NEB).  MAXK: register top-k list size (k <= MAXK).
template <typename T, int NEB, int MAXK>
__global__ __launch_bounds__(kRouteThreads) void route_kernel(
    const T* __restrict__ x, const T* __restrict__ wr, const float* __restrict__ br,
    const float* __restrict__ logits_in, float* __restrict__ logits_out, int32_t* __restrict__ ids,
    float* __restrict__ tw, float* __restrict__ tl, int ntok, int H, int E, int k) {
  extern __shared__ float lg[];  // [kRouteTokens][E + 1]
  const int ld = E + 1;
  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int tblk = blockIdx.x * kRouteTokens;

  if (logits_in != nullptr) {
    for (int idx = tid; idx < kRouteTokens * E; idx += kRouteThreads) {
      const int m = idx / E, e = idx - m * E;
      const int t = tblk + m;
      lg[m * ld + e] = t < ntok ? logits_in[size_t(t) * E + e] : 0.0f;
    }
  } else {
    using M = RouterMma<T>;
    const int row = lane & 15;     // A row (token) / B column (expert) this lane feeds
    const int kg = lane >> 4;      // lane group: which k slice of the step
    const int t = tblk + wave * 16 + row;
    const bool tok_ok = t < ntok;
    const T* xrow = x + size_t(tok_ok ? t : 0) * H;
    f32x4_t acc[NEB];
#pragma unroll
    for (int eb = 0; eb < NEB; ++eb) acc[eb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    const uint4 zero = make_uint4(0, 0, 0, 0);
    for (int k0 = 0; k0 < H; k0 += M::kStep) {
      const int kk = k0 + kg * M::kLaneK;
      const bool k_ok = kk < H;
      const uint4 a = (tok_ok && k_ok) ? *reinterpret_cast<const uint4*>(xrow + kk) : zero;
#pragma unroll
      for (int eb = 0; eb < NEB; ++eb) {
        const int e = eb * 16 + row;
        const uint4 b = (e < E && k_ok) ? *reinterpret_cast<const uint4*>(wr + size_t(e) * H + kk) : zero;
        M::mma(a, b, acc[eb]);
      }
    }
    // acc[eb][r] = logit(token wave*16 + 4*kg + r, expert eb*16 + row)
#pragma unroll
    for (int eb = 0; eb < NEB; ++eb) {
      const int e = eb * 16 + row;
      if (e < E) {
        const float bias = br != nullptr ? br[e] : 0.0f;
#pragma unroll
        for (int r = 0; r < 4; ++r) lg[(wave * 16 + 4 * kg + r) * ld + e] = acc[eb][r] + bias;
      }
    }
  }
  __syncthreads();

  if (logits_out != nullptr) {
    for (int idx = tid; idx < kRouteTokens * E; idx += kRouteThreads) {
      const int m = idx / E, e = idx - m * E;
      const int t = tblk + m;
      if (t < ntok) logits_out[size_t(t) * E + e] = lg[m * ld + e];
    }
  }

  if (tid < kRouteTokens) {
    const int t = tblk + tid;
    if (t < ntok) {
      float v[MAXK];
      int id[MAXK];
#pragma unroll
      for (int j = 0; j < MAXK; ++j) {
        v[j] = -INFINITY;
        id[j] = 0;
      }
      const float* my = lg + tid * ld;
      for (int e = 0; e < E; ++e) {
        const float xv = my[e];
        // insert into the descending list; a strict compare keeps earlier (lower) ids ahead of equal scores
#pragma unroll
        for (int j = MAXK - 1; j >= 0; --j) {
          const bool shift = (j > 0) && (v[j > 0 ? j - 1 : 0] < xv);
          if (shift) {
            v[j] = v[j - 1];
            id[j] = id[j - 1];
          } else if (v[j] < xv) {
            v[j] = xv;
            id[j] = e;
          }
        }
      }
      const float top = v[0];
      float ex[MAXK];
      float sum = 0.0f;
#pragma unroll
      for (int j = 0; j < MAXK; ++j) {
        if (j < k) {
          ex[j] = expf(v[j] - top);
          sum += ex[j];
        }
      }
      const float inv = 1.0f / sum;
#pragma unroll
      for (int j = 0; j < MAXK; ++j) {
        if (j < k) {
          const size_t o = size_t(t) * k + j;
          ids[o] = id[j];
          tw[o] = ex[j] * inv;
          if (tl != nullptr) tl[o] = v[j];
        }
      }
    }
  }
}

template <typename T, int NEB, int MAXK>
moe_status launch_route_t(const RouteArgs& a) {
  const moe_layer_desc* d = a.d;
  const int ntok = int(d->num_tokens);
  const int E = d->num_experts;
  const size_t lds = size_t(kRouteTokens) * (E + 1) * sizeof(float);
  auto kern = route_kernel<T, NEB, MAXK>;
  if (lds > 65536) {
    const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                             hipFuncAttributeMaxDynamicSharedMemorySize, int(lds));
    if (e != hipSuccess) return set_error(MOE_ERR_HIP, "route: LDS attribute: %s", hipGetErrorString(e));
  }
  const dim3 grid((ntok + kRouteTokens - 1) / kRouteTokens);
  MOE_LAUNCH("route_topk", kern, grid, dim3(kRouteThreads), lds, a.s, static_cast<const T*>(a.x),
             static_cast<const T*>(a.w_router), a.b_router, a.logits_in, a.logits_out, a.topk_ids, a.topk_w,
             a.topk_logit, ntok, d->hidden, E, d->top_k);
  return MOE_OK;
}

template <typename T, int NEB>
moe_status pick_k(const RouteArgs& a) {
  const int k = a.d->top_k;
  if (k <= 2) return launch_route_t<T, NEB, 2>(a);
  if (k <= 4) return launch_route_t<T, NEB, 4>(a);
  if (k <= 8) return launch_route_t<T, NEB, 8>(a);
  if (k <= 16) return launch_route_t<T, NEB, 16>(a);
  return launch_route_t<T, NEB, 32>(a);
}

template <typename T>
moe_status pick_e(const RouteArgs& a) {
  const int E = a.d->num_experts;
  if (E <= 16) return pick_k<T, 1>(a);
  if (E <= 32) return pick_k<T, 2>(a);
  if (E <= 64) return pick_k<T, 4>(a);
  if (E <= 128) return pick_k<T, 8>(a);
  return pick_k<T, 16>(a);
}

}  // namespace

moe_status launch_route(const RouteArgs& a) {
  return a.d->dtype == MOE_BF16 ? pick_e<bf16_t>(a) : pick_e<float>(a);
}

}  // namespace moe
