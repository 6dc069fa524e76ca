// Stage 4: combine.
//
// Ultralytics glossary "Expert Parallelism", section "How tokens move between
// GPUs", step 4: each token's expert results come back to it and are weighted
// by the router scores and summed (Transformers "Token dispatch": the rank
// combines them with the routing weights).  A pair that is not local or was
// cut by capacity contributes nothing, so a token whose pairs were all cut
// gets zero (its value then reaches the next layer only through the residual
// branch, which is outside this layer's output).
//
// One wave per token: the wave reads the token's k rows of y_sorted through
// pair_row (the inverse permutation), so the un-permute, the weighting and the
// sum are one pass with no atomics; each lane keeps a 16-byte slice of the
// row in float32, loads the slices of up to eight slots at once and adds them
// in slot order j = 0..k-1, then rounds once.
#include "common.h"
#include "kernels.h"

namespace moe {
namespace {

constexpr int kTokensPerBlock = 4;

// KB: slots whose rows are loaded together (k rounded up to 2, 4, 6 or 8; larger k goes in batches of 8);
// each lane takes kSlices 16-byte slices of the row per pass, so KB * kSlices loads are in flight
template <typename T, int KB, int kSlices>
__global__ __launch_bounds__(256) void combine_kernel(const uint4* __restrict__ ys, const int32_t* __restrict__ pair_row,
                                                      const float* __restrict__ tw, int64_t ntok, int k, int vec_per_row,
                                                      uint4* __restrict__ y) {
  constexpr int EPV = 16 / int(sizeof(T));
  const int lane = threadIdx.x & 63;
  const int64_t t = int64_t(blockIdx.x) * kTokensPerBlock + (threadIdx.x >> 6);
  if (t >= ntok) return;
  // lane j < k holds slot j's sorted row and weight; broadcast per slot below
  const int my_row = lane < k ? pair_row[t * k + lane] : -1;
  const float my_w = lane < k ? tw[t * k + lane] : 0.0f;
  uint4* dst = y + size_t(t) * vec_per_row;
  const u32x4_t* src = reinterpret_cast<const u32x4_t*>(ys);
  // every lane runs every pass (the slot broadcasts below read other lanes'
  // registers, so no lane may leave the loop early); slice c0 + 64u + lane
  for (int c0 = 0; c0 < vec_per_row; c0 += 64 * kSlices) {
    float acc[kSlices][EPV];
#pragma unroll
    for (int u = 0; u < kSlices; ++u)
#pragma unroll
      for (int e = 0; e < EPV; ++e) acc[u][e] = 0.0f;
    for (int j0 = 0; j0 < k; j0 += KB) {
      u32x4_t v[kSlices][KB];
#pragma unroll
      for (int jj = 0; jj < KB; ++jj) {
        const int r = __shfl(my_row, j0 + jj, 64);
#pragma unroll
        for (int u = 0; u < kSlices; ++u) {
          const int c = c0 + 64 * u + lane;
          if (j0 + jj < k && r >= 0 && c < vec_per_row) v[u][jj] = src[size_t(r) * vec_per_row + c];
        }
      }
      // accumulate in slot order
#pragma unroll
      for (int jj = 0; jj < KB; ++jj) {
        const int r = __shfl(my_row, j0 + jj, 64);
        const float wj = __shfl(my_w, j0 + jj, 64);
        if (j0 + jj < k && r >= 0) {
#pragma unroll
          for (int u = 0; u < kSlices; ++u) {
            float f[EPV];
            unpack16(make_uint4(v[u][jj][0], v[u][jj][1], v[u][jj][2], v[u][jj][3]), T(), f);
#pragma unroll
            for (int e = 0; e < EPV; ++e) acc[u][e] = fmaf(wj, f[e], acc[u][e]);
          }
        }
      }
    }
#pragma unroll
    for (int u = 0; u < kSlices; ++u) {
      const int c = c0 + 64 * u + lane;
      if (c < vec_per_row) dst[c] = pack16(acc[u], T());
    }
  }
}

template <typename T>
moe_status launch_t(const CombineArgs& a) {
  const moe_layer_desc* d = a.d;
  const int64_t T_ = d->num_tokens;
  const int vec_per_row = int(size_t(d->hidden) * dtype_bytes(d->dtype) / 16);
  const dim3 grid(unsigned((T_ + kTokensPerBlock - 1) / kTokensPerBlock));
  const int k = d->top_k;
  const uint4* ys = static_cast<const uint4*>(a.y_sorted);
  uint4* y = static_cast<uint4*>(a.y);
  // slices per lane and pass: 8 for pairs of slots (4: mixtral_like 35.7 -> 39.1 us, so not), 4 for
  // batches of six or eight; batches of four
  // take 6 when a row then fits fewer, fuller passes (a 2880-wide bf16 row: one pass of 384 slices
  // instead of two of 256; measured 31.0 -> 28.6 us on the gpt-oss-like share).  Five or six slots
  // load as one batch of six rather than eight: 150 registers instead of 184, three waves per SIMD
  // instead of two (skewed_capacity, k = 6: 78.6 -> 73.4 us, same box, interleaved runs)
  const auto waste = [&](int sl) { return (vec_per_row + 64 * sl - 1) / (64 * sl) * 64 * sl - vec_per_row; };
  if (k <= 2) {
    MOE_LAUNCH("combine", (combine_kernel<T, 2, 8>), grid, dim3(256), 0, a.s, ys, a.pair_row, a.topk_w, T_, k,
               vec_per_row, y);
  } else if (k <= 4) {
    if (waste(6) < waste(4)) {
      MOE_LAUNCH("combine", (combine_kernel<T, 4, 6>), grid, dim3(256), 0, a.s, ys, a.pair_row, a.topk_w, T_, k,
                 vec_per_row, y);
    } else {
      MOE_LAUNCH("combine", (combine_kernel<T, 4, 4>), grid, dim3(256), 0, a.s, ys, a.pair_row, a.topk_w, T_, k,
                 vec_per_row, y);
    }
  } else if (k <= 6) {
    MOE_LAUNCH("combine", (combine_kernel<T, 6, 4>), grid, dim3(256), 0, a.s, ys, a.pair_row, a.topk_w, T_, k,
               vec_per_row, y);
  } else {
    MOE_LAUNCH("combine", (combine_kernel<T, 8, 4>), grid, dim3(256), 0, a.s, ys, a.pair_row, a.topk_w, T_, k,
               vec_per_row, y);
  }
  return MOE_OK;
}

}  // namespace

moe_status launch_combine(const CombineArgs& a) {
  return a.d->dtype == MOE_BF16 ? launch_t<bf16_t>(a) : launch_t<float>(a);
}

}  // namespace moe
