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

template <typename T>
__global__ __launch_bounds__(256) void combine_kernel(const uint4* __restrict__ ys, const int32_t* __restrict__ pair_row,
                                                      const float* __restrict__ tw, int64_t ntok, int k, int vec_per_row,
                                                      uint4* __restrict__ y) {
  constexpr int EPV = 16 / int(sizeof(T));
  constexpr int kBatch = 8;  // slots whose rows are in flight together
  const int lane = threadIdx.x & 63;
  const int64_t t = int64_t(blockIdx.x) * kTokensPerBlock + (threadIdx.x >> 6);
  if (t >= ntok) return;
  // lane j < k holds slot j's sorted row and weight; broadcast per slot below
  const int my_row = lane < k ? pair_row[t * k + lane] : -1;
  const float my_w = lane < k ? tw[t * k + lane] : 0.0f;
  uint4* dst = y + size_t(t) * vec_per_row;
  for (int c = lane; c < vec_per_row; c += 64) {
    float acc[EPV];
#pragma unroll
    for (int e = 0; e < EPV; ++e) acc[e] = 0.0f;
    for (int j0 = 0; j0 < k; j0 += kBatch) {
      u32x4_t v[kBatch];
#pragma unroll
      for (int jj = 0; jj < kBatch; ++jj) {
        const int r = __shfl(my_row, j0 + jj, 64);
        if (j0 + jj < k && r >= 0) v[jj] = reinterpret_cast<const u32x4_t*>(ys)[size_t(r) * vec_per_row + c];
      }
      // accumulate in slot order
#pragma unroll
      for (int jj = 0; jj < kBatch; ++jj) {
        const int r = __shfl(my_row, j0 + jj, 64);
        const float wj = __shfl(my_w, j0 + jj, 64);
        if (j0 + jj < k && r >= 0) {
          float f[EPV];
          unpack16(make_uint4(v[jj][0], v[jj][1], v[jj][2], v[jj][3]), T(), f);
#pragma unroll
          for (int e = 0; e < EPV; ++e) acc[e] = fmaf(wj, f[e], acc[e]);
        }
      }
    }
    dst[c] = pack16(acc, T());
  }
}

}  // namespace

moe_status launch_combine(const CombineArgs& a) {
  const moe_layer_desc* d = a.d;
  const int64_t T = d->num_tokens;
  const int vec_per_row = int(size_t(d->hidden) * dtype_bytes(d->dtype) / 16);
  const dim3 grid(unsigned((T + kTokensPerBlock - 1) / kTokensPerBlock));
  if (d->dtype == MOE_BF16) {
    MOE_LAUNCH("combine", combine_kernel<bf16_t>, grid, dim3(256), 0, a.s, static_cast<const uint4*>(a.y_sorted),
               a.pair_row, a.topk_w, T, d->top_k, vec_per_row, static_cast<uint4*>(a.y));
  } else {
    MOE_LAUNCH("combine", combine_kernel<float>, grid, dim3(256), 0, a.s, static_cast<const uint4*>(a.y_sorted),
               a.pair_row, a.topk_w, T, d->top_k, vec_per_row, static_cast<uint4*>(a.y));
  }
  return MOE_OK;
}

}  // namespace moe
