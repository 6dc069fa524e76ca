// Stage 3, the skinny grouped-GEMM kernel for decode-sized batches (a few token
// rows per expert): Ultralytics glossary "Expert Parallelism", "How tokens move
// between GPUs", step 3 (each GPU runs its local experts on what it received).
#include <math.h>

#include <algorithm>

#include "ffn_common.h"
#include "kernels.h"

namespace moe {
namespace {

// ---------------------------------------------------------------------------
// Skinny kernel for segments of a few rows (decode-sized batches).
//
// With a handful of rows per expert the product is bound by streaming the
// expert weights from HBM, so the work is split over weight rows: one block
// of four waves owns one expert and 64 consecutive output columns (each wave
// 16 weight rows, or 16 gate + 16 up rows).  A wave multiplies up to 64 of the
// expert's token rows at a time (four MFMA 16x16x32 row blocks) and streams
// its weight rows straight from HBM into registers, eight k-steps of 32 in
// flight per matrix (16-byte loads; two consecutive steps cover a 128-byte
// line of each weight row).  The token rows come through the caches.  An
// expert that received no rows returns before touching its weights.
namespace skinny {

constexpr int kThreads = 256, kMaxRowBlocks = 4;

bool supported(int K) { return K % 32 == 0; }

// Each wave streams two sets of 16 weight rows: for gate/up the gate and the
// up rows of the same 16 output columns, for down two adjacent groups of 16
// output columns.  So a block (four waves) covers 64 gate/up columns or 128
// down columns.  The k loop is double-buffered in registers: the loads of the
// next four 32-k steps are in flight while the MFMAs of the current four run.
template <int NMAT>
constexpr int cols_per_block() { return NMAT == 2 ? 64 : 128; }

// SAVE (gate/up of the training forward): the gate and up pre-activations go to Gs, Us too.
// BKN: the weights are k-major (element (k, n) at B[k * N + n]): each lane then loads
// 16 bytes of one k row (a 32 x 16 block of a stream per step is 32 rows of 32 bytes),
// the wave parks the block in its own 1 KB of LDS and reads the fragments back with
// transposing reads, so the MFMAs see the same operands as with n-major weights.
template <int NMAT, bool SAVE, bool BKN>
__global__ __launch_bounds__(kThreads) void gemm_kernel(const bf16_t* __restrict__ A, const int32_t* __restrict__ offsets,
                                                        const bf16_t* __restrict__ B0, const bf16_t* __restrict__ B1,
                                                        bf16_t* __restrict__ C, int N, int K, bf16_t* __restrict__ Gs,
                                                        bf16_t* __restrict__ Us) {
  constexpr int kWaveCols = NMAT == 2 ? 16 : 32;
  constexpr int kPipe = 4;
  const int expert = blockIdx.y;
  const int seg0 = offsets[expert];
  const int seg_n = offsets[expert + 1] - seg0;
  if (seg_n <= 0) return;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int col0 = blockIdx.x * cols_per_block<NMAT>() + wave * kWaveCols;  // first output column of this wave
  if (col0 >= N) return;
  const size_t boff = size_t(expert) * N * K;
  const int kg = (lane >> 4) * 8;  // the lane's 8 k values within a step
  const bf16_t* bs0;
  const bf16_t* bs1;
  size_t kstride;  // elements between consecutive k of a lane's stream
  if constexpr (!BKN) {
    // stream 0 / 1 weight row of this lane (rows past N repeat row N-1; never stored)
    const int wrow0 = min(col0 + (lane & 15), N - 1);
    const int wrow1 = NMAT == 2 ? wrow0 : min(col0 + 16 + (lane & 15), N - 1);
    bs0 = B0 + boff + size_t(wrow0) * K + kg;
    bs1 = (NMAT == 2 ? B1 : B0) + boff + size_t(wrow1) * K + kg;
    kstride = 1;
  } else {
    // lane l loads k row l/2 of the step, columns c + 8 (l % 2) .. +7 of its stream's 16
    // (chunks past N re-read the last chunk of the row; never stored)
    const int c0 = min(col0 + 8 * (lane & 1), N - 8);
    const int c1 = NMAT == 2 ? c0 : min(col0 + 16 + 8 * (lane & 1), N - 8);
    bs0 = B0 + boff + size_t(lane >> 1) * N + c0;
    bs1 = (NMAT == 2 ? B1 : B0) + boff + size_t(lane >> 1) * N + c1;
    kstride = size_t(N);
  }
  // the wave's LDS blocks (k-major weights only): [stream][step] 1 KB each; row r of a
  // block at 32-byte slot r ^ 4 (r / 8 % 2), so a transposing read's two row quads per
  // half wave fall in different bank halves
  __shared__ __attribute__((aligned(1024))) char park[BKN ? 4 * 2 * kPipe * 1024 : 16];
  char* wpark = park + (BKN ? wave * 2 * kPipe * 1024 : 0);
  auto slot = [](int r) { return (r ^ (((r >> 3) & 1) << 2)) * 32; };
  const int woff = slot(lane >> 1) + 16 * (lane & 1);  // this lane's store
  // its transposing reads: k rows 8 (lane / 16) + (lane % 16) / 4 and four rows down
  const int roff0 = slot(8 * (lane >> 4) + ((lane & 15) >> 2)) + 8 * (lane & 3);
  const int roff1 = slot(8 * (lane >> 4) + ((lane & 15) >> 2) + 4) + 8 * (lane & 3);

  for (int m0 = 0; m0 < seg_n; m0 += 16 * kMaxRowBlocks) {
    const int nrb = min(kMaxRowBlocks, (seg_n - m0 + 15) / 16);
    // token row of each row block for this lane (rows past the segment repeat its last row)
    const bf16_t* arow[kMaxRowBlocks];
#pragma unroll
    for (int rb = 0; rb < kMaxRowBlocks; ++rb)
      arow[rb] = A + size_t(seg0 + min(m0 + rb * 16 + (lane & 15), seg_n - 1)) * K + kg;
    f32x4_t acc[2][kMaxRowBlocks];
#pragma unroll
    for (int m = 0; m < 2; ++m)
#pragma unroll
      for (int rb = 0; rb < kMaxRowBlocks; ++rb) acc[m][rb] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    // two register sets of kPipe k steps: the loads of the next set are in flight
    // while the MFMAs of the current one run (four steps per set: fewer waves
    // fit, but each keeps more in flight; same-box A/B on the decode-sized
    // layer: 0 to -4% per layer against two steps, while capping registers for
    // more waves per SIMD made it 12% slower)
    bf16x8_t w0[2][kPipe], w1[2][kPipe], a0[2][kPipe];
    const int nset = K / (32 * kPipe);
    auto load_set = [&](int b, int k0) {
#pragma unroll
      for (int u = 0; u < kPipe; ++u) {
        w0[b][u] = *reinterpret_cast<const bf16x8_t*>(bs0 + size_t(k0 + 32 * u) * kstride);
        w1[b][u] = *reinterpret_cast<const bf16x8_t*>(bs1 + size_t(k0 + 32 * u) * kstride);
        a0[b][u] = *reinterpret_cast<const bf16x8_t*>(arow[0] + k0 + 32 * u);
      }
    };
    // k-major weights: park the loaded blocks, then read the fragments back transposed
    auto transpose_set = [&](int b) {
      if constexpr (BKN) {
#pragma unroll
        for (int u = 0; u < kPipe; ++u) {
          *reinterpret_cast<bf16x8_t*>(wpark + u * 1024 + woff) = w0[b][u];
          *reinterpret_cast<bf16x8_t*>(wpark + (kPipe + u) * 1024 + woff) = w1[b][u];
        }
#pragma unroll
        for (int u = 0; u < kPipe; ++u) {
          w0[b][u] = read_kn_frag2(wpark + u * 1024 + roff0, wpark + u * 1024 + roff1);
          w1[b][u] = read_kn_frag2(wpark + (kPipe + u) * 1024 + roff0, wpark + (kPipe + u) * 1024 + roff1);
        }
      }
    };
    auto mma_set = [&](int b, int k0) {
      transpose_set(b);
#pragma unroll
      for (int u = 0; u < kPipe; ++u) {
#pragma unroll
        for (int rb = 0; rb < kMaxRowBlocks; ++rb) {
          if (rb < nrb) {
            const bf16x8_t a = rb == 0 ? a0[b][u] : *reinterpret_cast<const bf16x8_t*>(arow[rb] + k0 + 32 * u);
            acc[0][rb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, w0[b][u], acc[0][rb], 0, 0, 0);
            acc[1][rb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, w1[b][u], acc[1][rb], 0, 0, 0);
          }
        }
      }
    };
    if (nset > 0) load_set(0, 0);
    int set = 0;
    for (; set + 2 <= nset; set += 2) {
      load_set(1, (set + 1) * 32 * kPipe);
      mma_set(0, set * 32 * kPipe);
      if (set + 2 < nset) load_set(0, (set + 2) * 32 * kPipe);
      mma_set(1, (set + 1) * 32 * kPipe);
    }
    if (set < nset) mma_set(0, set * 32 * kPipe);
    int k0 = nset * 32 * kPipe;
    for (; k0 < K; k0 += 32) {
      bf16x8_t v0 = *reinterpret_cast<const bf16x8_t*>(bs0 + size_t(k0) * kstride);
      bf16x8_t v1 = *reinterpret_cast<const bf16x8_t*>(bs1 + size_t(k0) * kstride);
      if constexpr (BKN) {
        *reinterpret_cast<bf16x8_t*>(wpark + woff) = v0;
        *reinterpret_cast<bf16x8_t*>(wpark + kPipe * 1024 + woff) = v1;
        v0 = read_kn_frag2(wpark + roff0, wpark + roff1);
        v1 = read_kn_frag2(wpark + kPipe * 1024 + roff0, wpark + kPipe * 1024 + roff1);
      }
#pragma unroll
      for (int rb = 0; rb < kMaxRowBlocks; ++rb) {
        if (rb < nrb) {
          const bf16x8_t a = *reinterpret_cast<const bf16x8_t*>(arow[rb] + k0);
          acc[0][rb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, v0, acc[0][rb], 0, 0, 0);
          acc[1][rb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, v1, acc[1][rb], 0, 0, 0);
        }
      }
    }
    // 16x16 layout: lane -> weight row (column of the output) lane & 15,
    // register i -> token row 4*(lane/16) + i of the row block
#pragma unroll
    for (int rb = 0; rb < kMaxRowBlocks; ++rb) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = m0 + rb * 16 + 4 * (lane >> 4) + i;
        if (rb < nrb && r < seg_n) {
          bf16_t* crow = C + size_t(seg0 + r) * N;
          if (NMAT == 2) {
            const int col = col0 + (lane & 15);
            if (col < N) {
              crow[col] = f32_to_bf16(silu(acc[0][rb][i]) * acc[1][rb][i]);
              if constexpr (SAVE) {
                Gs[size_t(seg0 + r) * N + col] = f32_to_bf16(acc[0][rb][i]);
                Us[size_t(seg0 + r) * N + col] = f32_to_bf16(acc[1][rb][i]);
              }
            }
          } else {
#pragma unroll
            for (int s = 0; s < 2; ++s) {
              const int col = col0 + 16 * s + (lane & 15);
              if (col < N) crow[col] = f32_to_bf16(acc[s][rb][i]);
            }
          }
        }
      }
    }
  }
}

// bkn: k-major weights (see gemm_kernel)
template <int NMAT>
moe_status launch(const char* name, const bf16_t* A, const int32_t* offsets, const bf16_t* B0, const bf16_t* B1,
                  bf16_t* C, int L, int N, int K, bool bkn, hipStream_t s, bf16_t* Gs = nullptr, bf16_t* Us = nullptr) {
  const dim3 grid(unsigned((N + cols_per_block<NMAT>() - 1) / cols_per_block<NMAT>()), unsigned(L));
#define MOE_SKINNY(SAVE_)                                                                                          \
  do {                                                                                                             \
    if (bkn)                                                                                                       \
      MOE_LAUNCH(name, (gemm_kernel<NMAT, SAVE_, true>), grid, dim3(kThreads), 0, s, A, offsets, B0, B1, C, N, K, Gs, Us); \
    else                                                                                                           \
      MOE_LAUNCH(name, (gemm_kernel<NMAT, SAVE_, false>), grid, dim3(kThreads), 0, s, A, offsets, B0, B1, C, N, K, Gs, Us); \
  } while (0)
  if (NMAT == 2 && Gs != nullptr) {
    MOE_SKINNY(true);
  } else {
    MOE_SKINNY(false);
  }
#undef MOE_SKINNY
  return MOE_OK;
}

}  // namespace skinny

}  // namespace

bool skinny_ffn_fits(const moe_layer_desc* d, int64_t max_pairs) {
  return d->dtype == MOE_BF16 && max_pairs <= int64_t(32) * d->local_count && skinny::supported(d->hidden) &&
         skinny::supported(d->intermediate);
}

moe_status launch_skinny_ffn(const FfnArgs& a) {
  const moe_layer_desc* d = a.d;
  const int L = d->local_count, H = d->hidden, I = d->intermediate;
  bf16_t* h = static_cast<bf16_t*>(a.h);
  const bool kn = d->weight_layout == MOE_WEIGHTS_IN_OUT;
  moe_status st = skinny::launch<2>("ffn_gate_up", static_cast<const bf16_t*>(a.x_sorted), a.offsets,
                                    static_cast<const bf16_t*>(a.w_gate), static_cast<const bf16_t*>(a.w_up), h, L, I,
                                    H, kn, a.s, static_cast<bf16_t*>(a.g_out), static_cast<bf16_t*>(a.u_out));
  if (st != MOE_OK) return st;
  return skinny::launch<1>("ffn_down", h, a.offsets, static_cast<const bf16_t*>(a.w_down),
                           static_cast<const bf16_t*>(a.w_down), static_cast<bf16_t*>(a.y_sorted), L, H, I, kn, a.s);
}

}  // namespace moe
