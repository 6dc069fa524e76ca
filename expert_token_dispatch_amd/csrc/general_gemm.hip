// Stage 3, the general grouped-GEMM kernel: float32 layers and bf16 shapes off the
// large tile's grid (see grouped_gemm.hip for the path that picks it).
//
// Ultralytics glossary "Expert Parallelism", section "How tokens move between
// GPUs", step 3: each GPU runs its local experts on the tokens it received.
// The Transformers page names the expert kernel style "grouped_gemm" and says
// the expert weights are split along the expert dimension: they are stacked per
// local expert, n-major ([out, in], a linear layer's layout) or k-major
// ([in, out], the math form).  Expert i owns sorted rows [offsets[i],
// offsets[i+1]) and computes the SwiGLU feed-forward (math form)
//   h = silu(X Wg_i) * (X Wu_i)      (gate/up kernel, SwiGLU in its epilogue)
//   y = h Wd_i                       (down kernel)
// with float32 accumulation; h is rounded to the storage type once.
//
// Work split: one block computes a BM x BN output tile (both the gate and the
// up tile for the gate/up kernel, so SiLU(gate)*up is formed in registers).
// grid.x enumerates m-tile slots: expert i contributes ceil(n_i / BM) of them,
// found on the device from `offsets` (no host sync), and the grid is sized for
// the worst case ceil(P_max / BM) + L so surplus blocks exit at once.
// grid.y enumerates n-tiles.  Four waves split the tile 2 x 2; each wave owns
// 64 x 64 per matrix as 2 x 2 MFMA 32x32 blocks (bf16: v_mfma 32x32x16, the
// lane holds 8 consecutive k of its row/column; f32: eight 32x32x2 steps over
// the same 8 values).  A and B k-slices are staged through double-buffered LDS
// with rows padded to 80 bytes so the 16-byte fragment reads of eight lanes
// fall in distinct banks.
#include <math.h>

#include <algorithm>

#include "ffn_common.h"
#include "kernels.h"

namespace moe {
namespace {

constexpr int BM = 128, BN = 128, kThreads = 256;

template <typename T> struct Gemm;
template <> struct Gemm<bf16_t> {
  static constexpr int BK = 32;       // k per LDS stage
  static constexpr int kLd = BK + 8;  // LDS row stride in elements (80 bytes)
  static constexpr int kFragVec = 1;  // uint4 per lane per 16-k chunk
  __device__ static void mma(const uint4* a, const uint4* b, f32x16_t& c) {
    c = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a[0]), __builtin_bit_cast(bf16x8_t, b[0]),
                                                c, 0, 0, 0);
  }
};
template <> struct Gemm<float> {
  static constexpr int BK = 16;
  static constexpr int kLd = BK + 4;  // 80 bytes
  static constexpr int kFragVec = 2;
  __device__ static void mma(const uint4* a, const uint4* b, f32x16_t& c) {
#pragma unroll
    for (int v = 0; v < 2; ++v) {
      c = __builtin_amdgcn_mfma_f32_32x32x2f32(__uint_as_float(a[v].x), __uint_as_float(b[v].x), c, 0, 0, 0);
      c = __builtin_amdgcn_mfma_f32_32x32x2f32(__uint_as_float(a[v].y), __uint_as_float(b[v].y), c, 0, 0, 0);
      c = __builtin_amdgcn_mfma_f32_32x32x2f32(__uint_as_float(a[v].z), __uint_as_float(b[v].z), c, 0, 0, 0);
      c = __builtin_amdgcn_mfma_f32_32x32x2f32(__uint_as_float(a[v].w), __uint_as_float(b[v].w), c, 0, 0, 0);
    }
  }
};


// NMAT = 2: gate and up products with the SwiGLU epilogue; NMAT = 1: plain product.
// Tiles of BMT (128 or 64) token rows x BN weight rows; the waves split them 2 x 2,
// so a wave holds BMT/64 x 2 MFMA 32x32 blocks per matrix.  BKN: the weights are
// k-major (element (k, n) at B[k * N + n]); thread t then loads k rows 2p and 2p+1
// (p = t % (BK/2)) of 16-byte column chunk t / (BK/2) and stores them into the
// [BN][BK] tile as (k, k+1) pairs, so the tile is the one n-major weights give.
template <typename T, int NMAT, int BMT, bool BKN>
__global__ __launch_bounds__(kThreads) void grouped_gemm_kernel(const T* __restrict__ A,
                                                                const int32_t* __restrict__ offsets,
                                                                const T* __restrict__ B0, const T* __restrict__ B1,
                                                                T* __restrict__ C, int L, int N, int K,
                                                                T* __restrict__ Gs, T* __restrict__ Us) {
  using G = Gemm<T>;
  constexpr int BK = G::BK, kLd = G::kLd, FV = G::kFragVec;
  constexpr int EPV = 16 / int(sizeof(T));     // elements per 16-byte vector
  constexpr int CPR = BK / EPV;                // 16-byte chunks per tile row (4)
  constexpr int CPTA = BMT * CPR / kThreads;   // A chunks per thread (2 or 1)
  constexpr int CPTB = BN * CPR / kThreads;    // B chunks per thread per matrix (2)
  constexpr int MI = BMT / 64;                 // 32-row blocks per wave

  // ---- which expert and rows this block owns --------------------------------
  int g = blockIdx.x;
  int expert = -1, row0 = 0, rows = 0;
  {
    int prev = offsets[0];
    for (int i = 0; i < L; ++i) {
      const int nxt = offsets[i + 1];
      const int tiles = (nxt - prev + BMT - 1) / BMT;
      if (g < tiles) {
        expert = i;
        row0 = prev + g * BMT;
        rows = min(BMT, nxt - row0);
        break;
      }
      g -= tiles;
      prev = nxt;
    }
  }
  if (expert < 0) return;
  const int n0 = blockIdx.y * BN;
  const size_t boff = size_t(expert) * N * K;
  const T* Bm[2] = {B0 + boff, NMAT > 1 ? B1 + boff : B0 + boff};

  __shared__ __attribute__((aligned(16))) T As[2][BMT * kLd];
  __shared__ __attribute__((aligned(16))) T Bs[2][NMAT][BN * kLd];

  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int wm = wave >> 1, wn = wave & 1;
  const uint4 zero = make_uint4(0, 0, 0, 0);

  uint4 ra[CPTA], rb[NMAT][CPTB];
  constexpr int KP = BK / 2;  // k-major weights: (k, k+1) pairs per tile column
  static_assert(!BKN || (KP * (BN / EPV) == kThreads && CPTB == 2), "one pair unit per thread");
  auto gload = [&](int k0) {
#pragma unroll
    for (int j = 0; j < CPTA; ++j) {
      const int c = tid + j * kThreads;
      const int r = c / CPR, col = c % CPR;
      const int kk = k0 + col * EPV;
      const int ar = min(r, rows - 1);  // rows past the segment repeat its last row; never stored
      ra[j] = kk < K ? *reinterpret_cast<const uint4*>(A + size_t(row0 + ar) * K + kk) : zero;
    }
    if constexpr (!BKN) {
#pragma unroll
      for (int j = 0; j < CPTB; ++j) {
        const int c = tid + j * kThreads;
        const int r = c / CPR, col = c % CPR;
        const int kk = k0 + col * EPV;
#pragma unroll
        for (int m = 0; m < NMAT; ++m) {
          const int nr = n0 + r;
          rb[m][j] = (kk < K && nr < N) ? *reinterpret_cast<const uint4*>(Bm[m] + size_t(nr) * K + kk) : zero;
        }
      }
    } else {
      // N is a multiple of 8, so a chunk is wholly inside or wholly past column N
      const int p = tid % KP, n = n0 + (tid / KP) * EPV, kk = k0 + 2 * p;
#pragma unroll
      for (int m = 0; m < NMAT; ++m)
#pragma unroll
        for (int h = 0; h < 2; ++h)
          rb[m][h] = (n < N && kk + h < K) ? *reinterpret_cast<const uint4*>(Bm[m] + size_t(kk + h) * N + n) : zero;
    }
  };
  auto sstore = [&](int buf) {
#pragma unroll
    for (int j = 0; j < CPTA; ++j) {
      const int c = tid + j * kThreads;
      const int r = c / CPR, col = c % CPR;
      *reinterpret_cast<uint4*>(&As[buf][r * kLd + col * EPV]) = ra[j];
    }
    if constexpr (!BKN) {
#pragma unroll
      for (int j = 0; j < CPTB; ++j) {
        const int c = tid + j * kThreads;
        const int r = c / CPR, col = c % CPR;
#pragma unroll
        for (int m = 0; m < NMAT; ++m) *reinterpret_cast<uint4*>(&Bs[buf][m][r * kLd + col * EPV]) = rb[m][j];
      }
    } else {
      const int p = tid % KP, c0 = (tid / KP) * EPV;
#pragma unroll
      for (int m = 0; m < NMAT; ++m) {
        const uint32_t a[4] = {rb[m][0].x, rb[m][0].y, rb[m][0].z, rb[m][0].w};
        const uint32_t b[4] = {rb[m][1].x, rb[m][1].y, rb[m][1].z, rb[m][1].w};
        if constexpr (sizeof(T) == 2) {
#pragma unroll
          for (int w = 0; w < 4; ++w) {
            // column 2w: the low halves of rows k and k+1, column 2w+1: the high halves
            *reinterpret_cast<uint32_t*>(&Bs[buf][m][(c0 + 2 * w) * kLd + 2 * p]) = (a[w] & 0xFFFFu) | (b[w] << 16);
            *reinterpret_cast<uint32_t*>(&Bs[buf][m][(c0 + 2 * w + 1) * kLd + 2 * p]) =
                (a[w] >> 16) | (b[w] & 0xFFFF0000u);
          }
        } else {
#pragma unroll
          for (int w = 0; w < 4; ++w)
            *reinterpret_cast<uint2*>(&Bs[buf][m][(c0 + w) * kLd + 2 * p]) = make_uint2(a[w], b[w]);
        }
      }
    }
  };

  f32x16_t acc[NMAT][MI][2];
#pragma unroll
  for (int m = 0; m < NMAT; ++m)
#pragma unroll
    for (int i = 0; i < MI; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[m][i][j][r] = 0.0f;

  const int nk = (K + BK - 1) / BK;
  gload(0);
  sstore(0);
  __syncthreads();
  const int frow = lane & 31;            // row (A) / column (B) inside a 32-block
  const int fk = 8 * (lane >> 5);        // first of the lane's 8 k values in a 16-k chunk
  for (int kt = 0; kt < nk; ++kt) {
    const int buf = kt & 1;
    if (kt + 1 < nk) gload((kt + 1) * BK);
#pragma unroll
    for (int kc = 0; kc < BK / 16; ++kc) {
      uint4 af[MI][FV], bfr[NMAT][2][FV];
#pragma unroll
      for (int i = 0; i < MI; ++i) {
        const uint4* p =
            reinterpret_cast<const uint4*>(&As[buf][(wm * (BMT / 2) + i * 32 + frow) * kLd + kc * 16 + fk]);
#pragma unroll
        for (int v = 0; v < FV; ++v) af[i][v] = p[v];
      }
#pragma unroll
      for (int m = 0; m < NMAT; ++m)
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          const uint4* p =
              reinterpret_cast<const uint4*>(&Bs[buf][m][(wn * 64 + j * 32 + frow) * kLd + kc * 16 + fk]);
#pragma unroll
          for (int v = 0; v < FV; ++v) bfr[m][j][v] = p[v];
        }
#pragma unroll
      for (int m = 0; m < NMAT; ++m)
#pragma unroll
        for (int i = 0; i < MI; ++i)
#pragma unroll
          for (int j = 0; j < 2; ++j) G::mma(af[i], bfr[m][j], acc[m][i][j]);
    }
    if (kt + 1 < nk) sstore(buf ^ 1);
    __syncthreads();
  }

  // ---- epilogue: 32x32 accumulator layout, lane -> column (lane & 31),
  // register r -> row 8*(r/4) + 4*(lane/32) + r%4 ------------------------------
#pragma unroll
  for (int i = 0; i < MI; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int col = n0 + wn * 64 + j * 32 + (lane & 31);
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int rt = wm * (BMT / 2) + i * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
        if (rt < rows && col < N) {
          float v;
          if constexpr (NMAT == 2) {
            v = silu(acc[0][i][j][r]) * acc[1][i][j][r];
            if (Gs != nullptr) {  // training: keep the pre-activations for the backward
              Gs[size_t(row0 + rt) * N + col] = Elem<T>::from_f32(acc[0][i][j][r]);
              Us[size_t(row0 + rt) * N + col] = Elem<T>::from_f32(acc[1][i][j][r]);
            }
          } else {
            v = acc[0][i][j][r];
          }
          C[size_t(row0 + rt) * N + col] = Elem<T>::from_f32(v);
        }
      }
    }
}

template <typename T, int BMT, bool BKN>
moe_status launch_bm(const FfnArgs& a) {
  const moe_layer_desc* d = a.d;
  const int L = d->local_count, H = d->hidden, I = d->intermediate;
  const unsigned mslots = unsigned((a.max_pairs + BMT - 1) / BMT + L);
  MOE_LAUNCH("ffn_gate_up", (grouped_gemm_kernel<T, 2, BMT, BKN>), dim3(mslots, (I + BN - 1) / BN), dim3(kThreads), 0,
             a.s, static_cast<const T*>(a.x_sorted), a.offsets, static_cast<const T*>(a.w_gate),
             static_cast<const T*>(a.w_up), static_cast<T*>(a.h), L, I, H, static_cast<T*>(a.g_out),
             static_cast<T*>(a.u_out));
  MOE_LAUNCH("ffn_down", (grouped_gemm_kernel<T, 1, BMT, BKN>), dim3(mslots, (H + BN - 1) / BN), dim3(kThreads), 0,
             a.s, static_cast<const T*>(a.h), a.offsets, static_cast<const T*>(a.w_down),
             static_cast<const T*>(a.w_down), static_cast<T*>(a.y_sorted), L, H, I, static_cast<T*>(nullptr),
             static_cast<T*>(nullptr));
  return MOE_OK;
}

template <typename T, int BMT>
moe_status launch_bm(const FfnArgs& a) {
  return a.d->weight_layout == MOE_WEIGHTS_IN_OUT ? launch_bm<T, BMT, true>(a) : launch_bm<T, BMT, false>(a);
}

// 64-row tiles when 128-row tiles would leave fewer than two blocks per CU (the
// fp32 layer's 8 experts x ~1024 rows x 256 columns: 144 blocks of 128 rows)
template <typename T>
moe_status launch_t(const FfnArgs& a) {
  const moe_layer_desc* d = a.d;
  const int64_t nb = std::min((d->intermediate + BN - 1) / BN, (d->hidden + BN - 1) / BN);
  if (((a.max_pairs + BM - 1) / BM + d->local_count) * nb < 512) return launch_bm<T, 64>(a);
  return launch_bm<T, 128>(a);
}

}  // namespace

moe_status launch_general_ffn(const FfnArgs& a) {
  return a.d->dtype == MOE_BF16 ? launch_t<bf16_t>(a) : launch_t<float>(a);
}

}  // namespace moe
