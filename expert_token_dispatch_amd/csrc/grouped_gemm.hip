// Stage 3: the local experts as one grouped GEMM over ragged segments.
//
// Ultralytics glossary "Expert Parallelism", section "How tokens move between
// GPUs", step 3: each GPU runs its local experts on the tokens it received.
// The Transformers page names the expert kernel style "grouped_gemm" and says
// the expert weights are split along the expert dimension, which is the
// stacked [L, out, in] layout used here.  Expert i owns sorted rows
// [offsets[i], offsets[i+1]) and computes the SwiGLU feed-forward
//   h = silu(X Wg_i^T) * (X Wu_i^T)      (gate/up kernel, SwiGLU in its epilogue)
//   y = h Wd_i^T                         (down kernel)
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

#include "common.h"
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

__device__ __forceinline__ float silu(float z) { return z / (1.0f + __expf(-z)); }

// NMAT = 2: gate and up products with the SwiGLU epilogue; NMAT = 1: plain product.
template <typename T, int NMAT>
__global__ __launch_bounds__(kThreads) void grouped_gemm_kernel(const T* __restrict__ A,
                                                                const int32_t* __restrict__ offsets,
                                                                const T* __restrict__ B0, const T* __restrict__ B1,
                                                                T* __restrict__ C, int L, int N, int K) {
  using G = Gemm<T>;
  constexpr int BK = G::BK, kLd = G::kLd, FV = G::kFragVec;
  constexpr int EPV = 16 / int(sizeof(T));     // elements per 16-byte vector
  constexpr int CPR = BK / EPV;                // 16-byte chunks per tile row (4)
  constexpr int CPT = BM * CPR / kThreads;     // chunks per thread per matrix (2)
  static_assert(BM == BN, "one chunk map serves A and B");

  // ---- which expert and rows this block owns --------------------------------
  int g = blockIdx.x;
  int expert = -1, row0 = 0, rows = 0;
  {
    int prev = offsets[0];
    for (int i = 0; i < L; ++i) {
      const int nxt = offsets[i + 1];
      const int tiles = (nxt - prev + BM - 1) / BM;
      if (g < tiles) {
        expert = i;
        row0 = prev + g * BM;
        rows = min(BM, nxt - row0);
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

  __shared__ __attribute__((aligned(16))) T As[2][BM * kLd];
  __shared__ __attribute__((aligned(16))) T Bs[2][NMAT][BN * kLd];

  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int wm = wave >> 1, wn = wave & 1;
  const uint4 zero = make_uint4(0, 0, 0, 0);

  uint4 ra[CPT], rb[NMAT][CPT];
  auto gload = [&](int k0) {
#pragma unroll
    for (int j = 0; j < CPT; ++j) {
      const int c = tid + j * kThreads;
      const int r = c / CPR, col = c % CPR;
      const int kk = k0 + col * EPV;
      const bool kok = kk < K;
      const int ar = min(r, rows - 1);  // rows past the segment repeat its last row; never stored
      ra[j] = kok ? *reinterpret_cast<const uint4*>(A + size_t(row0 + ar) * K + kk) : zero;
#pragma unroll
      for (int m = 0; m < NMAT; ++m) {
        const int nr = n0 + r;
        rb[m][j] = (kok && nr < N) ? *reinterpret_cast<const uint4*>(Bm[m] + size_t(nr) * K + kk) : zero;
      }
    }
  };
  auto sstore = [&](int buf) {
#pragma unroll
    for (int j = 0; j < CPT; ++j) {
      const int c = tid + j * kThreads;
      const int r = c / CPR, col = c % CPR;
      *reinterpret_cast<uint4*>(&As[buf][r * kLd + col * EPV]) = ra[j];
#pragma unroll
      for (int m = 0; m < NMAT; ++m) *reinterpret_cast<uint4*>(&Bs[buf][m][r * kLd + col * EPV]) = rb[m][j];
    }
  };

  f32x16_t acc[NMAT][2][2];
#pragma unroll
  for (int m = 0; m < NMAT; ++m)
#pragma unroll
    for (int i = 0; i < 2; ++i)
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
      uint4 af[2][FV], bfr[NMAT][2][FV];
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const uint4* p = reinterpret_cast<const uint4*>(&As[buf][(wm * 64 + i * 32 + frow) * kLd + kc * 16 + fk]);
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
        for (int i = 0; i < 2; ++i)
#pragma unroll
          for (int j = 0; j < 2; ++j) G::mma(af[i], bfr[m][j], acc[m][i][j]);
    }
    if (kt + 1 < nk) sstore(buf ^ 1);
    __syncthreads();
  }

  // ---- epilogue: 32x32 accumulator layout, lane -> column (lane & 31),
  // register r -> row 8*(r/4) + 4*(lane/32) + r%4 ------------------------------
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int col = n0 + wn * 64 + j * 32 + (lane & 31);
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int rt = wm * 64 + i * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
        if (rt < rows && col < N) {
          float v;
          if constexpr (NMAT == 2) {
            v = silu(acc[0][i][j][r]) * acc[1][i][j][r];
          } else {
            v = acc[0][i][j][r];
          }
          C[size_t(row0 + rt) * N + col] = Elem<T>::from_f32(v);
        }
      }
    }
}

// ---------------------------------------------------------------------------
// Large-tile bf16 kernel for segments of hundreds of rows and more.
//
// 512 threads (8 waves, two per SIMD, so one wave's memory waits overlap the
// other's MFMAs) own a 256-row x 256-column tile of B rows: for the gate/up
// product that is 128 gate rows and the same 128 up rows (output 256 x 128),
// for the down product 256 output columns.  Waves are arranged 2 (M) x 4 (N);
// a wave holds 4 x 2 MFMA 32x32 accumulators (128 registers).  K advances 64
// at a time through two LDS stages of 72 KB each (rows padded to 144 bytes so
// 16-byte fragment reads of 16 lanes touch 64 distinct banks); the next
// stage's global loads are in flight while the current one is multiplied.
//
// Tile order: the blocks that run at the same time on one XCD (the hardware
// deals workgroups to the 8 XCDs round robin) get consecutive tile numbers,
// and tile numbers run over (expert, group of kGroupN n-tiles, m-tile, n-tile
// in group), so one XCD's L2 serves a few weight tiles to all m-tiles of an
// expert and a few activation tiles to several n-tiles.
namespace big {

constexpr int BM = 256, BNE = 256, BK = 64, LD = BK + 8, kThreads = 512;
constexpr int kStageA = BM * LD, kStageB = BNE * LD;  // elements
constexpr size_t kLdsBytes = size_t(2) * (kStageA + kStageB) * sizeof(bf16_t);
constexpr int kGroupN = 4;
constexpr int kXcds = 8;

template <int NMAT>
__global__ __launch_bounds__(kThreads) void gemm_kernel(const bf16_t* __restrict__ A, const int32_t* __restrict__ offsets,
                                                        const bf16_t* __restrict__ B0, const bf16_t* __restrict__ B1,
                                                        bf16_t* __restrict__ C, int L, int N, int K) {
  constexpr int ON = NMAT == 2 ? BNE / 2 : BNE;  // output columns per tile
  const int NT = (N + ON - 1) / ON;

  // ---- tile number -> (expert, m-tile, n-tile), all from device offsets ----
  int mt_total = 0;
  for (int i = 0; i < L; ++i) mt_total += (offsets[i + 1] - offsets[i] + BM - 1) / BM;
  const int R = mt_total * NT;
  const int id = blockIdx.x;
  if (id >= R) return;
  const int xcd = id % kXcds, loc = id / kXcds;
  const int q = R / kXcds, rr = R % kXcds;
  int t = xcd * q + min(xcd, rr) + loc;
  int expert = 0, seg0 = 0, seg_n = 0, mt_e = 0;
  for (int i = 0; i < L; ++i) {
    const int a = offsets[i], b = offsets[i + 1];
    const int m = (b - a + BM - 1) / BM;
    if (t < m * NT) {
      expert = i;
      seg0 = a;
      seg_n = b - a;
      mt_e = m;
      break;
    }
    t -= m * NT;
  }
  const int gfull = mt_e * kGroupN;
  const int ng = t / gfull;
  const int rem = t - ng * gfull;
  const int gsz = min(kGroupN, NT - ng * kGroupN);
  const int mt = rem / gsz;
  const int nt = ng * kGroupN + (rem - mt * gsz);
  const int row0 = seg0 + mt * BM;
  const int rows = min(BM, seg_n - mt * BM);
  const int n0 = nt * ON;
  const size_t boff = size_t(expert) * N * K;
  const bf16_t* Bg = B0 + boff;
  const bf16_t* Bu = (NMAT == 2 ? B1 : B0) + boff;

  extern __shared__ __attribute__((aligned(16))) bf16_t lds[];
  bf16_t* As = lds;                   // [2][BM][LD]
  bf16_t* Bs = lds + 2 * kStageA;     // [2][BNE][LD]

  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int wm = wave >> 2, wn = wave & 3;
  const u32x4_t zero = {0u, 0u, 0u, 0u};

  // global -> register staging: 4 A chunks and 4 B chunks of 16 bytes per
  // thread; chunk j of thread tid is row (tid + j*512) / 8, column (tid % 8)*8
  constexpr int CPR = BK / 8;  // 16-byte chunks per row (8)
  const int gcol = (tid % CPR) * 8;
  const int grow = tid / CPR;  // + j * 64
  const bf16_t* a_src = A + size_t(row0) * K + gcol;
  uint32_t a_row[4];
  uint32_t b_row[4];
  const bf16_t* b_base[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int r = grow + j * (kThreads / CPR);
    a_row[j] = uint32_t(min(r, rows - 1));
    if (NMAT == 2) {
      b_base[j] = r < BNE / 2 ? Bg : Bu;
      b_row[j] = uint32_t(n0 + (r & (BNE / 2 - 1)));
    } else {
      b_base[j] = Bg;
      b_row[j] = uint32_t(n0 + r);
    }
  }
  u32x4_t ra[4], rb[4];
#define MOE_BIG_GLOAD(k0)                                                                                   \
  do {                                                                                                      \
    const bool kok_ = (k0) + gcol < K;                                                                      \
    _Pragma("unroll") for (int j = 0; j < 4; ++j) {                                                         \
      ra[j] = kok_ ? *reinterpret_cast<const u32x4_t*>(a_src + size_t(a_row[j]) * K + (k0)) : zero;          \
      rb[j] = (kok_ && int(b_row[j]) < N)                                                                   \
                  ? *reinterpret_cast<const u32x4_t*>(b_base[j] + size_t(b_row[j]) * K + gcol + (k0))          \
                  : zero;                                                                                   \
    }                                                                                                       \
  } while (0)
#define MOE_BIG_SSTORE(st)                                                                                  \
  do {                                                                                                      \
    _Pragma("unroll") for (int j = 0; j < 4; ++j) {                                                         \
      const int r_ = grow + j * (kThreads / CPR);                                                           \
      *reinterpret_cast<u32x4_t*>(As + (st) * kStageA + r_ * LD + gcol) = ra[j];                              \
      *reinterpret_cast<u32x4_t*>(Bs + (st) * kStageB + r_ * LD + gcol) = rb[j];                              \
    }                                                                                                       \
  } while (0)

  f32x16_t acc[4][2];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

  // LDS rows this wave reads: A rows wm*128 + i*32 + (lane & 31); B rows below
  const int frow = lane & 31, fk = 8 * (lane >> 5);
  const int brow0 = NMAT == 2 ? wn * 32 : wn * 64;
  const int brow1 = NMAT == 2 ? BNE / 2 + wn * 32 : wn * 64 + 32;

  const int nk = (K + BK - 1) / BK;
  MOE_BIG_GLOAD(0);
  MOE_BIG_SSTORE(0);
  __syncthreads();
  for (int kt = 0; kt < nk; ++kt) {
    const int st = kt & 1;
    if (kt + 1 < nk) MOE_BIG_GLOAD((kt + 1) * BK);
    const bf16_t* as = As + st * kStageA + (wm * 128 + frow) * LD + fk;
    const bf16_t* bs = Bs + st * kStageB + frow * LD + fk;
#pragma unroll
    for (int kc = 0; kc < BK / 16; ++kc) {
      bf16x8_t af[4], bfr[2];
#pragma unroll
      for (int i = 0; i < 4; ++i) af[i] = *reinterpret_cast<const bf16x8_t*>(as + i * 32 * LD + kc * 16);
#pragma unroll
      for (int j = 0; j < 2; ++j) bfr[j] = *reinterpret_cast<const bf16x8_t*>(bs + (j ? brow1 : brow0) * LD + kc * 16);
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
    }
    if (kt + 1 < nk) MOE_BIG_SSTORE(st ^ 1);
    __syncthreads();
  }
#undef MOE_BIG_GLOAD
#undef MOE_BIG_SSTORE

  // ---- epilogue (32x32 layout: lane -> column lane & 31, register r -> row
  // 8*(r/4) + 4*(lane/32) + r%4) -----------------------------------------------
#pragma unroll
  for (int i = 0; i < 4; ++i) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int rt = wm * 128 + i * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
      if (rt >= rows) continue;
      bf16_t* crow = C + size_t(row0 + rt) * N;
      if (NMAT == 2) {
        const int col = n0 + wn * 32 + frow;
        if (col < N) crow[col] = f32_to_bf16(silu(acc[i][0][r]) * acc[i][1][r]);
      } else {
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          const int col = n0 + wn * 64 + j * 32 + frow;
          if (col < N) crow[col] = f32_to_bf16(acc[i][j][r]);
        }
      }
    }
  }
}

template <int NMAT>
moe_status launch(const char* name, const bf16_t* A, const int32_t* offsets, const bf16_t* B0, const bf16_t* B1,
                  bf16_t* C, int L, int N, int K, int64_t max_pairs, hipStream_t s) {
  auto kern = gemm_kernel<NMAT>;
  const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                           hipFuncAttributeMaxDynamicSharedMemorySize, int(kLdsBytes));
  if (e != hipSuccess) return set_error(MOE_ERR_HIP, "%s: LDS attribute: %s", name, hipGetErrorString(e));
  constexpr int ON = NMAT == 2 ? BNE / 2 : BNE;
  const int64_t mslots = (max_pairs + BM - 1) / BM + L;
  const int64_t grid = mslots * ((N + ON - 1) / ON);
  MOE_LAUNCH(name, kern, dim3(unsigned(grid)), dim3(kThreads), kLdsBytes, s, A, offsets, B0, B1, C, L, N, K);
  return MOE_OK;
}

}  // namespace big

template <typename T>
moe_status launch_t(const FfnArgs& a) {
  const moe_layer_desc* d = a.d;
  const int L = d->local_count, H = d->hidden, I = d->intermediate;
  const unsigned mslots = unsigned((a.max_pairs + BM - 1) / BM + L);
  MOE_LAUNCH("ffn_gate_up", (grouped_gemm_kernel<T, 2>), dim3(mslots, (I + BN - 1) / BN), dim3(kThreads), 0, a.s,
             static_cast<const T*>(a.x_sorted), a.offsets, static_cast<const T*>(a.w_gate),
             static_cast<const T*>(a.w_up), static_cast<T*>(a.h), L, I, H);
  MOE_LAUNCH("ffn_down", (grouped_gemm_kernel<T, 1>), dim3(mslots, (H + BN - 1) / BN), dim3(kThreads), 0, a.s,
             static_cast<const T*>(a.h), a.offsets, static_cast<const T*>(a.w_down), static_cast<const T*>(a.w_down),
             static_cast<T*>(a.y_sorted), L, H, I);
  return MOE_OK;
}

}  // namespace

moe_status launch_grouped_ffn(const FfnArgs& a) {
  if (a.max_pairs <= 0) return MOE_OK;
  const moe_layer_desc* d = a.d;
  // large tiles pay off once segments hold a few hundred rows; decode-sized
  // batches (a handful of rows per expert) keep the 128-row tiles
  if (d->dtype == MOE_BF16 && a.max_pairs >= int64_t(128) * d->local_count) {
    const int L = d->local_count, H = d->hidden, I = d->intermediate;
    const bf16_t* x = static_cast<const bf16_t*>(a.x_sorted);
    bf16_t* h = static_cast<bf16_t*>(a.h);
    moe_status st = big::launch<2>("ffn_gate_up", x, a.offsets, static_cast<const bf16_t*>(a.w_gate),
                                   static_cast<const bf16_t*>(a.w_up), h, L, I, H, a.max_pairs, a.s);
    if (st != MOE_OK) return st;
    return big::launch<1>("ffn_down", h, a.offsets, static_cast<const bf16_t*>(a.w_down),
                          static_cast<const bf16_t*>(a.w_down), static_cast<bf16_t*>(a.y_sorted), L, H, I,
                          a.max_pairs, a.s);
  }
  return d->dtype == MOE_BF16 ? launch_t<bf16_t>(a) : launch_t<float>(a);
}

}  // namespace moe
