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

// ---------------------------------------------------------------------------
// float32 products with a deep load ring.
//
// The general kernel above stages one k slice ahead in registers; a float32
// tile of 64 rows does ~1 us of MFMA work per 16-k slice, less than the load
// latency, so each slice waits on its loads.  This kernel keeps kSlots slices
// in flight instead: every stage is filled by direct global->LDS loads
// (buffer_load_dword ... lds: lane i of a load writes bytes [16i, 16i+16) of a
// 1 KB block), so the depth costs LDS, not registers, and a slice's loads are
// issued kSlots - 1 slices before it is used.  One barrier per slice frees the
// slot that was read the slice before, which is refilled at once.
//
// Stage layout: the tile's A rows (token rows) then its B rows (weight rows:
// gate then up for the gate/up product), 64 bytes (16 k) each; 16-byte chunk c
// of row r sits at chunk c ^ ((r / 4) % 4), so the fragment reads of 16 lanes
// (16 rows, one chunk) cover all 64 banks.  A 1 KB load fills 16 rows; block b
// of the stage is rows 16b..16b+15, all A or all B.  The waves split the tile
// 2 x 2 and each lane reads the 8 k values of its row as two 16-byte chunks,
// consumed by eight MFMA 32x32x2 steps as in the general kernel, so the
// products, their order and the epilogue are the general kernel's.
namespace ring {

constexpr int BK = 16, kRowBytes = 64;

// Ring depth: 128 x 128 tiles run one block per CU and keep six slices in flight;
// 64 x 64 tiles keep four, so that three blocks share a CU (gate/up: 48 KB instead of
// 72 KB of LDS).  A small layer's few hundred 64 x 64 tiles then all start at once:
// tiny_fp32 gate/up 60.4 -> 56.8 us, down 30.3 -> 29.4 us (same box; three slots
// measured the same as four).
template <int NMAT, int BMT, int BNR>
struct RS {
  static constexpr int kA = BMT, kB = NMAT * BNR;
  static constexpr int kSlots = BMT * BNR <= 64 * 64 ? 4 : 6;
  static constexpr int kStage = (kA + kB) * kRowBytes;
  static constexpr int kPerWave = kStage / 1024 / 4;  // 1 KB loads per wave per stage
  static constexpr size_t kLds = size_t(kSlots) * kStage;
  static_assert(kStage % 4096 == 0, "whole 1 KB loads for every wave");
};

// k of both operands is a multiple of BK (whole 64-byte rows); byte extents below 4 GiB
bool supported(const moe_layer_desc* d, int64_t max_pairs) {
  const int64_t H = d->hidden, I = d->intermediate;
  return d->dtype == MOE_F32 && d->weight_layout == MOE_WEIGHTS_OUT_IN && H % BK == 0 && I % BK == 0 &&
         max_pairs * std::max(H, I) * 4 < (int64_t(1) << 32) && H * I * 4 < (int64_t(1) << 32);
}

#define MOE_VMCNT(n) __builtin_amdgcn_s_waitcnt(((n) & 0xF) | (((n) >> 4) << 14) | (0x7 << 4) | (0xF << 8))

// Tiles of BMT token rows x BNR weight rows (per matrix); the waves split them 2 x 2.
template <int NMAT, int BMT, int BNR, bool SAVE>
__device__ __forceinline__ void ring_body(const float* __restrict__ A, int a_rows, const int32_t* __restrict__ offsets,
                                          const float* __restrict__ B0, const float* __restrict__ B1,
                                          float* __restrict__ C, int L, int N, int K, float* __restrict__ Gs,
                                          float* __restrict__ Us, char* lds) {
  using S = RS<NMAT, BMT, BNR>;
  constexpr int MI = BMT / 64;   // 32-row blocks per wave
  constexpr int NJ = BNR / 64;   // 32-column blocks per wave and matrix
  // ---- which expert and rows this block owns (as the general kernel) --------
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
  const int n0 = blockIdx.y * BNR;
  const int tid = threadIdx.x, wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  const int wm = wave >> 1, wn = wave & 1;
  const size_t boff = size_t(expert) * N * K;

  // ---- direct loads: buffer resources over the tile's token rows (up to the
  // buffer's last row) and each weight matrix; reads past them return zero.
  // Token rows past the segment and weight rows past N feed outputs that are
  // never stored.
  // the matrix of block j of this wave, as a base pointer and extent (uniform)
  const uint32_t wbytes = uint32_t(N) * uint32_t(K) * 4u;
  __amdgpu_buffer_rsrc_t rs[S::kPerWave];
  uint32_t vo[S::kPerWave];
#pragma unroll
  for (int j = 0; j < S::kPerWave; ++j) {
    const int b = S::kPerWave * wave + j;            // block of the stage
    const bool is_a = b < S::kA / 16, is_g = b < S::kA / 16 + BNR / 16;
    const float* base = is_a ? A + size_t(row0) * K : (is_g || NMAT == 1 ? B0 : B1) + boff;
    const uint32_t bytes = is_a ? uint32_t(a_rows - row0) * uint32_t(K) * 4u : wbytes;
    rs[j] = __builtin_amdgcn_make_buffer_rsrc(const_cast<float*>(base), 0, bytes, kRsrcFlags);
    const int r = 16 * b + (lane >> 2);              // stage row
    const int c = (lane & 3) ^ ((r >> 2) & 3);       // logical chunk of this lane
    const int mrow = is_a ? r : n0 + ((r - S::kA) % BNR);
    vo[j] = (uint32_t(mrow) * uint32_t(K) + uint32_t(4 * c)) * 4u;
  }
  const int nk = K / BK;
  auto issue = [&](int s) {  // stage min(s, nk-1) into its slot
    const int st = min(s, nk - 1);
    char* slot = lds + (s % S::kSlots) * S::kStage + S::kPerWave * wave * 1024;
    const uint32_t ko = uint32_t(st) * (BK * 4);
#pragma unroll
    for (int j = 0; j < S::kPerWave; ++j)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rs[j], (lds_ptr_t)(slot + j * 1024), 16, vo[j], ko, 0, 0);
  };

  f32x16_t acc[NMAT][MI][NJ];
#pragma unroll
  for (int m = 0; m < NMAT; ++m)
#pragma unroll
    for (int i = 0; i < MI; ++i)
#pragma unroll
      for (int j = 0; j < NJ; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[m][i][j][r] = 0.0f;

  // fragment rows of this lane: A rows wm*BMT/2 + i*32 + (lane & 31), B rows of
  // the wave's two 32-column blocks per matrix; chunks 2 (lane / 32) and +1
  const int fr = lane & 31, c0 = 2 * (lane >> 5);
  int aoff[MI][2], boffs[NMAT][NJ][2];
#pragma unroll
  for (int i = 0; i < MI; ++i) {
    const int r = wm * (BMT / 2) + i * 32 + fr;
#pragma unroll
    for (int h = 0; h < 2; ++h) aoff[i][h] = r * kRowBytes + (((c0 + h) ^ ((r >> 2) & 3)) * 16);
  }
#pragma unroll
  for (int m = 0; m < NMAT; ++m)
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      const int r = S::kA + m * BNR + wn * (BNR / 2) + j * 32 + fr;
#pragma unroll
      for (int h = 0; h < 2; ++h) boffs[m][j][h] = r * kRowBytes + (((c0 + h) ^ ((r >> 2) & 3)) * 16);
    }

#pragma unroll
  for (int s = 0; s < S::kSlots - 1; ++s) issue(s);
  for (int s = 0; s < nk; ++s) {
    MOE_VMCNT(S::kPerWave * (S::kSlots - 2));  // this wave's loads of stage s have landed
    block_barrier();                         // every wave's have, and stage s-1 is read out
    issue(s + S::kSlots - 1);                   // into the slot stage s-1 used
    const char* st = lds + (s % S::kSlots) * S::kStage;
    uint4 af[MI][2], bfr[NMAT][NJ][2];
#pragma unroll
    for (int i = 0; i < MI; ++i)
#pragma unroll
      for (int h = 0; h < 2; ++h) af[i][h] = *reinterpret_cast<const uint4*>(st + aoff[i][h]);
#pragma unroll
    for (int m = 0; m < NMAT; ++m)
#pragma unroll
      for (int j = 0; j < NJ; ++j)
#pragma unroll
        for (int h = 0; h < 2; ++h) bfr[m][j][h] = *reinterpret_cast<const uint4*>(st + boffs[m][j][h]);
#pragma unroll
    for (int m = 0; m < NMAT; ++m)
#pragma unroll
      for (int i = 0; i < MI; ++i)
#pragma unroll
        for (int j = 0; j < NJ; ++j) Gemm<float>::mma(af[i], bfr[m][j], acc[m][i][j]);
  }
  MOE_VMCNT(0);  // the ring's last (repeated) loads land before the block ends

  // ---- epilogue (the general kernel's): lane -> column (lane & 31), register
  // r -> row 8*(r/4) + 4*(lane/32) + r%4 -----------------------------------------
#pragma unroll
  for (int i = 0; i < MI; ++i)
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      const int col = n0 + wn * (BNR / 2) + j * 32 + (lane & 31);
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int rt = wm * (BMT / 2) + i * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
        if (rt < rows && col < N) {
          const size_t at = size_t(row0 + rt) * N + col;
          if constexpr (NMAT == 2) {
            C[at] = silu(acc[0][i][j][r]) * acc[1][i][j][r];
            if constexpr (SAVE) {
              Gs[at] = acc[0][i][j][r];
              Us[at] = acc[1][i][j][r];
            }
          } else {
            C[at] = acc[0][i][j][r];
          }
        }
      }
    }
}
#undef MOE_VMCNT

template <int NMAT, int BMT, int BNR, bool SAVE>
__global__ __launch_bounds__(kThreads) void ring_kernel(const float* __restrict__ A, int a_rows,
                                                       const int32_t* __restrict__ offsets,
                                                       const float* __restrict__ B0, const float* __restrict__ B1,
                                                       float* __restrict__ C, int L, int N, int K,
                                                       float* __restrict__ Gs, float* __restrict__ Us) {
  extern __shared__ __attribute__((aligned(1024))) char lds[];
  ring_body<NMAT, BMT, BNR, SAVE>(A, a_rows, offsets, B0, B1, C, L, N, K, Gs, Us, lds);
}

template <int NMAT, int BMT, int BNR, bool SAVE>
moe_status launch_one(const char* name, const float* A, int a_rows, const int32_t* offsets, const float* B0,
                      const float* B1, float* C, int L, int N, int K, float* Gs, float* Us, hipStream_t s) {
  auto kern = ring_kernel<NMAT, BMT, BNR, SAVE>;
  constexpr size_t lds = RS<NMAT, BMT, BNR>::kLds;
  const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                           hipFuncAttributeMaxDynamicSharedMemorySize, int(lds));
  if (e != hipSuccess) return set_error(MOE_ERR_HIP, "%s (float32): LDS attribute: %s", name, hipGetErrorString(e));
  const unsigned mslots = unsigned((a_rows + BMT - 1) / BMT + L);
  MOE_LAUNCH(name, kern, dim3(mslots, (N + BNR - 1) / BNR), dim3(kThreads), lds, s, A, a_rows, offsets, B0, B1, C, L,
             N, K, Gs, Us);
  return MOE_OK;
}

// Tile shape of one product: the blocks run in rounds over the CUs, so the product
// takes about (rounds) x (tile work); the expected m-tiles are P_max / BMT plus half
// a tile per expert.  64 x 64 tiles are taken when that estimate beats 128 x 128
// tiles by more than 10% (a small layer whose 128 x 128 tiles would leave most CUs
// idle or run one extra round); otherwise the larger tile, with half the loads per
// flop, is kept.
enum TileShape { k64x64, k128x128 };
TileShape pick(int64_t max_pairs, int L, int N) {
  const int64_t cus = 256;
  auto cost = [&](int bm, int bn) {
    const int64_t blocks = (max_pairs / bm + L / 2) * ((N + bn - 1) / bn);
    return (blocks + cus - 1) / cus * bm * bn;
  };
  return cost(64, 64) * 10 < cost(128, 128) * 9 ? k64x64 : k128x128;
}

template <int NMAT, bool SAVE>
moe_status launch_shape(TileShape sh, const char* name, const float* A, int a_rows, const int32_t* offsets,
                        const float* B0, const float* B1, float* C, int L, int N, int K, float* Gs, float* Us,
                        hipStream_t s) {
  if (sh == k64x64) return launch_one<NMAT, 64, 64, SAVE>(name, A, a_rows, offsets, B0, B1, C, L, N, K, Gs, Us, s);
  return launch_one<NMAT, 128, 128, SAVE>(name, A, a_rows, offsets, B0, B1, C, L, N, K, Gs, Us, s);
}

moe_status launch(const FfnArgs& a) {
  const moe_layer_desc* d = a.d;
  const int L = d->local_count, H = d->hidden, I = d->intermediate;
  const int arows = int(a.max_pairs);
  const float* x = static_cast<const float*>(a.x_sorted);
  const float* wg = static_cast<const float*>(a.w_gate);
  const float* wu = static_cast<const float*>(a.w_up);
  const float* wd = static_cast<const float*>(a.w_down);
  float* h = static_cast<float*>(a.h);
  const TileShape sgu = pick(a.max_pairs, L, I), sdn = pick(a.max_pairs, L, H);
  moe_status st = a.g_out != nullptr
                      ? launch_shape<2, true>(sgu, "ffn_gate_up", x, arows, a.offsets, wg, wu, h, L, I, H,
                                              static_cast<float*>(a.g_out), static_cast<float*>(a.u_out), a.s)
                      : launch_shape<2, false>(sgu, "ffn_gate_up", x, arows, a.offsets, wg, wu, h, L, I, H, nullptr,
                                               nullptr, a.s);
  if (st != MOE_OK) return st;
  return launch_shape<1, false>(sdn, "ffn_down", h, arows, a.offsets, wd, wd, static_cast<float*>(a.y_sorted), L, H, I,
                                nullptr, nullptr, a.s);
}

}  // namespace ring

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
  if (a.d->dtype == MOE_BF16) return launch_t<bf16_t>(a);
  if (ring::supported(a.d, a.max_pairs)) return ring::launch(a);
  return launch_t<float>(a);
}

}  // namespace moe
