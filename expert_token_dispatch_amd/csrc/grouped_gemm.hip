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
// One 256-thread block (four waves, one per SIMD) owns a tile of 256 rows by
// 256 B rows: for the gate/up product that is 128 gate rows and the same 128
// up rows (output 256 x 128), for the down product 256 output columns.  The
// waves split it 2 (M) x 2 (N); each holds 4 x 4 MFMA 32x32 accumulators
// (256 registers, kept in AGPRs), so every fragment read from LDS feeds four
// MFMAs.
//
// K advances 64 at a time through two 64 KB LDS stages filled by direct
// global->LDS loads (global_load_lds_dwordx4: lane i of a load writes bytes
// [16i, 16i+16) of a 1 KB block, no staging registers).  Rows are 128 bytes;
// 16-byte chunk c of row r sits at physical chunk c ^ ((r/2) % 8), so the
// fragment reads of 16 lanes (16 rows, one chunk) cover all 64 banks.
//
// Schedule of one stage (per wave): for each 16-k chunk, the fragments of the
// next chunk are read while this chunk's 16 MFMAs issue, one read between
// every two MFMAs (pinned with sched_group_barrier); reads bunched at the
// start of the group left the LDS and the matrix core taking turns.  Before the last chunk the wave waits for its own
// loads of the next stage and for its own reads of this stage, then a block
// barrier makes both true for every wave: the next stage's first fragments
// are read and this stage's slot is refilled (stage kt+2) while the last 16
// MFMAs run.  The barrier is a bare s_barrier: __syncthreads() would also
// drain every load in flight.
//
// The MFMAs take the weight fragment as the left operand, so each lane ends
// with four adjacent output columns of one token row; the epilogue parks the
// bf16 tile in LDS and writes it out in whole row pieces.
//
// Tile order: the blocks that run at once on one XCD (blocks are dealt to
// the 8 XCDs round robin) get consecutive tile numbers, and tile numbers run
// over (expert, group of kGroupN n-tiles, m-tile, n-tile in group), so one
// XCD's L2 serves a few weight tiles to all m-tiles of an expert and a few
// activation tiles to several n-tiles.
namespace big {

typedef __attribute__((address_space(3))) void* lds_ptr_t;
typedef __attribute__((address_space(1))) void* glb_ptr_t;

constexpr int BM = 256, BNE = 256, BK = 64, kStages = 2, kThreads = 256;
constexpr int kRowBytes = BK * 2;              // 128
constexpr int kStageA = BM * kRowBytes;        // 32 KB
constexpr int kStage = kStageA + BNE * kRowBytes;
constexpr size_t kLoopLds = size_t(kStages) * kStage;  // 128 KB
// epilogue staging: the output tile as bf16 rows of ON columns plus 16 bytes of padding
template <int NMAT>
constexpr int stage_row_bytes() { return (NMAT == 2 ? BNE / 2 : BNE) * 2 + 16; }
template <int NMAT>
constexpr size_t lds_bytes() {
  return kLoopLds > size_t(BM) * stage_row_bytes<NMAT>() ? kLoopLds : size_t(BM) * stage_row_bytes<NMAT>();
}
constexpr int kGroupN = 4;
constexpr int kXcds = 8;

// s_waitcnt on the vector-memory counter only (expcnt and lgkmcnt left at their maxima)
#define MOE_VMCNT(n) __builtin_amdgcn_s_waitcnt(((n) & 0xF) | (((n) >> 4) << 14) | (0x7 << 4) | (0xF << 8))
#define MOE_LGKMCNT0() __builtin_amdgcn_s_waitcnt(0xC07F)

bool supported(int K) { return K % BK == 0; }

// ---- work plan -------------------------------------------------------------
// Tiles are numbered over (expert, group of kGroupN n-tiles, m-tile, n-tile
// in group) and dealt to the XCDs in contiguous ranges (block b runs on XCD
// b % 8).  An XCD with q tiles runs them in rounds of `cpx` (its CU count);
// when the last round is only partly filled and K is long, its r tiles are
// cut into s pieces along K (s in {2, 4}, chosen to minimise the rounds the
// pieces take, ceil(r*s/cpx)/s), so the XCD finishes in F + ceil(r*s/cpx)/s
// tile times instead of F + 1.  Each piece writes its float32 accumulators;
// fixup_kernel adds the pieces in piece order (so the result does not depend
// on timing) and runs the usual epilogue.
constexpr int kSplitMinSteps = 128;  // K/BK from which the last round is split
constexpr int kMaxSplit = 4;
constexpr int kMaxParts = 96;        // pieces per XCD: s = 4 needs r <= 24, s = 2 needs r <= 16
constexpr int kMaxTail = kMaxParts / kMaxSplit;
constexpr size_t kPartBytes = size_t(kThreads) * 256 * sizeof(float);  // one piece's accumulators

__device__ __forceinline__ int split_of(int r, int cpx, int smax, int nk) {
  int best = 1;
  for (int s = 2; s <= smax; s *= 2) {
    if (r == 0 || r > kMaxTail || nk < 16 * s || r * s > kMaxParts) break;
    // ceil(r*s/cpx)/s < ceil(r*best/cpx)/best
    if (((r * s + cpx - 1) / cpx) * best < ((r * best + cpx - 1) / cpx) * s) best = s;
  }
  return best;
}

struct Job {
  int expert, row0, rows, n0;
  int kb, nks;     // k steps [kb, kb + nks)
  int part, nparts, pslot;
};

// The job of block (xcd, loc), or the tile of the XCD's u-th split tile when
// `tail >= 0`.  Returns false when the block has nothing to do.
__device__ __forceinline__ bool plan_job(const int32_t* __restrict__ offsets, int L, int NT, int nk, int cpx, int smax,
                                         int xcd, int loc, int tail, Job& jb) {
  int mt_total = 0;
  for (int i = 0; i < L; ++i) mt_total += (offsets[i + 1] - offsets[i] + BM - 1) / BM;
  const int R = mt_total * NT;
  const int q = R / kXcds, rr = R % kXcds;
  const int qx = q + (xcd < rr ? 1 : 0);
  const int base = xcd * q + min(xcd, rr);
  const int F = qx / cpx, r = qx - F * cpx;
  const int s = split_of(r, cpx, smax, nk);
  int t;
  if (tail >= 0) {
    if (s == 1 || tail >= r) return false;
    t = base + F * cpx + tail;
    jb.part = 0;
    jb.nparts = s;
    jb.pslot = xcd * kMaxParts + tail * s;
  } else if (loc < F * cpx || s == 1) {
    if (loc >= qx) return false;
    t = base + loc;
    jb.part = 0;
    jb.nparts = 1;
    jb.pslot = 0;
  } else {
    const int v = loc - F * cpx;
    if (v >= r * s) return false;
    const int u = v / s;
    t = base + F * cpx + u;
    jb.part = v - u * s;
    jb.nparts = s;
    jb.pslot = xcd * kMaxParts + v;
  }
  int seg0 = 0, seg_n = 0, mt_e = 0;
  jb.expert = 0;
  for (int i = 0; i < L; ++i) {
    const int a = offsets[i], b = offsets[i + 1];
    const int m = (b - a + BM - 1) / BM;
    if (t < m * NT) {
      jb.expert = i;
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
  jb.row0 = seg0 + mt * BM;
  jb.rows = min(BM, seg_n - mt * BM);
  jb.n0 = nt;  // n-tile index; the caller scales it by the tile's output columns
  jb.kb = (jb.part * nk) / jb.nparts;
  jb.nks = ((jb.part + 1) * nk) / jb.nparts - jb.kb;
  return true;
}

// ---- epilogue.  The products were formed as (weight rows) x (token rows), so
// in the 32x32 accumulator layout lane l holds token row l & 31 and register
// 4q+u holds output column 8q + 4*(l/32) + u: four adjacent columns per q.
// Each wave converts its part of the tile to bf16 (SwiGLU first for gate/up)
// and parks it in LDS, rows padded by 16 bytes; then every thread copies
// 16-byte row chunks out, so each store instruction writes whole 256-byte row
// pieces.  The caller has made sure no wave still reads the loop's LDS stages.
template <int NMAT>
__device__ __forceinline__ void epilogue(f32x16_t (&acc)[4][4], char* lds, bf16_t* __restrict__ C, int row0, int rows,
                                         int n0, int N) {
  constexpr int TC = NMAT == 2 ? BNE / 2 : BNE;  // output columns of the tile
  constexpr int RS = stage_row_bytes<NMAT>();
  constexpr int NJ = NMAT == 2 ? 2 : 4;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int wm = wave >> 1, wn = wave & 1, fr = lane & 31, g = lane >> 5;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int rt = wm * 128 + i * 32 + fr;
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        float v[4];
#pragma unroll
        for (int u = 0; u < 4; ++u)
          v[u] = NMAT == 2 ? silu(acc[i][j][4 * q + u]) * acc[i][j + 2][4 * q + u] : acc[i][j][4 * q + u];
        uint2 pk;
        pk.x = uint32_t(f32_to_bf16(v[0])) | (uint32_t(f32_to_bf16(v[1])) << 16);
        pk.y = uint32_t(f32_to_bf16(v[2])) | (uint32_t(f32_to_bf16(v[3])) << 16);
        const int cl = (NMAT == 2 ? wn * 64 : wn * 128) + j * 32 + 8 * q + 4 * g;
        *reinterpret_cast<uint2*>(lds + rt * RS + cl * 2) = pk;
      }
    }
  }
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
  block_barrier();
  constexpr int CPR = TC / 8;  // 16-byte chunks per row
#pragma unroll
  for (int u = 0; u < BM * CPR / kThreads; ++u) {
    const int id = tid + kThreads * u;
    const int r = id / CPR, c = id % CPR;
    const u32x4_t val = *reinterpret_cast<const u32x4_t*>(lds + r * RS + c * 16);
    // N is a multiple of 8, so a chunk is wholly inside or wholly past column N
    if (r < rows && n0 + c * 8 < N) *reinterpret_cast<u32x4_t*>(C + size_t(row0 + r) * N + n0 + c * 8) = val;
  }
}

// A piece's accumulators, thread-major: float4 number v of thread t at (v*256 + t)
__device__ __forceinline__ f32x4_t* part_ptr(float* __restrict__ parts, int pslot) {
  return reinterpret_cast<f32x4_t*>(parts + size_t(pslot) * (kPartBytes / sizeof(float)));
}

template <int NMAT>
__global__ __launch_bounds__(kThreads) void gemm_kernel(const bf16_t* __restrict__ A, const int32_t* __restrict__ offsets,
                                                        const bf16_t* __restrict__ B0, const bf16_t* __restrict__ B1,
                                                        bf16_t* __restrict__ C, int L, int N, int K, int cpx, int smax,
                                                        float* __restrict__ parts) {
  constexpr int ON = NMAT == 2 ? BNE / 2 : BNE;  // output columns per tile
  const int NT = (N + ON - 1) / ON;
  const int nk = K / BK;
  Job jb;
  if (!plan_job(offsets, L, NT, nk, cpx, smax, blockIdx.x % kXcds, blockIdx.x / kXcds, -1, jb)) return;
  const int row0 = jb.row0, rows = jb.rows, n0 = jb.n0 * ON, kb = jb.kb, nks = jb.nks;
  const size_t boff = size_t(jb.expert) * N * K;
  const bf16_t* Bg = B0 + boff;
  const bf16_t* Bu = (NMAT == 2 ? B1 : B0) + boff;

  extern __shared__ __attribute__((aligned(1024))) char lds[];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int wm = wave >> 1, wn = wave & 1;

  // ---- direct loads: 32 blocks of 8 rows (1 KB) for A and for B per stage;
  // wave w fills blocks 8w..8w+7 of each.  Lane i of block j writes row
  // 64w + 8j + i/8, physical chunk i%8, which holds logical chunk
  // (i%8) ^ ((row/2)%8); that depends on i and the parity of j only.
  const int lrow = 64 * wave + (lane >> 3);
  const int c_even = (lane & 7) ^ ((lane >> 4) & 7);
  const int c_odd = (lane & 7) ^ ((4 + (lane >> 4)) & 7);
  const bf16_t* a_base = A + size_t(row0) * K;
  const bf16_t* b_base;
  int b_lrow;
  if (NMAT == 2) {
    b_base = (wave < 2 ? Bg : Bu) + size_t(n0) * K;  // waves 0-1 load gate rows, 2-3 up rows
    b_lrow = lrow & (BNE / 2 - 1);
  } else {
    b_base = Bg + size_t(n0) * K;
    b_lrow = lrow;
  }
  const int b_lim = N - 1 - n0;  // B rows past N repeat row N-1: those columns are never stored
#define MOE_ISSUE(kt_)                                                                                      \
  do {                                                                                                      \
    char* sa_ = lds + ((kt_) % kStages) * kStage + (8 * wave) * 1024;                                       \
    const int k0_ = (kb + (kt_)) * BK;                                                                      \
    _Pragma("unroll") for (int j = 0; j < 8; ++j) {                                                         \
      const int cc_ = (j & 1) ? c_odd : c_even;                                                             \
      const int ar_ = min(lrow + 8 * j, rows - 1); /* rows past the segment repeat its last row */          \
      const int br_ = min(b_lrow + 8 * j, b_lim);                                                           \
      __builtin_amdgcn_global_load_lds((glb_ptr_t)(a_base + (uint32_t(ar_) * uint32_t(K) + cc_ * 8 + k0_)), \
                                       (lds_ptr_t)(sa_ + j * 1024), 16, 0, 0);                             \
      __builtin_amdgcn_global_load_lds((glb_ptr_t)(b_base + (uint32_t(br_) * uint32_t(K) + cc_ * 8 + k0_)), \
                                       (lds_ptr_t)(sa_ + kStageA + j * 1024), 16, 0, 0);                   \
    }                                                                                                       \
  } while (0)

  f32x16_t acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

  // ---- fragment addresses: A rows wm*128 + i*32 + (lane & 31); B rows of the
  // wave's four 32-column blocks (gate/up: two gate blocks, then the two up
  // blocks of the same columns) --------------------------------------------
  const int fr = lane & 31;
  const int sw = (fr >> 1) & 7;
  const int g = lane >> 5;
  int boffs[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int br = NMAT == 2 ? (j < 2 ? wn * 64 + j * 32 : BNE / 2 + wn * 64 + (j - 2) * 32) : wn * 128 + j * 32;
    boffs[j] = kStageA + (br + fr) * kRowBytes;
  }
  const int a_off = (wm * 128 + fr) * kRowBytes;
  bf16x8_t fa[2][4], fb[2][4];
#define MOE_LOADF(buf_, st_, kc_)                                                                         \
  do {                                                                                                    \
    const int co_ = ((2 * (kc_) + g) ^ sw) * 16;                                                          \
    _Pragma("unroll") for (int i = 0; i < 4; ++i)                                                         \
      fa[buf_][i] = *reinterpret_cast<const bf16x8_t*>((st_) + a_off + i * 32 * kRowBytes + co_);          \
    _Pragma("unroll") for (int j = 0; j < 4; ++j)                                                         \
      fb[buf_][j] = *reinterpret_cast<const bf16x8_t*>((st_) + boffs[j] + co_);                            \
  } while (0)
#define MOE_MMA(buf_)                                                                                     \
  do {                                                                                                    \
    _Pragma("unroll") for (int i = 0; i < 4; ++i)                                                         \
      _Pragma("unroll") for (int j = 0; j < 4; ++j)                                                       \
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fb[buf_][j], fa[buf_][i], acc[i][j], 0, 0, 0); \
  } while (0)
  // 8 x {MFMA, LDS read, MFMA}: the next chunk's fragment reads spread over the whole group
#define MOE_PIPE_DS()                                                                                     \
  do {                                                                                                    \
    _Pragma("unroll") for (int p_ = 0; p_ < 8; ++p_) {                                                    \
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);                                                  \
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);                                                  \
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);                                                  \
    }                                                                                                     \
  } while (0)

  MOE_ISSUE(0);
  if (nks > 1) {
    MOE_ISSUE(1);
    MOE_VMCNT(16);  // stage 0 landed (16 loads per stage per wave)
  } else {
    MOE_VMCNT(0);
  }
  block_barrier();
  MOE_LOADF(0, lds, 0);
  // every iteration has a next stage; the refill issued in it is stage kt+2,
  // or (near the end) a repeat of the last stage into the free slot
  for (int kt = 0; kt + 1 < nks; ++kt) {
    const char* st = lds + (kt % kStages) * kStage;
    MOE_LOADF(1, st, 1);
    MOE_MMA(0);
    MOE_LOADF(0, st, 2);
    MOE_MMA(1);
    MOE_LOADF(1, st, 3);
    MOE_MMA(0);
    MOE_PIPE_DS();
    MOE_PIPE_DS();
    MOE_PIPE_DS();
    __builtin_amdgcn_sched_barrier(0);
    MOE_VMCNT(0);     // this wave's loads of stage kt+1 have landed
    MOE_LGKMCNT0();   // and its reads of stage kt are done
    block_barrier();
    __builtin_amdgcn_sched_barrier(0);
    MOE_LOADF(0, lds + ((kt + 1) % kStages) * kStage, 0);
    MOE_ISSUE(min(kt + 2, nks - 1));
    MOE_MMA(1);
    __builtin_amdgcn_sched_group_barrier(0x100, 8, 0);
#pragma unroll
    for (int p = 0; p < 16; ++p) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
    }
  }
  {
    const char* st = lds + ((nks - 1) % kStages) * kStage;
    MOE_LOADF(1, st, 1);
    MOE_MMA(0);
    MOE_LOADF(0, st, 2);
    MOE_MMA(1);
    MOE_LOADF(1, st, 3);
    MOE_MMA(0);
    MOE_MMA(1);
  }
  MOE_VMCNT(0);  // the last refill repeated a stage; let it land before the block ends
#undef MOE_ISSUE
#undef MOE_LOADF
#undef MOE_MMA
#undef MOE_PIPE_DS

  if (jb.nparts > 1) {
    // one piece of a split tile: park the accumulators for fixup_kernel
    f32x4_t* dst = part_ptr(parts, jb.pslot);
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int c = 0; c < 4; ++c)
          dst[((i * 4 + j) * 4 + c) * kThreads + tid] =
              f32x4_t{acc[i][j][4 * c], acc[i][j][4 * c + 1], acc[i][j][4 * c + 2], acc[i][j][4 * c + 3]};
    return;
  }
  MOE_LGKMCNT0();
  block_barrier();  // every wave is done reading the last stage
  epilogue<NMAT>(acc, lds, C, row0, rows, n0, N);
}

// Adds the pieces of each split tile in piece order and writes the tile.
// kFixSub blocks share a tile; an item is one float4 of the accumulator
// layout (thread t, float4 v: i = v/16, j = v/4 % 4, q = v % 4), that is four
// adjacent output columns of one token row (for gate/up: the gate float4 and
// its up partner j + 2).
constexpr int kFixSub = 8;

template <int NMAT>
__global__ __launch_bounds__(kThreads) void fixup_kernel(const int32_t* __restrict__ offsets, bf16_t* __restrict__ C,
                                                         int L, int N, int K, int cpx, int smax,
                                                         const float* __restrict__ parts) {
  constexpr int ON = NMAT == 2 ? BNE / 2 : BNE;
  constexpr int NV = NMAT == 2 ? 32 : 64;                 // output float4s per thread of the tile
  constexpr int kPer = NV * kThreads / (kFixSub * kThreads);  // items per thread of this block
  const int NT = (N + ON - 1) / ON;
  const int sub = blockIdx.x % kFixSub, tile = blockIdx.x / kFixSub;
  Job jb;
  if (!plan_job(offsets, L, NT, K / BK, cpx, smax, tile % kXcds, 0, tile / kXcds, jb)) return;
  const int n0 = jb.n0 * ON;
  const size_t pstride = kPartBytes / sizeof(f32x4_t);  // float4s per piece
  const f32x4_t* base = reinterpret_cast<const f32x4_t*>(parts) + size_t(jb.pslot) * pstride;
#pragma unroll
  for (int it = 0; it < kPer; ++it) {
    const int item = (sub * kPer + it) * kThreads + threadIdx.x;  // consecutive threads: consecutive float4s
    const int t = item % kThreads, w = item / kThreads;
    // w -> (i, j, q) of the gate (or plain) float4
    const int i = NMAT == 2 ? w / 8 : w / 16;
    const int j = NMAT == 2 ? (w / 4) % 2 : (w / 4) % 4;
    const int q = w % 4;
    const int v = (i * 4 + j) * 4 + q;
    f32x4_t s = base[size_t(v) * kThreads + t];
    f32x4_t su = NMAT == 2 ? base[size_t(v + 8) * kThreads + t] : s;  // up partner: j + 2
    for (int p = 1; p < jb.nparts; ++p) {
      s += base[size_t(p) * pstride + size_t(v) * kThreads + t];
      if (NMAT == 2) su += base[size_t(p) * pstride + size_t(v + 8) * kThreads + t];
    }
    const int wave = t >> 6, lane = t & 63;
    const int wm = wave >> 1, wn = wave & 1, fr = lane & 31, g = lane >> 5;
    const int rt = wm * 128 + i * 32 + fr;
    const int cl = (NMAT == 2 ? wn * 64 : wn * 128) + j * 32 + 8 * q + 4 * g;
    if (rt < jb.rows && n0 + cl < N) {
      float o[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) o[u] = NMAT == 2 ? silu(s[u]) * su[u] : s[u];
      uint2 pk;
      pk.x = uint32_t(f32_to_bf16(o[0])) | (uint32_t(f32_to_bf16(o[1])) << 16);
      pk.y = uint32_t(f32_to_bf16(o[2])) | (uint32_t(f32_to_bf16(o[3])) << 16);
      *reinterpret_cast<uint2*>(C + size_t(jb.row0 + rt) * N + n0 + cl) = pk;
    }
  }
}
#undef MOE_VMCNT
#undef MOE_LGKMCNT0

int cus_per_xcd() {
  static int cached[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 32;
  if (cached[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n < kXcds) n = 256;
    cached[dev] = n / kXcds;
  }
  return cached[dev];
}

// K long enough for the split of a partly filled last round
bool splits(int K) { return K / BK >= kSplitMinSteps; }

template <int NMAT>
moe_status launch(const char* name, const bf16_t* A, const int32_t* offsets, const bf16_t* B0, const bf16_t* B1,
                  bf16_t* C, int L, int N, int K, int64_t max_pairs, float* parts, hipStream_t s) {
  auto kern = gemm_kernel<NMAT>;
  constexpr size_t lds = lds_bytes<NMAT>();
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern), hipFuncAttributeMaxDynamicSharedMemorySize,
                                     int(lds));
  if (e != hipSuccess) return set_error(MOE_ERR_HIP, "%s: LDS attribute: %s", name, hipGetErrorString(e));
  constexpr int ON = NMAT == 2 ? BNE / 2 : BNE;
  const int cpx = cus_per_xcd();
  const int smax = splits(K) && parts != nullptr ? kMaxSplit : 1;
  // every XCD's range holds at most ceil(R/8) tiles; splitting adds at most kMaxParts - kMaxTail blocks
  const int64_t tiles = ((max_pairs + BM - 1) / BM + L) * ((N + ON - 1) / ON);
  const int64_t per_xcd = (tiles + kXcds - 1) / kXcds + (smax > 1 ? kMaxParts - kMaxTail : 0);
  MOE_LAUNCH(name, kern, dim3(unsigned(per_xcd * kXcds)), dim3(kThreads), lds, s, A, offsets, B0, B1, C, L, N, K, cpx,
             smax, parts);
  if (smax > 1) {
    const char* fname = NMAT == 2 ? "ffn_gate_up_fixup" : "ffn_down_fixup";
    MOE_LAUNCH(fname, fixup_kernel<NMAT>, dim3(unsigned(kXcds * kMaxTail * kFixSub)), dim3(kThreads), 0, s, offsets, C,
               L, N, K, cpx, smax, static_cast<const float*>(parts));
  }
  return MOE_OK;
}

}  // namespace big

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

constexpr int kThreads = 256, kUnroll = 8, kMaxRowBlocks = 4;

bool supported(int K) { return K % 32 == 0; }

// Each wave streams two sets of 16 weight rows: for gate/up the gate and the
// up rows of the same 16 output columns, for down two adjacent groups of 16
// output columns.  So a block (four waves) covers 64 gate/up columns or 128
// down columns, and every lane keeps two weight loads per k step in flight.
template <int NMAT>
constexpr int cols_per_block() { return NMAT == 2 ? 64 : 128; }

template <int NMAT>
__global__ __launch_bounds__(kThreads) void gemm_kernel(const bf16_t* __restrict__ A, const int32_t* __restrict__ offsets,
                                                        const bf16_t* __restrict__ B0, const bf16_t* __restrict__ B1,
                                                        bf16_t* __restrict__ C, int N, int K) {
  constexpr int kWaveCols = NMAT == 2 ? 16 : 32;
  const int expert = blockIdx.y;
  const int seg0 = offsets[expert];
  const int seg_n = offsets[expert + 1] - seg0;
  if (seg_n <= 0) return;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int col0 = blockIdx.x * cols_per_block<NMAT>() + wave * kWaveCols;  // first output column of this wave
  if (col0 >= N) return;
  const size_t boff = size_t(expert) * N * K;
  const int kg = (lane >> 4) * 8;  // the lane's 8 k values within a step
  // stream 0 / 1 weight row of this lane (rows past N repeat row N-1; never stored)
  const int wrow0 = min(col0 + (lane & 15), N - 1);
  const int wrow1 = NMAT == 2 ? wrow0 : min(col0 + 16 + (lane & 15), N - 1);
  const bf16_t* bs0 = B0 + boff + size_t(wrow0) * K + kg;
  const bf16_t* bs1 = (NMAT == 2 ? B1 : B0) + boff + size_t(wrow1) * K + kg;

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

    int k0 = 0;
    for (; k0 + 32 * kUnroll <= K; k0 += 32 * kUnroll) {
      bf16x8_t w0[kUnroll], w1[kUnroll], a0[kUnroll];
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) {
        w0[u] = *reinterpret_cast<const bf16x8_t*>(bs0 + k0 + 32 * u);
        w1[u] = *reinterpret_cast<const bf16x8_t*>(bs1 + k0 + 32 * u);
        a0[u] = *reinterpret_cast<const bf16x8_t*>(arow[0] + k0 + 32 * u);  // first row block: loaded with the weights
      }
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) {
#pragma unroll
        for (int rb = 0; rb < kMaxRowBlocks; ++rb) {
          if (rb < nrb) {
            const bf16x8_t a = rb == 0 ? a0[u] : *reinterpret_cast<const bf16x8_t*>(arow[rb] + k0 + 32 * u);
            acc[0][rb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, w0[u], acc[0][rb], 0, 0, 0);
            acc[1][rb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, w1[u], acc[1][rb], 0, 0, 0);
          }
        }
      }
    }
    for (; k0 < K; k0 += 32) {
      const bf16x8_t w0 = *reinterpret_cast<const bf16x8_t*>(bs0 + k0);
      const bf16x8_t w1 = *reinterpret_cast<const bf16x8_t*>(bs1 + k0);
#pragma unroll
      for (int rb = 0; rb < kMaxRowBlocks; ++rb) {
        if (rb < nrb) {
          const bf16x8_t a = *reinterpret_cast<const bf16x8_t*>(arow[rb] + k0);
          acc[0][rb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, w0, acc[0][rb], 0, 0, 0);
          acc[1][rb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, w1, acc[1][rb], 0, 0, 0);
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
            if (col < N) crow[col] = f32_to_bf16(silu(acc[0][rb][i]) * acc[1][rb][i]);
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

template <int NMAT>
moe_status launch(const char* name, const bf16_t* A, const int32_t* offsets, const bf16_t* B0, const bf16_t* B1,
                  bf16_t* C, int L, int N, int K, hipStream_t s) {
  const dim3 grid(unsigned((N + cols_per_block<NMAT>() - 1) / cols_per_block<NMAT>()), unsigned(L));
  MOE_LAUNCH(name, gemm_kernel<NMAT>, grid, dim3(kThreads), 0, s, A, offsets, B0, B1, C, N, K);
  return MOE_OK;
}

}  // namespace skinny

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

// large tiles pay off once segments hold a few hundred rows; decode-sized
// batches (a handful of rows per expert) take the skinny kernel
bool use_big(const moe_layer_desc* d, int64_t max_pairs) {
  return d->dtype == MOE_BF16 && max_pairs >= int64_t(128) * d->local_count && big::supported(d->hidden) &&
         big::supported(d->intermediate);
}

moe_status launch_small(const FfnArgs& a) {
  const moe_layer_desc* d = a.d;
  const int L = d->local_count, H = d->hidden, I = d->intermediate;
  // decode-sized batches: a few rows per expert, bound by streaming the weights
  if (d->dtype == MOE_BF16 && a.max_pairs <= int64_t(32) * L && skinny::supported(H) && skinny::supported(I)) {
    bf16_t* h = static_cast<bf16_t*>(a.h);
    moe_status st = skinny::launch<2>("ffn_gate_up", static_cast<const bf16_t*>(a.x_sorted), a.offsets,
                                      static_cast<const bf16_t*>(a.w_gate), static_cast<const bf16_t*>(a.w_up), h, L, I,
                                      H, a.s);
    if (st != MOE_OK) return st;
    return skinny::launch<1>("ffn_down", h, a.offsets, static_cast<const bf16_t*>(a.w_down),
                             static_cast<const bf16_t*>(a.w_down), static_cast<bf16_t*>(a.y_sorted), L, H, I, a.s);
  }
  return d->dtype == MOE_BF16 ? launch_t<bf16_t>(a) : launch_t<float>(a);
}

}  // namespace

size_t ffn_parts_bytes(const moe_layer_desc* d, int64_t max_pairs) {
  if (!use_big(d, max_pairs) || !(big::splits(d->hidden) || big::splits(d->intermediate))) return 0;
  return size_t(big::kXcds) * big::kMaxParts * big::kPartBytes;
}

moe_status launch_grouped_ffn(const FfnArgs& a) {
  if (a.max_pairs <= 0) return MOE_OK;
  const moe_layer_desc* d = a.d;
  if (!use_big(d, a.max_pairs)) return launch_small(a);
  const int L = d->local_count, H = d->hidden, I = d->intermediate;
  const bf16_t* x = static_cast<const bf16_t*>(a.x_sorted);
  bf16_t* h = static_cast<bf16_t*>(a.h);
  moe_status st = big::launch<2>("ffn_gate_up", x, a.offsets, static_cast<const bf16_t*>(a.w_gate),
                                 static_cast<const bf16_t*>(a.w_up), h, L, I, H, a.max_pairs, a.parts, a.s);
  if (st != MOE_OK) return st;
  return big::launch<1>("ffn_down", h, a.offsets, static_cast<const bf16_t*>(a.w_down),
                        static_cast<const bf16_t*>(a.w_down), static_cast<bf16_t*>(a.y_sorted), L, H, I, a.max_pairs,
                        a.parts, a.s);
}

}  // namespace moe
