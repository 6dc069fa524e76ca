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

#include <algorithm>

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

// SiLU through the hardware reciprocal (1 ulp) rather than an IEEE division:
// five instructions instead of about fifteen.  Every FFN kernel here uses this
// one definition, so a token's result does not depend on which kernel ran it.
// Both ends stay exact: exp(-z) overflowing gives -0, underflowing gives z.
__device__ __forceinline__ float silu(float z) { return z * __builtin_amdgcn_rcpf(1.0f + __expf(-z)); }

// NMAT = 2: gate and up products with the SwiGLU epilogue; NMAT = 1: plain product.
// Tiles of BMT (128 or 64) token rows x BN weight rows; the waves split them 2 x 2,
// so a wave holds BMT/64 x 2 MFMA 32x32 blocks per matrix.
template <typename T, int NMAT, int BMT>
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
  auto gload = [&](int k0) {
#pragma unroll
    for (int j = 0; j < CPTA; ++j) {
      const int c = tid + j * kThreads;
      const int r = c / CPR, col = c % CPR;
      const int kk = k0 + col * EPV;
      const int ar = min(r, rows - 1);  // rows past the segment repeat its last row; never stored
      ra[j] = kk < K ? *reinterpret_cast<const uint4*>(A + size_t(row0 + ar) * K + kk) : zero;
    }
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
  };
  auto sstore = [&](int buf) {
#pragma unroll
    for (int j = 0; j < CPTA; ++j) {
      const int c = tid + j * kThreads;
      const int r = c / CPR, col = c % CPR;
      *reinterpret_cast<uint4*>(&As[buf][r * kLd + col * EPV]) = ra[j];
    }
#pragma unroll
    for (int j = 0; j < CPTB; ++j) {
      const int c = tid + j * kThreads;
      const int r = c / CPR, col = c % CPR;
#pragma unroll
      for (int m = 0; m < NMAT; ++m) *reinterpret_cast<uint4*>(&Bs[buf][m][r * kLd + col * EPV]) = rb[m][j];
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

constexpr int BM = 256, BNE = 256, BK = 64, kStages = 2;
constexpr int kRowBytes = BK * 2;              // 128
constexpr int kGroupN = 4;
constexpr int kXcds = 8;

// s_waitcnt on the vector-memory counter only (expcnt and lgkmcnt left at their maxima)
#define MOE_VMCNT(n) __builtin_amdgcn_s_waitcnt(((n) & 0xF) | (((n) >> 4) << 14) | (0x7 << 4) | (0xF << 8))
#define MOE_LGKMCNT0() __builtin_amdgcn_s_waitcnt(0xC07F)

bool supported(int K) { return K % BK == 0; }
// word 3 of a buffer descriptor on this family: 32-bit data format, raw byte addressing
constexpr int kRsrcFlags = 0x00020000;
// the direct loads address a weight matrix with 32-bit byte offsets
bool addressable(int64_t rows, int64_t K) { return rows * K * 2 < (int64_t(1) << 32); }

// ---- work plan -------------------------------------------------------------
// Tiles are numbered over (expert, group of kGroupN n-tiles, m-tile, n-tile
// in group) and dealt to the XCDs in contiguous ranges (block b runs on XCD
// b % 8).  An XCD with q tiles runs them in rounds of `cpx` (its CU count);
// when the last round is only partly filled, its r tiles may be cut into s
// pieces along K, so the XCD finishes in F + ceil(r*s/cpx)/s tile times
// instead of F + 1.  Each piece writes its float32 accumulators and
// fixup_kernel adds the pieces in piece order (so the result does not depend
// on timing) and runs the usual epilogue.  A cut pays when the tile time it
// saves, (1 - ceil(r*s/cpx)/s) * nk steps, exceeds the pieces' write and
// re-read, which cost about kPieceSteps steps each (256 KB out and back per
// piece against the tile's 64 KB per step from L2 and MALL).
constexpr int kSplitMinSteps = 32;   // K/BK from which the last round may be cut
constexpr int kMaxSplit = 4;
constexpr int kMaxParts = 96;        // pieces per XCD
constexpr int kMaxTail = kMaxParts / kMaxSplit;
constexpr size_t kPartBytes = size_t(65536) * sizeof(float);  // one piece's accumulators (a 256 x 256 tile)
constexpr float kPieceSteps = 0.4f;

__device__ __forceinline__ int split_of(int r, int cpx, int smax, int nk) {
  int best = 1;
  float best_net = 0.0f;
  for (int s = 2; s <= smax; s *= 2) {
    if (r == 0 || r > kMaxTail || nk < 16 * s || r * s > kMaxParts) break;
    const float rounds = float((r * s + cpx - 1) / cpx) / float(s);  // tile times the pieces take
    const float net = (1.0f - rounds) * float(nk) - kPieceSteps * float(r * s);
    if (net > best_net) {
      best = s;
      best_net = net;
    }
  }
  return best;
}

struct Job {
  int expert, row0, rows, n0;
  bool wide;       // a segment's tail of at most 128 rows: 128 rows x 512 B rows (two n-tiles)
  int kb, nks;     // k steps [kb, kb + nks)
  int part, nparts, pslot;
};

// Tiles of one expert with n rows: in every group of up to kGroupN n-tiles,
// the full 256-row m-tiles, then the tail m-tile: a regular tile per n-tile
// when the tail has more than 128 rows, else one wide tile per two n-tiles.
__device__ __forceinline__ int tail_tiles(int tail, int gsz) {
  return tail == 0 ? 0 : (tail <= BM / 2 ? (gsz + 1) / 2 : gsz);
}
__device__ __forceinline__ int expert_tiles(int n, int NT) {
  const int mf = n / BM, tail = n - mf * BM;
  const int nfull = NT / kGroupN, last = NT - nfull * kGroupN;
  return nfull * (mf * kGroupN + tail_tiles(tail, kGroupN)) + (last ? mf * last + tail_tiles(tail, last) : 0);
}

// One XCD's share of the work: tiles [base, base + qx) in rounds of cpx; the r
// tiles of a partly filled last round are cut into s pieces (s = 1: not cut).
struct XcdPlan {
  int base, qx, F, r, s, units;
};

__device__ __forceinline__ XcdPlan plan_xcd(int R, int nk, int cpx, int smax, int xcd) {
  XcdPlan xp;
  const int q = R / kXcds, rr = R % kXcds;
  xp.qx = q + (xcd < rr ? 1 : 0);
  xp.base = xcd * q + min(xcd, rr);
  xp.F = xp.qx / cpx;
  xp.r = xp.qx - xp.F * cpx;
  xp.s = split_of(xp.r, cpx, smax, nk);
  xp.units = xp.s == 1 ? xp.qx : xp.F * cpx + xp.r * xp.s;
  return xp;
}

// Per-expert tile counts of both products, as exclusive prefix sums
// (pre[0..L] for gate/up, pre[L+1..2L+1] for down), so that a GEMM block
// finds the total and its tile's expert without walking all the offsets.
__global__ __launch_bounds__(1024) void plan_kernel(const int32_t* __restrict__ offsets, int L, int NT_gu, int NT_dn,
                                                    int32_t* __restrict__ pre) {
  __shared__ int wa[16], wb[16];  // per-wave totals
  int carry_gu = 0, carry_dn = 0;
  for (int i0 = 0; i0 < L; i0 += 1024) {
    const int i = i0 + threadIdx.x;
    const int n = i < L ? offsets[i + 1] - offsets[i] : 0;
    const int a = i < L ? expert_tiles(n, NT_gu) : 0;
    const int b = i < L ? expert_tiles(n, NT_dn) : 0;
    // two block scans (inclusive within waves, then over the wave totals)
    int va = a, vb = b;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    for (int d = 1; d < 64; d <<= 1) {
      const int ta = __shfl_up(va, d, 64), tb = __shfl_up(vb, d, 64);
      if (lane >= d) {
        va += ta;
        vb += tb;
      }
    }
    if (lane == 63) {
      wa[wave] = va;
      wb[wave] = vb;
    }
    __syncthreads();
    int ba = 0, bb = 0, ta = 0, tb = 0;
    for (int w = 0; w < 16; ++w) {
      if (w < wave) {
        ba += wa[w];
        bb += wb[w];
      }
      ta += wa[w];
      tb += wb[w];
    }
    if (i < L) {
      pre[i] = carry_gu + ba + va - a;
      pre[L + 1 + i] = carry_dn + bb + vb - b;
    }
    carry_gu += ta;
    carry_dn += tb;
    __syncthreads();
  }
  if (threadIdx.x == 0) {
    pre[L] = carry_gu;
    pre[2 * L + 1] = carry_dn;
  }
}

// expert, rows and columns of tile t; tpre = the product's tile prefix (L + 1 entries)
__device__ __forceinline__ void tile_of(const int32_t* __restrict__ offsets, const int32_t* tpre, int L, int NT, int t,
                                        Job& jb) {
  // the expert: the last i with tpre[i] <= t (experts with no tiles have tpre[i] == tpre[i+1])
  int lo = 0, hi = L - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (tpre[mid] <= t) lo = mid; else hi = mid - 1;
  }
  jb.expert = lo;
  t -= tpre[lo];
  const int seg0 = offsets[lo];
  const int seg_n = offsets[lo + 1] - seg0;
  const int mf = seg_n / BM, tl = seg_n - mf * BM;
  const int nfull = NT / kGroupN;
  const int per_group = mf * kGroupN + tail_tiles(tl, kGroupN);
  int ng = t / per_group;
  if (ng > nfull) ng = nfull;  // past the full groups: the last, partial group
  const int rem = t - ng * per_group;
  const int gsz = ng < nfull ? kGroupN : NT - nfull * kGroupN;
  if (rem < mf * gsz) {
    const int mt = rem / gsz;
    jb.n0 = ng * kGroupN + (rem - mt * gsz);
    jb.row0 = seg0 + mt * BM;
    jb.rows = BM;
    jb.wide = false;
  } else {
    const int r2 = rem - mf * gsz;
    jb.row0 = seg0 + mf * BM;
    jb.rows = tl;
    jb.wide = tl <= BM / 2;
    jb.n0 = ng * kGroupN + (jb.wide ? 2 * r2 : r2);
  }
}

// Unit u of the XCD (u < xp.units): a whole tile, or one K piece of a tile of the last round.
__device__ __forceinline__ void unit_job(const int32_t* __restrict__ offsets, const int32_t* tpre, int L, int NT, int nk,
                                         int cpx, int xcd, const XcdPlan& xp, int u, Job& jb) {
  int t;
  if (u < xp.F * cpx || xp.s == 1) {
    t = xp.base + u;
    jb.part = 0;
    jb.nparts = 1;
    jb.pslot = 0;
  } else {
    const int v = u - xp.F * cpx;
    const int w = v / xp.s;
    t = xp.base + xp.F * cpx + w;
    jb.part = v - w * xp.s;
    jb.nparts = xp.s;
    jb.pslot = xcd * kMaxParts + v;
  }
  tile_of(offsets, tpre, L, NT, t, jb);
  jb.kb = (jb.part * nk) / jb.nparts;
  jb.nks = ((jb.part + 1) * nk) / jb.nparts - jb.kb;
}

// Tile shapes: regular 256 A rows x 256 B rows, wide 128 A rows x 512 B rows.  With
// NW = 4 waves (one per SIMD) a wave owns 128 A rows x 128 B rows (4 x 4 MFMA 32x32
// accumulators, waves 2 x 2, or 1 x 4 for the wide tile); with NW = 8 (two per SIMD)
// 128 A rows x 64 B rows (4 x 2 accumulators, waves 2 x 4, or 1 x 8).  NB = 16 / NW
// B fragments per wave.
template <bool WIDE, int NW>
struct Shape {
  static constexpr int kThreads = NW * 64;
  static constexpr int NB = 16 / NW;
  static constexpr int kA = WIDE ? BM / 2 : BM;          // A rows
  static constexpr int kB = WIDE ? 2 * BNE : BNE;        // B rows
  static constexpr int kStageA = kA * kRowBytes;
  static constexpr int kStage = (kA + kB) * kRowBytes;   // 64 KB regular, 80 KB wide
  static constexpr int kLdA = kA / (8 * NW), kLdB = kB / (8 * NW);  // 1 KB direct loads per wave per stage
  static constexpr int kLd = kLdA + kLdB;
  __device__ static int wm(int wave) { return WIDE ? 0 : wave / (NW / 2); }
  __device__ static int wn(int wave) { return WIDE ? wave : wave % (NW / 2); }
};
constexpr size_t kLoopLdsMax = size_t(kStages) * Shape<true, 4>::kStage;  // 160 KB

// ---- epilogue.  The products were formed as (weight rows) x (token rows), so
// in the 32x32 accumulator layout lane l holds token row l & 31 and register
// 4q+u holds output column 8q + 4*(l/32) + u: four adjacent columns per q.
// Each wave converts its part of the tile to bf16 (SwiGLU first for gate/up)
// and parks it in LDS, rows padded by 16 bytes; then every thread copies
// 16-byte row chunks out, so each store instruction writes whole row pieces.
// The caller has made sure no wave still reads the loop's LDS stages.
// EP: kPlain; kSave (gate/up of the training forward: the gate and up
// pre-activations are written too, to Gs and Us); kSwigluBwd (the down
// product's dgrad dh = dy_sorted Wd: reads the saved gate and up values Gs, Us
// and writes dg and du side by side into C, rows of 2N).
constexpr int kPlain = 0, kSave = 1, kSwigluBwd = 2;
// the weight-gradient products (see wgrad_k): gemm_kernel decodes its own jobs
constexpr int kWgrad = 3;

template <int NMAT, bool WIDE, int NW, int EP>
__device__ __forceinline__ void epilogue(f32x16_t (&acc)[4][16 / NW], char* lds, bf16_t* __restrict__ C, int row0,
                                         int rows, int n0, int N, bf16_t* __restrict__ Gs, bf16_t* __restrict__ Us) {
  if constexpr (EP == kPlain || EP == kWgrad) {
  using S = Shape<WIDE, NW>;
  constexpr int NB = S::NB, kThreads = S::kThreads;
  constexpr int TC = NMAT == 2 ? S::kB / 2 : S::kB;  // output columns of the tile
  constexpr int RS = TC * 2 + 16;
  constexpr int NJ = NMAT == 2 ? NB / 2 : NB;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int wm = S::wm(wave), wn = S::wn(wave), fr = lane & 31, g = lane >> 5;
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
          v[u] = NMAT == 2 ? silu(acc[i][j][4 * q + u]) * acc[i][j + NB / 2][4 * q + u] : acc[i][j][4 * q + u];
        uint2 pk;
        pk.x = pack_bf16x2(v[0], v[1]);
        pk.y = pack_bf16x2(v[2], v[3]);
        const int cl = (NMAT == 2 ? wn * NB * 16 : wn * NB * 32) + j * 32 + 8 * q + 4 * g;
        *reinterpret_cast<uint2*>(lds + rt * RS + cl * 2) = pk;
      }
    }
  }
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
  block_barrier();
  constexpr int CPR = TC / 8;  // 16-byte chunks per row
#pragma unroll
  for (int u = 0; u < S::kA * CPR / kThreads; ++u) {
    const int id = tid + kThreads * u;
    const int r = id / CPR, c = id % CPR;
    const u32x4_t val = *reinterpret_cast<const u32x4_t*>(lds + r * RS + c * 16);
    // N is a multiple of 8, so a chunk is wholly inside or wholly past column N
    if (r < rows && n0 + c * 8 < N) *reinterpret_cast<u32x4_t*>(C + size_t(row0 + r) * N + n0 + c * 8) = val;
  }
  } else if constexpr (EP == kSave) {
  using S = Shape<WIDE, NW>;
  constexpr int NB = S::NB, kThreads = S::kThreads;
  constexpr int TC = NMAT == 2 ? S::kB / 2 : S::kB;  // output columns of the tile
  constexpr int RS = TC * 2 + 16;
  constexpr int NJ = NMAT == 2 ? NB / 2 : NB;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int wm = S::wm(wave), wn = S::wn(wave), fr = lane & 31, g = lane >> 5;
  // sel 0: the output (SwiGLU for gate/up); sel 1, 2: the gate, up pre-activations
  auto park = [&](int sel) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int rt = wm * 128 + i * 32 + fr;
#pragma unroll
      for (int j = 0; j < NJ; ++j) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          float v[4];
#pragma unroll
          for (int u = 0; u < 4; ++u) {
            if constexpr (NMAT == 1) {
              v[u] = acc[i][j][4 * q + u];
            } else {
              const float gv = acc[i][j][4 * q + u], uv = acc[i][j + NB / 2][4 * q + u];
              v[u] = sel == 0 ? silu(gv) * uv : (sel == 1 ? gv : uv);
            }
          }
          uint2 pk;
          pk.x = pack_bf16x2(v[0], v[1]);
          pk.y = pack_bf16x2(v[2], v[3]);
          const int cl = (NMAT == 2 ? wn * NB * 16 : wn * NB * 32) + j * 32 + 8 * q + 4 * g;
          *reinterpret_cast<uint2*>(lds + rt * RS + cl * 2) = pk;
        }
      }
    }
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
    block_barrier();
  };
  constexpr int CPR = TC / 8;  // 16-byte chunks per row
  auto copy_out = [&](bf16_t* __restrict__ dst) {
#pragma unroll
    for (int u = 0; u < S::kA * CPR / kThreads; ++u) {
      const int id = tid + kThreads * u;
      const int r = id / CPR, c = id % CPR;
      const u32x4_t val = *reinterpret_cast<const u32x4_t*>(lds + r * RS + c * 16);
      // N is a multiple of 8, so a chunk is wholly inside or wholly past column N
      if (r < rows && n0 + c * 8 < N) *reinterpret_cast<u32x4_t*>(dst + size_t(row0 + r) * N + n0 + c * 8) = val;
    }
  };
  park(0);
  copy_out(C);
  if (NMAT == 2) {
    // training: the pre-activations too, through the same LDS tile once every
    // wave has read the previous one out
#pragma unroll 1
    for (int sel = 1; sel <= 2; ++sel) {
      __builtin_amdgcn_s_waitcnt(0xC07F);
      block_barrier();
      park(sel);
      copy_out(sel == 1 ? Gs : Us);
    }
  }
  } else {
  // SwiGLU backward (NMAT == 1): dh is parked as bf16 like a plain output; the
  // copy-out reads the saved gate and up values of the same 8 columns and
  // writes dg = dh up silu'(gate) and du = dh silu(gate), silu'(g) = s (1 + g (1 - s)).
  static_assert(NMAT == 1, "the SwiGLU backward epilogue follows the down product's dgrad");
  using S = Shape<WIDE, NW>;
  constexpr int NB = S::NB, kThreads = S::kThreads;
  constexpr int TC = S::kB;
  constexpr int RS = TC * 2 + 16;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int wm = S::wm(wave), wn = S::wn(wave), fr = lane & 31, g = lane >> 5;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int rt = wm * 128 + i * 32 + fr;
#pragma unroll
    for (int j = 0; j < NB; ++j) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        uint2 pk;
        pk.x = pack_bf16x2(acc[i][j][4 * q], acc[i][j][4 * q + 1]);
        pk.y = pack_bf16x2(acc[i][j][4 * q + 2], acc[i][j][4 * q + 3]);
        const int cl = wn * NB * 32 + j * 32 + 8 * q + 4 * g;
        *reinterpret_cast<uint2*>(lds + rt * RS + cl * 2) = pk;
      }
    }
  }
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
  block_barrier();
  constexpr int CPR = TC / 8;
#pragma unroll
  for (int u = 0; u < S::kA * CPR / kThreads; ++u) {
    const int id = tid + kThreads * u;
    const int r = id / CPR, c = id % CPR;
    if (r < rows && n0 + c * 8 < N) {
      const u32x4_t dh = *reinterpret_cast<const u32x4_t*>(lds + r * RS + c * 16);
      const size_t at = size_t(row0 + r) * N + n0 + c * 8;
      const u32x4_t gv = *reinterpret_cast<const u32x4_t*>(Gs + at);
      const u32x4_t uv = *reinterpret_cast<const u32x4_t*>(Us + at);
      u32x4_t dg, du;
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        float o_g[2], o_u[2];
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const float fd = __uint_as_float(h ? dh[w] & 0xFFFF0000u : dh[w] << 16);
          const float fg = __uint_as_float(h ? gv[w] & 0xFFFF0000u : gv[w] << 16);
          const float fu = __uint_as_float(h ? uv[w] & 0xFFFF0000u : uv[w] << 16);
          const float sg = __builtin_amdgcn_rcpf(1.0f + __expf(-fg));
          o_g[h] = fd * fu * (sg * (1.0f + fg * (1.0f - sg)));
          o_u[h] = fd * (fg * sg);
        }
        dg[w] = pack_bf16x2(o_g[0], o_g[1]);
        du[w] = pack_bf16x2(o_u[0], o_u[1]);
      }
      bf16_t* o = C + size_t(row0 + r) * 2 * N + n0 + c * 8;
      *reinterpret_cast<u32x4_t*>(o) = dg;
      *reinterpret_cast<u32x4_t*>(o + N) = du;
    }
  }
  }
}

template <int NMAT>
constexpr size_t lds_bytes() {
  constexpr size_t reg = size_t(Shape<false, 4>::kA) * ((NMAT == 2 ? BNE / 2 : BNE) * 2 + 16);
  constexpr size_t wide = size_t(Shape<true, 4>::kA) * ((NMAT == 2 ? BNE : 2 * BNE) * 2 + 16);
  constexpr size_t st = reg > wide ? reg : wide;
  return kLoopLdsMax > st ? kLoopLdsMax : st;
}

// A piece's accumulators, thread-major: float4 number v of thread t at (v*256 + t)
__device__ __forceinline__ f32x4_t* part_ptr(float* __restrict__ parts, int pslot) {
  return reinterpret_cast<f32x4_t*>(parts + size_t(pslot) * (kPartBytes / sizeof(float)));
}

// One tile (or one K piece of it): the main loop, then the epilogue or the piece write-out.
template <int NMAT, bool WIDE, int NW, int EP>
__device__ __forceinline__ void tile_body(const bf16_t* __restrict__ A, int a_rows, const bf16_t* __restrict__ Bg,
                                          const bf16_t* __restrict__ Bu, bf16_t* __restrict__ C, int N, int K,
                                          const Job& jb, float* __restrict__ parts, char* lds,
                                          bf16_t* __restrict__ Gs, bf16_t* __restrict__ Us) {
  using S = Shape<WIDE, NW>;
  constexpr int NB = S::NB, kThreads = S::kThreads;
  constexpr int ON = NMAT == 2 ? BNE / 2 : BNE;
  const int row0 = jb.row0, rows = jb.rows, n0 = jb.n0 * ON, kb = jb.kb, nks = jb.nks;
  // the wave index is uniform: keeping it in a scalar register makes every LDS
  // target of the direct loads scalar arithmetic
  const int tid = threadIdx.x, wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  const int wm = S::wm(wave), wn = S::wn(wave);

  // ---- direct loads: per stage kLdA 1 KB blocks of 8 A rows and kLdB of 8 B
  // rows per wave; wave w fills A blocks kLdA*w.. and B blocks kLdB*w.. .  Lane
  // i of block j writes row (first row of the wave) + 8j + i/8, physical chunk
  // i%8, which holds logical chunk (i%8) ^ ((row/2)%8); as the wave's first row
  // is a multiple of 16, that depends on i and the parity of j only.
  const int c_even = (lane & 7) ^ ((lane >> 4) & 7);
  const int c_odd = (lane & 7) ^ ((4 + (lane >> 4)) & 7);
  const int a_lrow = (S::kA / NW) * wave + (lane >> 3);
  // buffer resources over the tile's rows of A and over the whole weight matrix
  // (its extent is under 4 GiB); a read outside either returns zeros
  const uint32_t a_bytes = uint32_t(min(int64_t(a_rows - row0) * K * 2, int64_t(0xFFFFFFFF)));
  const __amdgpu_buffer_rsrc_t a_rsrc =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<bf16_t*>(A + size_t(row0) * K), 0, a_bytes, kRsrcFlags);
  int b_lrow;
  if (NMAT == 2) b_lrow = ((S::kB / NW) * wave + (lane >> 3)) & (S::kB / 2 - 1);  // first half of the waves: gate rows
  else b_lrow = (S::kB / NW) * wave + (lane >> 3);
  const __amdgpu_buffer_rsrc_t b_rsrc = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<bf16_t*>(NMAT == 2 && wave >= NW / 2 ? Bu : Bg), 0, uint32_t(N) * uint32_t(K) * 2u, kRsrcFlags);
  // Rows past the segment (A) or past N (B) feed only outputs that are never
  // stored, so they may read any valid row: A takes the rows that follow (up
  // to the last row of the buffer), B wraps around to the first rows.  Letting
  // them all repeat one row would send every lane of the padding to the same
  // 128 bytes, one L2 channel, on every step.
  // Each lane's byte offsets are fixed for the whole loop (A from the tile's
  // first row, B from the matrix); a step only moves the scalar offset by k0,
  // so a load costs no vector arithmetic.
  const int a_lim = a_rows - 1 - row0;
  uint32_t a_vo[S::kLdA], b_vo[S::kLdB];
#pragma unroll
  for (int j = 0; j < S::kLdA; ++j) {
    const int cc = (j & 1) ? c_odd : c_even;
    a_vo[j] = (uint32_t(min(a_lrow + 8 * j, a_lim)) * uint32_t(K) + uint32_t(cc * 8)) * 2u;
  }
#pragma unroll
  for (int j = 0; j < S::kLdB; ++j) {
    const int cc = (j & 1) ? c_odd : c_even;
    int r = n0 + b_lrow + 8 * j;
    if (r >= N) r %= N;
    b_vo[j] = (uint32_t(r) * uint32_t(K) + uint32_t(cc * 8)) * 2u;
  }
// loads q0..q1-1 of stage kt_, in the order A0 B0 A1 B1 ... (then the B rows
// past the last A block)
#define MOE_ISSUE(kt_, q0_, q1_)                                                                            \
  do {                                                                                                      \
    char* sa_ = lds + ((kt_) % kStages) * S::kStage + (S::kLdA * wave) * 1024;                              \
    char* sb_ = lds + ((kt_) % kStages) * S::kStage + S::kStageA + (S::kLdB * wave) * 1024;                 \
    const uint32_t k0_ = uint32_t(kb + (kt_)) * (BK * 2);                                                   \
    _Pragma("unroll") for (int q = (q0_); q < (q1_); ++q) {                                                 \
      const int j_ = q < 2 * S::kLdA ? q / 2 : q - S::kLdA;                                                 \
      if (q < 2 * S::kLdA && q % 2 == 0)                                                                    \
        __builtin_amdgcn_raw_ptr_buffer_load_lds(a_rsrc, (lds_ptr_t)(sa_ + j_ * 1024), 16, a_vo[j_], k0_, 0, 0); \
      else                                                                                                  \
        __builtin_amdgcn_raw_ptr_buffer_load_lds(b_rsrc, (lds_ptr_t)(sb_ + j_ * 1024), 16, b_vo[j_], k0_, 0, 0); \
    }                                                                                                       \
  } while (0)

  f32x16_t acc[4][NB];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < NB; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

  // ---- fragment addresses: A rows wm*128 + i*32 + (lane & 31); B rows of the
  // wave's four 32-column blocks (gate/up: two gate blocks, then the two up
  // blocks of the same columns) --------------------------------------------
  const int fr = lane & 31;
  const int sw = (fr >> 1) & 7;
  const int g = lane >> 5;
  int boffs[NB];
#pragma unroll
  for (int j = 0; j < NB; ++j) {
    const int br = NMAT == 2 ? (j < NB / 2 ? wn * NB * 16 + j * 32 : S::kB / 2 + wn * NB * 16 + (j - NB / 2) * 32)
                             : wn * NB * 32 + j * 32;
    boffs[j] = S::kStageA + (br + fr) * kRowBytes;
  }
  const int a_off = (wm * 128 + fr) * kRowBytes;
  bf16x8_t fa[2][4], fb[2][NB];
#define MOE_LOADF(buf_, st_, kc_)                                                                         \
  do {                                                                                                    \
    const int co_ = ((2 * (kc_) + g) ^ sw) * 16;                                                          \
    _Pragma("unroll") for (int i = 0; i < 4; ++i)                                                         \
      fa[buf_][i] = *reinterpret_cast<const bf16x8_t*>((st_) + a_off + i * 32 * kRowBytes + co_);          \
    _Pragma("unroll") for (int j = 0; j < NB; ++j)                                                        \
      fb[buf_][j] = *reinterpret_cast<const bf16x8_t*>((st_) + boffs[j] + co_);                            \
  } while (0)
#define MOE_MMA(buf_)                                                                                     \
  do {                                                                                                    \
    _Pragma("unroll") for (int i = 0; i < 4; ++i)                                                         \
      _Pragma("unroll") for (int j = 0; j < NB; ++j)                                                      \
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fb[buf_][j], fa[buf_][i], acc[i][j], 0, 0, 0); \
  } while (0)
  // 8 x {MFMA, LDS read, MFMA}: the next chunk's fragment reads spread over the whole group
#define MOE_PIPE_DS()                                                                                     \
  do {                                                                                                    \
    if constexpr (NB == 4) {                                                                              \
      _Pragma("unroll") for (int p_ = 0; p_ < 8; ++p_) {                                                  \
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);                                                \
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);                                                \
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);                                                \
      }                                                                                                   \
    } else {                                                                                              \
      _Pragma("unroll") for (int p_ = 0; p_ < 4 + NB; ++p_) {                                             \
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);                                                \
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);                                                \
      }                                                                                                   \
      __builtin_amdgcn_sched_group_barrier(0x008, 4 * NB - (4 + NB), 0);                                  \
    }                                                                                                     \
  } while (0)

  // The refill of a stage goes out in two halves: the first right after the
  // barrier that frees its slot (beside the last chunk of the stage before),
  // the second beside the first chunk of the stage in between.  Against one
  // burst of all kLd loads per step this halves the rate at which the 32 CUs
  // of an XCD hit L2 together, and the second half still has three chunks to
  // land before the barrier that waits for it.
  constexpr int kHalf = S::kLd / 2;
  // a chunk that also issues half a refill: its fragment reads first, then the loads
  // spread over its 4 * NB MFMAs
#define MOE_CHUNK_LOADS()                                                                                 \
  do {                                                                                                    \
    __builtin_amdgcn_sched_group_barrier(0x100, 4 + NB, 0);                                               \
    if constexpr (NB == 4) {                                                                              \
      _Pragma("unroll") for (int p_ = 0; p_ < 8; ++p_) {                                                  \
        __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);                                                \
        __builtin_amdgcn_sched_group_barrier(0x020, kHalf / 8, 0);                                        \
      }                                                                                                   \
      if constexpr (kHalf % 8 != 0) __builtin_amdgcn_sched_group_barrier(0x020, kHalf % 8, 0);           \
    } else {                                                                                              \
      _Pragma("unroll") for (int p_ = 0; p_ < kHalf; ++p_) {                                              \
        __builtin_amdgcn_sched_group_barrier(0x008, 4 * NB / kHalf, 0);                                   \
        __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);                                                \
      }                                                                                                   \
    }                                                                                                     \
  } while (0)
  MOE_ISSUE(0, 0, S::kLd);
  if (nks > 1) {
    MOE_ISSUE(1, 0, kHalf);
    MOE_VMCNT(kHalf);  // stage 0 landed
  } else {
    MOE_VMCNT(0);
  }
  block_barrier();
  MOE_LOADF(0, lds, 0);
  // every iteration has a next stage; the refill issued in it is stage kt+2,
  // or (near the end) a repeat of the last stage into the free slot
  for (int kt = 0; kt + 1 < nks; ++kt) {
    const char* st = lds + (kt % kStages) * S::kStage;
    MOE_LOADF(1, st, 1);
    MOE_ISSUE(min(kt + 1, nks - 1), kHalf, S::kLd);
    MOE_MMA(0);
    MOE_CHUNK_LOADS();
    __builtin_amdgcn_sched_barrier(0);
    MOE_LOADF(0, st, 2);
    MOE_MMA(1);
    MOE_LOADF(1, st, 3);
    MOE_MMA(0);
    MOE_PIPE_DS();
    MOE_PIPE_DS();
    __builtin_amdgcn_sched_barrier(0);
    MOE_VMCNT(0);     // this wave's loads of stage kt+1 have landed
    MOE_LGKMCNT0();   // and its reads of stage kt are done
    block_barrier();
    __builtin_amdgcn_sched_barrier(0);
    MOE_LOADF(0, lds + ((kt + 1) % kStages) * S::kStage, 0);
    MOE_ISSUE(min(kt + 2, nks - 1), 0, kHalf);
    MOE_MMA(1);
    MOE_CHUNK_LOADS();
  }
  {
    const char* st = lds + ((nks - 1) % kStages) * S::kStage;
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
#undef MOE_CHUNK_LOADS

  if (jb.nparts > 1) {
    // one piece of a split tile: park the accumulators for fixup_kernel
    f32x4_t* dst = part_ptr(parts, jb.pslot);
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < NB; ++j)
#pragma unroll
        for (int c = 0; c < 4; ++c)
          dst[((i * NB + j) * 4 + c) * kThreads + tid] =
              f32x4_t{acc[i][j][4 * c], acc[i][j][4 * c + 1], acc[i][j][4 * c + 2], acc[i][j][4 * c + 3]};
    return;
  }
  MOE_LGKMCNT0();
  block_barrier();  // every wave is done reading the last stage
  epilogue<NMAT, WIDE, NW, EP>(acc, lds, C, row0, rows, n0, N, Gs, Us);
}

// ---- weight gradients on the large tile --------------------------------------
// Expert e's dW = A_e B_e^T reduces over its rows.  The caller has copied the
// operands transposed into per-expert blocks [rows, K_e] with K_e the segment
// length rounded up to 64 (at least 64; the padding is zero), at element offset
// rows * Q_e (Q_e = sum of K_e' over e' < e), so each expert's product has
// the forward's operand layout with its own K.  In gemm_kernel's kWgrad mode:
// blockIdx x = tile (m major), y = expert, z = which of up to two (A, C) pairs
// (A rows [z M, (z+1) M)); A = the transposed blocks (a_rows of them per
// expert), B0 = B's blocks, C and Gs = the two outputs, K = M.
__device__ __forceinline__ int wgrad_k(int n) { return n <= 64 ? 64 : (n + 63) / 64 * 64; }

template <int NMAT, int NW, int EP>
__global__ __launch_bounds__(NW * 64) void gemm_kernel(const bf16_t* __restrict__ A, const int32_t* __restrict__ offsets,
                                                       const bf16_t* __restrict__ B0, const bf16_t* __restrict__ B1,
                                                       bf16_t* __restrict__ C, int L, int N, int K, int a_rows,
                                                        const int32_t* __restrict__ tpre, int cpx, int smax,
                                                        float* __restrict__ parts, bf16_t* __restrict__ Gs,
                                                        bf16_t* __restrict__ Us) {
  extern __shared__ __attribute__((aligned(1024))) char lds[];
  if constexpr (EP == kWgrad) {
    const int e = blockIdx.y, z = blockIdx.z, M = K;
    int64_t q = 0;
    for (int i = 0; i < e; ++i) q += wgrad_k(offsets[i + 1] - offsets[i]);
    const int Ke = wgrad_k(offsets[e + 1] - offsets[e]);
    const int tn = (N + BNE - 1) / BNE;
    Job jb;
    jb.expert = e;
    jb.row0 = (blockIdx.x / tn) * BM;
    jb.rows = min(BM, M - jb.row0);
    jb.n0 = blockIdx.x % tn;
    jb.wide = false;
    jb.kb = 0;
    jb.nks = Ke / BK;
    jb.part = 0;
    jb.nparts = 1;
    jb.pslot = 0;
    const bf16_t* Ae = A + q * a_rows + size_t(z) * M * Ke;
    const bf16_t* Be = B0 + q * N;
    bf16_t* Ce = (z ? Gs : C) + size_t(e) * M * N;
    // (EP, not kPlain, as the template argument: hipcc's host pass rejects the literal
    // here; the epilogue treats kWgrad as kPlain)
    tile_body<NMAT, false, NW, EP>(Ae, M, Be, Be, Ce, N, Ke, jb, parts, lds, Us, Us);
    return;
  }
  constexpr int ON = NMAT == 2 ? BNE / 2 : BNE;  // output columns per regular tile
  const int NT = (N + ON - 1) / ON;
  const int nk = K / BK;
  // block (xcd, loc) runs unit loc of its XCD (blocks are dealt to the XCDs round robin)
  const int xcd = blockIdx.x % kXcds, loc = blockIdx.x / kXcds;
  const XcdPlan xp = plan_xcd(tpre[L], nk, cpx, smax, xcd);
  if (loc >= xp.units) return;
  // the tile prefix into LDS for the search (the loop's stages overwrite it later)
  int32_t* spre = reinterpret_cast<int32_t*>(lds);
  for (int i = threadIdx.x; i <= L; i += NW * 64) spre[i] = tpre[i];
  __syncthreads();
  Job jb;
  unit_job(offsets, spre, L, NT, nk, cpx, xcd, xp, loc, jb);
  __syncthreads();  // every wave has its job before the first loads land in the LDS
  const size_t boff = size_t(jb.expert) * N * K;
  const bf16_t* Bg = B0 + boff;
  const bf16_t* Bu = (NMAT == 2 ? B1 : B0) + boff;
  if (jb.wide)
    tile_body<NMAT, true, NW, EP>(A, a_rows, Bg, Bu, C, N, K, jb, parts, lds, Gs, Us);
  else
    tile_body<NMAT, false, NW, EP>(A, a_rows, Bg, Bu, C, N, K, jb, parts, lds, Gs, Us);
}


// Adds the pieces of each split tile in piece order and writes the tile.
// kFixSub blocks share a tile; an item is one float4 of the accumulator
// layout of the NW-wave kernel (thread t, float4 v: i = v / (4 NB), j = v/4 % NB,
// q = v % 4), that is four adjacent output columns of one token row (for
// gate/up: the gate float4 and its up partner j + NB/2).
constexpr int kFixSub = 8;

template <int NMAT, int NW, int EP>
__global__ __launch_bounds__(NW * 64) void fixup_kernel(const int32_t* __restrict__ offsets, bf16_t* __restrict__ C,
                                                         int L, int N, int K, const int32_t* __restrict__ tpre, int cpx,
                                                         int smax, const float* __restrict__ parts,
                                                         bf16_t* __restrict__ Gs, bf16_t* __restrict__ Us) {
  constexpr int ON = NMAT == 2 ? BNE / 2 : BNE;
  constexpr int kThreads = NW * 64, NB = 16 / NW;
  constexpr int NJ = NMAT == 2 ? NB / 2 : NB;   // output column blocks per wave
  constexpr int NV = 16 * NJ;                   // output float4s per thread of the tile
  constexpr int kPer = NV / kFixSub;            // items per thread of this block
  const int NT = (N + ON - 1) / ON;
  const int sub = blockIdx.x % kFixSub, tile = blockIdx.x / kFixSub;
  const int xcd = tile % kXcds, w = tile / kXcds;  // w-th split tile of the XCD
  const XcdPlan xp = plan_xcd(tpre[L], K / BK, cpx, smax, xcd);
  if (xp.s == 1 || w >= xp.r) return;
  Job jb;
  tile_of(offsets, tpre, L, NT, xp.base + xp.F * cpx + w, jb);
  jb.nparts = xp.s;
  jb.pslot = xcd * kMaxParts + w * xp.s;
  const int n0 = jb.n0 * ON;
  const size_t pstride = kPartBytes / sizeof(f32x4_t);  // float4s per piece
  const f32x4_t* base = reinterpret_cast<const f32x4_t*>(parts) + size_t(jb.pslot) * pstride;
#pragma unroll
  for (int it = 0; it < kPer; ++it) {
    const int f = sub * kPer + it;  // float4 slot; consecutive threads read consecutive float4s
    const int t = threadIdx.x;
    const int i = f / (4 * NJ);
    const int j = (f / 4) % NJ;
    const int q = f % 4;
    const int v = (i * NB + j) * 4 + q;
    constexpr int UP = (NB / 2) * 4;  // up partner: j + NB/2
    f32x4_t s = base[size_t(v) * kThreads + t];
    f32x4_t su = NMAT == 2 ? base[size_t(v + UP) * kThreads + t] : s;
    for (int p = 1; p < jb.nparts; ++p) {
      s += base[size_t(p) * pstride + size_t(v) * kThreads + t];
      if (NMAT == 2) su += base[size_t(p) * pstride + size_t(v + UP) * kThreads + t];
    }
    const int wave = t >> 6, lane = t & 63;
    const int wm = jb.wide ? Shape<true, NW>::wm(wave) : Shape<false, NW>::wm(wave);
    const int wn = jb.wide ? Shape<true, NW>::wn(wave) : Shape<false, NW>::wn(wave);
    const int fr = lane & 31, g = lane >> 5;
    const int rt = wm * 128 + i * 32 + fr;
    const int cl = (NMAT == 2 ? wn * NB * 16 : wn * NB * 32) + j * 32 + 8 * q + 4 * g;
    if (rt < jb.rows && n0 + cl < N) {
      float o[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) o[u] = NMAT == 2 ? silu(s[u]) * su[u] : s[u];
      uint2 pk;
      pk.x = pack_bf16x2(o[0], o[1]);
      pk.y = pack_bf16x2(o[2], o[3]);
      *reinterpret_cast<uint2*>(C + size_t(jb.row0 + rt) * N + n0 + cl) = pk;
      if constexpr (NMAT == 2 && EP == kSave) {  // training: the pre-activations too
        const size_t at = size_t(jb.row0 + rt) * N + n0 + cl;
        *reinterpret_cast<uint2*>(Gs + at) = make_uint2(pack_bf16x2(s[0], s[1]), pack_bf16x2(s[2], s[3]));
        *reinterpret_cast<uint2*>(Us + at) = make_uint2(pack_bf16x2(su[0], su[1]), pack_bf16x2(su[2], su[3]));
      }
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

// K long enough to cut a partly filled last round
bool splits(int K) { return K / BK >= kSplitMinSteps; }

// Eight waves (two per SIMD) for products shorter than kEightWaveSteps k steps, where
// the per-tile fixed costs weigh most (same-box A/B: gpt-oss-like layer -4.5%,
// skewed layer -1.5%); four for longer ones (mixtral-like layer: eight are 1% slower).
constexpr int kEightWaveSteps = 64;

template <int NMAT, int NW, int EP>
moe_status launch_nws(const char* name, const bf16_t* A, const int32_t* offsets, const bf16_t* B0, const bf16_t* B1,
                      bf16_t* C, int L, int N, int K, int64_t max_pairs, const int32_t* tpre, float* parts,
                      hipStream_t s, bf16_t* Gs, bf16_t* Us);

template <int NMAT, int NW>
moe_status launch_nw(const char* name, const bf16_t* A, const int32_t* offsets, const bf16_t* B0, const bf16_t* B1,
                     bf16_t* C, int L, int N, int K, int64_t max_pairs, const int32_t* tpre, float* parts,
                     hipStream_t s, bf16_t* Gs, bf16_t* Us, int ep) {
  if constexpr (NMAT == 2) {
    if (ep == kSave) return launch_nws<NMAT, NW, kSave>(name, A, offsets, B0, B1, C, L, N, K, max_pairs, tpre, parts, s, Gs, Us);
  } else {
    if (ep == kSwigluBwd)
      return launch_nws<NMAT, NW, kSwigluBwd>(name, A, offsets, B0, B1, C, L, N, K, max_pairs, tpre, nullptr, s, Gs, Us);
  }
  return launch_nws<NMAT, NW, kPlain>(name, A, offsets, B0, B1, C, L, N, K, max_pairs, tpre, parts, s, Gs, Us);
}

// EP: the epilogue (kSave: the training forward's gate/up, which also writes the
// pre-activations; kSwigluBwd: the backward's down dgrad, never split along K)
template <int NMAT, int NW, int EP>
moe_status launch_nws(const char* name, const bf16_t* A, const int32_t* offsets, const bf16_t* B0, const bf16_t* B1,
                      bf16_t* C, int L, int N, int K, int64_t max_pairs, const int32_t* tpre, float* parts,
                      hipStream_t s, bf16_t* Gs, bf16_t* Us) {
  constexpr int kThreads = NW * 64;
  auto kern = gemm_kernel<NMAT, NW, EP>;
  constexpr size_t lds = lds_bytes<NMAT>();
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern), hipFuncAttributeMaxDynamicSharedMemorySize,
                                     int(lds));
  if (e != hipSuccess) return set_error(MOE_ERR_HIP, "%s: LDS attribute: %s", name, hipGetErrorString(e));
  const int cpx = cus_per_xcd();
  const int smax = splits(K) && parts != nullptr ? kMaxSplit : 1;
  // every XCD's range holds at most ceil(R/8) tiles (R counts regular tiles, an upper bound on the
  // mix of regular and wide ones); splitting adds at most kMaxParts - kMaxTail blocks
  constexpr int ON = NMAT == 2 ? BNE / 2 : BNE;
  const int64_t tiles = ((max_pairs + BM - 1) / BM + L) * ((N + ON - 1) / ON);
  const int64_t per_xcd = (tiles + kXcds - 1) / kXcds + (smax > 1 ? kMaxParts - kMaxTail : 0);
  // A holds max_pairs rows (the caller's x_sorted or h)
  MOE_LAUNCH(name, kern, dim3(unsigned(per_xcd * kXcds)), dim3(kThreads), lds, s, A, offsets, B0, B1, C, L, N, K,
             int(max_pairs), tpre, cpx, smax, parts, Gs, Us);
  if (smax > 1) {
    const char* fname = NMAT == 2 ? "ffn_gate_up_fixup" : "ffn_down_fixup";
    MOE_LAUNCH(fname, (fixup_kernel<NMAT, NW, EP>), dim3(unsigned(kXcds * kMaxTail * kFixSub)), dim3(kThreads), 0, s,
               offsets, C, L, N, K, tpre, cpx, smax, static_cast<const float*>(parts), Gs, Us);
  }
  return MOE_OK;
}

template <int NW>
moe_status launch_wgrad_nw(const char* name, const moe_layer_desc* d, const int32_t* offsets, const bf16_t* At,
                           int a_rows_total, const bf16_t* Bt, bf16_t* C0, bf16_t* C1, int M, int N, int Z,
                           hipStream_t s) {
  auto kern = gemm_kernel<1, NW, kWgrad>;
  constexpr size_t lds = lds_bytes<1>();
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern), hipFuncAttributeMaxDynamicSharedMemorySize,
                                     int(lds));
  if (e != hipSuccess) return set_error(MOE_ERR_HIP, "%s: LDS attribute: %s", name, hipGetErrorString(e));
  const unsigned tiles = unsigned(((M + BM - 1) / BM) * ((N + BNE - 1) / BNE));
  MOE_LAUNCH(name, kern, dim3(tiles, unsigned(d->local_count), unsigned(Z)), dim3(NW * 64), lds, s, At, offsets, Bt,
             Bt, C0, d->local_count, N, M, a_rows_total, static_cast<const int32_t*>(nullptr), 0, 1,
             static_cast<float*>(nullptr), C1, static_cast<bf16_t*>(nullptr));
  return MOE_OK;
}

template <int NMAT>
moe_status launch(const char* name, const bf16_t* A, const int32_t* offsets, const bf16_t* B0, const bf16_t* B1,
                  bf16_t* C, int L, int N, int K, int64_t max_pairs, const int32_t* tpre, float* parts,
                  hipStream_t s, bf16_t* Gs = nullptr, bf16_t* Us = nullptr, int ep = kPlain) {
  if (K / BK < kEightWaveSteps)
    return launch_nw<NMAT, 8>(name, A, offsets, B0, B1, C, L, N, K, max_pairs, tpre, parts, s, Gs, Us, ep);
  return launch_nw<NMAT, 4>(name, A, offsets, B0, B1, C, L, N, K, max_pairs, tpre, parts, s, Gs, Us, ep);
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
template <int NMAT, bool SAVE>
__global__ __launch_bounds__(kThreads) void gemm_kernel(const bf16_t* __restrict__ A, const int32_t* __restrict__ offsets,
                                                        const bf16_t* __restrict__ B0, const bf16_t* __restrict__ B1,
                                                        bf16_t* __restrict__ C, int N, int K, bf16_t* __restrict__ Gs,
                                                        bf16_t* __restrict__ Us) {
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

    // two register sets of kPipe k steps: the loads of the next set are in flight
    // while the MFMAs of the current one run (four steps per set: fewer waves
    // fit, but each keeps more in flight; same-box A/B on the decode-sized
    // layer: 0 to -4% per layer against two steps, while capping registers for
    // more waves per SIMD made it 12% slower)
    constexpr int kPipe = 4;
    bf16x8_t w0[2][kPipe], w1[2][kPipe], a0[2][kPipe];
    const int nset = K / (32 * kPipe);
    auto load_set = [&](int b, int k0) {
#pragma unroll
      for (int u = 0; u < kPipe; ++u) {
        w0[b][u] = *reinterpret_cast<const bf16x8_t*>(bs0 + k0 + 32 * u);
        w1[b][u] = *reinterpret_cast<const bf16x8_t*>(bs1 + k0 + 32 * u);
        a0[b][u] = *reinterpret_cast<const bf16x8_t*>(arow[0] + k0 + 32 * u);
      }
    };
    auto mma_set = [&](int b, int k0) {
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

template <int NMAT>
moe_status launch(const char* name, const bf16_t* A, const int32_t* offsets, const bf16_t* B0, const bf16_t* B1,
                  bf16_t* C, int L, int N, int K, hipStream_t s, bf16_t* Gs = nullptr, bf16_t* Us = nullptr) {
  const dim3 grid(unsigned((N + cols_per_block<NMAT>() - 1) / cols_per_block<NMAT>()), unsigned(L));
  if (NMAT == 2 && Gs != nullptr) {
    MOE_LAUNCH(name, (gemm_kernel<NMAT, true>), grid, dim3(kThreads), 0, s, A, offsets, B0, B1, C, N, K, Gs, Us);
  } else {
    MOE_LAUNCH(name, (gemm_kernel<NMAT, false>), grid, dim3(kThreads), 0, s, A, offsets, B0, B1, C, N, K, Gs, Us);
  }
  return MOE_OK;
}

}  // namespace skinny

template <typename T, int BMT>
moe_status launch_bm(const FfnArgs& a) {
  const moe_layer_desc* d = a.d;
  const int L = d->local_count, H = d->hidden, I = d->intermediate;
  const unsigned mslots = unsigned((a.max_pairs + BMT - 1) / BMT + L);
  MOE_LAUNCH("ffn_gate_up", (grouped_gemm_kernel<T, 2, BMT>), dim3(mslots, (I + BN - 1) / BN), dim3(kThreads), 0,
             a.s, static_cast<const T*>(a.x_sorted), a.offsets, static_cast<const T*>(a.w_gate),
             static_cast<const T*>(a.w_up), static_cast<T*>(a.h), L, I, H, static_cast<T*>(a.g_out),
             static_cast<T*>(a.u_out));
  MOE_LAUNCH("ffn_down", (grouped_gemm_kernel<T, 1, BMT>), dim3(mslots, (H + BN - 1) / BN), dim3(kThreads), 0, a.s,
             static_cast<const T*>(a.h), a.offsets, static_cast<const T*>(a.w_down), static_cast<const T*>(a.w_down),
             static_cast<T*>(a.y_sorted), L, H, I, static_cast<T*>(nullptr), static_cast<T*>(nullptr));
  return MOE_OK;
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

// large tiles pay off once segments hold a few hundred rows; decode-sized
// batches (a handful of rows per expert) take the skinny kernel
bool use_big(const moe_layer_desc* d, int64_t max_pairs) {
  return d->dtype == MOE_BF16 && max_pairs >= int64_t(128) * d->local_count && big::supported(d->hidden) &&
         big::supported(d->intermediate) && big::addressable(d->intermediate, d->hidden);
}

moe_status launch_small(const FfnArgs& a) {
  const moe_layer_desc* d = a.d;
  const int L = d->local_count, H = d->hidden, I = d->intermediate;
  // decode-sized batches: a few rows per expert, bound by streaming the weights
  if (d->dtype == MOE_BF16 && a.max_pairs <= int64_t(32) * L && skinny::supported(H) && skinny::supported(I)) {
    bf16_t* h = static_cast<bf16_t*>(a.h);
    moe_status st = skinny::launch<2>("ffn_gate_up", static_cast<const bf16_t*>(a.x_sorted), a.offsets,
                                      static_cast<const bf16_t*>(a.w_gate), static_cast<const bf16_t*>(a.w_up), h, L, I,
                                      H, a.s, static_cast<bf16_t*>(a.g_out), static_cast<bf16_t*>(a.u_out));
    if (st != MOE_OK) return st;
    return skinny::launch<1>("ffn_down", h, a.offsets, static_cast<const bf16_t*>(a.w_down),
                             static_cast<const bf16_t*>(a.w_down), static_cast<bf16_t*>(a.y_sorted), L, H, I, a.s);
  }
  return d->dtype == MOE_BF16 ? launch_t<bf16_t>(a) : launch_t<float>(a);
}

}  // namespace

size_t ffn_scratch_bytes(const moe_layer_desc* d, int64_t max_pairs) {
  if (!use_big(d, max_pairs)) return 0;
  const size_t plan = align_up(size_t(2) * (d->local_count + 1) * sizeof(int32_t), 256);
  const bool split = big::splits(d->hidden) || big::splits(d->intermediate);
  return plan + (split ? size_t(big::kXcds) * big::kMaxParts * big::kPartBytes : 0);
}

// ---- the backward's dgrad products on the large-tile kernel ---------------------
// With the expert weights transposed to [N, K] rows (wdT [L, I, H]; wguT [L, H, 2I],
// the gate's transpose then the up's), both dgrad products have the forward's
// operand layout: dh = dy_sorted wdT_e^T with the SwiGLU backward in the epilogue
// (writing dg | du as [P, 2I]), then dx_sorted = [dg | du] wguT_e^T, one product
// over K = 2I.
bool big_backward_supported(const moe_layer_desc* d, int64_t max_pairs) {
  return use_big(d, max_pairs) && big::supported(2 * d->intermediate) &&
         big::addressable(d->hidden, 2 * int64_t(d->intermediate));
}

size_t big_backward_scratch_bytes(const moe_layer_desc* d) {
  const size_t plan = align_up(size_t(2) * (d->local_count + 1) * sizeof(int32_t), 256);
  return plan + (big::splits(2 * d->intermediate) ? size_t(big::kXcds) * big::kMaxParts * big::kPartBytes : 0);
}

moe_status launch_big_backward_dgrad(const moe_layer_desc* d, const bf16_t* dy_sorted, const int32_t* offsets,
                                     const bf16_t* wdT, const bf16_t* gate, const bf16_t* up, bf16_t* dgu,
                                     const bf16_t* wguT, bf16_t* dx_sorted, int64_t max_pairs, void* scratch,
                                     hipStream_t s) {
  const int L = d->local_count, H = d->hidden, I = d->intermediate;
  int32_t* pre = static_cast<int32_t*>(scratch);
  float* parts = big::splits(2 * I) ? reinterpret_cast<float*>(static_cast<char*>(scratch) +
                                                               align_up(size_t(2) * (L + 1) * sizeof(int32_t), 256))
                                    : nullptr;
  MOE_LAUNCH("ffn_bwd_plan", big::plan_kernel, dim3(1), dim3(1024), 0, s, offsets, L, (I + big::BNE - 1) / big::BNE,
             (H + big::BNE - 1) / big::BNE, pre);
  moe_status st = big::launch<1>("ffn_down_dgrad", dy_sorted, offsets, wdT, wdT, dgu, L, I, H, max_pairs, pre, nullptr,
                                 s, const_cast<bf16_t*>(gate), const_cast<bf16_t*>(up), big::kSwigluBwd);
  if (st != MOE_OK) return st;
  return big::launch<1>("ffn_gate_up_dgrad", dgu, offsets, wguT, wguT, dx_sorted, L, H, 2 * I, max_pairs, pre + L + 1,
                        parts, s);
}

bool big_wgrad_supported(const moe_layer_desc* d, int64_t max_pairs) {
  const int64_t kmax = (max_pairs + 63) / 64 * 64 + 64;
  return big_backward_supported(d, max_pairs) && big::addressable(std::max(d->hidden, 2 * d->intermediate), kmax);
}

moe_status launch_big_backward_wgrad(const char* name, const moe_layer_desc* d, const int32_t* offsets,
                                     const bf16_t* At, int a_rows_total, const bf16_t* Bt, bf16_t* C0, bf16_t* C1,
                                     int M, int N, int Z, int64_t max_pairs, hipStream_t s) {
  // eight waves when the average segment is under 64 k steps, as for the forward
  const int64_t avg = max_pairs / std::max(1, d->local_count);
  if (avg / big::BK < big::kEightWaveSteps)
    return big::launch_wgrad_nw<8>(name, d, offsets, At, a_rows_total, Bt, C0, C1, M, N, Z, s);
  return big::launch_wgrad_nw<4>(name, d, offsets, At, a_rows_total, Bt, C0, C1, M, N, Z, s);
}

moe_status launch_grouped_ffn(const FfnArgs& a) {
  if (a.max_pairs <= 0) return MOE_OK;
  const moe_layer_desc* d = a.d;
  if (!use_big(d, a.max_pairs)) return launch_small(a);
  const int L = d->local_count, H = d->hidden, I = d->intermediate;
  const bf16_t* x = static_cast<const bf16_t*>(a.x_sorted);
  bf16_t* h = static_cast<bf16_t*>(a.h);
  // scratch: the tile plan, then (long K) the split pieces
  int32_t* pre = static_cast<int32_t*>(a.scratch);
  float* parts = big::splits(H) || big::splits(I)
                     ? reinterpret_cast<float*>(static_cast<char*>(a.scratch) +
                                                align_up(size_t(2) * (L + 1) * sizeof(int32_t), 256))
                     : nullptr;
  MOE_LAUNCH("ffn_plan", big::plan_kernel, dim3(1), dim3(1024), 0, a.s, a.offsets, L, (I + big::BNE / 2 - 1) / (big::BNE / 2),
             (H + big::BNE - 1) / big::BNE, pre);
  moe_status st = big::launch<2>("ffn_gate_up", x, a.offsets, static_cast<const bf16_t*>(a.w_gate),
                                 static_cast<const bf16_t*>(a.w_up), h, L, I, H, a.max_pairs, pre, parts, a.s,
                                 static_cast<bf16_t*>(a.g_out), static_cast<bf16_t*>(a.u_out),
                                 a.g_out != nullptr ? big::kSave : big::kPlain);
  if (st != MOE_OK) return st;
  return big::launch<1>("ffn_down", h, a.offsets, static_cast<const bf16_t*>(a.w_down),
                        static_cast<const bf16_t*>(a.w_down), static_cast<bf16_t*>(a.y_sorted), L, H, I, a.max_pairs,
                        pre + L + 1, parts, a.s);
}

}  // namespace moe
