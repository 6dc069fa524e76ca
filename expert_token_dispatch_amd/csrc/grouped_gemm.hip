// Stage 3: the local experts as one grouped GEMM over ragged segments.
//
// Ultralytics glossary "Expert Parallelism", section "How tokens move between
// GPUs", step 3: each GPU runs its local experts on the tokens it received.
// The Transformers page names the expert kernel style "grouped_gemm" and says
// the expert weights are split along the expert dimension: they are stacked
// per local expert.  Expert i owns sorted rows [offsets[i], offsets[i+1]) and
// computes the SwiGLU feed-forward (math form)
//   h = silu(X Wg_i) * (X Wu_i)      (gate/up product, SwiGLU in its epilogue)
//   y = h Wd_i                       (down product)
// with float32 accumulation; h is rounded to the storage type once.
//
// Three kernels, picked from the largest segment the caller allows (P_max) and
// the dtype: the large-tile bf16 kernel below for segments of hundreds of rows,
// the skinny kernel (skinny_gemm.hip) for decode-sized batches, and the general
// kernel (general_gemm.hip) for float32 and shapes off the large tile's grid.
#include <math.h>

#include <algorithm>
#include <cstring>

#include "ffn_common.h"
#include "kernels.h"

namespace moe {
namespace {

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
// K advances 64 at a time through LDS filled by direct global->LDS loads
// (buffer_load_dwordx4 ... lds: lane i of a load writes bytes [16i, 16i+16) of
// a 1 KB block, no staging registers): the 256 activation rows of a step in
// two 32 KB slots, the 256 weight rows in three, so the weight rows (which
// miss L2 far more often) are asked for two steps ahead (a wide tile keeps two
// whole stages).  Rows are 128 bytes; 16-byte chunk c of row r sits at physical
// chunk c ^ ((r/2) % 8), so the fragment reads of 16 lanes (16 rows, one
// chunk) cover all 64 banks.
//
// Schedule of one step (per wave): for each 16-k chunk, the fragments of the
// next chunk are read while this chunk's 16 MFMAs issue, one read between
// every two MFMAs (pinned with sched_group_barrier); reads bunched at the
// start of the group left the LDS and the matrix core taking turns.  Before
// the last chunk the wave waits for its own loads of the next step and for its
// own reads of this one, then a block barrier makes both true for every wave:
// the next step's first fragments are read and the freed slots are refilled
// while the last 16 MFMAs run.  The barrier is a bare s_barrier:
// __syncthreads() would also drain every load in flight.
//
// The MFMAs take the weight fragment as the left operand, so each lane ends
// with four adjacent output columns of one token row; the epilogue parks the
// bf16 tile in LDS and writes it out in whole row pieces.
//
// Tile order: the blocks that run at once on one XCD (blocks are dealt to
// the 8 XCDs round robin) get consecutive tile numbers, and tile numbers run
// over (expert, group of gn n-tiles, m-tile, n-tile in group), so one XCD's L2
// serves a few weight tiles to all m-tiles of an expert and a few activation
// tiles to several n-tiles.
namespace big {

constexpr int BM = 256, BNE = 256, BK = 64, kStages = 2;

constexpr int kRowBytes = BK * 2;              // 128
constexpr int kXcds = 8;

// n-tiles per group of the tile order (gn): 2 for products of fewer than 8192 k, 4 for
// longer ones (same-box interleaved runs: with 2 instead of 4, mixtral_like's gate/up
// (K = 4096) -2.2% and the gpt-oss-like share's products (K = 2880) -1.4 to -2.4%, but
// mixtral_like's down (K = 14336) +1.7 to +2.7%; groups of 1 or 8 were slower).
__host__ __device__ constexpr int group_width(int K) { return K >= 8192 ? 4 : 2; }

// s_waitcnt on the vector-memory counter only (expcnt and lgkmcnt left at their maxima)
#define MOE_VMCNT(n) __builtin_amdgcn_s_waitcnt(((n) & 0xF) | (((n) >> 4) << 14) | (0x7 << 4) | (0xF << 8))
#define MOE_LGKMCNT0() __builtin_amdgcn_s_waitcnt(0xC07F)

bool supported(int K) { return K % BK == 0; }
// the direct loads address a weight matrix with 32-bit byte offsets
bool addressable(int64_t rows, int64_t K) { return rows * K * 2 < (int64_t(1) << 32); }

// ---- work plan -------------------------------------------------------------
// Tiles are numbered over (expert, group of gn n-tiles, m-tile, n-tile
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

// Tiles of one expert with n rows: in every group of up to gn n-tiles, the
// full 256-row m-tiles, then the tail m-tile: a regular tile per n-tile when
// the tail has more than 128 rows, else one wide tile per two n-tiles.
__device__ __forceinline__ int tail_tiles(int tail, int gsz) {
  return tail == 0 ? 0 : (tail <= BM / 2 ? (gsz + 1) / 2 : gsz);
}
__device__ __forceinline__ int expert_tiles(int n, int NT, int gn) {
  const int mf = n / BM, tail = n - mf * BM;
  const int nfull = NT / gn, last = NT - nfull * gn;
  return nfull * (mf * gn + tail_tiles(tail, gn)) + (last ? mf * last + tail_tiles(tail, last) : 0);
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
// K_gu, K_dn: each product's K (its group width follows from it).
__global__ __launch_bounds__(1024) void plan_kernel(const int32_t* __restrict__ offsets, int L, int NT_gu, int NT_dn,
                                                    int K_gu, int K_dn, int32_t* __restrict__ pre) {
  __shared__ int wa[16], wb[16];  // per-wave totals
  int carry_gu = 0, carry_dn = 0;
  for (int i0 = 0; i0 < L; i0 += 1024) {
    const int i = i0 + threadIdx.x;
    const int n = i < L ? offsets[i + 1] - offsets[i] : 0;
    const int a = i < L ? expert_tiles(n, NT_gu, group_width(K_gu)) : 0;
    const int b = i < L ? expert_tiles(n, NT_dn, group_width(K_dn)) : 0;
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

// expert, rows and columns of tile t; tpre = the product's tile prefix (L + 1 entries),
// gn its group width
__device__ __forceinline__ void tile_of(const int32_t* __restrict__ offsets, const int32_t* tpre, int L, int NT, int gn,
                                        int t, Job& jb) {
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
  const int nfull = NT / gn;
  const int per_group = mf * gn + tail_tiles(tl, gn);
  int ng = t / per_group;
  if (ng > nfull) ng = nfull;  // past the full groups: the last, partial group
  const int rem = t - ng * per_group;
  const int gsz = ng < nfull ? gn : NT - nfull * gn;
  if (rem < mf * gsz) {
    const int mt = rem / gsz;
    jb.n0 = ng * gn + (rem - mt * gsz);
    jb.row0 = seg0 + mt * BM;
    jb.rows = BM;
    jb.wide = false;
  } else {
    const int r2 = rem - mf * gsz;
    jb.row0 = seg0 + mf * BM;
    jb.rows = tl;
    jb.wide = tl <= BM / 2;
    jb.n0 = ng * gn + (jb.wide ? 2 * r2 : r2);
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
  tile_of(offsets, tpre, L, NT, group_width(nk * BK), t, jb);
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
  static constexpr int kStageB = kB * kRowBytes;
  static constexpr int kStage = (kA + kB) * kRowBytes;   // 64 KB regular, 80 KB wide
  static constexpr int kLdA = kA / (8 * NW), kLdB = kB / (8 * NW);  // 1 KB direct loads per wave per stage
  static constexpr int kLd = kLdA + kLdB;
  __device__ static int wm(int wave) { return WIDE ? 0 : wave / (NW / 2); }
  __device__ static int wn(int wave) { return WIDE ? wave : wave % (NW / 2); }
};
constexpr size_t kLoopLdsMax = size_t(kStages) * Shape<true, 4>::kStage;  // 160 KB
// a regular tile's two A slots and three B slots fit in the same space
static_assert(2 * Shape<false, 4>::kStageA + 3 * Shape<false, 4>::kStageB <= int(kLoopLdsMax), "regular ring");

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
// the weight-gradient products (wgrad_kernel); the epilogue treats them as kPlain
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

// The operands of one tile.  Each is stored one of two ways, with rows of ld elements:
//   A, AKM false: m-major, element (m, k) at A[m * lda + k]; the buffer holds a_rows rows
//      of m (rows past them read zero);
//   A, AKM true:  k-major, element (k, m) at A[k * lda + m]; a_rows rows of k;
//   B, BKN false: n-major, element (n, k) at B[n * ldb + k] (a linear layer's [out, in]);
//   B, BKN true:  k-major, element (k, n) at B[k * ldb + n] (the math form's [in, out]);
//      b_rows rows (of n or k) either way.
// Bg, and Bu for the up rows of gate/up; with kcat > 0 (one-matrix products only) the
// k steps from kcat on read Bu at step - kcat (a product over two matrices side by side
// along K, such as dg Wg + du Wu).
struct Operands {
  const bf16_t* A;
  int a_rows, lda;
  const bf16_t* Bg;
  const bf16_t* Bu;
  int b_rows, ldb;
};

// One tile (or one K piece of it): the main loop, then the epilogue or the piece write-out.
template <int NMAT, bool WIDE, int NW, int EP, bool BKN, bool AKM>
__device__ __forceinline__ void tile_body(const Operands& op, bf16_t* __restrict__ C, int N, int K, int kcat,
                                          const Job& jb, float* __restrict__ parts, char* lds,
                                          bf16_t* __restrict__ Gs, bf16_t* __restrict__ Us) {
  const bf16_t* __restrict__ A = op.A;
  const bf16_t* __restrict__ Bg = op.Bg;
  const bf16_t* __restrict__ Bu = op.Bu;
  const int a_rows = op.a_rows, lda = op.lda, ldb = op.ldb;
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
  // buffer resources over A (from the tile's first row when m-major) and over the whole
  // weight matrix (its extent is under 4 GiB); a read outside either returns zeros
  const int64_t a_span = AKM ? int64_t(a_rows) * lda : int64_t(a_rows - row0) * lda;
  const uint32_t a_bytes = uint32_t(min(a_span * 2, int64_t(0xFFFFFFFF)));
  const __amdgpu_buffer_rsrc_t a_rsrc = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<bf16_t*>(AKM ? A : A + size_t(row0) * lda), 0, a_bytes, kRsrcFlags);
  // the first half of the waves loads gate rows (or the only matrix), the second half up rows;
  // b_rsrc2 is the second matrix of a product split along K
  const uint32_t b_bytes = uint32_t(min(int64_t(op.b_rows) * ldb * 2, int64_t(0xFFFFFFFF)));
  const __amdgpu_buffer_rsrc_t b_rsrc = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<bf16_t*>(NMAT == 2 && wave >= NW / 2 ? Bu : Bg), 0, b_bytes, kRsrcFlags);
  const __amdgpu_buffer_rsrc_t b_rsrc2 = __builtin_amdgcn_make_buffer_rsrc(const_cast<bf16_t*>(Bu), 0, b_bytes,
                                                                           kRsrcFlags);
  // Rows past the segment (A) or past N (B) feed only outputs that are never
  // stored, so they may read any valid row: A takes the rows that follow (up
  // to the last row of the buffer), B wraps around to the first rows.  Letting
  // them all repeat one row would send every lane of the padding to the same
  // 128 bytes, one L2 channel, on every step.
  // Each lane's byte offsets are fixed for the whole loop (A from the tile's
  // first row, B from the matrix); a step only moves the scalar offset by k0,
  // so a load costs no vector arithmetic.
  uint32_t a_vo[S::kLdA], b_vo[S::kLdB];
  if constexpr (!AKM) {
    const int a_lim = a_rows - 1 - row0;
#pragma unroll
    for (int j = 0; j < S::kLdA; ++j) {
      const int cc = (j & 1) ? c_odd : c_even;
      a_vo[j] = (uint32_t(min(a_lrow + 8 * j, a_lim)) * uint32_t(lda) + uint32_t(cc * 8)) * 2u;
    }
  } else {
    // k-major stage, laid out as the k-major B stage below: regions of 128 m columns,
    // 64 k rows of 256 bytes each, 64-byte units swizzled by row
#pragma unroll
    for (int j = 0; j < S::kLdA; ++j) {
      const int gb = S::kLdA * wave + j;
      const int krow = 4 * (gb & 15) + (lane >> 4);
      const int u = ((lane & 15) >> 2) ^ ((lane >> 4) & 3);
      // columns past the tile's rows read what follows (or zeros past the buffer): never stored
      a_vo[j] = (uint32_t(krow) * uint32_t(lda) + uint32_t(row0 + 128 * (gb >> 4) + 32 * u + 8 * (lane & 3))) * 2u;
    }
  }
  if constexpr (!BKN) {
    int b_lrow;
    if (NMAT == 2) b_lrow = ((S::kB / NW) * wave + (lane >> 3)) & (S::kB / 2 - 1);
    else b_lrow = (S::kB / NW) * wave + (lane >> 3);
#pragma unroll
    for (int j = 0; j < S::kLdB; ++j) {
      const int cc = (j & 1) ? c_odd : c_even;
      int r = n0 + b_lrow + 8 * j;
      if (r >= N) r %= N;
      b_vo[j] = (uint32_t(r) * uint32_t(ldb) + uint32_t(cc * 8)) * 2u;
    }
  } else {
    // k-major stage: the tile's B rows in regions of 128 columns (gate regions, then
    // up regions), each 64 k rows of 256 bytes; 64-byte unit u (32 columns) of k row
    // r sits at physical unit u ^ (r % 4), so the four rows a transposing read
    // touches per half wave fall in four different bank groups.  Block j of the wave
    // (1 KB: four k rows of one region) is global block kLdB*wave + j; its lane l
    // writes k row 4*(block % 16) + l/16, physical 16-byte chunk l % 16.
#pragma unroll
    for (int j = 0; j < S::kLdB; ++j) {
      const int gb = S::kLdB * wave + j;
      const int reg = gb >> 4, krow = 4 * (gb & 15) + (lane >> 4);
      const int u = ((lane & 15) >> 2) ^ ((lane >> 4) & 3);
      const int col = n0 + 128 * (NMAT == 2 ? reg % (S::kB / 256) : reg) + 32 * u + 8 * (lane & 3);
      // columns past N read what follows in memory (or zeros past the matrix): never stored
      b_vo[j] = (uint32_t(krow) * uint32_t(ldb) + uint32_t(col)) * 2u;
    }
  }
  // LDS stages.  A wide tile keeps two whole stages (A and B rows of a step together).
  // A regular tile keeps its A rows in two slots and its B rows in three (2 x 32 + 3 x
  // 32 KB): the weight rows, which miss L2 far more often than the activation rows,
  // are asked for two steps before they are used instead of one.  a_slot(s) is where
  // stage s's A rows start; b_slot(s) + kStageA is where its B rows start (the B
  // fragment offsets count from a whole stage's base).
  constexpr bool kRing3 = !WIDE;
  const auto a_slot = [&](int st) -> char* {
    return kRing3 ? lds + (st & 1) * S::kStageA : lds + (st % kStages) * S::kStage;
  };
  const auto b_slot = [&](int st) -> char* {
    return kRing3 ? lds + S::kStageA + (st % 3) * S::kStageB : lds + (st % kStages) * S::kStage;
  };
// loads q0..q1-1 of stage kt_, in the order A0 B0 A1 B1 ... (then the B rows
// past the last A block)
#define MOE_ISSUE(kt_, q0_, q1_)                                                                            \
  do {                                                                                                      \
    char* sa_ = a_slot(kt_) + (S::kLdA * wave) * 1024;                                                      \
    char* sb_ = b_slot(kt_) + S::kStageA + (S::kLdB * wave) * 1024;                                         \
    const int s_ = kb + (kt_);                                                                              \
    const uint32_t k0_ = uint32_t(s_) * (AKM ? uint32_t(BK * 2) * uint32_t(lda) : uint32_t(BK * 2));          \
    const bool sec_ = kcat > 0 && s_ >= kcat;                                                               \
    const uint32_t kbo_ = uint32_t(sec_ ? s_ - kcat : s_) * (BKN ? uint32_t(BK * 2) * uint32_t(ldb) : uint32_t(BK * 2)); \
    _Pragma("unroll") for (int q = (q0_); q < (q1_); ++q) {                                                 \
      const int j_ = q < 2 * S::kLdA ? q / 2 : q - S::kLdA;                                                 \
      if (q < 2 * S::kLdA && q % 2 == 0)                                                                    \
        __builtin_amdgcn_raw_ptr_buffer_load_lds(a_rsrc, (lds_ptr_t)(sa_ + j_ * 1024), 16, a_vo[j_], k0_, 0, 0); \
      else                                                                                                  \
        __builtin_amdgcn_raw_ptr_buffer_load_lds(sec_ ? b_rsrc2 : b_rsrc, (lds_ptr_t)(sb_ + j_ * 1024), 16, b_vo[j_], \
                                                 kbo_, 0, 0);                                              \
    }                                                                                                       \
  } while (0)

#define MOE_ISSUE_A1(kt_, j_)                                                                               \
  do {                                                                                                      \
    char* sa_ = a_slot(kt_) + (S::kLdA * wave) * 1024;                                                      \
    const uint32_t k0_ = uint32_t(kb + (kt_)) * (AKM ? uint32_t(BK * 2) * uint32_t(lda) : uint32_t(BK * 2)); \
    __builtin_amdgcn_raw_ptr_buffer_load_lds(a_rsrc, (lds_ptr_t)(sa_ + (j_) * 1024), 16, a_vo[j_], k0_, 0, 0);   \
  } while (0)
#define MOE_ISSUE_B1(kt_, j_)                                                                               \
  do {                                                                                                      \
    char* sb_ = b_slot(kt_) + S::kStageA + (S::kLdB * wave) * 1024;                                         \
    const int s_ = kb + (kt_);                                                                              \
    const bool sec_ = kcat > 0 && s_ >= kcat;                                                               \
    const uint32_t kbo_ = uint32_t(sec_ ? s_ - kcat : s_) * (BKN ? uint32_t(BK * 2) * uint32_t(ldb) : uint32_t(BK * 2)); \
    __builtin_amdgcn_raw_ptr_buffer_load_lds(sec_ ? b_rsrc2 : b_rsrc, (lds_ptr_t)(sb_ + (j_) * 1024), 16, b_vo[j_], \
                                             kbo_, 0, 0);                                                   \
  } while (0)
// all A loads (MOE_ISSUE_A) or all B loads (MOE_ISSUE_B) of stage kt_
#define MOE_ISSUE_A(kt_)                                                                                    \
  do {                                                                                                      \
    char* sa_ = a_slot(kt_) + (S::kLdA * wave) * 1024;                                                      \
    const uint32_t k0_ = uint32_t(kb + (kt_)) * (AKM ? uint32_t(BK * 2) * uint32_t(lda) : uint32_t(BK * 2)); \
    _Pragma("unroll") for (int j_ = 0; j_ < S::kLdA; ++j_)                                                  \
      __builtin_amdgcn_raw_ptr_buffer_load_lds(a_rsrc, (lds_ptr_t)(sa_ + j_ * 1024), 16, a_vo[j_], k0_, 0, 0);  \
  } while (0)
#define MOE_ISSUE_B(kt_)                                                                                    \
  do {                                                                                                      \
    char* sb_ = b_slot(kt_) + S::kStageA + (S::kLdB * wave) * 1024;                                         \
    const int s_ = kb + (kt_);                                                                              \
    const bool sec_ = kcat > 0 && s_ >= kcat;                                                               \
    const uint32_t kbo_ = uint32_t(sec_ ? s_ - kcat : s_) * (BKN ? uint32_t(BK * 2) * uint32_t(ldb) : uint32_t(BK * 2)); \
    _Pragma("unroll") for (int j_ = 0; j_ < S::kLdB; ++j_)                                                  \
      __builtin_amdgcn_raw_ptr_buffer_load_lds(sec_ ? b_rsrc2 : b_rsrc, (lds_ptr_t)(sb_ + j_ * 1024), 16, b_vo[j_], \
                                               kbo_, 0, 0);                                                 \
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
    if constexpr (!BKN) {
      boffs[j] = S::kStageA + (br + fr) * kRowBytes;
    } else {
      // 32-column block br: region br / 128, unit (br % 128) / 32; lane group G = lane / 16
      // reads k rows 8 (G / 2) + i / 4 (i = lane % 16) and columns 16 (G % 2) + 4 (i % 4)
      const int G = lane >> 4, i = lane & 15, u = (br & 127) >> 5;
      boffs[j] = S::kStageA + (br >> 7) * 16384 + (8 * (G >> 1) + (i >> 2)) * 256 + 64 * (u ^ (i >> 2)) +
                 32 * (G & 1) + 8 * (i & 3);
    }
  }
  // A rows wm*128 + i*32: m-major, one row per lane; k-major, region wm, unit i
  int aoffs[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    if constexpr (!AKM) {
      aoffs[i] = (wm * 128 + i * 32 + fr) * kRowBytes;
    } else {
      const int G = lane >> 4, il = lane & 15;
      aoffs[i] = wm * 16384 + (8 * (G >> 1) + (il >> 2)) * 256 + 64 * (i ^ (il >> 2)) + 32 * (G & 1) + 8 * (il & 3);
    }
  }
  bf16x8_t fa[2][4], fb[2][NB];
#define MOE_LOADF(buf_, sta_, stb_, kc_)                                                                  \
  do {                                                                                                    \
    const int co_ = ((2 * (kc_) + g) ^ sw) * 16;                                                          \
    _Pragma("unroll") for (int i = 0; i < 4; ++i)                                                         \
      fa[buf_][i] = AKM ? read_kn_frag((sta_) + aoffs[i] + (kc_) * 16 * 256)                               \
                        : *reinterpret_cast<const bf16x8_t*>((sta_) + aoffs[i] + co_);                     \
    _Pragma("unroll") for (int j = 0; j < NB; ++j)                                                        \
      fb[buf_][j] = BKN ? read_kn_frag((stb_) + boffs[j] + (kc_) * 16 * 256)                               \
                        : *reinterpret_cast<const bf16x8_t*>((stb_) + boffs[j] + co_);                     \
  } while (0)
#define MOE_MMA(buf_)                                                                                     \
  do {                                                                                                    \
    _Pragma("unroll") for (int i = 0; i < 4; ++i)                                                         \
      _Pragma("unroll") for (int j = 0; j < NB; ++j)                                                      \
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fb[buf_][j], fa[buf_][i], acc[i][j], 0, 0, 0); \
  } while (0)
#define MOE_LOADF_Q(buf_, sta_, stb_, kc_, q_)                                                            \
  do {                                                                                                    \
    const int co_ = ((2 * (kc_) + g) ^ sw) * 16;                                                          \
    fa[buf_][q_] = AKM ? read_kn_frag((sta_) + aoffs[q_] + (kc_) * 16 * 256)                                \
                       : *reinterpret_cast<const bf16x8_t*>((sta_) + aoffs[q_] + co_);                      \
    if ((q_) < NB)                                                                                        \
      fb[buf_][(q_) % NB] = BKN ? read_kn_frag((stb_) + boffs[(q_) % NB] + (kc_) * 16 * 256)                \
                                : *reinterpret_cast<const bf16x8_t*>((stb_) + boffs[(q_) % NB] + co_);      \
  } while (0)
#define MOE_MMA_Q(buf_, q_)                                                                               \
  do {                                                                                                    \
    _Pragma("unroll") for (int j = 0; j < NB; ++j)                                                        \
      acc[q_][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fb[buf_][j], fa[buf_][q_], acc[q_][j], 0, 0, 0); \
  } while (0)
// the order inside a quarter of a four-wave tile: its MFMAs with the fragment reads and the load
// between them (mixtral_like gate/up -1.6 to -2.4%; the same for the eight-wave tile was 2-4%
// slower, so it keeps the compiler's order inside each quarter)
#define MOE_QUARTER_ORDER()                                                                               \
  do {                                                                                                    \
    if constexpr (NB == 4 && !AKM && !BKN) {                                                              \
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);                                                  \
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);                                                  \
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);                                                  \
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);                                                  \
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);                                                  \
      __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);                                                  \
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);                                                  \
    }                                                                                                     \
  } while (0)
  // LDS reads per chunk (a k-major B fragment takes two transposing reads) and MFMAs per chunk
  constexpr int kDs = 4 * (AKM ? 2 : 1) + NB * (BKN ? 2 : 1), kMf = 4 * NB;
  // {MFMA, LDS read, MFMA} (or {MFMA, LDS read} when the reads outnumber half the
  // MFMAs): the next chunk's fragment reads spread over the whole group
#define MOE_PIPE_DS()                                                                                     \
  do {                                                                                                    \
    if constexpr (kMf >= 2 * kDs) {                                                                       \
      _Pragma("unroll") for (int p_ = 0; p_ < kDs; ++p_) {                                                \
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);                                                \
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);                                                \
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);                                                \
      }                                                                                                   \
      if constexpr (kMf > 2 * kDs) __builtin_amdgcn_sched_group_barrier(0x008, kMf - 2 * kDs, 0);         \
    } else {                                                                                              \
      _Pragma("unroll") for (int p_ = 0; p_ < kDs; ++p_) {                                                \
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);                                                \
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);                                                \
      }                                                                                                   \
      if constexpr (kMf > kDs) __builtin_amdgcn_sched_group_barrier(0x008, kMf - kDs, 0);                 \
    }                                                                                                     \
  } while (0)

  // The refill of a stage goes out in two halves: the first right after the
  // barrier that frees its slot (beside the last chunk of the stage before),
  // the second beside the first chunk of the stage in between.  Against one
  // burst of all kLd loads per step this halves the rate at which the 32 CUs
  // of an XCD hit L2 together, and the second half still has three chunks to
  // land before the barrier that waits for it.
  constexpr int kHalf = S::kLd / 2;
  static_assert(!kRing3 || (S::kLdA == kHalf && S::kLdB == kHalf), "a regular tile's A and B loads are the halves");
  // a chunk that also issues half a refill: its fragment reads first, then the loads
  // spread over its 4 * NB MFMAs
#define MOE_CHUNK_LOADS()                                                                                 \
  do {                                                                                                    \
    __builtin_amdgcn_sched_group_barrier(0x100, kDs, 0);                                                  \
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
  // Load order (the vector-memory counter retires loads in issue order).  Wide tile:
  // stage 0, the first half of stage 1; each iteration kt then issues the second half of
  // stage kt+1 at its top and the first half of stage kt+2 after its barrier, and the
  // barrier waits for everything (stage kt+1).  Regular tile: A0 B0 B1 and the first
  // half of A1; iteration kt issues the second half of A(kt+1) in its chunk 0, B(kt+2)
  // in chunks 1 and 2, and the first half of A(kt+2) in chunk 3 (after its barrier), so
  // at the barrier only B(kt+2) may still be in flight.  One load per quarter chunk
  // keeps the texture addresser's queue from filling (with a chunk's loads issued
  // together it was full several times as often as the vendor library's; spreading
  // them: mixtral_like down −2 to −3%, gate/up −0.3%).  Near the end a stage past the
  // last repeats the last one (same bytes into the same slot).
  if constexpr (kRing3) {
    // within a chunk, per quarter: one row of MFMAs, the next chunk's fragments of that
    // quarter, at most one load; the fences pin the order
    constexpr int hA = S::kLdA / 2, hB = S::kLdB / 2;
    static_assert(hA <= 4 && hB <= 4 && 4 % hA == 0 && 4 % hB == 0, "loads per quarter");
    MOE_ISSUE_A(0);
    MOE_ISSUE_B(0);
    MOE_ISSUE_B(min(1, nks - 1));
    _Pragma("unroll") for (int j = 0; j < hA; ++j) MOE_ISSUE_A1(min(1, nks - 1), j);
    MOE_VMCNT(S::kLdB + hA);  // stage 0 landed
    block_barrier();
    MOE_LOADF(0, a_slot(0), b_slot(0), 0);
    for (int kt = 0; kt + 1 < nks; ++kt) {
      const char* sta = a_slot(kt);
      const char* stb = b_slot(kt);
      const int sa1 = min(kt + 1, nks - 1), s2 = min(kt + 2, nks - 1);
      __builtin_amdgcn_sched_barrier(0);
      // chunk 0 (fragments of chunk 1 into buffer 1)
      _Pragma("unroll") for (int q = 0; q < 4; ++q) {
        MOE_MMA_Q(0, q);
        MOE_LOADF_Q(1, sta, stb, 1, q);
        if (q % (4 / hA) == 4 / hA - 1) MOE_ISSUE_A1(sa1, hA + q / (4 / hA));
        MOE_QUARTER_ORDER();
        __builtin_amdgcn_sched_barrier(0);
      }
      // chunk 1
      _Pragma("unroll") for (int q = 0; q < 4; ++q) {
        MOE_MMA_Q(1, q);
        MOE_LOADF_Q(0, sta, stb, 2, q);
        if (q % (4 / hB) == 4 / hB - 1) MOE_ISSUE_B1(s2, q / (4 / hB));
        MOE_QUARTER_ORDER();
        __builtin_amdgcn_sched_barrier(0);
      }
      // chunk 2
      _Pragma("unroll") for (int q = 0; q < 4; ++q) {
        MOE_MMA_Q(0, q);
        MOE_LOADF_Q(1, sta, stb, 3, q);
        if (q % (4 / hB) == 4 / hB - 1) MOE_ISSUE_B1(s2, hB + q / (4 / hB));
        MOE_QUARTER_ORDER();
        __builtin_amdgcn_sched_barrier(0);
      }
      MOE_VMCNT(S::kLdB);  // all but B(kt+2)
      MOE_LGKMCNT0();
      block_barrier();
      __builtin_amdgcn_sched_barrier(0);
      // chunk 3 (fragments of the next stage's chunk 0 into buffer 0)
      {
        const char* nta = a_slot(kt + 1);
        const char* ntb = b_slot(kt + 1);
        _Pragma("unroll") for (int q = 0; q < 4; ++q) {
          MOE_MMA_Q(1, q);
          MOE_LOADF_Q(0, nta, ntb, 0, q);
          if (q % (4 / hA) == 4 / hA - 1) MOE_ISSUE_A1(s2, q / (4 / hA));
          MOE_QUARTER_ORDER();
          __builtin_amdgcn_sched_barrier(0);
        }
      }
    }
  } else {
    MOE_ISSUE(0, 0, S::kLd);
    if (nks > 1) {
      MOE_ISSUE(1, 0, kHalf);
      MOE_VMCNT(kHalf);  // stage 0 landed
    } else {
      MOE_VMCNT(0);
    }
    block_barrier();
    MOE_LOADF(0, a_slot(0), b_slot(0), 0);
    for (int kt = 0; kt + 1 < nks; ++kt) {
      const char* sta = a_slot(kt);
      const char* stb = b_slot(kt);
      MOE_LOADF(1, sta, stb, 1);
      MOE_ISSUE(min(kt + 1, nks - 1), kHalf, S::kLd);
      MOE_MMA(0);
      MOE_CHUNK_LOADS();
      __builtin_amdgcn_sched_barrier(0);
      MOE_LOADF(0, sta, stb, 2);
      MOE_MMA(1);
      MOE_LOADF(1, sta, stb, 3);
      MOE_MMA(0);
      MOE_PIPE_DS();
      MOE_PIPE_DS();
      __builtin_amdgcn_sched_barrier(0);
      MOE_VMCNT(0);
      MOE_LGKMCNT0();
      block_barrier();
      __builtin_amdgcn_sched_barrier(0);
      MOE_LOADF(0, a_slot(kt + 1), b_slot(kt + 1), 0);
      MOE_ISSUE(min(kt + 2, nks - 1), 0, kHalf);
      MOE_MMA(1);
      MOE_CHUNK_LOADS();
    }
  }
  {
    const char* sta = a_slot(nks - 1);
    const char* stb = b_slot(nks - 1);
    MOE_LOADF(1, sta, stb, 1);
    MOE_MMA(0);
    MOE_LOADF(0, sta, stb, 2);
    MOE_MMA(1);
    MOE_LOADF(1, sta, stb, 3);
    MOE_MMA(0);
    MOE_MMA(1);
  }
  MOE_VMCNT(0);  // the last refill repeated a stage; let it land before the block ends
#undef MOE_ISSUE
#undef MOE_ISSUE_A
#undef MOE_ISSUE_A1
#undef MOE_ISSUE_B1
#undef MOE_LOADF_Q
#undef MOE_MMA_Q
#undef MOE_QUARTER_ORDER
#undef MOE_ISSUE_B
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
// Expert e's dW = A_e^T B_e reduces over its rows [o_e, o_e + n_e): both operands are
// read in place, k-major (row p of x_sorted, h, dy_sorted or dg | du is k = p), with the
// buffer resources ending at the segment's end so the last, partial k step reads
// zeros past it.  Grid: x = output tile (m major), y = expert, z = which of up to two
// outputs (C0, C1), the z-th reading A and B at column offsets z * a_zoff, z * b_zoff.
struct WgradOps {
  const bf16_t* A;
  int lda, a_zoff;
  const bf16_t* B;
  int ldb, b_zoff;
  bf16_t* C0;
  bf16_t* C1;
  int M, N;
};

template <int NW>
__global__ __launch_bounds__(NW * 64) void wgrad_kernel(WgradOps w, const int32_t* __restrict__ offsets) {
  extern __shared__ __attribute__((aligned(1024))) char lds[];
  const int e = blockIdx.y, z = blockIdx.z;
  const int o = offsets[e], n = offsets[e + 1] - o;
  const int tn = (w.N + BNE - 1) / BNE;
  Job jb;
  jb.expert = e;
  jb.row0 = (blockIdx.x / tn) * BM;
  jb.rows = min(BM, w.M - jb.row0);
  jb.n0 = blockIdx.x % tn;
  jb.wide = false;
  jb.kb = 0;
  jb.nks = max(1, (n + BK - 1) / BK);  // an empty segment reads zeros and writes a zero gradient
  jb.part = 0;
  jb.nparts = 1;
  jb.pslot = 0;
  Operands op;
  op.A = w.A + size_t(o) * w.lda + size_t(z) * w.a_zoff;
  op.a_rows = n;
  op.lda = w.lda;
  op.Bg = op.Bu = w.B + size_t(o) * w.ldb + size_t(z) * w.b_zoff;
  op.b_rows = n;
  op.ldb = w.ldb;
  bf16_t* Ce = (z ? w.C1 : w.C0) + size_t(e) * w.M * w.N;
  tile_body<1, false, NW, kWgrad, true, true>(op, Ce, w.N, jb.nks * BK, 0, jb, nullptr, lds, nullptr, nullptr);
}

// BKN, kcat: the weight operand's layout and K split (see tile_body)
template <int NMAT, int NW, int EP, bool BKN>
__global__ __launch_bounds__(NW * 64) void gemm_kernel(const bf16_t* __restrict__ A, const int32_t* __restrict__ offsets,
                                                       const bf16_t* __restrict__ B0, const bf16_t* __restrict__ B1,
                                                       bf16_t* __restrict__ C, int L, int N, int K, int kcat, int a_rows,
                                                        const int32_t* __restrict__ tpre, int cpx, int smax,
                                                        float* __restrict__ parts, bf16_t* __restrict__ Gs,
                                                        bf16_t* __restrict__ Us) {
  extern __shared__ __attribute__((aligned(1024))) char lds[];
  static_assert(EP != kWgrad, "the weight-gradient products run wgrad_kernel");
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
  // K of one weight matrix: K, or 64 kcat for a product over two matrices side by side along K
  const int kw = kcat > 0 ? kcat * BK : K;
  const size_t boff = size_t(jb.expert) * N * kw;
  Operands op;
  op.A = A;
  op.a_rows = a_rows;
  op.lda = K;
  op.Bg = B0 + boff;
  op.Bu = (NMAT == 2 || kcat > 0 ? B1 : B0) + boff;
  op.b_rows = BKN ? kw : N;
  op.ldb = BKN ? N : kw;
  if (jb.wide)
    tile_body<NMAT, true, NW, EP, BKN, false>(op, C, N, K, kcat, jb, parts, lds, Gs, Us);
  else
    tile_body<NMAT, false, NW, EP, BKN, false>(op, C, N, K, kcat, jb, parts, lds, Gs, Us);
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
  tile_of(offsets, tpre, L, NT, group_width(K), xp.base + xp.F * cpx + w, jb);
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

template <int NMAT, int NW, int EP, bool BKN>
moe_status launch_nws(const char* name, const bf16_t* A, const int32_t* offsets, const bf16_t* B0, const bf16_t* B1,
                      bf16_t* C, int L, int N, int K, int kcat, int64_t max_pairs, const int32_t* tpre, float* parts,
                      hipStream_t s, bf16_t* Gs, bf16_t* Us);

template <int NMAT, int NW>
moe_status launch_nw(const char* name, const bf16_t* A, const int32_t* offsets, const bf16_t* B0, const bf16_t* B1,
                     bf16_t* C, int L, int N, int K, int kcat, bool bkn, int64_t max_pairs, const int32_t* tpre,
                     float* parts, hipStream_t s, bf16_t* Gs, bf16_t* Us, int ep) {
#define MOE_NWS(EP_, PARTS_)                                                                                      \
  (bkn ? launch_nws<NMAT, NW, EP_, true>(name, A, offsets, B0, B1, C, L, N, K, kcat, max_pairs, tpre, PARTS_, s, Gs, Us) \
       : launch_nws<NMAT, NW, EP_, false>(name, A, offsets, B0, B1, C, L, N, K, kcat, max_pairs, tpre, PARTS_, s, Gs, Us))
  if constexpr (NMAT == 2) {
    if (ep == kSave) return MOE_NWS(kSave, parts);
  } else {
    if (ep == kSwigluBwd) return MOE_NWS(kSwigluBwd, nullptr);
  }
  return MOE_NWS(kPlain, parts);
#undef MOE_NWS
}

// EP: the epilogue (kSave: the training forward's gate/up, which also writes the
// pre-activations; kSwigluBwd: the backward's down dgrad, never split along K)
template <int NMAT, int NW, int EP, bool BKN>
moe_status launch_nws(const char* name, const bf16_t* A, const int32_t* offsets, const bf16_t* B0, const bf16_t* B1,
                      bf16_t* C, int L, int N, int K, int kcat, int64_t max_pairs, const int32_t* tpre, float* parts,
                      hipStream_t s, bf16_t* Gs, bf16_t* Us) {
  constexpr int kThreads = NW * 64;
  auto kern = gemm_kernel<NMAT, NW, EP, BKN>;
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
  MOE_LAUNCH(name, kern, dim3(unsigned(per_xcd * kXcds)), dim3(kThreads), lds, s, A, offsets, B0, B1, C, L, N, K, kcat,
             int(max_pairs), tpre, cpx, smax, parts, Gs, Us);
  if (smax > 1) {
    const char* fname = std::strcmp(name, "ffn_gate_up") == 0         ? "ffn_gate_up_fixup"
                        : std::strcmp(name, "ffn_gate_up_dgrad") == 0 ? "ffn_gate_up_dgrad_fixup"
                        : std::strcmp(name, "ffn_down") == 0          ? "ffn_down_fixup"
                                                                       : "ffn_fixup";
    MOE_LAUNCH(fname, (fixup_kernel<NMAT, NW, EP>), dim3(unsigned(kXcds * kMaxTail * kFixSub)), dim3(kThreads), 0, s,
               offsets, C, L, N, K, tpre, cpx, smax, static_cast<const float*>(parts), Gs, Us);
  }
  return MOE_OK;
}

template <int NW>
moe_status launch_wgrad_nw(const char* name, const moe_layer_desc* d, const int32_t* offsets, const WgradOps& w, int Z,
                           hipStream_t s) {
  auto kern = wgrad_kernel<NW>;
  constexpr size_t lds = lds_bytes<1>();
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern), hipFuncAttributeMaxDynamicSharedMemorySize,
                                     int(lds));
  if (e != hipSuccess) return set_error(MOE_ERR_HIP, "%s: LDS attribute: %s", name, hipGetErrorString(e));
  const unsigned tiles = unsigned(((w.M + BM - 1) / BM) * ((w.N + BNE - 1) / BNE));
  MOE_LAUNCH(name, kern, dim3(tiles, unsigned(d->local_count), unsigned(Z)), dim3(NW * 64), lds, s, w, offsets);
  return MOE_OK;
}

// bkn: the weight operand is k-major (element (k, n) at B[k * N + n]); kcat > 0: a
// one-matrix product over B0 for the first 64 * kcat of K, then B1 (see tile_body)
template <int NMAT>
moe_status launch(const char* name, const bf16_t* A, const int32_t* offsets, const bf16_t* B0, const bf16_t* B1,
                  bf16_t* C, int L, int N, int K, int kcat, bool bkn, int64_t max_pairs, const int32_t* tpre,
                  float* parts, hipStream_t s, bf16_t* Gs = nullptr, bf16_t* Us = nullptr, int ep = kPlain) {
  if (K / BK < kEightWaveSteps)
    return launch_nw<NMAT, 8>(name, A, offsets, B0, B1, C, L, N, K, kcat, bkn, max_pairs, tpre, parts, s, Gs, Us, ep);
  return launch_nw<NMAT, 4>(name, A, offsets, B0, B1, C, L, N, K, kcat, bkn, max_pairs, tpre, parts, s, Gs, Us, ep);
}

}  // namespace big

// large tiles pay off once segments hold a few hundred rows; decode-sized
// batches (a handful of rows per expert) take the skinny kernel
bool use_big(const moe_layer_desc* d, int64_t max_pairs) {
  return d->dtype == MOE_BF16 && max_pairs >= int64_t(128) * d->local_count && big::supported(d->hidden) &&
         big::supported(d->intermediate) && big::addressable(d->intermediate, d->hidden);
}

moe_status launch_small(const FfnArgs& a) {
  // decode-sized batches: a few rows per expert, bound by streaming the weights
  if (skinny_ffn_fits(a.d, a.max_pairs)) return launch_skinny_ffn(a);
  return launch_general_ffn(a);
}

}  // namespace

size_t ffn_scratch_bytes(const moe_layer_desc* d, int64_t max_pairs) {
  if (!use_big(d, max_pairs)) return 0;
  const size_t plan = align_up(size_t(2) * (d->local_count + 1) * sizeof(int32_t), 256);
  const bool split = big::splits(d->hidden) || big::splits(d->intermediate);
  return plan + (split ? size_t(big::kXcds) * big::kMaxParts * big::kPartBytes : 0);
}

// ---- the backward's dgrad products on the large-tile kernel ---------------------
// dh = dy_sorted Wd^T (math form: Wd_e is [I, H]) with the SwiGLU backward in the
// epilogue (writing dg | du as [P, 2I]), then dx_sorted = [dg | du] [Wg_e | Wu_e]^T, one
// product over K = 2I whose first I read Wg_e and the rest Wu_e.  Each weight is read
// in place: the math-form layout gives these products n-major operands (Wd_e rows are
// the I outputs, Wg_e rows the H outputs), the linear layout k-major ones.
bool big_backward_supported(const moe_layer_desc* d, int64_t max_pairs) {
  return use_big(d, max_pairs) && big::supported(2 * d->intermediate) &&
         big::addressable(d->hidden, 2 * int64_t(d->intermediate));
}

size_t big_backward_scratch_bytes(const moe_layer_desc* d) {
  const size_t plan = align_up(size_t(2) * (d->local_count + 1) * sizeof(int32_t), 256);
  return plan + (big::splits(2 * d->intermediate) ? size_t(big::kXcds) * big::kMaxParts * big::kPartBytes : 0);
}

moe_status launch_big_backward_dgrad(const moe_layer_desc* d, const bf16_t* dy_sorted, const int32_t* offsets,
                                     const bf16_t* w_down, const bf16_t* w_gate, const bf16_t* w_up,
                                     const bf16_t* gate, const bf16_t* up, bf16_t* dgu, bf16_t* dx_sorted,
                                     int64_t max_pairs, void* scratch, hipStream_t s) {
  const int L = d->local_count, H = d->hidden, I = d->intermediate;
  const bool kn = d->weight_layout != MOE_WEIGHTS_IN_OUT;
  int32_t* pre = static_cast<int32_t*>(scratch);
  float* parts = big::splits(2 * I) ? reinterpret_cast<float*>(static_cast<char*>(scratch) +
                                                               align_up(size_t(2) * (L + 1) * sizeof(int32_t), 256))
                                    : nullptr;
  MOE_LAUNCH("ffn_bwd_plan", big::plan_kernel, dim3(1), dim3(1024), 0, s, offsets, L, (I + big::BNE - 1) / big::BNE,
             (H + big::BNE - 1) / big::BNE, H, 2 * I, pre);
  moe_status st = big::launch<1>("ffn_down_dgrad", dy_sorted, offsets, w_down, w_down, dgu, L, I, H, 0, kn, max_pairs,
                                 pre, nullptr, s, const_cast<bf16_t*>(gate), const_cast<bf16_t*>(up), big::kSwigluBwd);
  if (st != MOE_OK) return st;
  return big::launch<1>("ffn_gate_up_dgrad", dgu, offsets, w_gate, w_up, dx_sorted, L, H, 2 * I, I / big::BK, kn,
                        max_pairs, pre + L + 1, parts, s);
}

// The weight gradients read their operands in place, k-major, with 32-bit offsets
// from a segment's first row: every segment must be addressable that way.
bool big_wgrad_supported(const moe_layer_desc* d, int64_t max_pairs) {
  return big_backward_supported(d, max_pairs) &&
         big::addressable(max_pairs + 64, std::max<int64_t>(d->hidden, 2 * int64_t(d->intermediate)));
}

// dW_e = A_e^T B_e for each local expert e (Z outputs; see big::WgradOps).
moe_status launch_big_backward_wgrad(const char* name, const moe_layer_desc* d, const int32_t* offsets,
                                     const bf16_t* A, int lda, int a_zoff, const bf16_t* B, int ldb, int b_zoff,
                                     bf16_t* C0, bf16_t* C1, int M, int N, int Z, int64_t max_pairs, hipStream_t s) {
  big::WgradOps w{A, lda, a_zoff, B, ldb, b_zoff, C0, C1, M, N};
  // eight waves when the average segment is under 64 k steps, as for the forward
  const int64_t avg = max_pairs / std::max(1, d->local_count);
  if (avg / big::BK < big::kEightWaveSteps) return big::launch_wgrad_nw<8>(name, d, offsets, w, Z, s);
  return big::launch_wgrad_nw<4>(name, d, offsets, w, Z, s);
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
             (H + big::BNE - 1) / big::BNE, H, I, pre);
  // the math-form layout stores the weights k-major
  const bool kn = d->weight_layout == MOE_WEIGHTS_IN_OUT;
  moe_status st = big::launch<2>("ffn_gate_up", x, a.offsets, static_cast<const bf16_t*>(a.w_gate),
                                 static_cast<const bf16_t*>(a.w_up), h, L, I, H, 0, kn, a.max_pairs, pre, parts, a.s,
                                 static_cast<bf16_t*>(a.g_out), static_cast<bf16_t*>(a.u_out),
                                 a.g_out != nullptr ? big::kSave : big::kPlain);
  if (st != MOE_OK) return st;
  return big::launch<1>("ffn_down", h, a.offsets, static_cast<const bf16_t*>(a.w_down),
                        static_cast<const bf16_t*>(a.w_down), static_cast<bf16_t*>(a.y_sorted), L, H, I, 0, kn,
                        a.max_pairs, pre + L + 1, parts, a.s);
}

}  // namespace moe
