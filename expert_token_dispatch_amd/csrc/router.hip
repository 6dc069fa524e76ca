// Stage 1: router logits, top-k and routing weights.
//
// Ultralytics glossary "Expert Parallelism", section "How tokens move between
// GPUs", step 1: the router scores every token against every expert and keeps
// the k best.  Here the scores are a linear layer, logits = x Wr^T + b, with
// float32 accumulation; the k best are taken in descending order with ties to
// the lower expert id, and the routing weights are a softmax over the k chosen
// logits.
//
// Two kernels:
//  route_logits  a skinny GEMM [T, H] x [H, E].  A block owns 64 tokens (four
//                waves of 16), a group of up to 64 experts and one slice of H;
//                the grid spans token tiles x expert groups x H slices so that
//                even a decode batch keeps a few hundred blocks streaming.
//                x rows and router-weight rows (128 bytes of k per stage) go
//                through a 4-slot LDS ring filled by direct global->LDS loads
//                three stages ahead, so the only waits are the explicit ones;
//                the router-weight rows are shared by the four waves.  MFMA
//                16x16x32 bf16 (f32: 8 x 16x16x4 per stage).  Each block
//                writes its partial logits to partial[slice][t][e].
//  route_topk    sums the slices in slice order (so the logits do not depend
//                on scheduling) and adds the bias; then a row of 16 lanes per
//                token takes the k best in k rounds, each a row-wide maximum and
//                a row-wide minimum of the expert ids holding it (so equal
//                scores go to the lower id), both by DPP within the row, and
//                forms the softmax over the k chosen.
#include <math.h>

#include "common.h"
#include "kernels.h"

namespace moe {

namespace {

constexpr int kTok = 64;        // tokens per logits block (4 waves x 16)
constexpr int kThreads = 256;
constexpr int kMaxGroup = 64;   // experts per logits block
constexpr int kRowBytes = 128;  // bytes of k per router-weight row and stage
constexpr int kSlots = 4;       // LDS ring depth

typedef __attribute__((address_space(3))) void* lds_ptr_t;
typedef __attribute__((address_space(1))) void* glb_ptr_t;

#define MOE_VMCNT(n) __builtin_amdgcn_s_waitcnt(((n) & 0xF) | (((n) >> 4) << 14) | (0x7 << 4) | (0xF << 8))

template <typename T> struct RouterMma;
template <> struct RouterMma<bf16_t> {
  static constexpr int kStepK = 64;  // k per 128-byte chunk
  // one MFMA 16x16x32 per 16-byte piece s (two per chunk); the lane supplies
  // k = 32*s + 8*(lane/16) .. +7
  __device__ static void mma(const u32x4_t& a, const u32x4_t& b, f32x4_t& c) {
    c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a), __builtin_bit_cast(bf16x8_t, b), c,
                                                0, 0, 0);
  }
  // byte offset inside a 128-byte chunk of the lane's 16-byte piece s (s = 0, 1)
  __device__ static int piece(int lane, int s) { return s * 64 + (lane >> 4) * 16; }
};
template <> struct RouterMma<float> {
  static constexpr int kStepK = 32;
  // four MFMA 16x16x4 per 16-byte piece s (eight per chunk); the lane supplies
  // k = 16*s + 4*(lane/16) .. +3
  __device__ static void mma(const u32x4_t& a, const u32x4_t& b, f32x4_t& c) {
#pragma unroll
    for (int v = 0; v < 4; ++v) c = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a[v]), __uint_as_float(b[v]), c, 0, 0, 0);
  }
  __device__ static int piece(int lane, int s) { return s * 64 + (lane >> 4) * 16; }
};

// 16-byte chunk c of router-weight row r lives at physical chunk c ^ ((r/2) % 8)
__device__ __forceinline__ int swz(int r, int c) { return c ^ ((r >> 1) & 7); }

// partial[slice][t][e] = sum over the slice's k of x[t,k] * Wr[e,k]
//
// Stage layout in LDS: 64 x rows then G router-weight rows, 128 bytes each,
// 16-byte chunk c of row r at physical chunk c ^ ((r/2) % 8).  Both operands
// arrive by direct global->LDS loads; wave w loads its own 16 x rows (two
// 1 KB loads) and router-weight loads w, w+4, ... of the G/8 per stage.
template <typename T, int NEB>
__global__ __launch_bounds__(kThreads) void logits_kernel(const T* __restrict__ x, const T* __restrict__ wr,
                                                          float* __restrict__ partial, int ntok, int H, int E,
                                                          int k_per_slice) {
  using M = RouterMma<T>;
  constexpr int G = NEB * 16;                       // expert rows per block (<= 64)
  constexpr int kRows = kTok + G;
  constexpr int kSlotBytes = kRows * kRowBytes;     // <= 16 KB
  constexpr int EPC = 16 / int(sizeof(T));          // elements per 16-byte chunk
  constexpr int kWrLoads = G / 8;
  __shared__ __attribute__((aligned(1024))) char ring[kSlots * kSlotBytes];

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int t0 = blockIdx.x * kTok;
  const int e0 = blockIdx.y * G;
  const int k_begin = blockIdx.z * k_per_slice;
  const int k_end = min(H, k_begin + k_per_slice);
  const int nstep = (k_end - k_begin + M::kStepK - 1) / M::kStepK;

  // per-lane source rows and chunk of each direct load (chunks past H re-read
  // the row start: the matching x values are zeroed after the LDS read)
  const int lr = lane >> 3;                         // row within a 1 KB load
  const T* xsrc[2];
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int r = 16 * wave + 8 * j + lr;           // x row within the tile
    xsrc[j] = x + size_t(min(t0 + r, ntok - 1)) * H + swz(r, lane & 7) * EPC;  // rows past T repeat the last token
  }
  // direct loads this wave issues per stage: 2 for x, 0-2 for the router weight
  const int my_wr = wave < kWrLoads ? (kWrLoads - 1 - wave) / 4 + 1 : 0;
  auto issue = [&](int s) {
    char* slot = ring + (s % kSlots) * kSlotBytes;
    const int kb = k_begin + s * M::kStepK;
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int kk = kb + swz(16 * wave + 8 * j + lr, lane & 7) * EPC;
      __builtin_amdgcn_global_load_lds((glb_ptr_t)(xsrc[j] - swz(16 * wave + 8 * j + lr, lane & 7) * EPC +
                                                   (kk < H ? kk : 0)),
                                       (lds_ptr_t)(slot + (2 * wave + j) * 1024), 16, 0, 0);
    }
#pragma unroll
    for (int j0 = 0; j0 < 2; ++j0) {
      const int j = wave + 4 * j0;
      if (j < kWrLoads) {
        const int r = 8 * j + lr;                   // router-weight row within the group
        const int kk = kb + swz(kTok + r, lane & 7) * EPC;
        const int e = min(e0 + r, E - 1);           // rows past E repeat expert E-1 (never stored)
        __builtin_amdgcn_global_load_lds((glb_ptr_t)(wr + size_t(e) * H + (kk < H ? kk : 0)),
                                         (lds_ptr_t)(slot + kTok * kRowBytes + j * 1024), 16, 0, 0);
      }
    }
  };

  f32x4_t acc[NEB];
#pragma unroll
  for (int i = 0; i < NEB; ++i) acc[i] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  const int arow = 16 * wave + (lane & 15);
  for (int s = 0; s < kSlots - 1 && s < nstep; ++s) issue(s);
  for (int s = 0; s < nstep; ++s) {
    // this wave's loads of stage s have landed once only the later stages'
    // loads (stages s+1 and s+2, 2 + my_wr each) may still be in flight
    const int later = (2 + my_wr) * min(2, nstep - 1 - s);
    switch (later) {
      case 8: MOE_VMCNT(8); break;
      case 7: MOE_VMCNT(7); break;
      case 6: MOE_VMCNT(6); break;
      case 5: MOE_VMCNT(5); break;
      case 4: MOE_VMCNT(4); break;
      case 3: MOE_VMCNT(3); break;
      case 2: MOE_VMCNT(2); break;
      default: MOE_VMCNT(0); break;
    }
    // all waves' parts of stage s are in LDS; all waves are done with stage s-1
    block_barrier();
    if (s + kSlots - 1 < nstep) issue(s + kSlots - 1);
    const char* slot = ring + (s % kSlots) * kSlotBytes;
    const int kb = k_begin + s * M::kStepK;
    u32x4_t a[2];
#pragma unroll
    for (int p = 0; p < 2; ++p) {
      const int c = M::piece(lane, p) >> 4;
      a[p] = *reinterpret_cast<const u32x4_t*>(slot + arow * kRowBytes + swz(arow, c) * 16);
      if (kb + M::kStepK > k_end && kb + c * EPC >= k_end) a[p] = u32x4_t{0u, 0u, 0u, 0u};
    }
    // every fragment of the stage first, then the products with the expert
    // blocks interleaved (each accumulator still takes piece 0, then piece 1,
    // so the sums are those of one expert block at a time); independent
    // products back to back keep the matrix pipe from waiting on a result
    // (same-box A/B: route stage 42.0 -> 39.1 us on the gpt-oss-like layer)
    u32x4_t b[NEB][2];
#pragma unroll
    for (int nb = 0; nb < NEB; ++nb) {
      const int r = kTok + nb * 16 + (lane & 15);
#pragma unroll
      for (int p = 0; p < 2; ++p) {
        const int c = M::piece(lane, p) >> 4;
        b[nb][p] = *reinterpret_cast<const u32x4_t*>(slot + r * kRowBytes + swz(r, c) * 16);
      }
    }
    __builtin_amdgcn_sched_barrier(0);  // keep the reads ahead of the products
#pragma unroll
    for (int p = 0; p < 2; ++p)
#pragma unroll
      for (int nb = 0; nb < NEB; ++nb) M::mma(a[p], b[nb][p], acc[nb]);
  }
  MOE_VMCNT(0);

  // acc[nb][i] = partial logit of (token t0 + 16*wave + 4*(lane/16) + i, expert e0 + 16*nb + (lane & 15))
  float* out = partial + size_t(blockIdx.z) * ntok * E;
#pragma unroll
  for (int nb = 0; nb < NEB; ++nb) {
    const int e = e0 + nb * 16 + (lane & 15);
    if (e < E) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int t = t0 + 16 * wave + 4 * (lane >> 4) + i;
        if (t < ntok) out[size_t(t) * E + e] = acc[nb][i];
      }
    }
  }
}

constexpr int kTopkTok = 64;      // tokens per top-k block

static_assert(kTopkTok == kDispatchTokens, "a top-k block is one dispatch chunk");

// Sum a 64-token tile of partial logits over the slices in slice order, add the
// bias, optionally store the logits, and keep the tile in LDS with row stride ld.
template <int NTHR>
__device__ __forceinline__ void load_logit_tile(const float* __restrict__ partial, int nslice,
                                                const float* __restrict__ br, float* __restrict__ logits_out,
                                                int ntok, int E, int t0, int rows, int ld, float* lg, int tid) {
  const int n = rows * E;  // the tile's logits are contiguous in every slice
  const size_t slice_stride = size_t(ntok) * E;
  const float* base = partial + size_t(t0) * E;
  if ((E & 3) == 0) {
    const int n4 = n >> 2;
    // four float4s per thread per round, their slices' loads issued together and added in slice order
    for (int i0 = tid; i0 < n4; i0 += 4 * NTHR) {
      f32x4_t v[4];
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const int i = i0 + c * NTHR;
        if (i < n4) v[c] = reinterpret_cast<const f32x4_t*>(base)[i];
      }
      for (int s0 = 1; s0 < nslice; s0 += 4) {
        f32x4_t t[4][4];
#pragma unroll
        for (int c = 0; c < 4; ++c)
#pragma unroll
          for (int u = 0; u < 4; ++u) {
            const int i = i0 + c * NTHR;
            if (i < n4 && s0 + u < nslice) t[c][u] = reinterpret_cast<const f32x4_t*>(base + (s0 + u) * slice_stride)[i];
          }
#pragma unroll
        for (int c = 0; c < 4; ++c)
#pragma unroll
          for (int u = 0; u < 4; ++u)
            if (i0 + c * NTHR < n4 && s0 + u < nslice) v[c] += t[c][u];
      }
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const int i = i0 + c * NTHR;
        if (i >= n4) continue;
        const int m = (4 * i) / E, e = 4 * i - m * E;
        if (br != nullptr) {
#pragma unroll
          for (int q = 0; q < 4; ++q) v[c][q] += br[e + q];
        }
        if (logits_out != nullptr) reinterpret_cast<f32x4_t*>(logits_out + size_t(t0) * E)[i] = v[c];
#pragma unroll
        for (int q = 0; q < 4; ++q) lg[m * ld + e + q] = v[c][q];
      }
    }
  } else {
    for (int i = tid; i < n; i += NTHR) {
      float v = base[i];
      for (int sl = 1; sl < nslice; ++sl) v += base[sl * slice_stride + i];
      const int m = i / E, e = i - m * E;
      if (br != nullptr) v += br[e];
      if (logits_out != nullptr) logits_out[size_t(t0) * E + i] = v;
      lg[m * ld + e] = v;
    }
  }
}

// ---- top-k with one 16-lane row per token (E <= 16 * VPL) ----------------
// A block of 1024 threads takes the same 64-token tile; each wave's four rows
// of 16 lanes take one token each, lane r holding experts r*VPL .. r*VPL+VPL-1.
// Each of the k rounds finds the row's largest remaining logit with four DPP
// steps, then the lowest expert id holding it with four more (so equal scores
// go to the lower id, the order the pages' top-k implies), and the lane owning
// that expert marks it taken.  The weights are a softmax over the k chosen
// logits, shifted by the largest.
constexpr int kRowThreads = 1024;

template <int CTRL>
__device__ __forceinline__ int dpp(int x) {
  return __builtin_amdgcn_update_dpp(0, x, CTRL, 0xF, 0xF, false);
}
// maximum / minimum over the 16 lanes of a row, left in every lane of the row
__device__ __forceinline__ float row_max(float x) {
  x = fmaxf(x, __int_as_float(dpp<0xB1>(__float_as_int(x))));   // quad_perm [1,0,3,2]
  x = fmaxf(x, __int_as_float(dpp<0x4E>(__float_as_int(x))));   // quad_perm [2,3,0,1]
  x = fmaxf(x, __int_as_float(dpp<0x141>(__float_as_int(x))));  // row_half_mirror
  x = fmaxf(x, __int_as_float(dpp<0x140>(__float_as_int(x))));  // row_mirror
  return x;
}
__device__ __forceinline__ int row_min(int x) {
  x = min(x, dpp<0xB1>(x));
  x = min(x, dpp<0x4E>(x));
  x = min(x, dpp<0x141>(x));
  x = min(x, dpp<0x140>(x));
  return x;
}

template <int MAXK, int VPL>
__global__ __launch_bounds__(kRowThreads) void topk_row_kernel(const float* __restrict__ partial, int nslice,
                                                               const float* __restrict__ br, float* __restrict__ logits_out,
                                                               int32_t* __restrict__ ids, float* __restrict__ tw,
                                                               float* __restrict__ tl, int32_t* __restrict__ blk_counts,
                                                               int ntok, int E, int k, const float* __restrict__ sel_bias,
                                                               int gsize, int max_groups) {
  extern __shared__ float sh[];
  const int ld = 16 * VPL + 4;                 // row stride: a lane's VPL logits are 16-byte aligned
  float* lg = sh;                              // [64][ld]
  int* hist = reinterpret_cast<int*>(sh + kTopkTok * ld);  // [E]
  float* sb = sh + kTopkTok * ld + E;          // [E] selection bias, staged once per block
  const int tid = threadIdx.x;
  if (blk_counts != nullptr)
    for (int e = tid; e < E; e += kRowThreads) hist[e] = 0;
  if (sel_bias != nullptr)
    for (int e = tid; e < E; e += kRowThreads) sb[e] = sel_bias[e];
  const int t0 = blockIdx.x * kTopkTok;
  const int rows = min(kTopkTok, ntok - t0);
  load_logit_tile<kRowThreads>(partial, nslice, br, logits_out, ntok, E, t0, rows, ld, lg, tid);
  __syncthreads();

  const int wave = tid >> 6, lane = tid & 63, r = lane & 15;
  const int m = wave * 4 + (lane >> 4);        // token of this row within the tile
  if (m < rows) {
    float v[VPL];
    const f32x4_t* src = reinterpret_cast<const f32x4_t*>(lg + m * ld + r * VPL);
#pragma unroll
    for (int c4 = 0; c4 < VPL / 4; ++c4) {
      const f32x4_t q = src[c4];
#pragma unroll
      for (int u = 0; u < 4; ++u) v[4 * c4 + u] = q[u] == q[u] ? q[u] : -INFINITY;  // a NaN ranks last
    }
    unsigned taken = 0;
#pragma unroll
    for (int c = 0; c < VPL; ++c)
      if (r * VPL + c >= E) taken |= 1u << c;  // past the last expert
    // selection scores: the logits plus the selection bias (a float32 sum), if any
    float sc[VPL];
#pragma unroll
    for (int c = 0; c < VPL; ++c) {
      sc[c] = v[c];
      if (sel_bias != nullptr && r * VPL + c < E) {
        const float t = v[c] + sb[r * VPL + c];
        sc[c] = t == t ? t : -INFINITY;
      }
    }
    if (gsize > 0) {
      // group-limited routing: lane g < G scores group g (its best selection score), then
      // max_groups rounds of row max / lowest group keep the best groups; experts of
      // the other groups count as taken
      const int G = E / gsize;
      float gs = -INFINITY;
      if (r < G) {
        const float* row = lg + m * ld + r * gsize;
        for (int i = 0; i < gsize; ++i) {
          float t = row[i];
          t = t == t ? t : -INFINITY;
          if (sel_bias != nullptr) {
            t += sb[r * gsize + i];
            t = t == t ? t : -INFINITY;
          }
          gs = fmaxf(gs, t);
        }
      }
      bool avail = r < G;
      unsigned chosen = 0;
      for (int q = 0; q < max_groups; ++q) {
        const float mx = row_max(avail ? gs : -INFINITY);
        const int cand = (avail && gs == mx) ? r : 0x7FFFFFFF;
        const int win = row_min(cand);
        chosen |= 1u << win;
        if (r == win) avail = false;
      }
      // slots past the last expert are already taken (and their group index could
      // exceed the mask's 32 bits)
#pragma unroll
      for (int c = 0; c < VPL; ++c)
        if (r * VPL + c < E && !((chosen >> ((r * VPL + c) / gsize)) & 1u)) taken |= 1u << c;
    }
    float sel_v[MAXK];
    int sel_i[MAXK];
#pragma unroll
    for (int j = 0; j < MAXK; ++j) {
      sel_v[j] = 0.0f;
      sel_i[j] = 0;
      if (j < k) {
        // this lane's best untaken logit; a strict compare keeps the lower id on ties
        float bv = -INFINITY, bl = -INFINITY;
        int bc = -1;
#pragma unroll
        for (int c = 0; c < VPL; ++c)
          if (!((taken >> c) & 1u) && (bc < 0 || sc[c] > bv)) {
            bv = sc[c];
            bl = v[c];
            bc = c;
          }
        const float mx = row_max(bv);
        const int cand = (bc >= 0 && bv == mx) ? r * VPL + bc : 0x7FFFFFFF;
        const int win = row_min(cand);
        if (cand == win) taken |= 1u << bc;
        // the chosen expert's logit without the bias (the winner lane's)
        sel_v[j] = sel_bias != nullptr ? row_max(cand == win ? bl : -INFINITY) : mx;
        sel_i[j] = win;
        if (r == 0 && blk_counts != nullptr) atomicAdd(&hist[win], 1);
      }
    }
    // the largest chosen logit (the first one, unless a selection bias reordered them)
    float top = sel_v[0];
#pragma unroll
    for (int j = 1; j < MAXK; ++j)
      if (j < k) top = fmaxf(top, sel_v[j]);
    float ex[MAXK];
    float sum = 0.0f;
#pragma unroll
    for (int j = 0; j < MAXK; ++j) {
      if (j < k) {
        ex[j] = expf(sel_v[j] - top);
        sum += ex[j];
      }
    }
    const float inv = 1.0f / sum;
    const int t = t0 + m;
    // lane r of the row writes entries r and r + 16
#pragma unroll
    for (int h = 0; h < (MAXK + 15) / 16; ++h) {
      const int j = r + 16 * h;
      if (j < k) {
        float ov = sel_v[0], oe = ex[0];
        int oi = sel_i[0];
#pragma unroll
        for (int jj = 1; jj < MAXK; ++jj)
          if (j == jj) {
            ov = sel_v[jj];
            oe = ex[jj];
            oi = sel_i[jj];
          }
        const size_t o = size_t(t) * k + j;
        ids[o] = oi;
        tw[o] = oe * inv;
        if (tl != nullptr) tl[o] = ov;
      }
    }
  }
  // the chunk's expert histogram for dispatch (integer counts: order-free)
  if (blk_counts != nullptr) {
    __syncthreads();
    for (int e = tid; e < E; e += kRowThreads) blk_counts[size_t(blockIdx.x) * E + e] = hist[e];
  }
}

// ---- one balancing step on the selection bias --------------------------------
// Ultralytics glossary "Expert Parallelism", section "Load balancing and
// capacity": after each step the bias goes down for overloaded experts and up
// for idle ones.  Overloaded means more than the mean load, tested on integers
// (counts[e] * E > total); at the mean the bias stays.
__global__ __launch_bounds__(1024) void bias_update_kernel(const int32_t* __restrict__ counts, float* __restrict__ bias,
                                                           int E, float gamma) {
  __shared__ long long part[16];
  long long t = 0;
  for (int e = threadIdx.x; e < E; e += 1024) t += counts[e];
  for (int o = 32; o > 0; o >>= 1) t += __shfl_xor(t, o, 64);
  if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = t;
  __syncthreads();
  long long total = 0;
  for (int w = 0; w < 16; ++w) total += part[w];
  for (int e = threadIdx.x; e < E; e += 1024) {
    const long long c = (long long)counts[e] * E;
    if (c > total) bias[e] = bias[e] - gamma;
    else if (c < total) bias[e] = bias[e] + gamma;
  }
}

// Work split of the logits kernel: token tiles x expert groups x H slices.
struct Split {
  int groups, neb, slices, k_per_slice;
};

template <typename T>
Split plan(const moe_layer_desc* d) {
  Split s;
  const int E = d->num_experts, H = d->hidden;
  const int e16 = (E + 15) / 16 * 16;
  const int64_t tiles = (d->num_tokens + kTok - 1) / kTok;
  // widest expert group that still leaves a few hundred blocks (narrower groups re-read the
  // token tile once per group, which only small batches can afford)
  int g = e16 < kMaxGroup ? e16 : kMaxGroup;
  while (g > 16 && tiles * ((E + g - 1) / g) * 4 < 256) g /= 2;
  g = (g + 15) / 16 * 16;
  s.neb = g / 16;
  s.groups = (E + g - 1) / g;
  const int step = RouterMma<T>::kStepK;
  const int nsteps = (H + step - 1) / step;
  // enough blocks to keep every CU streaming, but each slice at least 4 chunks deep, and no
  // more than 128 KB of partial logits for one top-k block to add up
  int slices = 1;
  while (tiles * s.groups * slices < 512 && nsteps / (slices * 2) >= 4 &&
         int64_t(slices) * 2 * kTopkTok * E * int64_t(sizeof(float)) <= 128 * 1024)
    slices *= 2;
  s.slices = slices;
  s.k_per_slice = (nsteps + slices - 1) / slices * step;
  return s;
}

template <typename T, int NEB>
moe_status launch_logits(const RouteArgs& a, const Split& sp, float* partial) {
  const moe_layer_desc* d = a.d;
  const int ntok = int(d->num_tokens);
  const dim3 grid(unsigned((ntok + kTok - 1) / kTok), unsigned(sp.groups), unsigned(sp.slices));
  MOE_LAUNCH("route_logits", (logits_kernel<T, NEB>), grid, dim3(kThreads), 0, a.s, static_cast<const T*>(a.x),
             static_cast<const T*>(a.w_router), partial, ntok, d->hidden, d->num_experts, sp.k_per_slice);
  return MOE_OK;
}

template <int MAXK, int VPL>
moe_status launch_topk_rows(const RouteArgs& a, const float* partial, int nslice, const float* bias) {
  const moe_layer_desc* d = a.d;
  const int ntok = int(d->num_tokens);
  const int E = d->num_experts;
  const size_t lds = (size_t(kTopkTok) * (16 * VPL + 4) + 2 * size_t(E)) * sizeof(float);
  auto kern = topk_row_kernel<MAXK, VPL>;
  if (lds > 65536) {
    const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                             hipFuncAttributeMaxDynamicSharedMemorySize, int(lds));
    if (e != hipSuccess) return set_error(MOE_ERR_HIP, "route_topk: LDS attribute: %s", hipGetErrorString(e));
  }
  const dim3 grid(unsigned((ntok + kTopkTok - 1) / kTopkTok));
  MOE_LAUNCH("route_topk", kern, grid, dim3(kRowThreads), lds, a.s, partial, nslice, bias, a.logits_out,
             a.topk_ids, a.topk_w, a.topk_logit, a.blk_counts, ntok, E, d->top_k, a.sel_bias, a.group_size,
             a.max_groups);
  return MOE_OK;
}

template <int MAXK>
moe_status launch_topk(const RouteArgs& a, const float* partial, int nslice, const float* bias) {
  // one 16-lane row per token, 4, 8 or 16 logits per lane (the router takes up to 256 experts);
  // four for E <= 64 halves each round's per-lane scan (same box, interleaved: skewed_capacity
  // 18.4 -> 15.6 us, mixtral_like 7.0 -> 6.2, tiny_fp32 5.9 -> 5.1)
  if (a.d->num_experts <= 64) return launch_topk_rows<MAXK, 4>(a, partial, nslice, bias);
  if (a.d->num_experts <= 128) return launch_topk_rows<MAXK, 8>(a, partial, nslice, bias);
  return launch_topk_rows<MAXK, 16>(a, partial, nslice, bias);
}

moe_status pick_topk(const RouteArgs& a, const float* partial, int nslice, const float* bias) {
  const int k = a.d->top_k;
  if (k <= 2) return launch_topk<2>(a, partial, nslice, bias);
  if (k <= 4) return launch_topk<4>(a, partial, nslice, bias);
  if (k <= 8) return launch_topk<8>(a, partial, nslice, bias);
  if (k <= 16) return launch_topk<16>(a, partial, nslice, bias);
  return launch_topk<32>(a, partial, nslice, bias);
}

template <typename T>
moe_status route_t(const RouteArgs& a) {
  const Split sp = plan<T>(a.d);
  moe_status st;
  switch (sp.neb) {
    case 1: st = launch_logits<T, 1>(a, sp, a.partial); break;
    case 2: st = launch_logits<T, 2>(a, sp, a.partial); break;
    case 3: st = launch_logits<T, 3>(a, sp, a.partial); break;
    default: st = launch_logits<T, 4>(a, sp, a.partial); break;
  }
  if (st != MOE_OK) return st;
  return pick_topk(a, a.partial, sp.slices, a.b_router);
}

}  // namespace

size_t route_scratch_bytes(const moe_layer_desc* d) {
  const Split sp = d->dtype == MOE_BF16 ? plan<bf16_t>(d) : plan<float>(d);
  return align_up(size_t(sp.slices) * size_t(d->num_tokens) * d->num_experts * sizeof(float), 256);
}

moe_status launch_selection_bias_update(const moe_layer_desc* d, const int32_t* counts, float* bias, float gamma,
                                        hipStream_t s) {
  MOE_LAUNCH("route_bias_update", bias_update_kernel, dim3(1), dim3(1024), 0, s, counts, bias, d->num_experts, gamma);
  return MOE_OK;
}

moe_status launch_route(const RouteArgs& a) {
  if (a.logits_in != nullptr) return pick_topk(a, a.logits_in, 1, nullptr);
  return a.d->dtype == MOE_BF16 ? route_t<bf16_t>(a) : route_t<float>(a);
}

}  // namespace moe
