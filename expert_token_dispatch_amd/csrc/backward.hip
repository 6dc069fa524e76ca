// The backward pass of the layer.
//
// Hugging Face Transformers "Expert parallelism", section "Token dispatch":
// every rank trains on its own share of the batch, and an expert's weight
// gradient is the sum over all the pairs that reached it (an expert that got
// no tokens still takes part, contributing zero).  The gradients follow the
// chain rule through the forward (Ultralytics glossary "Expert Parallelism",
// "How tokens move between GPUs": route, dispatch, compute, combine):
//
//   combine   y[t] = sum_j w[t,j] y_sorted[q(t,j)]
//             -> dy_sorted[q] = w[t,j] dy[t],  dw[t,j] = <dy[t], y_sorted[q]>
//   softmax   w = softmax over the k chosen logits
//             -> dl[t,j] = w[t,j] (dw[t,j] - sum_i w[t,i] dw[t,i])
//   experts   g = v Wg^T, u = v Wu^T, h = silu(g) u, out = h Wd^T
//             -> dh = dout Wd, dg = dh u silu'(g), du = dh silu(g),
//                dWd = dout^T h, dWg = dg^T v, dWu = du^T v, dv = dg Wg + du Wu
//   router    logits = x Wr^T + b -> dWr = dlogits^T x, db = sum_t dlogits
//   dispatch  x_sorted[q] = x[t]  -> dx[t] = sum_j dx_sorted[q(t,j)] + sum_j dl[t,j] Wr[e(t,j)]
//
// Which experts a token uses is a discrete choice and carries no gradient.
//
// The grouped GEMMs come in two forms.  dgrad (dh, dv): rows are the sorted
// pairs, ragged by expert segment as in the forward, and the weight operand is
// read along its output dimension (B[k][n] with n contiguous).  wgrad (dW):
// the reduction runs over an expert's segment (ragged K) and both operands are
// contiguous along the output dimensions (A[k][m], B[k][n]).  Both stage their
// tiles into LDS as rows of K so the MFMA fragment reads are the forward's:
// an operand contiguous along M or N is loaded as two k rows of one 16-byte
// chunk per thread and written to LDS transposed, as (k, k+1) pairs.
#include <math.h>

#include <algorithm>
#include <type_traits>

#include "common.h"
#include "kernels.h"

namespace moe {
namespace {

// ---------------------------------------------------------------------------
// combine backward + softmax backward: one wave per token
// ---------------------------------------------------------------------------
constexpr int kTokensPerBlock = 4;

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

// KB: slots whose rows are loaded together (k rounded up to 2, 4 or 8; larger k in batches of 8);
// each lane takes kSlices 16-byte slices of a row per pass, so KB * kSlices loads are in flight
template <int KB>
constexpr int slices_for() { return KB <= 2 ? 8 : 4; }

template <typename T, int KB>
__global__ __launch_bounds__(256) void combine_bwd_kernel(const u32x4_t* __restrict__ dy, const u32x4_t* __restrict__ ys,
                                                          const int32_t* __restrict__ pair_row,
                                                          const float* __restrict__ tw, int64_t ntok, int k,
                                                          int vec_per_row, u32x4_t* __restrict__ dys,
                                                          float* __restrict__ dl) {
  constexpr int EPV = 16 / int(sizeof(T));
  constexpr int kSlices = slices_for<KB>();
  const int lane = threadIdx.x & 63;
  const int64_t t = int64_t(blockIdx.x) * kTokensPerBlock + (threadIdx.x >> 6);
  if (t >= ntok) return;
  const int my_row = lane < k ? pair_row[t * k + lane] : -1;
  const float my_w = lane < k ? tw[t * k + lane] : 0.0f;
  float my_dot = 0.0f;  // lane j: <dy[t], y_sorted[row of slot j]>
  const u32x4_t* src = dy + size_t(t) * vec_per_row;
  // every lane runs every pass (slot broadcasts and wave sums read other
  // lanes' registers); slice c0 + 64u + lane
  for (int c0 = 0; c0 < vec_per_row; c0 += 64 * kSlices) {
    float g[kSlices][EPV];
#pragma unroll
    for (int u = 0; u < kSlices; ++u) {
      const int c = c0 + 64 * u + lane;
      u32x4_t v = {0u, 0u, 0u, 0u};
      if (c < vec_per_row) v = src[c];
      unpack16(make_uint4(v[0], v[1], v[2], v[3]), T(), g[u]);
    }
    for (int j0 = 0; j0 < k; j0 += KB) {
      u32x4_t v[KB][kSlices];
#pragma unroll
      for (int jj = 0; jj < KB; ++jj) {
        const int r = __shfl(my_row, j0 + jj, 64);
#pragma unroll
        for (int u = 0; u < kSlices; ++u) {
          const int c = c0 + 64 * u + lane;
          if (j0 + jj < k && r >= 0 && c < vec_per_row) v[jj][u] = ys[size_t(r) * vec_per_row + c];
        }
      }
#pragma unroll
      for (int jj = 0; jj < KB; ++jj) {
        const int r = __shfl(my_row, j0 + jj, 64);
        if (j0 + jj >= k || r < 0) continue;  // uniform over the wave
        const float wj = __shfl(my_w, j0 + jj, 64);
        float p = 0.0f;
#pragma unroll
        for (int u = 0; u < kSlices; ++u) {
          const int c = c0 + 64 * u + lane;
          if (c < vec_per_row) {
            float f[EPV], o[EPV];
            unpack16(make_uint4(v[jj][u][0], v[jj][u][1], v[jj][u][2], v[jj][u][3]), T(), f);
#pragma unroll
            for (int e = 0; e < EPV; ++e) {
              p = fmaf(g[u][e], f[e], p);
              o[e] = wj * g[u][e];
            }
            const uint4 pk = pack16(o, T());
            dys[size_t(r) * vec_per_row + c] = u32x4_t{pk.x, pk.y, pk.z, pk.w};
          }
        }
        p = wave_sum(p);
        if (lane == j0 + jj) my_dot += p;
      }
    }
  }
  const float inner = wave_sum(my_w * my_dot);
  if (lane < k) dl[t * k + lane] = my_w * (my_dot - inner);
}

// ---------------------------------------------------------------------------
// dispatch backward: dx[t] = sum_j dx_sorted[q(t,j)] + sum_j dl[t,j] Wr[e(t,j)]
// (float32, the expert part in slot order, then the router part in slot
// order, rounded once); rows of KB slots are loaded together
// ---------------------------------------------------------------------------
template <typename T, int KB>
__global__ __launch_bounds__(256) void dispatch_bwd_kernel(const u32x4_t* __restrict__ dxs,
                                                           const int32_t* __restrict__ pair_row,
                                                           const int32_t* __restrict__ ids,
                                                           const float* __restrict__ dl, const u32x4_t* __restrict__ wr,
                                                           int64_t ntok, int k, int vec_per_row,
                                                           u32x4_t* __restrict__ dx) {
  constexpr int EPV = 16 / int(sizeof(T));
  constexpr int kSlices = slices_for<KB>();
  const int lane = threadIdx.x & 63;
  const int64_t t = int64_t(blockIdx.x) * kTokensPerBlock + (threadIdx.x >> 6);
  if (t >= ntok) return;
  const int my_row = lane < k ? pair_row[t * k + lane] : -1;
  const int my_e = lane < k ? ids[t * k + lane] : 0;
  const float my_dl = lane < k ? dl[t * k + lane] : 0.0f;
  // every lane runs every pass (slot broadcasts and wave sums read other
  // lanes' registers); slice c0 + 64u + lane
  for (int c0 = 0; c0 < vec_per_row; c0 += 64 * kSlices) {
    float acc[kSlices][EPV];
#pragma unroll
    for (int u = 0; u < kSlices; ++u)
#pragma unroll
      for (int e = 0; e < EPV; ++e) acc[u][e] = 0.0f;
    // the expert part, then the router part (pass 0, 1)
#pragma unroll
    for (int pass = 0; pass < 2; ++pass) {
      for (int j0 = 0; j0 < k; j0 += KB) {
        u32x4_t v[KB][kSlices];
#pragma unroll
        for (int jj = 0; jj < KB; ++jj) {
          const int r = pass == 0 ? __shfl(my_row, j0 + jj, 64) : __shfl(my_e, j0 + jj, 64);
          const u32x4_t* base = pass == 0 ? dxs : wr;
#pragma unroll
          for (int u = 0; u < kSlices; ++u) {
            const int c = c0 + 64 * u + lane;
            if (j0 + jj < k && r >= 0 && c < vec_per_row) v[jj][u] = base[size_t(r) * vec_per_row + c];
          }
        }
#pragma unroll
        for (int jj = 0; jj < KB; ++jj) {
          const int r = pass == 0 ? __shfl(my_row, j0 + jj, 64) : 0;
          if (j0 + jj >= k || r < 0) continue;  // uniform over the wave
          const float d = pass == 0 ? 1.0f : __shfl(my_dl, j0 + jj, 64);
#pragma unroll
          for (int u = 0; u < kSlices; ++u) {
            const int c = c0 + 64 * u + lane;
            if (c < vec_per_row) {
              float f[EPV];
              unpack16(make_uint4(v[jj][u][0], v[jj][u][1], v[jj][u][2], v[jj][u][3]), T(), f);
#pragma unroll
              for (int e = 0; e < EPV; ++e) acc[u][e] = pass == 0 ? acc[u][e] + f[e] : fmaf(d, f[e], acc[u][e]);
            }
          }
        }
      }
    }
#pragma unroll
    for (int u = 0; u < kSlices; ++u) {
      const int c = c0 + 64 * u + lane;
      if (c < vec_per_row) {
        const uint4 pk = pack16(acc[u], T());
        dx[size_t(t) * vec_per_row + c] = u32x4_t{pk.x, pk.y, pk.z, pk.w};
      }
    }
  }
}

// ---------------------------------------------------------------------------
// router: dlogits [T, Ep] (zero except the chosen experts; Ep = E rounded up
// to 8, the padding columns zero) in the layer's type for the dWr product and
// in float32 for the bias gradient, whose column sums run in two fixed-order
// passes (per chunk of tokens, then over the chunks).
// ---------------------------------------------------------------------------
template <typename T>
__global__ __launch_bounds__(256) void dlogits_kernel(const int32_t* __restrict__ ids, const float* __restrict__ dl,
                                                      int64_t ntok, int k, int E, int Ep, T* __restrict__ dlog,
                                                      float* __restrict__ dlog32) {
  const int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i >= ntok * Ep) return;
  const int64_t t = i / Ep;
  const int e = int(i % Ep);
  float v = 0.0f;
  if (e < E)
    for (int j = 0; j < k; ++j)
      if (ids[t * k + j] == e) v += dl[t * k + j];
  dlog[i] = Elem<T>::from_f32(v);
  if (dlog32 != nullptr) dlog32[i] = v;
}

constexpr int kColChunks = 128;

__global__ __launch_bounds__(256) void colsum_part_kernel(const float* __restrict__ dlog32, int64_t ntok, int Ep,
                                                          float* __restrict__ part) {
  const int c = blockIdx.x;
  const int64_t per = (ntok + kColChunks - 1) / kColChunks;
  const int64_t t0 = c * per, t1 = t0 + per < ntok ? t0 + per : ntok;
  for (int e = threadIdx.x; e < Ep; e += blockDim.x) {
    float s = 0.0f;
    for (int64_t t = t0; t < t1; ++t) s += dlog32[t * Ep + e];
    part[size_t(c) * Ep + e] = s;
  }
}

__global__ __launch_bounds__(256) void colsum_final_kernel(const float* __restrict__ part, int E, int Ep,
                                                           float* __restrict__ db) {
  for (int e = threadIdx.x; e < E; e += blockDim.x) {
    float s = 0.0f;
    for (int c = 0; c < kColChunks; ++c) s += part[size_t(c) * Ep + e];
    db[e] = s;
  }
}

// zero fill (a kernel rather than a memset, so callers may capture it in a graph)
__global__ __launch_bounds__(256) void zero_kernel(u32x4_t* __restrict__ p, int64_t n16, uint32_t* __restrict__ tail,
                                                   int64_t ntail) {
  const int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i < n16) p[i] = u32x4_t{0u, 0u, 0u, 0u};
  if (i < ntail) tail[i] = 0u;
}

// ---------------------------------------------------------------------------
// grouped GEMMs
// ---------------------------------------------------------------------------
constexpr int BM = 128, BN = 128, kThreads = 256;

template <typename T> struct Mma;
template <> struct Mma<bf16_t> {
  static constexpr int BK = 32;       // k per LDS stage
  static constexpr int kLd = BK + 8;  // LDS row stride in elements (80 bytes)
  static constexpr int FV = 1;        // 16-byte vectors per lane per 16-k chunk
  __device__ static void mma(const uint4* a, const uint4* b, f32x16_t& c) {
    c = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a[0]), __builtin_bit_cast(bf16x8_t, b[0]),
                                                c, 0, 0, 0);
  }
};
template <> struct Mma<float> {
  static constexpr int BK = 16;
  static constexpr int kLd = BK + 4;  // 80 bytes
  static constexpr int FV = 2;
  // eight 32x32x2 steps over the lane's eight k values (the same k for A and B)
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

// A tile of 128 rows x BK stored along K in memory (row r at base + (r0+r)*ld).
// Rows past `rows` repeat the last valid row (their results are never
// stored); k at or past K reads zero.  K is a multiple of the vector width.
template <typename T>
struct RowTile {
  static constexpr int BK = Mma<T>::BK, kLd = Mma<T>::kLd;
  static constexpr int EPV = 16 / int(sizeof(T)), CPR = BK / EPV, CPT = BM * CPR / kThreads;
  u32x4_t r[CPT];  // native vectors: a select of HIP's struct uint4 goes through scratch
  __device__ __forceinline__ void load(const T* __restrict__ base, int64_t ld, int64_t r0, int rows, int k0, int K) {
    const u32x4_t zero = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int j = 0; j < CPT; ++j) {
      const int c = threadIdx.x + j * kThreads;
      const int rr = min(c / CPR, rows - 1), kk = k0 + (c % CPR) * EPV;
      r[j] = kk < K ? *reinterpret_cast<const u32x4_t*>(base + (r0 + rr) * ld + kk) : zero;
    }
  }
  __device__ __forceinline__ void store(T* lds) const {
#pragma unroll
    for (int j = 0; j < CPT; ++j) {
      const int c = threadIdx.x + j * kThreads;
      *reinterpret_cast<u32x4_t*>(&lds[(c / CPR) * kLd + (c % CPR) * EPV]) = r[j];
    }
  }
};

// A tile of BK x 128 stored along M (or N) in memory: element (k, i) at
// base[(k0+k)*ld + i0 + i].  Thread t loads k rows 2p and 2p+1 (p = t % (BK/2))
// of the 16-byte chunk t / (BK/2) and writes the pairs to LDS as row i,
// columns 2p and 2p+1, so the LDS tile is [128][BK] like a RowTile's.
// k at or past kvalid and chunks at or past ivalid (a multiple of the vector
// width) read zero.
template <typename T>
struct ColTile {
  static constexpr int BK = Mma<T>::BK, kLd = Mma<T>::kLd;
  static constexpr int EPV = 16 / int(sizeof(T)), KP = BK / 2;
  static_assert(KP * (BM / EPV) == kThreads, "one unit per thread");
  u32x4_t lo, hi;
  __device__ __forceinline__ void load(const T* __restrict__ base, int64_t ld, int k0, int64_t kvalid, int i0, int ivalid) {
    const int p = threadIdx.x % KP, ch = threadIdx.x / KP;
    const int i = i0 + ch * EPV;
    const int64_t k = k0 + 2 * p;
    const u32x4_t zero = {0u, 0u, 0u, 0u};
    const bool ok = i < ivalid;
    lo = ok && k < kvalid ? *reinterpret_cast<const u32x4_t*>(base + k * ld + i) : zero;
    hi = ok && k + 1 < kvalid ? *reinterpret_cast<const u32x4_t*>(base + (k + 1) * ld + i) : zero;
  }
  __device__ __forceinline__ void store(T* lds) const {
    const int p = threadIdx.x % KP, ch = threadIdx.x / KP;
    const uint32_t a[4] = {lo[0], lo[1], lo[2], lo[3]}, b[4] = {hi[0], hi[1], hi[2], hi[3]};
    if constexpr (sizeof(T) == 2) {
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        // element 2w: low halves, element 2w+1: high halves
        const uint32_t ev = (a[w] & 0xFFFFu) | (b[w] << 16);
        const uint32_t od = (a[w] >> 16) | (b[w] & 0xFFFF0000u);
        *reinterpret_cast<uint32_t*>(&lds[(ch * EPV + 2 * w) * kLd + 2 * p]) = ev;
        *reinterpret_cast<uint32_t*>(&lds[(ch * EPV + 2 * w + 1) * kLd + 2 * p]) = od;
      }
    } else {
#pragma unroll
      for (int w = 0; w < 4; ++w)
        *reinterpret_cast<uint2*>(&lds[(ch * EPV + w) * kLd + 2 * p]) = make_uint2(a[w], b[w]);
    }
  }
};

// One 16-k chunk of MFMAs: waves split the 128 x 128 tile 2 x 2, each owning
// 2 x 2 blocks of 32 x 32.
template <typename T>
__device__ __forceinline__ void mma_stage(const T* As, const T* Bs, f32x16_t (&acc)[2][2], int wm, int wn, int lane) {
  using G = Mma<T>;
  constexpr int kLd = G::kLd, FV = G::FV;
  const int frow = lane & 31, fk = 8 * (lane >> 5);
#pragma unroll
  for (int kc = 0; kc < G::BK / 16; ++kc) {
    uint4 af[2][FV], bf[2][FV];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const uint4* p = reinterpret_cast<const uint4*>(&As[(wm * 64 + i * 32 + frow) * kLd + kc * 16 + fk]);
#pragma unroll
      for (int v = 0; v < FV; ++v) af[i][v] = p[v];
    }
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const uint4* p = reinterpret_cast<const uint4*>(&Bs[(wn * 64 + j * 32 + frow) * kLd + kc * 16 + fk]);
#pragma unroll
      for (int v = 0; v < FV; ++v) bf[j][v] = p[v];
    }
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j) G::mma(af[i], bf[j], acc[i][j]);
  }
}

// SiLU and its derivative through the hardware reciprocal, the same formula
// as the forward's gate: s = 1/(1+e^-g), silu = g s, silu' = s (1 + g (1 - s)).
__device__ __forceinline__ void silu_and_grad(float g, float& a, float& da) {
  const float s = __builtin_amdgcn_rcpf(1.0f + __expf(-g));
  a = g * s;
  da = s * (1.0f + g * (1.0f - s));
}

template <typename T>
struct DgradArgs {
  const T* A[2];         // [P, K[p]] rows = sorted pairs, row stride lda
  int K[2];
  int lda;
  const T* B[2];         // expert e: B[p] + e * b_estride, element (k, n) at [k * N + n]
  int64_t b_estride;     //   (BNK: at [n * K[p] + k])
  int N;
  T* C;                  // [P, N] (plain epilogue)
  const T* G;            // SwiGLU epilogue: saved pre-activations [P, N] ...
  const T* U;
  T* DGU;                // ... and their gradients side by side: [P, 2N], dg then du
  const int32_t* offsets;
  int L;
};

// C = sum_p A[p] B[p]_e over the sorted rows of each expert (EPI 0), or the
// SwiGLU backward of the result (EPI 1: C is dh; writes dg, du).  BNK: the
// weight operand is n-major (rows of K), else k-major (rows of N).
template <typename T, int EPI, int NPROD, bool BNK>
__global__ __launch_bounds__(kThreads) void dgrad_kernel(DgradArgs<T> p) {
  using G = Mma<T>;
  constexpr int BK = G::BK, kLd = G::kLd;
  int g = blockIdx.x, expert = -1, row0 = 0, rows = 0;
  {
    int prev = p.offsets[0];
    for (int i = 0; i < p.L; ++i) {
      const int nxt = p.offsets[i + 1];
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
  __shared__ __attribute__((aligned(16))) T As[2][BM * kLd];
  __shared__ __attribute__((aligned(16))) T Bs[2][BN * kLd];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, wm = wave >> 1, wn = wave & 1;

  f32x16_t acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

  // the argument fields as locals: a lambda capturing the argument struct
  // itself would need its address and copy it to scratch
  const T* const A0 = p.A[0];
  const T* const A1 = p.A[1];
  const T* const B0 = p.B[0] + size_t(expert) * p.b_estride;
  const T* const B1 = p.B[1] + size_t(expert) * p.b_estride;
  const int K0 = p.K[0], K1 = p.K[1], N = p.N, lda = p.lda;
  const int nk0 = (K0 + BK - 1) / BK;
  const int nks = nk0 + (NPROD > 1 ? (K1 + BK - 1) / BK : 0);
  RowTile<T> ta;
  typename std::conditional<BNK, RowTile<T>, ColTile<T>>::type tb;
  auto gload = [&](int s) {
    const bool q = NPROD > 1 && s >= nk0;
    const int k0 = (s - (q ? nk0 : 0)) * BK;
    const int Kq = q ? K1 : K0;
    ta.load(q ? A1 : A0, lda, row0, rows, k0, Kq);
    if constexpr (BNK)
      tb.load(q ? B1 : B0, Kq, n0, N - n0, k0, Kq);
    else
      tb.load(q ? B1 : B0, N, k0, Kq, n0, N);
  };
  if (nks > 0) {
    gload(0);
    ta.store(As[0]);
    tb.store(Bs[0]);
  }
  __syncthreads();
  for (int s = 0; s < nks; ++s) {
    const int buf = s & 1;
    if (s + 1 < nks) gload(s + 1);
    mma_stage<T>(As[buf], Bs[buf], acc, wm, wn, lane);
    if (s + 1 < nks) {
      ta.store(As[buf ^ 1]);
      tb.store(Bs[buf ^ 1]);
    }
    __syncthreads();
  }

  // accumulator layout: lane -> column (lane & 31), register r -> row 8*(r/4) + 4*(lane/32) + r%4
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int col = n0 + wn * 64 + j * 32 + (lane & 31);
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int rt = wm * 64 + i * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
        if (rt < rows && col < p.N) {
          const size_t at = size_t(row0 + rt) * p.N + col;
          const float v = acc[i][j][r];
          if constexpr (EPI == 0) {
            p.C[at] = Elem<T>::from_f32(v);
          } else {
            const float gv = Elem<T>::to_f32(p.G[at]), uv = Elem<T>::to_f32(p.U[at]);
            float a, da;
            silu_and_grad(gv, a, da);
            const size_t o2 = size_t(row0 + rt) * 2 * p.N + col;
            p.DGU[o2] = Elem<T>::from_f32(v * uv * da);
            p.DGU[o2 + p.N] = Elem<T>::from_f32(v * a);
          }
        }
      }
    }
}

template <typename T>
struct WgradArgs {
  const T* A[2];          // element (m, k) of expert e at A[z][(o_e + k) * lda + m]
  int lda;
  int m_load;             // columns of A that may be read (a multiple of the vector width)
  const T* B[2];          // element (k, n) at B[z][(o_e + k) * ldb + n] (B[1] NULL: B[0] for both)
  int ldb;
  T* C[2];                // expert e: C[z] + e * M * N, [M, N]
  int M, N;
  const int32_t* offsets; // NULL: one segment [0, k_total)
  int64_t k_total;
  float* partial;         // split-K (one segment): [gridDim.z, M, N] float32 pieces, else NULL
};

// C[z]_e = A[z]_e^T B_e, the reduction over expert e's segment; an empty
// segment writes zeros.  blockIdx.z picks the (A, C) pair.
template <typename T>
__global__ __launch_bounds__(kThreads) void wgrad_kernel(WgradArgs<T> p) {
  using G = Mma<T>;
  constexpr int BK = G::BK;
  // split-K: blockIdx.z picks a K slice instead of the (A, C) pair
  const bool split = p.partial != nullptr;
  const int z = split ? 0 : blockIdx.z, e = blockIdx.y;
  const int tiles_n = (p.N + BN - 1) / BN;
  const int m0 = (blockIdx.x / tiles_n) * BM, n0 = (blockIdx.x % tiles_n) * BN;
  int64_t o = p.offsets ? p.offsets[e] : 0;
  int64_t kseg = p.offsets ? p.offsets[e + 1] - o : p.k_total;
  if (split) {
    const int64_t per = ((kseg + gridDim.z - 1) / gridDim.z + BK - 1) / BK * BK;
    const int64_t lo = min(kseg, per * blockIdx.z);
    o += lo;
    kseg = min(kseg - lo, per);
  }
  const T* A = (z ? p.A[1] : p.A[0]) + o * p.lda;
  const T* B = (z && p.B[1] != nullptr ? p.B[1] : p.B[0]) + o * p.ldb;
  __shared__ __attribute__((aligned(16))) T As[2][BM * G::kLd];
  __shared__ __attribute__((aligned(16))) T Bs[2][BN * G::kLd];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, wm = wave >> 1, wn = wave & 1;

  f32x16_t acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

  const int nks = int((kseg + BK - 1) / BK);
  const int lda = p.lda, m_load = p.m_load, ldb = p.ldb, N = p.N;
  ColTile<T> ta, tb;
  auto gload = [&](int s) {
    ta.load(A, lda, s * BK, kseg, m0, m_load);
    tb.load(B, ldb, s * BK, kseg, n0, N);
  };
  if (nks > 0) {
    gload(0);
    ta.store(As[0]);
    tb.store(Bs[0]);
  }
  __syncthreads();
  for (int s = 0; s < nks; ++s) {
    const int buf = s & 1;
    if (s + 1 < nks) gload(s + 1);
    mma_stage<T>(As[buf], Bs[buf], acc, wm, wn, lane);
    if (s + 1 < nks) {
      ta.store(As[buf ^ 1]);
      tb.store(Bs[buf ^ 1]);
    }
    __syncthreads();
  }

  T* C = (z ? p.C[1] : p.C[0]) + size_t(e) * p.M * p.N;
  float* part = split ? p.partial + size_t(blockIdx.z) * p.M * p.N : nullptr;
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int col = n0 + wn * 64 + j * 32 + (lane & 31);
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int mt = m0 + wm * 64 + i * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
        if (mt < p.M && col < p.N) {
          if (split)
            part[size_t(mt) * p.N + col] = acc[i][j][r];
          else
            C[size_t(mt) * p.N + col] = Elem<T>::from_f32(acc[i][j][r]);
        }
      }
    }
}

// Sums the split-K pieces in slice order and rounds once.
template <typename T>
__global__ __launch_bounds__(256) void splitk_sum_kernel(const float* __restrict__ partial, int pieces, int64_t n,
                                                         T* __restrict__ C) {
  const int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i >= n) return;
  float v = 0.0f;
  for (int z = 0; z < pieces; ++z) v += partial[size_t(z) * n + i];
  C[i] = Elem<T>::from_f32(v);
}

// ---------------------------------------------------------------------------
// host launchers
// ---------------------------------------------------------------------------
int padded_experts(int E) { return (E + 7) / 8 * 8; }

template <typename T>
moe_status combine_bwd_t(const CombineBwdArgs& a) {
  const moe_layer_desc* d = a.d;
  const int vpr = int(size_t(d->hidden) * sizeof(T) / 16);
  const dim3 grid(unsigned((d->num_tokens + kTokensPerBlock - 1) / kTokensPerBlock));
  const u32x4_t* dy = static_cast<const u32x4_t*>(a.dy);
  const u32x4_t* ys = static_cast<const u32x4_t*>(a.y_sorted);
  u32x4_t* dys = static_cast<u32x4_t*>(a.dy_sorted);
  const int k = d->top_k;
  if (k <= 2) {
    MOE_LAUNCH("combine_bwd", (combine_bwd_kernel<T, 2>), grid, dim3(256), 0, a.s, dy, ys, a.pair_row, a.topk_w,
               d->num_tokens, k, vpr, dys, a.dl);
  } else if (k <= 4) {
    MOE_LAUNCH("combine_bwd", (combine_bwd_kernel<T, 4>), grid, dim3(256), 0, a.s, dy, ys, a.pair_row, a.topk_w,
               d->num_tokens, k, vpr, dys, a.dl);
  } else {
    MOE_LAUNCH("combine_bwd", (combine_bwd_kernel<T, 8>), grid, dim3(256), 0, a.s, dy, ys, a.pair_row, a.topk_w,
               d->num_tokens, k, vpr, dys, a.dl);
  }
  return MOE_OK;
}

template <typename T>
moe_status dispatch_bwd_t(const DispatchBwdArgs& a) {
  const moe_layer_desc* d = a.d;
  const int vpr = int(size_t(d->hidden) * sizeof(T) / 16);
  const dim3 grid(unsigned((d->num_tokens + kTokensPerBlock - 1) / kTokensPerBlock));
  const u32x4_t* dxs = static_cast<const u32x4_t*>(a.dx_sorted);
  const u32x4_t* wr = static_cast<const u32x4_t*>(a.w_router);
  u32x4_t* dx = static_cast<u32x4_t*>(a.dx);
  const int k = d->top_k;
  if (k <= 2) {
    MOE_LAUNCH("dispatch_bwd", (dispatch_bwd_kernel<T, 2>), grid, dim3(256), 0, a.s, dxs, a.pair_row, a.topk_ids,
               a.dl, wr, d->num_tokens, k, vpr, dx);
  } else if (k <= 4) {
    MOE_LAUNCH("dispatch_bwd", (dispatch_bwd_kernel<T, 4>), grid, dim3(256), 0, a.s, dxs, a.pair_row, a.topk_ids,
               a.dl, wr, d->num_tokens, k, vpr, dx);
  } else {
    MOE_LAUNCH("dispatch_bwd", (dispatch_bwd_kernel<T, 8>), grid, dim3(256), 0, a.s, dxs, a.pair_row, a.topk_ids,
               a.dl, wr, d->num_tokens, k, vpr, dx);
  }
  return MOE_OK;
}

// Scratch of the FFN backward: dg | du [P_max, 2I], then on the large-tile path the
// tile plan and split-K pieces.
struct FfnBwdScratch {
  void* dgu;
  void* big;  // big_backward_scratch_bytes
  bool big_wgrad;  // the weight gradients on the large tile (no scratch of their own)
};

FfnBwdScratch carve_ffn_bwd(const moe_layer_desc* d, int64_t max_pairs, void* base, size_t* bytes) {
  const size_t dt = dtype_bytes(d->dtype);
  char* p = static_cast<char*>(base);
  size_t o = 0;
  auto take = [&](size_t n) -> void* {
    void* r = p ? p + o : nullptr;
    o += align_up(n, 256);
    return r;
  };
  FfnBwdScratch w{};
  w.dgu = take(size_t(max_pairs) * 2 * d->intermediate * dt);
  if (big_backward_supported(d, max_pairs)) {
    w.big = take(big_backward_scratch_bytes(d));
    w.big_wgrad = big_wgrad_supported(d, max_pairs);
  }
  if (bytes) *bytes = o;
  return w;
}

// With the math-form weights (MOE_WEIGHTS_IN_OUT) Wd_e is [I, H] and Wg_e, Wu_e [H, I];
// the linear layout stores their transposes.  dh = dy_sorted Wd_e^T and
// dx_sorted = dg Wg_e^T + du Wu_e^T read the weights in place either way (n-major
// operands for the math form, k-major for the linear layout); the weight gradients
// are written in the weights' layout: dWd_e = h^T dy_sorted [I, H] or its transpose
// dy_sorted^T h [H, I], and likewise x_sorted^T dg or dg^T x_sorted.
template <typename T>
moe_status ffn_bwd_t(const FfnBwdArgs& a) {
  const moe_layer_desc* d = a.d;
  const int L = d->local_count, H = d->hidden, I = d->intermediate;
  const bool io = d->weight_layout == MOE_WEIGHTS_IN_OUT;
  const FfnBwdScratch w = carve_ffn_bwd(d, a.max_pairs, a.scratch, nullptr);
  T* dgu = static_cast<T*>(w.dgu);
  bool big = false;
  if constexpr (sizeof(T) == 2) {
    if (w.big != nullptr) {
      // the dgrad products on the large-tile kernel, reading the weights in place
      big = true;
      const moe_status st = launch_big_backward_dgrad(
          d, static_cast<const bf16_t*>(a.dy_sorted), a.offsets, static_cast<const bf16_t*>(a.w_down),
          static_cast<const bf16_t*>(a.w_gate), static_cast<const bf16_t*>(a.w_up), static_cast<const bf16_t*>(a.gate),
          static_cast<const bf16_t*>(a.up), dgu, static_cast<bf16_t*>(a.dx_sorted), a.max_pairs, w.big, a.s);
      if (st != MOE_OK) return st;
    }
  }
  const unsigned mslots = unsigned((a.max_pairs + BM - 1) / BM + L);
  if (!big) {  // dh = dy_sorted Wd_e^T, then dg, du
    DgradArgs<T> p{};
    p.A[0] = static_cast<const T*>(a.dy_sorted);
    p.K[0] = H;
    p.lda = H;
    p.B[0] = static_cast<const T*>(a.w_down);
    p.b_estride = int64_t(H) * I;
    p.N = I;
    p.G = static_cast<const T*>(a.gate);
    p.U = static_cast<const T*>(a.up);
    p.DGU = dgu;
    p.offsets = a.offsets;
    p.L = L;
    if (io) {
      MOE_LAUNCH("ffn_down_dgrad", (dgrad_kernel<T, 1, 1, true>), dim3(mslots, (I + BN - 1) / BN), dim3(kThreads), 0,
                 a.s, p);
    } else {
      MOE_LAUNCH("ffn_down_dgrad", (dgrad_kernel<T, 1, 1, false>), dim3(mslots, (I + BN - 1) / BN), dim3(kThreads), 0,
                 a.s, p);
    }
  }
  bool big_w = false;
  if constexpr (sizeof(T) == 2) {
    if (w.big_wgrad) {
      // the weight gradients on the large tile, every operand read in place
      big_w = true;
      const bf16_t* dys = static_cast<const bf16_t*>(a.dy_sorted);
      const bf16_t* h = static_cast<const bf16_t*>(a.h);
      const bf16_t* xs = static_cast<const bf16_t*>(a.x_sorted);
      bf16_t* dwd = static_cast<bf16_t*>(a.dw_down);
      bf16_t* dwg = static_cast<bf16_t*>(a.dw_gate);
      bf16_t* dwu = static_cast<bf16_t*>(a.dw_up);
      const bf16_t* g = reinterpret_cast<const bf16_t*>(dgu);
      moe_status st = io ? launch_big_backward_wgrad("ffn_down_wgrad", d, a.offsets, h, I, 0, dys, H, 0, dwd, nullptr,
                                                     I, H, 1, a.max_pairs, a.s)
                         : launch_big_backward_wgrad("ffn_down_wgrad", d, a.offsets, dys, H, 0, h, I, 0, dwd, nullptr,
                                                     H, I, 1, a.max_pairs, a.s);
      if (st == MOE_OK) {
        st = io ? launch_big_backward_wgrad("ffn_gate_up_wgrad", d, a.offsets, xs, H, 0, g, 2 * I, I, dwg, dwu, H, I, 2,
                                            a.max_pairs, a.s)
                : launch_big_backward_wgrad("ffn_gate_up_wgrad", d, a.offsets, g, 2 * I, I, xs, H, 0, dwg, dwu, I, H, 2,
                                            a.max_pairs, a.s);
      }
      if (st != MOE_OK) return st;
    }
  }
  if (!big_w) {  // dWd_e = h_e^T dy_sorted_e [I, H] (math form) or dy_sorted_e^T h_e [H, I]
    WgradArgs<T> p{};
    const T* dys = static_cast<const T*>(a.dy_sorted);
    const T* h = static_cast<const T*>(a.h);
    p.A[0] = io ? h : dys;
    p.lda = io ? I : H;
    p.m_load = io ? I : H;
    p.B[0] = io ? dys : h;
    p.ldb = io ? H : I;
    p.C[0] = static_cast<T*>(a.dw_down);
    p.M = io ? I : H;
    p.N = io ? H : I;
    p.offsets = a.offsets;
    const unsigned tiles = unsigned(((p.M + BM - 1) / BM) * ((p.N + BN - 1) / BN));
    MOE_LAUNCH("ffn_down_wgrad", wgrad_kernel<T>, dim3(tiles, L, 1), dim3(kThreads), 0, a.s, p);
  }
  if (!big) {  // dx_sorted = dg Wg_e^T + du Wu_e^T, one product over K = 2I
    DgradArgs<T> p{};
    p.A[0] = dgu;
    p.A[1] = dgu + I;
    p.K[0] = p.K[1] = I;
    p.lda = 2 * I;
    p.B[0] = static_cast<const T*>(a.w_gate);
    p.B[1] = static_cast<const T*>(a.w_up);
    p.b_estride = int64_t(I) * H;
    p.N = H;
    p.C = static_cast<T*>(a.dx_sorted);
    p.offsets = a.offsets;
    p.L = L;
    if (io) {
      MOE_LAUNCH("ffn_gate_up_dgrad", (dgrad_kernel<T, 0, 2, true>), dim3(mslots, (H + BN - 1) / BN), dim3(kThreads), 0,
                 a.s, p);
    } else {
      MOE_LAUNCH("ffn_gate_up_dgrad", (dgrad_kernel<T, 0, 2, false>), dim3(mslots, (H + BN - 1) / BN), dim3(kThreads),
                 0, a.s, p);
    }
  }
  if (!big_w) {  // dWg_e = x_e^T dg_e, dWu_e = x_e^T du_e [H, I] (math form), or dg_e^T x_e, du_e^T x_e [I, H]
    WgradArgs<T> p{};
    const T* xs = static_cast<const T*>(a.x_sorted);
    if (io) {
      p.A[0] = p.A[1] = xs;
      p.lda = H;
      p.m_load = H;
      p.B[0] = dgu;
      p.B[1] = dgu + I;
      p.ldb = 2 * I;
      p.M = H;
      p.N = I;
    } else {
      p.A[0] = dgu;
      p.A[1] = dgu + I;
      p.lda = 2 * I;
      p.m_load = I;
      p.B[0] = xs;
      p.ldb = H;
      p.M = I;
      p.N = H;
    }
    p.C[0] = static_cast<T*>(a.dw_gate);
    p.C[1] = static_cast<T*>(a.dw_up);
    p.offsets = a.offsets;
    const unsigned tiles = unsigned(((p.M + BM - 1) / BM) * ((p.N + BN - 1) / BN));
    MOE_LAUNCH("ffn_gate_up_wgrad", wgrad_kernel<T>, dim3(tiles, L, 2), dim3(kThreads), 0, a.s, p);
  }
  return MOE_OK;
}

// The router's dW = dlogits^T x reduces over every token: K slices of at least
// 256 tokens, enough to give ~1024 blocks, summed in slice order.
int route_bwd_pieces(const moe_layer_desc* d) {
  const int64_t tiles = int64_t((d->num_experts + BM - 1) / BM) * ((d->hidden + BN - 1) / BN);
  int64_t z = (1024 + tiles - 1) / tiles;
  z = std::min<int64_t>(z, (d->num_tokens + 255) / 256);
  return int(std::max<int64_t>(1, std::min<int64_t>(z, 64)));
}

template <typename T>
moe_status route_bwd_t(const RouteBwdArgs& a) {
  const moe_layer_desc* d = a.d;
  const int E = d->num_experts, Ep = padded_experts(E), H = d->hidden;
  const int64_t T_ = d->num_tokens;
  const RouteBwdScratch w = carve_route_bwd_scratch(d, a.ws);
  T* dlog = static_cast<T*>(w.dlogits);
  const int64_t n = T_ * Ep;
  MOE_LAUNCH("route_bwd_dlogits", dlogits_kernel<T>, dim3(unsigned((n + 255) / 256)), dim3(256), 0, a.s, a.topk_ids,
             a.dl, T_, d->top_k, E, Ep, dlog, a.db_router ? w.dlogits32 : static_cast<float*>(nullptr));
  WgradArgs<T> p{};
  p.A[0] = dlog;
  p.lda = Ep;
  p.m_load = Ep;
  p.B[0] = static_cast<const T*>(a.x);
  p.ldb = H;
  p.C[0] = static_cast<T*>(a.dw_router);
  p.M = E;
  p.N = H;
  p.offsets = nullptr;
  p.k_total = T_;
  const int pieces = route_bwd_pieces(d);
  p.partial = pieces > 1 ? w.pieces : nullptr;
  const unsigned tiles = unsigned(((E + BM - 1) / BM) * ((H + BN - 1) / BN));
  MOE_LAUNCH("route_bwd_wgrad", wgrad_kernel<T>, dim3(tiles, 1, unsigned(pieces)), dim3(kThreads), 0, a.s, p);
  if (pieces > 1) {
    const int64_t n = int64_t(E) * H;
    MOE_LAUNCH("route_bwd_wgrad_sum", splitk_sum_kernel<T>, dim3(unsigned((n + 255) / 256)), dim3(256), 0, a.s, w.pieces,
               pieces, n, static_cast<T*>(a.dw_router));
  }
  if (a.db_router != nullptr) {
    MOE_LAUNCH("route_bwd_bias", colsum_part_kernel, dim3(kColChunks), dim3(256), 0, a.s, w.dlogits32, T_, Ep,
               w.part);
    MOE_LAUNCH("route_bwd_bias_final", colsum_final_kernel, dim3(1), dim3(256), 0, a.s, w.part, E, Ep, a.db_router);
  }
  return MOE_OK;
}

}  // namespace

size_t route_bwd_scratch_bytes(const moe_layer_desc* d) {
  const int Ep = padded_experts(d->num_experts);
  const size_t n = size_t(d->num_tokens) * Ep;
  const int pieces = route_bwd_pieces(d);
  return align_up(n * dtype_bytes(d->dtype), 256) + align_up(n * 4, 256) + align_up(size_t(kColChunks) * Ep * 4, 256) +
         (pieces > 1 ? align_up(size_t(pieces) * d->num_experts * d->hidden * 4, 256) : 0);
}

RouteBwdScratch carve_route_bwd_scratch(const moe_layer_desc* d, void* ws) {
  const int Ep = padded_experts(d->num_experts);
  const size_t n = size_t(d->num_tokens) * Ep;
  char* p = static_cast<char*>(ws);
  RouteBwdScratch w;
  w.dlogits = p;
  p += align_up(n * dtype_bytes(d->dtype), 256);
  w.dlogits32 = reinterpret_cast<float*>(p);
  p += align_up(n * 4, 256);
  w.part = reinterpret_cast<float*>(p);
  p += align_up(size_t(kColChunks) * Ep * 4, 256);
  w.pieces = route_bwd_pieces(d) > 1 ? reinterpret_cast<float*>(p) : nullptr;
  return w;
}

size_t ffn_bwd_scratch_bytes(const moe_layer_desc* d, int64_t max_pairs) {
  size_t n = 0;
  carve_ffn_bwd(d, max_pairs, nullptr, &n);
  return n;
}

moe_status launch_zero(const char* name, void* p, size_t bytes, hipStream_t s) {
  if (p == nullptr || bytes == 0) return MOE_OK;
  // bytes is a multiple of 4; p is 16-byte aligned
  const int64_t n16 = int64_t(bytes / 16), ntail = int64_t(bytes % 16) / 4;
  uint32_t* tail = reinterpret_cast<uint32_t*>(static_cast<char*>(p) + n16 * 16);
  const int64_t n = n16 > ntail ? n16 : ntail;
  MOE_LAUNCH(name, zero_kernel, dim3(unsigned((n + 255) / 256)), dim3(256), 0, s, static_cast<u32x4_t*>(p), n16, tail,
             ntail);
  return MOE_OK;
}

moe_status launch_combine_backward(const CombineBwdArgs& a) {
  return a.d->dtype == MOE_BF16 ? combine_bwd_t<bf16_t>(a) : combine_bwd_t<float>(a);
}
moe_status launch_dispatch_backward(const DispatchBwdArgs& a) {
  return a.d->dtype == MOE_BF16 ? dispatch_bwd_t<bf16_t>(a) : dispatch_bwd_t<float>(a);
}
moe_status launch_grouped_ffn_backward(const FfnBwdArgs& a) {
  return a.d->dtype == MOE_BF16 ? ffn_bwd_t<bf16_t>(a) : ffn_bwd_t<float>(a);
}
moe_status launch_route_backward(const RouteBwdArgs& a) {
  return a.d->dtype == MOE_BF16 ? route_bwd_t<bf16_t>(a) : route_bwd_t<float>(a);
}

}  // namespace moe
