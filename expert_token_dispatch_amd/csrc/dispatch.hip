// Stage 2: token dispatch on one GPU.
//
// Hugging Face Transformers "Expert parallelism", section "Token dispatch":
// every (token, expert) pair is sent to the owner of its expert, which runs
// its local experts on what it receives.  On one GPU that is a permutation of
// the pairs into contiguous per-expert segments: a histogram of pairs per
// expert (the glossary snippet's bincount), an exclusive scan into segment
// offsets, and a stable scatter; the glossary's "Load balancing and capacity"
// adds an optional per-expert limit whose overflow skips the expert.
//
// Pair p = t*k + j.  Within a segment, pairs keep ascending p, so the result is
// unique and matches a stable counting sort exactly.  Work goes by chunks of
// 64 tokens (their 64*k pairs):
//   count     per chunk, counts over all E experts (the router's top-k kernel
//             writes these itself inside moe_layer_forward), built
//             with a wave64 match-any (ballot over the id bits) so only one
//             lane per distinct id touches the LDS histogram;
//   scan      one block: totals per expert, (capacity), exclusive scans into
//             segment offsets, and for every (chunk, expert) the first row of
//             that chunk's pairs (range sums over chunks, then prefixes);
//   scatter   per block again, in rounds of 256 pairs: the rank of a pair
//             among equal experts is its rank within its wave (match-any +
//             popcount of lower lanes) plus the counts of earlier waves and
//             earlier rounds -- no atomics, so the order is deterministic;
//   capacity  (only with a limit) one block per local expert: the expert's
//             keys sit in registers (element j*1024 + thread); radix select of
//             the C-th largest key (logit desc, then token asc), then a stable
//             compaction from per-wave ballots and two scans over the 512
//             (register, wave) slots;
//   place     without a capacity cut, scatter and row copy in one kernel:
//             ranks as in scatter, then token-major copies (one read of x[t],
//             one write per kept local pair, 16-byte vectors); when the chunk
//             histogram table is small (chunks x experts <= 16384) every place
//             block also sums the columns it needs itself, so no scan launch
//             sits between the router and the copy;
//   gather    with a capacity cut, the same token-major copy after it.
// The gather writes x_sorted with nontemporal stores: a capacity-limited layer
// has many pairs (hundreds of MB of rows, more than the last-level cache), so
// the rows stream to memory instead of evicting what the caches hold (same-box
// A/B on the skewed layer with capacity: dispatch stage 151 -> 130 us).  The
// place kernel keeps ordinary stores: there the rows are read back from the
// caches by the grouped GEMM.
#include "common.h"
#include "kernels.h"

namespace moe {

size_t dispatch_scratch_bytes(const moe_layer_desc* d) {
  const int64_t n = d->num_tokens * d->top_k;
  const int64_t nblk = dispatch_blocks(d->num_tokens);
  size_t b = 0;
  b += align_up(size_t(nblk) * d->num_experts * 4, 256);
  b += align_up(size_t(nblk) * d->local_count * 4, 256);
  b += align_up(size_t(d->local_count + 1) * 4, 256);
  if (d->capacity_factor > 0) b += align_up(size_t(n) * 4, 256);
  return b;
}

DispatchScratch carve_dispatch_scratch(const moe_layer_desc* d, void* ws) {
  const int64_t nblk = dispatch_blocks(d->num_tokens);
  char* p = static_cast<char*>(ws);
  DispatchScratch s{};
  s.blk_all = reinterpret_cast<int32_t*>(p);
  p += align_up(size_t(nblk) * d->num_experts * 4, 256);
  s.blk_base = reinterpret_cast<int32_t*>(p);
  p += align_up(size_t(nblk) * d->local_count * 4, 256);
  s.pre_off = reinterpret_cast<int32_t*>(p);
  p += align_up(size_t(d->local_count + 1) * 4, 256);
  s.tmp_sorted = d->capacity_factor > 0 ? reinterpret_cast<int32_t*>(p) : nullptr;
  return s;
}

namespace {

__device__ __forceinline__ int bits_for(int maxval) { return 32 - __clz(maxval); }

// Sum of col[b * stride] for b = b_lo, b_lo + step, ... < b_hi, eight loads in flight
// (integer sums: the grouping does not change the result).
__device__ __forceinline__ int column_sum(const int32_t* __restrict__ col, size_t stride, int b_lo, int b_hi, int step) {
  int s[8] = {0, 0, 0, 0, 0, 0, 0, 0};
  int b = b_lo;
  for (; b + 7 * step < b_hi; b += 8 * step) {
#pragma unroll
    for (int u = 0; u < 8; ++u) s[u] += col[size_t(b + u * step) * stride];
  }
  for (; b < b_hi; b += step) s[0] += col[size_t(b) * stride];
  return ((s[0] + s[1]) + (s[2] + s[3])) + ((s[4] + s[5]) + (s[6] + s[7]));
}

// Exclusive scan over the block; *total receives the block sum.  `wsum` holds
// one int per wave.  Every thread of the block must call it.
__device__ int block_exclusive_scan(int v, int* wsum, int* total) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int nw = blockDim.x >> 6;
  const int incl = wave_inclusive_scan(v);
  if (lane == 63) wsum[wave] = incl;
  __syncthreads();
  if (wave == 0) {
    int s = lane < nw ? wsum[lane] : 0;
    s = wave_inclusive_scan(s);
    if (lane < nw) wsum[lane] = s;
  }
  __syncthreads();
  const int before = wave > 0 ? wsum[wave - 1] : 0;
  *total = wsum[nw - 1];
  __syncthreads();
  return before + incl - v;
}

// ---- count ------------------------------------------------------------------
__global__ __launch_bounds__(kDispatchThreads) void count_kernel(const int32_t* __restrict__ ids, int64_t n_pairs,
                                                                 int E, int chunk, int32_t* __restrict__ blk_all) {
  extern __shared__ int32_t hist[];  // [E]
  for (int e = threadIdx.x; e < E; e += blockDim.x) hist[e] = 0;
  __syncthreads();
  const int64_t p0 = int64_t(blockIdx.x) * chunk;
  const int64_t p1 = min(n_pairs, p0 + chunk);
  const int bits = bits_for(E);
  for (int64_t base = p0; base < p1; base += blockDim.x) {
    const int64_t p = base + threadIdx.x;
    int id = p < p1 ? ids[p] : E;
    if (id < 0 || id >= E) id = E;  // sentinel: not counted
    const uint64_t m = match_any(uint32_t(id), bits, ~uint64_t(0));
    if (id < E && (m & lanemask_lt()) == 0) atomicAdd(&hist[id], int(__popcll(m)));
  }
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += blockDim.x) blk_all[size_t(blockIdx.x) * E + e] = hist[e];
}

// ---- scan -------------------------------------------------------------------
constexpr int kScanThreads = 1024;
constexpr int kScanGroups = 16;  // chunk ranges per column: short serial prefixes over the range sums

__global__ __launch_bounds__(kScanThreads) void scan_kernel(const int32_t* __restrict__ blk_all, int nblk, int E,
                                                            int begin, int L, int64_t cap, int32_t* __restrict__ counts,
                                                            int32_t* __restrict__ offsets, int32_t* __restrict__ pre_off,
                                                            int32_t* __restrict__ blk_base,
                                                            int64_t* __restrict__ num_dropped) {
  extern __shared__ int32_t sh[];
  int32_t* cnt = sh;          // [E]
  int32_t* pre = sh + E;      // [L + 1]
  __shared__ int wsum[kScanThreads / 64];
  __shared__ long long dsum[kScanThreads / 64];
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;

  __shared__ int rsum[kScanThreads];
  // totals per expert: columns in groups of up to 1024; thread t sums column
  // t % Ec over a contiguous range of chunks (coalesced across the columns)
  for (int c0 = 0; c0 < E; c0 += kScanThreads) {
    const int Ec = min(kScanThreads, E - c0);
    const int G = min(kScanGroups, kScanThreads / Ec);
    const int per = (nblk + G - 1) / G;
    const int e = tid % Ec, g = tid / Ec;
    int sum = 0;
    if (g < G) {
      const int b_lo = min(nblk, g * per), b_hi = min(nblk, b_lo + per);
      sum = column_sum(blk_all + c0 + e, size_t(E), b_lo, b_hi, 1);
      rsum[tid] = sum;
    }
    __syncthreads();
    if (tid < Ec) {
      int tot = 0;
      for (int gg = 0; gg < G; ++gg) tot += rsum[gg * Ec + tid];
      cnt[c0 + tid] = tot;
      counts[c0 + tid] = tot;
    }
    __syncthreads();
  }

  // segment offsets before (pre) and after (offsets) the capacity cut
  int carry_pre = 0, carry_post = 0;
  long long dropped = 0;
  for (int i0 = 0; i0 < L; i0 += kScanThreads) {
    const int i = i0 + tid;
    const int n = i < L ? cnt[begin + i] : 0;
    const int kept = cap < 0 ? n : int(min<int64_t>(n, cap));
    dropped += n - kept;
    int tot_n, tot_k;
    const int ex_n = block_exclusive_scan(n, wsum, &tot_n);
    const int ex_k = block_exclusive_scan(kept, wsum, &tot_k);
    if (i < L) {
      pre[i] = carry_pre + ex_n;
      pre_off[i] = carry_pre + ex_n;
      offsets[i] = carry_post + ex_k;
    }
    carry_pre += tot_n;
    carry_post += tot_k;
  }
  if (tid == 0) {
    pre[L] = carry_pre;
    pre_off[L] = carry_pre;
    offsets[L] = carry_post;
  }
  // dropped pairs: sum over threads
  for (int d = 1; d < 64; d <<= 1) dropped += __shfl_xor(dropped, d, 64);
  if (lane == 0) dsum[wave] = dropped;
  __syncthreads();
  if (tid == 0 && num_dropped != nullptr) {
    long long s = 0;
    for (int w = 0; w < kScanThreads / 64; ++w) s += dsum[w];
    *num_dropped = s;
  }

  // first pre-capacity row of every chunk's pairs of local expert i:
  // pre[i] + sum over earlier chunks of their count of expert begin+i.
  // Columns in groups of up to 1024: thread t takes column t % Lc and a
  // contiguous range of chunks (group t / Lc); range sums go through LDS.
  for (int c0 = 0; c0 < L; c0 += kScanThreads) {
    const int Lc = min(kScanThreads, L - c0);
    const int G = min(kScanGroups, kScanThreads / Lc);
    const int per = (nblk + G - 1) / G;
    const int i = tid % Lc, g = tid / Lc;
    const bool act = g < G;
    const int b_lo = act ? min(nblk, g * per) : 0, b_hi = act ? min(nblk, b_lo + per) : 0;
    const int32_t* col = blk_all + begin + c0 + i;
    const int s = act ? column_sum(col, size_t(E), b_lo, b_hi, 1) : 0;
    if (act) rsum[tid] = s;
    __syncthreads();
    if (act) {
      int run = pre[c0 + i];
      for (int gg = 0; gg < g; ++gg) run += rsum[gg * Lc + i];
      for (int b = b_lo; b < b_hi; ++b) {
        blk_base[size_t(b) * L + c0 + i] = run;
        run += col[size_t(b) * E];
      }
    }
    __syncthreads();
  }
}

// ---- scatter ----------------------------------------------------------------
// CAP: the positions are pre-capacity rows in tmp_sorted; the capacity kernel
// finishes pair_row for local pairs.
template <bool CAP>
__global__ __launch_bounds__(kDispatchThreads) void scatter_kernel(const int32_t* __restrict__ ids, int64_t n_pairs,
                                                                   int begin, int L, int chunk,
                                                                   const int32_t* __restrict__ blk_base,
                                                                   int32_t* __restrict__ out_sorted,
                                                                   int32_t* __restrict__ pair_row) {
  extern __shared__ int32_t sh[];
  int32_t* run = sh;       // [L]      next row of each local expert for this block
  int32_t* cnt = sh + L;   // [4][L]   pairs of each expert in each wave of this round
  constexpr int kWaves = kDispatchThreads / 64;
  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  for (int i = tid; i < L; i += kDispatchThreads) run[i] = blk_base[size_t(blockIdx.x) * L + i];
  for (int i = tid; i < kWaves * L; i += kDispatchThreads) cnt[i] = 0;
  __syncthreads();
  const int64_t p0 = int64_t(blockIdx.x) * chunk;
  const int64_t p1 = min(n_pairs, p0 + chunk);
  const int bits = bits_for(L);
  for (int64_t base = p0; base < p1; base += kDispatchThreads) {
    const int64_t p = base + tid;
    const bool valid = p < p1;
    const int id = valid ? ids[p] : -1;
    const int li = (id >= begin && id < begin + L) ? id - begin : L;  // L: not local
    const uint64_t m = match_any(uint32_t(li), bits, ~uint64_t(0));
    const uint64_t lower = m & lanemask_lt();
    if (li < L && lower == 0) cnt[wave * L + li] = int(__popcll(m));
    __syncthreads();
    if (li < L) {
      int pos = run[li] + int(__popcll(lower));
      for (int w = 0; w < wave; ++w) pos += cnt[w * L + li];
      out_sorted[pos] = int32_t(p);
      if (!CAP) pair_row[p] = pos;
    } else if (valid) {
      pair_row[p] = -1;
    }
    __syncthreads();
    for (int i = tid; i < L; i += kDispatchThreads) {
      int s = 0;
#pragma unroll
      for (int w = 0; w < kWaves; ++w) {
        s += cnt[w * L + i];
        cnt[w * L + i] = 0;
      }
      run[i] += s;
    }
    __syncthreads();
  }
}

// ---- capacity -----------------------------------------------------------------
// Order-preserving key of a float32 logit (larger logit -> larger key); -0.0
// and +0.0 map to one key because they compare equal.
__device__ __forceinline__ uint32_t logit_key(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7FFFFFFFu) == 0) u = 0;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

constexpr int kCapThreads = 1024;
constexpr int kCapPerThread = 32;  // register-resident keys per thread (segments up to 32768 pairs)
constexpr int kCapWaves = kCapThreads / 64;
constexpr int kCapSlots = kCapPerThread * kCapWaves;  // (register, wave) slots in segment order

// Finds the digit (bits [shift, shift+8) of keys matching `prefix` on `mask`)
// at which the count from the largest digit down reaches `want`; the block's
// histogram is in hist[256].  Returns the digit and leaves in *left how many
// of the wanted keys still have to come from that digit.  Wave 0 does a
// suffix scan over the 256 bins (4 per lane); the result goes through LDS.
__device__ void pick_digit(const int* hist, int want, uint32_t* s_digit, int* s_want) {
  if (threadIdx.x < 64) {
    const int lane = threadIdx.x;
    // lane L owns bins 255-4L .. 252-4L (largest digits first)
    int c[4];
    int tot = 0;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      c[q] = hist[255 - 4 * lane - q];
      tot += c[q];
    }
    const int incl = wave_inclusive_scan(tot);
    int before = incl - tot;  // keys in larger digits than this lane's bins
    // the first lane whose range reaches `want` holds the digit
    const uint64_t hit = __ballot(before < want && incl >= want);
    if (hit != 0 && lane == __ffsll((unsigned long long)hit) - 1) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        if (before + c[q] >= want) {
          *s_digit = uint32_t(255 - 4 * lane - q);
          *s_want = want - before;
          break;
        }
        before += c[q];
      }
    }
  }
}

__global__ __launch_bounds__(kCapThreads) void capacity_kernel(const int32_t* __restrict__ tmp_sorted,
                                                               const int32_t* __restrict__ pre_off,
                                                               const int32_t* __restrict__ offsets,
                                                               const float* __restrict__ topk_logit, int cap,
                                                               int32_t* __restrict__ sorted_pairs,
                                                               int32_t* __restrict__ pair_row) {
  __shared__ int hist[256];
  __shared__ int wsum[kCapThreads / 64];
  __shared__ int slot_cnt[kCapSlots];
  __shared__ uint32_t s_digit;
  __shared__ int s_want;
  const int tid = threadIdx.x;
  const int i = blockIdx.x;
  const int a = pre_off[i];
  const int n = pre_off[i + 1] - a;
  const int out0 = offsets[i];
  const int32_t* seg = tmp_sorted + a;

  if (n <= cap) {
    for (int r = tid; r < n; r += kCapThreads) {
      const int p = seg[r];
      sorted_pairs[out0 + r] = p;
      pair_row[p] = out0 + r;
    }
    return;
  }

  if (cap == 0) {  // nothing is kept
    for (int r = tid; r < n; r += kCapThreads) pair_row[seg[r]] = -1;
    return;
  }

  // element r = j*1024 + tid of the segment sits in this thread's register j
  // (coalesced loads; segment order is j-major, then wave, then lane)
  const int lane = tid & 63, wave = tid >> 6;
  int pid[kCapPerThread];
  uint32_t key[kCapPerThread];
#pragma unroll
  for (int j = 0; j < kCapPerThread; ++j) {
    const int r = j * kCapThreads + tid;
    pid[j] = r < n ? seg[r] : -1;
  }
#pragma unroll
  for (int j = 0; j < kCapPerThread; ++j) key[j] = pid[j] >= 0 ? logit_key(topk_logit[pid[j]]) : 0u;

  // radix select, most significant byte first: threshold key thr of the cap-th
  // largest key, and how many keys equal to thr are still wanted
  uint32_t prefix = 0, mask = 0;
  int want = cap;
  for (int shift = 24; shift >= 0; shift -= 8) {
    for (int b = tid; b < 256; b += kCapThreads) hist[b] = 0;
    __syncthreads();
#pragma unroll
    for (int j = 0; j < kCapPerThread; ++j)
      if (pid[j] >= 0 && (key[j] & mask) == prefix) atomicAdd(&hist[(key[j] >> shift) & 0xFFu], 1);
    __syncthreads();
    pick_digit(hist, want, &s_digit, &s_want);
    __syncthreads();
    prefix |= s_digit << shift;
    mask |= 0xFFu << shift;
    want = s_want;
    __syncthreads();
  }
  const uint32_t thr = prefix;
  const int need_eq = want;  // keys equal to thr kept: the first need_eq in segment (= token) order

  // rank of each key equal to thr among the equal keys before it, in segment order:
  // per (j, wave) counts from ballots, one exclusive scan over the 512 (j, wave) slots
  uint64_t eqm[kCapPerThread];
#pragma unroll
  for (int j = 0; j < kCapPerThread; ++j) {
    eqm[j] = __ballot(pid[j] >= 0 && key[j] == thr);
    if (lane == 0) slot_cnt[j * kCapWaves + wave] = int(__popcll(eqm[j]));
  }
  __syncthreads();
  int tot;
  {
    const int v = tid < kCapSlots ? slot_cnt[tid] : 0;
    const int ex = block_exclusive_scan(v, wsum, &tot);
    if (tid < kCapSlots) slot_cnt[tid] = ex;
  }
  __syncthreads();
  uint64_t keepm[kCapPerThread];
  const uint64_t below = lanemask_lt();
#pragma unroll
  for (int j = 0; j < kCapPerThread; ++j) {
    const bool in = pid[j] >= 0;
    const bool eq = in && key[j] == thr;
    const int eq_before = slot_cnt[j * kCapWaves + wave] + int(__popcll(eqm[j] & below));
    keepm[j] = __ballot(in && (key[j] > thr || (eq && eq_before < need_eq)));
  }
  __syncthreads();
#pragma unroll
  for (int j = 0; j < kCapPerThread; ++j)
    if (lane == 0) slot_cnt[j * kCapWaves + wave] = int(__popcll(keepm[j]));
  __syncthreads();
  {
    const int v = tid < kCapSlots ? slot_cnt[tid] : 0;
    const int ex = block_exclusive_scan(v, wsum, &tot);
    if (tid < kCapSlots) slot_cnt[tid] = ex;
  }
  __syncthreads();
#pragma unroll
  for (int j = 0; j < kCapPerThread; ++j) {
    if (pid[j] < 0) continue;
    if ((keepm[j] >> lane) & 1u) {
      const int pos = out0 + slot_cnt[j * kCapWaves + wave] + int(__popcll(keepm[j] & below));
      sorted_pairs[pos] = pid[j];
      pair_row[pid[j]] = pos;
    } else {
      pair_row[pid[j]] = -1;
    }
  }
}

// ---- gather -----------------------------------------------------------------
// Token-major: one wave per token reads the token's row once and writes it to
// the sorted row of each of its kept local pairs (pair_row), so x is read once
// however many experts a token picked.
constexpr int kGatherTokensPerBlock = 4;

__global__ __launch_bounds__(256) void gather_kernel(const u32x4_t* __restrict__ x, const int32_t* __restrict__ pair_row,
                                                     int64_t ntok, int k, int vec_per_row, u32x4_t* __restrict__ xs) {
  const int lane = threadIdx.x & 63;
  const int64_t t = int64_t(blockIdx.x) * kGatherTokensPerBlock + (threadIdx.x >> 6);
  if (t >= ntok) return;
  const int my_row = lane < k ? pair_row[t * k + lane] : -1;
  // destinations as a bit mask over slots (k <= 32)
  const uint64_t kept = __ballot(my_row >= 0);
  if (kept == 0) return;
  const u32x4_t* src = x + size_t(t) * vec_per_row;
  constexpr int kUnroll = 4;
  for (int c0 = 0; c0 < vec_per_row; c0 += 64 * kUnroll) {
    u32x4_t v[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int c = c0 + u * 64 + lane;
      if (c < vec_per_row) v[u] = src[c];
    }
    for (uint64_t m = kept; m != 0; m &= m - 1) {
      const int j = __ffsll((unsigned long long)m) - 1;
      const int r = __shfl(my_row, j, 64);
      u32x4_t* dst = xs + size_t(r) * vec_per_row;
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) {
        const int c = c0 + u * 64 + lane;
        if (c < vec_per_row) __builtin_nontemporal_store(v[u], dst + c);
      }
    }
  }
}

// ---- place (scatter + gather in one pass, no capacity cut) -------------------
// `split` blocks share one chunk of kDispatchTokens tokens: each ranks all of
// the chunk's pairs exactly like the scatter kernel (so the rows are the same),
// the first also writes sorted_pairs/pair_row, and each copies the rows of its
// share of the chunk's tokens, token-major (one read of x[t], one write per
// kept local pair).  The split is at least 8 (same-box A/B against 4 and 16:
// mixtral-like layer 36.6 us against 36.8 and 37.8) and large enough that a small
// batch still spreads its row copies over ~256 CUs (a decode batch of one
// chunk: 64 blocks of one token each).
constexpr int kMinPlaceSplit = 8, kMaxPlaceSplit = kDispatchTokens;
int place_split(int nblk) {  // power of two, kDispatchTokens divisible by it
  int s = kMinPlaceSplit;
  while (s < kMaxPlaceSplit && int64_t(nblk) * s < 256) s *= 2;
  return s;
}
// With few chunks and experts the place blocks find their own bases: every
// block sums the chunk histograms it needs (no separate scan launch).
constexpr int kFuseEntries = 65536;  // chunks x experts up to which the scan is folded in (gpt-oss-like
                                     // share, 256 x 128: layer -2% against a scan launch)

// FUSED: run[i] = (pairs of local experts before i) + (pairs of local expert i
// in earlier chunks), from the chunk histograms; block 0 also writes counts,
// offsets and the (zero) drop count.  Otherwise blk_base holds them.
template <bool FUSED>
__global__ __launch_bounds__(kDispatchThreads) void place_kernel(const int32_t* __restrict__ ids, int64_t ntok, int k,
                                                                 int begin, int L, const int32_t* __restrict__ blk_base,
                                                                 const int32_t* __restrict__ blk_all, int nblk, int E,
                                                                 int32_t* __restrict__ counts, int32_t* __restrict__ offsets,
                                                                 int64_t* __restrict__ num_dropped,
                                                                 int32_t* __restrict__ sorted_pairs,
                                                                 int32_t* __restrict__ pair_row,
                                                                 const u32x4_t* __restrict__ x, int vec_per_row,
                                                                 u32x4_t* __restrict__ xs, int split) {
  extern __shared__ int32_t sh[];
  constexpr int kWaves = kDispatchThreads / 64;
  int32_t* run = sh;                      // [L]
  int32_t* cnt = sh + L;                  // [kWaves][L]
  int32_t* pos = sh + L * (1 + kWaves);   // [kDispatchTokens * k] row of each of the chunk's pairs, -1 if none
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int chunk = blockIdx.x / split, part = blockIdx.x % split;
  const int64_t t0 = int64_t(chunk) * kDispatchTokens;
  const int ntk = int(min<int64_t>(kDispatchTokens, ntok - t0));
  const int np = ntk * k;
  const int64_t p0 = t0 * k;

  if (FUSED) {
    // per local expert i: total over all chunks and over the chunks before this one;
    // run[i] = (exclusive scan of the totals)[i] + (this expert's pairs in earlier chunks).
    // Experts in groups of up to 256; within a group, thread t takes expert t % Lg and
    // every G-th chunk row from t / Lg (rows read coalesced), partial sums meet in LDS.
    __shared__ int wsum[kWaves];
    __shared__ int ptot[kDispatchThreads], pbef[kDispatchThreads];
    int carry = 0;
    for (int i0 = 0; i0 < L; i0 += kDispatchThreads) {
      const int Lg = min(kDispatchThreads, L - i0);
      const int G = kDispatchThreads / Lg;
      const int il = tid % Lg, g = tid / Lg;
      int tot = 0, before = 0;
      if (g < G) {
        // chunks g, g + G, ...: those before this chunk, then the rest
        const int32_t* col = blk_all + begin + i0 + il;
        const int split = g < chunk ? g + (chunk - g + G - 1) / G * G : g;  // first of this group's chunks >= chunk
        before = column_sum(col, size_t(E), g, min(split, nblk), G);
        tot = before + column_sum(col, size_t(E), split, nblk, G);
      }
      ptot[tid] = tot;
      pbef[tid] = before;
      __syncthreads();
      tot = 0;
      before = 0;
      if (tid < Lg) {
        for (int gg = 0; gg < G; ++gg) {
          tot += ptot[gg * Lg + tid];
          before += pbef[gg * Lg + tid];
        }
      }
      int all;
      const int ex = carry + block_exclusive_scan(tid < Lg ? tot : 0, wsum, &all);
      if (tid < Lg) {
        run[i0 + tid] = ex + before;
        if (blockIdx.x == 0) {
          offsets[i0 + tid] = ex;
          counts[begin + i0 + tid] = tot;
        }
      }
      carry += all;
    }
    if (blockIdx.x == 0) {
      if (tid == 0) {
        offsets[L] = carry;
        if (num_dropped != nullptr) *num_dropped = 0;
      }
      // experts outside the local range (their totals were not needed above), grouped like the local ones
      for (int e0 = 0; e0 < E; e0 += kDispatchThreads) {
        const int Eg = min(kDispatchThreads, E - e0);
        const int G = kDispatchThreads / Eg;
        const int el = tid % Eg, g = tid / Eg;
        const int e = e0 + el;
        const bool outside = e < begin || e >= begin + L;
        int tot = 0;
        if (g < G && outside) tot = column_sum(blk_all + e, size_t(E), g, nblk, G);
        __syncthreads();
        ptot[tid] = tot;
        __syncthreads();
        if (tid < Eg && (e0 + tid < begin || e0 + tid >= begin + L)) {
          int s = 0;
          for (int gg = 0; gg < G; ++gg) s += ptot[gg * Eg + tid];
          counts[e0 + tid] = s;
        }
      }
    }
  } else {
    for (int q = tid; q < L; q += kDispatchThreads) run[q] = blk_base[size_t(chunk) * L + q];
  }
  for (int q = tid; q < kWaves * L; q += kDispatchThreads) cnt[q] = 0;
  __syncthreads();
  const int bits = bits_for(L);
  for (int base = 0; base < np; base += kDispatchThreads) {
    const int r = base + tid;
    const bool valid = r < np;
    const int id = valid ? ids[p0 + r] : -1;
    const int li = (id >= begin && id < begin + L) ? id - begin : L;  // L: not local
    const uint64_t m = match_any(uint32_t(li), bits, ~uint64_t(0));
    const uint64_t lower = m & lanemask_lt();
    if (li < L && lower == 0) cnt[wave * L + li] = int(__popcll(m));
    __syncthreads();
    if (li < L) {
      int ps = run[li] + int(__popcll(lower));
      for (int w = 0; w < wave; ++w) ps += cnt[w * L + li];
      pos[r] = ps;
      if (part == 0) {
        sorted_pairs[ps] = int32_t(p0 + r);
        pair_row[p0 + r] = ps;
      }
    } else if (valid) {
      pos[r] = -1;
      if (part == 0) pair_row[p0 + r] = -1;
    }
    __syncthreads();
    for (int q = tid; q < L; q += kDispatchThreads) {
      int sum = 0;
#pragma unroll
      for (int w = 0; w < kWaves; ++w) {
        sum += cnt[w * L + q];
        cnt[w * L + q] = 0;
      }
      run[q] += sum;
    }
    __syncthreads();
  }

  // copy this part's tokens (tpp of the chunk): with at least one token per wave each
  // wave takes whole tokens, else the waves on a token split its columns
  const int tpp = kDispatchTokens / split;
  const int wpt = tpp >= kWaves ? 1 : kWaves / tpp;  // waves per token
  const int tpw = tpp >= kWaves ? tpp / kWaves : 1;  // tokens per wave
  const int tw0 = part * tpp + (tpp >= kWaves ? wave * tpw : wave / wpt);
  const int cper = (vec_per_row + wpt - 1) / wpt;
  const int c_lo = (wave % wpt) * cper, c_hi = min(vec_per_row, c_lo + cper);
  constexpr int kUnroll = 4;
  for (int tt = tw0; tt < tw0 + tpw && tt < ntk; ++tt) {
    const int my_row = lane < k ? pos[tt * k + lane] : -1;
    const uint64_t kept = __ballot(my_row >= 0);
    if (kept == 0) continue;
    const u32x4_t* src = x + size_t(t0 + tt) * vec_per_row;
    for (int c0 = c_lo; c0 < c_hi; c0 += 64 * kUnroll) {
      u32x4_t v[kUnroll];
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) {
        const int c = c0 + u * 64 + lane;
        if (c < c_hi) v[u] = src[c];
      }
      for (uint64_t mk = kept; mk != 0; mk &= mk - 1) {
        const int j = __ffsll((unsigned long long)mk) - 1;
        const int rrow = __shfl(my_row, j, 64);
        u32x4_t* dst = xs + size_t(rrow) * vec_per_row;
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
          const int c = c0 + u * 64 + lane;
          if (c < c_hi) dst[c] = v[u];
        }
      }
    }
  }
}

}  // namespace

moe_status launch_dispatch(const DispatchArgs& a) {
  const moe_layer_desc* d = a.d;
  const int64_t n = d->num_tokens * d->top_k;
  const int chunk = kDispatchTokens * d->top_k;  // pairs per chunk
  const int nblk = int(dispatch_blocks(d->num_tokens));
  const int E = d->num_experts, L = d->local_count, begin = d->local_begin;
  const bool cap = a.capacity >= 0;
  const int vec_per_row = int(size_t(d->hidden) * dtype_bytes(d->dtype) / 16);

  if (!a.counts_ready) {
    MOE_LAUNCH("dispatch_count", count_kernel, dim3(nblk), dim3(kDispatchThreads), size_t(E) * 4, a.s, a.topk_ids, n, E,
               chunk, a.scr.blk_all);
  }
  // without a capacity cut and with a small chunk-histogram table the place kernel finds its own bases
  const bool fused = !cap && int64_t(nblk) * E <= kFuseEntries;
  if (!fused) {
    MOE_LAUNCH("dispatch_scan", scan_kernel, dim3(1), dim3(kScanThreads), size_t(E + L + 1) * 4, a.s, a.scr.blk_all,
               nblk, E, begin, L, a.capacity, a.counts, a.offsets, a.scr.pre_off, a.scr.blk_base, a.num_dropped);
  }
  if (cap) {
    const size_t scat_lds = size_t(L) * (1 + kDispatchThreads / 64) * 4;
    MOE_LAUNCH("dispatch_scatter", scatter_kernel<true>, dim3(nblk), dim3(kDispatchThreads), scat_lds, a.s, a.topk_ids, n,
               begin, L, chunk, a.scr.blk_base, a.scr.tmp_sorted, a.pair_row);
    MOE_LAUNCH("dispatch_capacity", capacity_kernel, dim3(L), dim3(kCapThreads), 0, a.s, a.scr.tmp_sorted, a.scr.pre_off,
               a.offsets, a.topk_logit, int(a.capacity), a.sorted_pairs, a.pair_row);
    const dim3 grid(unsigned((d->num_tokens + kGatherTokensPerBlock - 1) / kGatherTokensPerBlock));
    MOE_LAUNCH("dispatch_gather", gather_kernel, grid, dim3(256), 0, a.s, static_cast<const u32x4_t*>(a.x), a.pair_row,
               d->num_tokens, d->top_k, vec_per_row, static_cast<u32x4_t*>(a.x_sorted));
  } else {
    const size_t lds = (size_t(L) * (1 + kDispatchThreads / 64) + size_t(chunk)) * 4;
    auto kern = fused ? place_kernel<true> : place_kernel<false>;
    if (lds > 65536) {
      const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                               hipFuncAttributeMaxDynamicSharedMemorySize, int(lds));
      if (e != hipSuccess) return set_error(MOE_ERR_HIP, "dispatch_place: LDS attribute: %s", hipGetErrorString(e));
    }
    const int split = place_split(nblk);
    MOE_LAUNCH("dispatch_place", kern, dim3(unsigned(nblk) * split), dim3(kDispatchThreads), lds, a.s,
               a.topk_ids, d->num_tokens, d->top_k, begin, L, a.scr.blk_base, a.scr.blk_all, nblk, E, a.counts,
               a.offsets, a.num_dropped, a.sorted_pairs, a.pair_row, static_cast<const u32x4_t*>(a.x), vec_per_row,
               static_cast<u32x4_t*>(a.x_sorted), split);
  }
  return MOE_OK;
}

}  // namespace moe
