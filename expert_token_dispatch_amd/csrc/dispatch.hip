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
//             that chunk's pairs (range sums over chunks, then prefixes); when
//             the chunk histogram table is small (chunks x experts <= 65536)
//             the place or scatter kernel's blocks each sum the columns they
//             need instead, so no scan launch sits after the router;
//   scatter   (with a capacity limit) per block again, in rounds of 256 pairs:
//             the rank of a pair among equal experts is its rank within its
//             wave (match-any + popcount of lower lanes) plus the counts of
//             earlier waves and earlier rounds -- no atomics, so the order is
//             deterministic; each pair's logit key goes beside it;
//   capacity  (only with a limit) per 4096-row slice of an expert's segment: a
//             leading-digit histogram of each slice, then a radix select of the
//             C-th largest key (logit desc, then token asc) and a stable
//             compaction of the slice (see the capacity section below);
//   place     without a capacity cut, scatter and row copy in one kernel:
//             ranks as in scatter, then token-major copies (one read of x[t],
//             one write per kept local pair, 16-byte vectors);
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

// The capacity cut works on slices of kCapSlice consecutive pre-capacity rows of
// one expert's segment; an upper bound on their number over all local experts.
constexpr int kCapSlice = 4096;
constexpr int kCapBins = 4096;  // 12-bit radix digits
int64_t cap_slices_max(const moe_layer_desc* d) {
  return (d->num_tokens * d->top_k + kCapSlice - 1) / kCapSlice + d->local_count;
}

size_t dispatch_scratch_bytes(const moe_layer_desc* d) {
  const int64_t n = d->num_tokens * d->top_k;
  const int64_t nblk = dispatch_blocks(d->num_tokens);
  size_t b = 0;
  b += align_up(size_t(nblk) * d->num_experts * 4, 256);
  b += align_up(size_t(nblk) * d->local_count * 4, 256);
  if (d->capacity_factor > 0) {
    b += 3 * align_up(size_t(n) * 4, 256);
    b += align_up(size_t(d->local_count + 1) * 4, 256);
    b += align_up(size_t(cap_slices_max(d)) * 16, 256);
    b += align_up(size_t(cap_slices_max(d)) * kCapBins * 4, 256);
  }
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
  const int64_t n = d->num_tokens * d->top_k;
  if (d->capacity_factor > 0) {
    s.tmp_sorted = reinterpret_cast<int32_t*>(p);
    p += align_up(size_t(n) * 4, 256);
    s.tmp_key = reinterpret_cast<uint32_t*>(p);
    p += align_up(size_t(n) * 4, 256);
    s.tmp_final = reinterpret_cast<int32_t*>(p);
    p += align_up(size_t(n) * 4, 256);
    s.slice_off = reinterpret_cast<int32_t*>(p);
    p += align_up(size_t(d->local_count + 1) * 4, 256);
    s.slice_desc = reinterpret_cast<int32_t*>(p);
    p += align_up(size_t(cap_slices_max(d)) * 16, 256);
    s.slice_hist = reinterpret_cast<uint32_t*>(p);
  }
  return s;
}

namespace {

// The descriptors of local expert i's capacity slices: {its first slice, pre-capacity
// segment start, segment length, first kept row}, one per slice.
__device__ __forceinline__ void write_slice_desc(int32_t* __restrict__ slice_desc, int first, int pre, int n, int out0) {
  const int ns = (n + kCapSlice - 1) / kCapSlice;
  for (int q = 0; q < ns; ++q) reinterpret_cast<int4*>(slice_desc)[first + q] = make_int4(first, pre, n, out0);
}

__device__ __forceinline__ int bits_for(int maxval) { return 32 - __clz(maxval); }

// Sum of col[b * stride] for b = b_lo, b_lo + step, ... < b_hi, eight loads in flight
// (integer sums: the grouping does not change the result).  Sixteen in flight was
// slower (the capacity path's fused scatter: 15.9 -> 25.5 us; every block reads the
// same rows, so more requests only queue at the same L2 channels).
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

// Inclusive prefix sum over the wave (modulo 2^32) by DPP lane moves, no LDS
// round trips: Hillis-Steele within each row of 16 lanes (row_shr 1, 2, 4, 8; a
// lane shifted in from outside its row reads 0), then the last lane of row 0 is
// added to row 1 and that of row 2 to row 3 (row_bcast:15), then the last lane of
// row 1 to rows 2 and 3 (row_bcast:31).  The cross-lane operations are those of
// AMD's GCN3/Vega ISA documents (DPP_CTRL row_shr, row_bcast15, row_bcast31).
__device__ __forceinline__ uint32_t wave_scan_u32(uint32_t v) {
  int x = int(v);
  x = int(uint32_t(x) + uint32_t(__builtin_amdgcn_update_dpp(0, x, 0x111, 0xf, 0xf, true)));  // row_shr:1
  x = int(uint32_t(x) + uint32_t(__builtin_amdgcn_update_dpp(0, x, 0x112, 0xf, 0xf, true)));  // row_shr:2
  x = int(uint32_t(x) + uint32_t(__builtin_amdgcn_update_dpp(0, x, 0x114, 0xf, 0xf, true)));  // row_shr:4
  x = int(uint32_t(x) + uint32_t(__builtin_amdgcn_update_dpp(0, x, 0x118, 0xf, 0xf, true)));  // row_shr:8
  x = int(uint32_t(x) + uint32_t(__builtin_amdgcn_update_dpp(0, x, 0x142, 0xa, 0xf, false)));  // row_bcast:15
  x = int(uint32_t(x) + uint32_t(__builtin_amdgcn_update_dpp(0, x, 0x143, 0xc, 0xf, false)));  // row_bcast:31
  return uint32_t(x);
}

// Exclusive scan over the block (modulo 2^32); *total receives the block sum.
// `wsum` holds one word per wave.  Every thread of the block must call it.
__device__ uint32_t block_exclusive_scan_u32(uint32_t v, uint32_t* wsum, uint32_t* total) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int nw = blockDim.x >> 6;
  const uint32_t incl = wave_scan_u32(v);
  if (lane == 63) wsum[wave] = incl;
  __syncthreads();
  if (wave == 0) {
    uint32_t s = lane < nw ? wsum[lane] : 0u;
    s = wave_scan_u32(s);
    if (lane < nw) wsum[lane] = s;
  }
  __syncthreads();
  const uint32_t before = wave > 0 ? wsum[wave - 1] : 0u;
  *total = wsum[nw - 1];
  __syncthreads();
  return before + incl - v;
}

// The same for non-negative int sums that fit an int.
__device__ int block_exclusive_scan(int v, int* wsum, int* total) {
  uint32_t t;
  const uint32_t ex = block_exclusive_scan_u32(uint32_t(v), reinterpret_cast<uint32_t*>(wsum), &t);
  *total = int(t);
  return int(ex);
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
constexpr int kScanCache = 32;   // chunk counts a thread keeps in registers between the two passes

__global__ __launch_bounds__(kScanThreads) void scan_kernel(const int32_t* __restrict__ blk_all, int nblk, int E,
                                                            int begin, int L, int64_t cap, int32_t* __restrict__ counts,
                                                            int32_t* __restrict__ offsets,
                                                            int32_t* __restrict__ blk_base,
                                                            int32_t* __restrict__ slice_off,
                                                            int32_t* __restrict__ slice_desc,
                                                            int64_t* __restrict__ num_dropped) {
  extern __shared__ int32_t sh[];
  int32_t* cnt = sh;          // [E]
  int32_t* pre = sh + E;      // [L + 1]
  __shared__ int wsum[kScanThreads / 64];
  __shared__ long long dsum[kScanThreads / 64];
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;

  __shared__ int rsum[kScanThreads];
  // When every column fits one pass (E <= 1024) and a thread's range of chunks fits
  // kScanCache registers, the thread loads its counts once, all in flight, and keeps
  // them for the per-chunk bases below (the histogram was just written by another
  // kernel, so each dependent round of loads costs a trip past this XCD's L2).
  const int G1 = min(kScanGroups, kScanThreads / max(1, min(E, kScanThreads)));
  const int per1 = (nblk + G1 - 1) / G1;
  const bool cached = E <= kScanThreads && per1 <= kScanCache;
  int v[kScanCache];
  if (cached) {
    const int e = tid % E, g = tid / E;
    int sum = 0;
    if (g < G1) {
      const int b_lo = min(nblk, g * per1), b_hi = min(nblk, b_lo + per1);
#pragma unroll
      for (int u = 0; u < kScanCache; ++u) v[u] = b_lo + u < b_hi ? blk_all[size_t(b_lo + u) * E + e] : 0;
#pragma unroll
      for (int u = 0; u < kScanCache; ++u) sum += v[u];
      rsum[tid] = sum;
    }
    __syncthreads();
    if (tid < E) {
      int tot = 0;
      for (int gg = 0; gg < G1; ++gg) tot += rsum[gg * E + tid];
      cnt[tid] = tot;
      counts[tid] = tot;
    }
    __syncthreads();
  }
  // totals per expert: columns in groups of up to 1024; thread t sums column
  // t % Ec over a contiguous range of chunks (coalesced across the columns)
  for (int c0 = 0; !cached && c0 < E; c0 += kScanThreads) {
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

  // segment offsets before (pre) and after (offsets) the capacity cut; with a cut,
  // also the first capacity slice of each expert
  int carry_pre = 0, carry_post = 0, carry_sl = 0;
  long long dropped = 0;
  for (int i0 = 0; i0 < L; i0 += kScanThreads) {
    const int i = i0 + tid;
    const int n = i < L ? cnt[begin + i] : 0;
    const int kept = cap < 0 ? n : int(min<int64_t>(n, cap));
    dropped += n - kept;
    int tot_n, tot_k, tot_s = 0, ex_s = 0;
    const int ex_n = block_exclusive_scan(n, wsum, &tot_n);
    const int ex_k = block_exclusive_scan(kept, wsum, &tot_k);
    if (cap >= 0) ex_s = block_exclusive_scan((n + kCapSlice - 1) / kCapSlice, wsum, &tot_s);
    if (i < L) {
      pre[i] = carry_pre + ex_n;
      offsets[i] = carry_post + ex_k;
      if (cap >= 0) {
        slice_off[i] = carry_sl + ex_s;
        write_slice_desc(slice_desc, carry_sl + ex_s, carry_pre + ex_n, n, carry_post + ex_k);
      }
    }
    carry_pre += tot_n;
    carry_post += tot_k;
    carry_sl += tot_s;
  }
  if (tid == 0) {
    pre[L] = carry_pre;
    offsets[L] = carry_post;
    if (cap >= 0) slice_off[L] = carry_sl;
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
  if (cached) {
    // the first pass's threads and registers: thread (column e, group g) of a local e
    const int e = tid % E, g = tid / E;
    if (g < G1 && e >= begin && e < begin + L) {
      const int b_lo = min(nblk, g * per1), b_hi = min(nblk, b_lo + per1);
      int run = pre[e - begin];
      for (int gg = 0; gg < g; ++gg) run += rsum[gg * E + e];
#pragma unroll
      for (int u = 0; u < kScanCache; ++u) {
        if (b_lo + u < b_hi) blk_base[size_t(b_lo + u) * L + e - begin] = run;
        run += v[u];
      }
    }
    return;
  }
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

// ---- bases of one chunk without a scan launch ----------------------------------
// For small chunk-histogram tables a block finds the bases of its own chunk:
// run[i] = (pairs of the local experts before i) + (pairs of local expert i in
// the chunks before this one), in pre-capacity rows.  Experts go in groups of up
// to 256; within a group thread t takes expert t % Lg and every G-th chunk row from
// t / Lg (rows read coalesced), and the partial sums meet in LDS.  Block 0 also
// writes counts [E] (the experts outside the local range one per block, its threads
// splitting the column: one block summing them all would be the last to finish),
// the segment offsets (after the cut when cap >= 0) and the drop count; with a cut,
// also the first capacity slice of each expert and the slices' descriptors.
// Every thread of the block must call it.
__device__ void chunk_bases(const int32_t* __restrict__ blk_all, int nblk, int E, int begin, int L, int chunk,
                            int64_t cap, int32_t* run, int32_t* __restrict__ counts, int32_t* __restrict__ offsets,
                            int32_t* __restrict__ slice_off, int32_t* __restrict__ slice_desc,
                            int64_t* __restrict__ num_dropped) {
  constexpr int kWaves = kDispatchThreads / 64;
  __shared__ int wsum[kWaves];
  __shared__ int ptot[kDispatchThreads], pbef[kDispatchThreads];
  const int tid = threadIdx.x;
  const bool first = blockIdx.x == 0;
  int carry = 0, carry_post = 0, carry_sl = 0, dropped = 0;
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
      if (first) counts[begin + i0 + tid] = tot;
    }
    if (cap < 0) {
      if (first && tid < Lg) offsets[i0 + tid] = ex;
    } else {
      const int kept = int(min<int64_t>(tot, cap));
      dropped += tot - kept;
      int all_k, all_s;
      const int ex_k = carry_post + block_exclusive_scan(kept, wsum, &all_k);
      const int ex_s = carry_sl + block_exclusive_scan((tot + kCapSlice - 1) / kCapSlice, wsum, &all_s);
      if (first && tid < Lg) {
        offsets[i0 + tid] = ex_k;
        slice_off[i0 + tid] = ex_s;
        write_slice_desc(slice_desc, ex_s, ex, tot, ex_k);
      }
      carry_post += all_k;
      carry_sl += all_s;
    }
    carry += all;
  }
  if (first) {
    int all_d = 0;
    if (cap >= 0) (void)block_exclusive_scan(dropped, wsum, &all_d);
    if (tid == 0) {
      offsets[L] = cap < 0 ? carry : carry_post;
      if (cap >= 0) slice_off[L] = carry_sl;
      if (num_dropped != nullptr) *num_dropped = all_d;
    }
  }
  for (int e = int(blockIdx.x); e < E; e += int(gridDim.x)) {
    if (e >= begin && e < begin + L) continue;
    int tot = 0;
    for (int b = tid; b < nblk; b += kDispatchThreads) tot += blk_all[size_t(b) * E + e];
    int all;
    (void)block_exclusive_scan(tot, wsum, &all);
    if (tid == 0) counts[e] = all;
  }
}

// ---- scatter ----------------------------------------------------------------
// Order-preserving key of a float32 logit (larger logit -> larger key); -0.0
// and +0.0 map to one key because they compare equal.
__device__ __forceinline__ uint32_t logit_key(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7FFFFFFFu) == 0) u = 0;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// With a capacity limit: the positions are pre-capacity rows in tmp_sorted, with
// each pair's logit key beside it in tmp_key (so the capacity cut reads its
// segment's keys in order); pair_row holds the pre-capacity row until the gather
// resolves it.  FUSED: the block finds its own bases (chunk_bases), else blk_base
// holds them.
template <bool FUSED>
__global__ __launch_bounds__(kDispatchThreads) void scatter_kernel(const int32_t* __restrict__ ids, int64_t n_pairs,
                                                                   int begin, int L, int chunk,
                                                                   const int32_t* __restrict__ blk_base,
                                                                   const int32_t* __restrict__ blk_all, int nblk, int E,
                                                                   int64_t cap, int32_t* __restrict__ counts,
                                                                   int32_t* __restrict__ offsets,
                                                                   int32_t* __restrict__ slice_off,
                                                                   int32_t* __restrict__ slice_desc,
                                                                   int64_t* __restrict__ num_dropped,
                                                                   int32_t* __restrict__ out_sorted,
                                                                   int32_t* __restrict__ pair_row,
                                                                   const float* __restrict__ topk_logit,
                                                                   uint32_t* __restrict__ tmp_key) {
  extern __shared__ int32_t sh[];
  int32_t* run = sh;       // [L]      next row of each local expert for this block
  int32_t* cnt = sh + L;   // [4][L]   pairs of each expert in each wave of this round
  constexpr int kWaves = kDispatchThreads / 64;
  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  if (FUSED) {
    chunk_bases(blk_all, nblk, E, begin, L, int(blockIdx.x), cap, run, counts, offsets, slice_off,
                slice_desc, num_dropped);
  } else {
    for (int i = tid; i < L; i += kDispatchThreads) run[i] = blk_base[size_t(blockIdx.x) * L + i];
  }
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
      pair_row[p] = pos;
      tmp_key[pos] = logit_key(topk_logit[p]);
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
// The cut keeps the cap pairs with the largest keys of each expert over capacity
// (logit descending, equal keys in segment = token order).  Its blocks each take
// one slice of kCapSlice consecutive pre-capacity rows of one expert (the slice
// descriptors are written with the offsets), so a hot expert's segment is spread
// over several CUs:
//   cap_hist    per slice of an expert over capacity, the histogram of the keys'
//               leading 12-bit digit (bits 31..20);
//   cap_select  per slice: an expert within capacity copies its rows; otherwise the
//               block takes the whole segment's keys into registers, sums the
//               slices' histograms, and finishes the radix select of the cap-th
//               largest key from them (two 10-bit digits over the few keys that
//               share the leading one), redundantly in every block of the expert
//               (no grid-wide wait); then it ranks the rows of its own slice from
//               one scan over per-wave counts of the earlier slices and ballot
//               counts of its own (register, wave) slots.
constexpr int kCapThreads = 1024;
constexpr int kCapPerThread = 32;  // register-resident keys per thread (segments up to 32768 pairs)
constexpr int kCapWaves = kCapThreads / 64;
constexpr int kSliceRegs = kCapSlice / kCapThreads;   // a slice is registers [4s, 4s + 4) of the segment
constexpr int kCapCopies = 8;                         // counter copies per digit (lane mod 8)
constexpr int kCapWords = kCapBins * kCapCopies;      // 128 KB of LDS
constexpr size_t kCapLds = size_t(kCapWords + 1) * 4;  // cap_hist: the counters and one word
constexpr int kLowBins = 1024;                          // 10-bit digits of the select's last two passes
constexpr int kRankSlots = kCapWaves + kSliceRegs * kCapWaves;  // earlier-slice sums per wave, then the slice's slots
static_assert(kRankSlots > 64 && kRankSlots <= 128, "one wave scans the rank slots, two per lane");
constexpr size_t kSelLds = size_t(kCapBins + 2 * kLowBins + kRankSlots + kCapWaves + 3) * 4;
static_assert(kCapSlice % kCapThreads == 0 && kCapPerThread % kSliceRegs == 0, "slices are whole register groups");
static_assert(kCapBins == 4 * kCapThreads, "each thread owns four digits of a pass");

// Digit counts of a radix-select pass are gathered in hist[8 d + c]: copy c of
// digit d (lane l adds to copy l mod 8, so the lanes of a wave that share a digit
// spread over eight words).  compact_counts sums the copies into cnt[d]: lanes take
// consecutive 16-byte chunks (chunk q holds four copies of digit q / 2, so a wave's
// reads cover the banks without conflicts; per-thread runs of 128 bytes made every
// read a 32-way bank conflict, ~7k cycles per pass) and neighbouring lanes add their
// halves.  nbins is a multiple of 32, so whole waves run each round.
__device__ void compact_counts(const uint32_t* hist, int nbins, uint32_t* cnt) {
  const u32x4_t* h4 = reinterpret_cast<const u32x4_t*>(hist);
  for (int q = threadIdx.x; q < 2 * nbins; q += blockDim.x) {
    const u32x4_t x = h4[q];
    uint32_t v = (x[0] + x[1]) + (x[2] + x[3]);
    v += uint32_t(__shfl_xor(int(v), 1, 64));
    if ((q & 1) == 0) cnt[q >> 1] = v;
  }
}

// The digit of a radix-select pass from cnt[d], the candidate keys of digit d: the
// wanted key is the want-th largest candidate.  `pad` keys counted in digit 0 are not
// candidates (padding) and are taken off.  One wave walks the digits from the top,
// 256 per step (lane l holds digits top-1-4l .. top-4-4l: one 16-byte read, lanes
// contiguous), with a DPP scan of the lanes' sums; the lane whose digits reach `want`
// leaves the digit in *s_digit and, in *s_want, how many of the wanted keys still have
// to come from it.  nbins is a multiple of 256.  Called by one whole wave; the block
// waits at a barrier meanwhile (a block-wide scan here cost three barriers a pass).
__device__ void wave_pick_digit(const uint32_t* cnt, int nbins, int want, uint32_t pad, uint32_t* s_digit,
                                int* s_want) {
  const int lane = threadIdx.x & 63;
  uint32_t before = 0;  // candidates in larger digits (the same in every lane)
  for (int top = nbins; top > 0; top -= 256) {
    const u32x4_t x = reinterpret_cast<const u32x4_t*>(cnt + top - 4 - 4 * lane)[0];
    uint32_t c[4] = {x[3], x[2], x[1], x[0]};  // digits top-1-4l, ..., top-4-4l
    if (top - 4 - 4 * lane == 0) c[3] -= pad;
    const uint32_t tot = (c[0] + c[1]) + (c[2] + c[3]);
    const uint32_t incl = wave_scan_u32(tot);
    const uint32_t all = uint32_t(__builtin_amdgcn_readlane(int(incl), 63));
    if (before + all >= uint32_t(want)) {
      uint32_t ex = before + incl - tot;
      if (ex < uint32_t(want) && ex + tot >= uint32_t(want)) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          if (ex + c[q] >= uint32_t(want)) {
            *s_digit = uint32_t(top - 1 - 4 * lane - q);
            *s_want = int(uint32_t(want) - ex);
            break;
          }
          ex += c[q];
        }
      }
      return;
    }
    before += all;
  }
}

// Capacity block b's slice: false when b is past the last slice (slice_off[L]);
// else its descriptor {expert's first slice, segment start, length, first kept row}.
// Both loads are in flight together: the grid has one block per descriptor entry, so
// entry b is in bounds even when it is not in use (its contents are then ignored).
__device__ __forceinline__ bool slice_of(const int32_t* __restrict__ slice_off, const int32_t* __restrict__ slice_desc,
                                         int L, int b, int4* dsc) {
  const int total = slice_off[L];
  *dsc = reinterpret_cast<const int4*>(slice_desc)[b];
  return b < total;
}

// Leading-digit histogram of one slice of an expert over capacity:
// slice_hist[b][d] = keys of slice b whose bits 31..20 are d.
__global__ __launch_bounds__(kCapThreads) void cap_hist_kernel(const uint32_t* __restrict__ tmp_key,
                                                               const int32_t* __restrict__ slice_off,
                                                               const int32_t* __restrict__ slice_desc, int L, int cap,
                                                               uint32_t* __restrict__ slice_hist) {
  // all of the block's LDS is dynamic, so the counters start at offset 0 (aligned 16-byte accesses)
  extern __shared__ int32_t sh[];
  uint32_t* hist = reinterpret_cast<uint32_t*>(sh);  // [kCapWords]
  const int tid = threadIdx.x;
  const int b = blockIdx.x;
  int4 dsc;
  if (!slice_of(slice_off, slice_desc, L, b, &dsc)) return;
  const int a = dsc.y, n = dsc.z;
  if (n <= cap) return;
  const int r0 = (b - dsc.x) * kCapSlice;
  uint32_t key[kSliceRegs];
#pragma unroll
  for (int u = 0; u < kSliceRegs; ++u) {
    const int r = r0 + u * kCapThreads + tid;
    key[u] = r < n ? tmp_key[a + r] : 0u;
  }
  u32x4_t* hist4 = reinterpret_cast<u32x4_t*>(hist);
  const u32x4_t zero4 = {0u, 0u, 0u, 0u};
  for (int q = tid; q < kCapWords / 4; q += kCapThreads) hist4[q] = zero4;
  __syncthreads();
  const int copy = tid & (kCapCopies - 1);
#pragma unroll
  for (int u = 0; u < kSliceRegs; ++u)
    if (r0 + u * kCapThreads + tid < n) atomicAdd(&hist[(key[u] >> 20) * kCapCopies + copy], 1u);
  __syncthreads();
  compact_counts(hist, kCapBins, slice_hist + size_t(b) * kCapBins);
}

// One slice of an expert's pre-capacity segment, rows [r0, r0 + kCapSlice) of
// tmp_sorted (pair ids, in pair order) and tmp_key (their logit keys), segment
// [a, a + n).  Writes sorted_pairs for the slice's kept pairs (at their rows from
// the expert's first kept row out0) and, for every row of the slice, its final row
// or -1 in tmp_final; the gather resolves pair_row through tmp_final.
// A kept key's row is (keys above the threshold before it) + min(keys equal to it
// before it, equal keys kept), from one scan over the (register, wave) slots of the
// slices up to this one, of packed counts (keys above the threshold in the low half,
// equal in the high half), and the lanes below the key in its slot.
__global__ __launch_bounds__(kCapThreads) void cap_select_kernel(const int32_t* __restrict__ tmp_sorted,
                                                                 const uint32_t* __restrict__ tmp_key,
                                                                 const int32_t* __restrict__ slice_off,
                                                                 const int32_t* __restrict__ slice_desc,
                                                                 const uint32_t* __restrict__ slice_hist, int L,
                                                                 int cap, int32_t* __restrict__ sorted_pairs,
                                                                 int32_t* __restrict__ tmp_final) {
  extern __shared__ int32_t sh[];
  uint32_t* cnt = reinterpret_cast<uint32_t*>(sh);   // [kCapBins]   leading-digit counts
  uint32_t* low = cnt + kCapBins;                    // [2][kLowBins] counts of the two 10-bit passes
  uint32_t* slot_cnt = low + 2 * kLowBins;           // [kRankSlots]
  uint32_t* wsum = slot_cnt + kRankSlots;            // [kCapWaves]
  uint32_t& s_digit = wsum[kCapWaves];
  int& s_want = reinterpret_cast<int*>(wsum)[kCapWaves + 1];
  const int tid = threadIdx.x;
  const int b = blockIdx.x;
  int4 dsc;
  if (!slice_of(slice_off, slice_desc, L, b, &dsc)) return;
  const int s0 = dsc.x, a = dsc.y, n = dsc.z, out0 = dsc.w;
  const int sl = b - s0;
  const int r0 = sl * kCapSlice;
  const int32_t* seg = tmp_sorted + a;

  if (n <= cap) {  // every row kept, in place
    int32_t v[kSliceRegs];
#pragma unroll
    for (int u = 0; u < kSliceRegs; ++u) {
      const int r = r0 + u * kCapThreads + tid;
      v[u] = r < n ? seg[r] : 0;
    }
#pragma unroll
    for (int u = 0; u < kSliceRegs; ++u) {
      const int r = r0 + u * kCapThreads + tid;
      if (r < n) {
        sorted_pairs[out0 + r] = v[u];
        tmp_final[a + r] = out0 + r;
      }
    }
    return;
  }
  if (cap == 0) {  // nothing is kept
#pragma unroll
    for (int u = 0; u < kSliceRegs; ++u) {
      const int r = r0 + u * kCapThreads + tid;
      if (r < n) tmp_final[a + r] = -1;
    }
    return;
  }

  // element r = j*1024 + tid of the segment sits in this thread's register j
  // (coalesced loads; segment order is j-major, then wave, then lane).  Rows past the
  // segment hold key 0 as padding; the digit passes skip registers with no row of the
  // segment (j*1024 >= n, a wave-uniform test), and the rest's npad padding keys are
  // candidates while the digits chosen so far are all 0, always in digit 0, which the
  // digit pick takes off.  A padding key is never above a threshold and comes after
  // every real row in segment order, so it never takes a kept row.
  const int lane = tid & 63, wave = tid >> 6;
  const int nreg = (n + kCapThreads - 1) / kCapThreads;
  const uint32_t npad = uint32_t(nreg * kCapThreads - n);
  const uint32_t* kseg = tmp_key + a;
  uint32_t key[kCapPerThread];
#pragma unroll
  for (int j = 0; j < kCapPerThread; ++j) {
    const uint32_t r = uint32_t(j * kCapThreads + tid);
    key[j] = r < uint32_t(n) ? kseg[r] : 0u;
  }

  // leading digit: the slices' histograms summed (thread t takes digits 4t .. 4t+3),
  // no padding counted; the counters of the later passes cleared meanwhile
  {
    const int s1 = s0 + nreg / kSliceRegs + (nreg % kSliceRegs != 0);  // the expert's slices: ceil(n / kCapSlice)
    u32x4_t acc = {0u, 0u, 0u, 0u};
#pragma unroll 4
    for (int s = s0; s < s1; ++s) {
      const u32x4_t h = reinterpret_cast<const u32x4_t*>(slice_hist + size_t(s) * kCapBins)[tid];
      acc[0] += h[0];
      acc[1] += h[1];
      acc[2] += h[2];
      acc[3] += h[3];
    }
    reinterpret_cast<u32x4_t*>(cnt)[tid] = acc;
    for (int q = tid; q < 2 * kLowBins; q += kCapThreads) low[q] = 0u;
  }
  __syncthreads();
  if (wave == 0) wave_pick_digit(cnt, kCapBins, cap, 0u, &s_digit, &s_want);
  __syncthreads();
  uint32_t prefix = s_digit << 20, mask = 0xFFF00000u;
  int want = s_want;
  // the remaining 20 bits in two 10-bit digits over the keys that share the digits so
  // far.  Those are few, so each pass counts into one word per digit (ties of many
  // equal keys only make their atomics queue); the next pass has counters of its own,
  // so the digit and count read here are not overwritten before every wave has them.
#pragma unroll
  for (int ps = 0; ps < 2; ++ps) {
    const int shift = 10 - 10 * ps;
    uint32_t* h = low + ps * kLowBins;
#pragma unroll
    for (int j = 0; j < kCapPerThread; ++j)
      if (j < nreg && (key[j] & mask) == prefix) atomicAdd(&h[(key[j] >> shift) & uint32_t(kLowBins - 1)], 1u);
    __syncthreads();
    if (wave == 0) wave_pick_digit(h, kLowBins, want, prefix == 0 ? npad : 0u, &s_digit, &s_want);
    __syncthreads();
    prefix |= s_digit << shift;
    mask |= uint32_t(kLowBins - 1) << shift;
    want = s_want;
  }
  const uint32_t thr = prefix;
  const uint32_t need_eq = uint32_t(want);  // keys equal to thr kept: the first need_eq in segment order

  // One scan over packed counts (keys above thr in the low half, equal to it in the high
  // half; halves stay below 2^16, so no carry): first, per wave, its threads' keys in the
  // slices before this one (every element there is a row of the segment), then per
  // (register, wave) slot of this slice; per key of the slice, the same counts over the
  // lanes below it in its slot.
  uint32_t mine = 0;
#pragma unroll
  for (int j = 0; j < kCapPerThread; ++j)
    if (j < kSliceRegs * sl) mine += (key[j] > thr ? 1u : 0u) + (key[j] == thr ? 0x10000u : 0u);
  mine = wave_scan_u32(mine);
  if (lane == 63) slot_cnt[wave] = mine;
  const uint64_t below = lanemask_lt();
  uint32_t lcnt[kSliceRegs], skey[kSliceRegs];
#pragma unroll
  for (int j = 0; j < kCapPerThread; ++j) {
    if (j / kSliceRegs == sl) {  // wave-uniform
      const int jj = j % kSliceRegs;
      const uint64_t gm = __ballot(key[j] > thr), em = __ballot(key[j] == thr);
      lcnt[jj] = uint32_t(__popcll(gm & below)) | (uint32_t(__popcll(em & below)) << 16);
      skey[jj] = key[j];
      if (lane == 0)
        slot_cnt[kCapWaves + jj * kCapWaves + wave] = uint32_t(__popcll(gm)) | (uint32_t(__popcll(em)) << 16);
    }
  }
  __syncthreads();
  if (wave == 0) {  // exclusive scan of the kRankSlots slots by one wave: lane l holds slots l and 64 + l
    const uint32_t v0 = slot_cnt[lane], v1 = lane < kRankSlots - 64 ? slot_cnt[64 + lane] : 0u;
    const uint32_t i0 = wave_scan_u32(v0), i1 = wave_scan_u32(v1);
    const uint32_t t0 = uint32_t(__builtin_amdgcn_readlane(int(i0), 63));
    slot_cnt[lane] = i0 - v0;
    if (lane < kRankSlots - 64) slot_cnt[64 + lane] = t0 + i1 - v1;
  }
  __syncthreads();
  // every pair-id load in flight at once, then the stores (a kept row always lands in
  // [out0, out_end); the test only keeps this kernel and the gather in bounds)
  const int out_end = out0 + cap;  // an expert over capacity keeps exactly cap rows
  int32_t f[kSliceRegs], v[kSliceRegs];
#pragma unroll
  for (int jj = 0; jj < kSliceRegs; ++jj) {
    const int r = r0 + jj * kCapThreads + tid;
    const bool gt = skey[jj] > thr, eq = skey[jj] == thr;
    const uint32_t c = slot_cnt[kCapWaves + jj * kCapWaves + wave] + lcnt[jj];
    const uint32_t gb = c & 0xffffu, eb = c >> 16;
    f[jj] = (r < n && (gt || (eq && eb < need_eq))) ? out0 + int(gb + min(eb, need_eq)) : -1;
    v[jj] = f[jj] >= 0 ? seg[r] : 0;
  }
#pragma unroll
  for (int jj = 0; jj < kSliceRegs; ++jj) {
    const int r = r0 + jj * kCapThreads + tid;
    if (r < n) {
      const bool kept = f[jj] >= out0 && f[jj] < out_end;
      if (kept) sorted_pairs[f[jj]] = v[jj];
      tmp_final[a + r] = kept ? f[jj] : -1;
    }
  }
}

// ---- gather -----------------------------------------------------------------
// Token-major: one wave per token reads the token's row once and writes it to
// the sorted row of each of its kept local pairs (pair_row), so x is read once
// however many experts a token picked.
constexpr int kGatherTokensPerBlock = 4;

// After the capacity cut pair_row holds each local pair's pre-capacity row; the
// gather first resolves it through tmp_final (final row, or -1 if the pair was cut)
// and writes the final pair_row.
__global__ __launch_bounds__(256) void gather_kernel(const u32x4_t* __restrict__ x, int32_t* __restrict__ pair_row,
                                                     const int32_t* __restrict__ tmp_final, int64_t ntok, int k,
                                                     int vec_per_row, u32x4_t* __restrict__ xs) {
  const int lane = threadIdx.x & 63;
  const int64_t t = int64_t(blockIdx.x) * kGatherTokensPerBlock + (threadIdx.x >> 6);
  if (t >= ntok) return;
  int my_row = lane < k ? pair_row[t * k + lane] : -1;
  if (my_row >= 0) my_row = tmp_final[my_row];
  if (lane < k) pair_row[t * k + lane] = my_row;
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
constexpr int kMinPlaceSplit = 2, kMaxPlaceSplit = kDispatchTokens;
// Blocks per chunk: a power of two (kDispatchTokens divisible by it) giving about 1024 blocks.
// More blocks copy in smaller pieces and, fused, each re-reads the chunk histograms for its
// bases; fewer leave the copy too few loads in flight (measured on the gpt-oss-like share,
// 256 chunks: 2048 blocks 24.4 us, 1024 21.8, 512 23.2; mixtral_like, 128 chunks: 1024
// blocks 35.1 us, 512 35.6, 2048 37.0).
int place_split(int nblk) {
  int s = kMinPlaceSplit;
  while (s < kMaxPlaceSplit && int64_t(nblk) * s < 1024) s *= 2;
  return s;
}
// With few chunks and experts the place blocks find their own bases: every
// block sums the chunk histograms it needs (no separate scan launch).
constexpr int kFuseEntries = 65536;  // chunks x experts up to which the scan is folded in (gpt-oss-like
                                     // share, 256 x 128: layer -2% against a scan launch)

// FUSED: run[i] = (pairs of local experts before i) + (pairs of local expert i
// in earlier chunks), from the chunk histograms; block 0 also writes counts,
// offsets and the (zero) drop count.  Otherwise blk_base holds them.
template <bool FUSED, int kUnroll>
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
    chunk_bases(blk_all, nblk, E, begin, L, chunk, -1, run, counts, offsets, nullptr, nullptr, num_dropped);
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
  // with a small chunk-histogram table the place (or scatter) kernel finds its own bases
  const bool fused = int64_t(nblk) * E <= kFuseEntries;
  if (!fused) {
    MOE_LAUNCH("dispatch_scan", scan_kernel, dim3(1), dim3(kScanThreads), size_t(E + L + 1) * 4, a.s, a.scr.blk_all,
               nblk, E, begin, L, a.capacity, a.counts, a.offsets, a.scr.blk_base, a.scr.slice_off,
               a.scr.slice_desc, a.num_dropped);
  }
  if (cap) {
    const size_t scat_lds = size_t(L) * (1 + kDispatchThreads / 64) * 4;
    auto scatter = fused ? scatter_kernel<true> : scatter_kernel<false>;
    if (scat_lds > 65536 - 4096) {  // thousands of local experts (the block also holds ~2 KB of static LDS)
      const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(scatter),
                                               hipFuncAttributeMaxDynamicSharedMemorySize, int(scat_lds));
      if (e != hipSuccess) return set_error(MOE_ERR_HIP, "dispatch_scatter: LDS attribute: %s", hipGetErrorString(e));
    }
    MOE_LAUNCH("dispatch_scatter", scatter, dim3(nblk), dim3(kDispatchThreads), scat_lds, a.s, a.topk_ids, n, begin, L, chunk, a.scr.blk_base, a.scr.blk_all,
               nblk, E, a.capacity, a.counts, a.offsets, a.scr.slice_off, a.scr.slice_desc,
               a.num_dropped,
               a.scr.tmp_sorted, a.pair_row, a.topk_logit, a.scr.tmp_key);
    {
      const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(cap_hist_kernel),
                                               hipFuncAttributeMaxDynamicSharedMemorySize, int(kCapLds));
      if (e != hipSuccess) return set_error(MOE_ERR_HIP, "dispatch_cap_hist: LDS attribute: %s", hipGetErrorString(e));
    }
    // one block per slice slot; blocks past the last slice return at once
    const dim3 slices(unsigned(cap_slices_max(d)));
    MOE_LAUNCH("dispatch_cap_hist", cap_hist_kernel, slices, dim3(kCapThreads), kCapLds, a.s, a.scr.tmp_key,
               a.scr.slice_off, a.scr.slice_desc, L, int(a.capacity), a.scr.slice_hist);
    MOE_LAUNCH("dispatch_capacity", cap_select_kernel, slices, dim3(kCapThreads), kSelLds, a.s, a.scr.tmp_sorted,
               a.scr.tmp_key, a.scr.slice_off, a.scr.slice_desc, a.scr.slice_hist, L, int(a.capacity),
               a.sorted_pairs, a.scr.tmp_final);
    const dim3 grid(unsigned((d->num_tokens + kGatherTokensPerBlock - 1) / kGatherTokensPerBlock));
    MOE_LAUNCH("dispatch_gather", gather_kernel, grid, dim3(256), 0, a.s, static_cast<const u32x4_t*>(a.x), a.pair_row,
               a.scr.tmp_final, d->num_tokens, d->top_k, vec_per_row, static_cast<u32x4_t*>(a.x_sorted));
  } else {
    const size_t lds = (size_t(L) * (1 + kDispatchThreads / 64) + size_t(chunk)) * 4;
    // 16-byte slices per lane and pass over a row: 4, or 6 when the row then fits fewer, fuller
    // passes (a 2880-wide bf16 row: one pass of 384 instead of two of 256; 21.6 -> 20.2 us on the
    // gpt-oss-like share)
    const int split = place_split(nblk);
    const int tpp = kDispatchTokens / split, waves = kDispatchThreads / 64;
    const int wpt = tpp >= waves ? 1 : waves / tpp;  // waves per token, as in the kernel
    const int cper = (vec_per_row + wpt - 1) / wpt;
    const auto waste = [&](int u) { return (cper + 64 * u - 1) / (64 * u) * 64 * u - cper; };
    const bool six = waste(6) < waste(4);
    auto kern = fused ? (six ? place_kernel<true, 6> : place_kernel<true, 4>)
                      : (six ? place_kernel<false, 6> : place_kernel<false, 4>);
    if (lds > 65536) {
      const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                               hipFuncAttributeMaxDynamicSharedMemorySize, int(lds));
      if (e != hipSuccess) return set_error(MOE_ERR_HIP, "dispatch_place: LDS attribute: %s", hipGetErrorString(e));
    }
    MOE_LAUNCH("dispatch_place", kern, dim3(unsigned(nblk) * split), dim3(kDispatchThreads), lds, a.s,
               a.topk_ids, d->num_tokens, d->top_k, begin, L, a.scr.blk_base, a.scr.blk_all, nblk, E, a.counts,
               a.offsets, a.num_dropped, a.sorted_pairs, a.pair_row, static_cast<const u32x4_t*>(a.x), vec_per_row,
               static_cast<u32x4_t*>(a.x_sorted), split);
  }
  return MOE_OK;
}

}  // namespace moe
