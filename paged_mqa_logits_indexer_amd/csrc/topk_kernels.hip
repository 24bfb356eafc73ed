// Exact per-row top-k driven by the coarse histogram, for gfx950.
//
// DeepGEMM PR #94, "Motivation" and the SGLang commit "Replace the CuTe DSL
// selector with a JIT CUDA selector; add verify": the selector takes the
// threshold bin from the producer's 1024-bin histogram instead of making its
// own first pass, collects the columns above that bin, refines the threshold
// bin, and falls back to an exact whole-row radix select when the histogram
// is stale or the threshold bin holds more candidates than the capacity
// (8192); equal keys go to the lower column.  vLLM PR #52696 "Summary": the
// same selection on FP16 score keys, refining only the key bits the bin has
// not fixed.
//
// Launch sequence of one topk_rows call (one stream, no host sync):
//   [hist == NULL only] topk_zero_hist + topk_hist: build the row histograms
//                  in the workspace (the first pass the producer's fused
//                  histogram normally replaces)
//   topk_count     many workgroups per row, one 4096-score chunk each: the
//                  threshold bin b* from the histogram; counts of the chunk's
//                  scores above b* and in b* go to counts[row][chunk] (plain
//                  stores, no atomics); chunk 0 publishes b*
//   topk_write     the same chunks again: each workgroup adds up the counts of
//                  the chunks before it, rescans its chunk and writes the
//                  columns above b* to the output and the (key, column)
//                  candidates of b* to the row's candidate list, at exact
//                  positions (a block-wide scan keeps column order)
//   topk_refine    one workgroup per row checks the real counts against b*:
//                  if they confirm it, a radix select on the candidates'
//                  remaining key bits finishes the row; otherwise an exact
//                  radix select over the whole row does.  A kernel of its own:
//                  a last-workgroup handoff inside topk_write would need a
//                  device-scope fence per workgroup, which on this multi-die
//                  part writes back and invalidates the L2 under the others.
//
// Why the result is exact whatever the histogram holds: bin() is
// non-increasing in the score and in its FP16 rounding, so every column of a
// lower bin has a strictly larger key than every column of a higher bin.  If
// the scan counts n_gt columns above b* and n_eq in it with
// n_gt < k <= n_gt + n_eq, the top-k is those n_gt columns plus the best
// k - n_gt of the candidates.  Any other count means the histogram was not the
// histogram of these scores, and the row is selected from scratch.
#include "indexer_common.h"

namespace pmqa {
namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / kWave;
constexpr int kChunk = 4096;                // scores per workgroup
constexpr int kPerIter = kThreads * 4;      // scores per block-wide step
constexpr int kAllBins = kBins;             // threshold meaning "every live score"
constexpr int kRefineThreads = 512;         // one workgroup per row finishes it

struct RowMeta {
  int bstar;  // threshold bin the count pass used
  int pad0, pad1, pad2;
};

struct Workspace {
  RowMeta* meta;   // [rows]
  int2* counts;    // [rows][max_chunks]: (above b*, in b*) per chunk
  int* hist;       // [rows][1024]: histograms built when the caller has none
  uint2* cand;     // [rows][kCandCap]: (key, column) of the threshold bin
  int max_chunks;
};

__host__ __device__ inline size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

__host__ __device__ inline int chunks_for(int64_t stride) {
  return static_cast<int>((stride + kChunk - 1) / kChunk);
}

__host__ __device__ inline size_t workspace_size(int rows, int max_chunks) {
  return align256(sizeof(RowMeta) * rows) + align256(sizeof(int2) * static_cast<size_t>(rows) * max_chunks) +
         align256(sizeof(int) * kBins * static_cast<size_t>(rows)) +
         sizeof(uint2) * kCandCap * static_cast<size_t>(rows);
}

inline Workspace carve(void* base, int rows, int max_chunks) {
  char* p = static_cast<char*>(base);
  Workspace w;
  w.meta = reinterpret_cast<RowMeta*>(p);
  p += align256(sizeof(RowMeta) * rows);
  w.counts = reinterpret_cast<int2*>(p);
  p += align256(sizeof(int2) * static_cast<size_t>(rows) * max_chunks);
  w.hist = reinterpret_cast<int*>(p);
  p += align256(sizeof(int) * kBins * static_cast<size_t>(rows));
  w.cand = reinterpret_cast<uint2*>(p);
  w.max_chunks = max_chunks;
  return w;
}

template <int KEY>
__device__ __forceinline__ uint32_t score_key(float x) {
  if constexpr (KEY == IDX_KEY_FP32) return key_f32(x);
  else return key_f16(f16_bits_rn(x));
}

__device__ __forceinline__ int clamp_len(const int32_t* lens, int row, int64_t stride) {
  const int64_t l = lens[row];
  return static_cast<int>(l < 0 ? 0 : (l > stride ? stride : l));
}

// Workgroups a row uses: one per started chunk, at least one (an empty row
// still needs its finishing workgroup).
__device__ __forceinline__ int row_chunks(int len) { return len > 0 ? (len + kChunk - 1) / kChunk : 1; }

// ---------------------------------------------------------------------------
// Block-wide helpers for NT threads (s_red holds NT / 64 entries at least).
template <int NT = kThreads>
__device__ __forceinline__ int block_sum(int v, int* s_red) {
  v = wave_sum(v);
  const int wave = threadIdx.x / kWave;
  if (__lane_id() == 0) s_red[wave] = v;
  __syncthreads();
  int t = 0;
#pragma unroll
  for (int w = 0; w < NT / kWave; ++w) t += s_red[w];
  __syncthreads();
  return t;
}

// Exclusive prefix of v in thread order; *total = block sum.
template <int NT = kThreads>
__device__ __forceinline__ int block_excl_scan(int v, int* s_red, int* total) {
  const int inc = wave_inclusive_scan(v);
  const int wave = threadIdx.x / kWave;
  if (__lane_id() == kWave - 1) s_red[wave] = inc;
  __syncthreads();
  int before = 0, all = 0;
#pragma unroll
  for (int w = 0; w < NT / kWave; ++w) {
    const int t = s_red[w];
    before += (w < wave) ? t : 0;
    all += t;
  }
  __syncthreads();
  *total = all;
  return before + inc - v;
}

// Threshold bin of a row: the first bin whose inclusive prefix count reaches
// k, or kAllBins when the histogram holds at most k scores.
__device__ int threshold_bin(const int* __restrict__ h, int k, int* s_red) {
  constexpr int per = kBins / kThreads;  // 4 bins per thread
  int c[per];
  int sum = 0;
#pragma unroll
  for (int i = 0; i < per; ++i) {
    c[i] = h[threadIdx.x * per + i];
    sum += c[i];
  }
  int total = 0;
  int run = block_excl_scan(sum, s_red, &total);
  if (total <= k) return kAllBins;
  // The crossing lies in exactly one thread's bins (counts are non-negative
  // in any histogram this call produced; for a foreign one any bin is fine,
  // the counts checked later decide).
  if (threadIdx.x == 0) s_red[kWaves] = kAllBins;
  __syncthreads();
#pragma unroll
  for (int i = 0; i < per; ++i) {
    if (run < k && run + c[i] >= k) s_red[kWaves] = threadIdx.x * per + i;
    run += c[i];
  }
  __syncthreads();
  const int bstar = s_red[kWaves];
  __syncthreads();
  return bstar;
}

// Classify four consecutive scores against b*.
__device__ __forceinline__ void classify4(const f32x4& v, int s, int s1, int bstar, bool (&gt)[4],
                                          bool (&eq)[4]) {
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const uint32_t hb = f16_bits_rn(v[e]);
    const bool live = (s + e < s1) && !f16_is_nan(hb);
    const int bin = coarse_bin_f16(hb);
    gt[e] = live && bin < bstar;
    eq[e] = live && bin == bstar;
  }
}

// ---------------------------------------------------------------------------
__global__ void topk_zero_hist_kernel(int* hist, int rows) {
  const int64_t n = static_cast<int64_t>(rows) * kBins;
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; i < n;
       i += static_cast<int64_t>(gridDim.x) * blockDim.x)
    hist[i] = 0;
}

// Histogram of each row's live non-NaN scores, added to hist_out.
__global__ __launch_bounds__(kThreads) void topk_hist_kernel(const float* __restrict__ logits,
                                                             int64_t stride,
                                                             const int32_t* __restrict__ lens,
                                                             int* __restrict__ hist_out) {
  __shared__ int s_hist[kBins];
  const int row = blockIdx.y;
  const int len = clamp_len(lens, row, stride);
  const int s0 = blockIdx.x * kChunk;
  if (s0 >= len) return;
  for (int i = threadIdx.x; i < kBins; i += kThreads) s_hist[i] = 0;
  __syncthreads();
  const float* x = logits + static_cast<int64_t>(row) * stride;
  const int s1 = min(len, s0 + kChunk);
  for (int s = s0 + threadIdx.x * 4; s < s1; s += kPerIter) {
    const f32x4 v = *reinterpret_cast<const f32x4*>(x + s);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      if (s + e < s1) {
        const uint32_t hb = f16_bits_rn(v[e]);
        if (!f16_is_nan(hb)) atomicAdd(&s_hist[coarse_bin_f16(hb)], 1);
      }
    }
  }
  __syncthreads();
  unsigned long long* gh = reinterpret_cast<unsigned long long*>(hist_out + static_cast<int64_t>(row) * kBins);
  const uint2* sh = reinterpret_cast<const uint2*>(s_hist);
  for (int i = threadIdx.x; i < kBins / 2; i += kThreads) {
    const uint2 v = sh[i];
    if (v.x | v.y) atomicAdd(gh + i, (static_cast<unsigned long long>(v.y) << 32) | v.x);
  }
}

// ---------------------------------------------------------------------------
__global__ __launch_bounds__(kThreads) void topk_count_kernel(const float* __restrict__ logits,
                                                              int64_t stride,
                                                              const int32_t* __restrict__ hist,
                                                              const int32_t* __restrict__ lens, int k,
                                                              Workspace ws) {
  __shared__ int s_red[kWaves + 1];
  const int row = blockIdx.y;
  const int c = blockIdx.x;
  const int len = clamp_len(lens, row, stride);
  if (c >= row_chunks(len)) return;
  const int* h = (hist ? hist : ws.hist) + static_cast<int64_t>(row) * kBins;
  const int bstar = threshold_bin(h, k, s_red);
  if (c == 0 && threadIdx.x == 0) ws.meta[row] = RowMeta{bstar, 0, 0, 0};

  const float* x = logits + static_cast<int64_t>(row) * stride;
  const int s0 = c * kChunk;
  const int s1 = min(len, s0 + kChunk);
  int ng = 0, ne = 0;
  for (int base = s0; base < s1; base += kPerIter) {
    const int s = base + threadIdx.x * 4;
    f32x4 v = {0.f, 0.f, 0.f, 0.f};
    if (s < s1) v = *reinterpret_cast<const f32x4*>(x + s);
    bool gt[4], eq[4];
    classify4(v, s, s1, bstar, gt, eq);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      ng += gt[e];
      ne += eq[e];
    }
  }
  // Both counts at once: each is at most kChunk < 2^16.
  const int both = block_sum(ng | (ne << 16), s_red);
  if (threadIdx.x == 0)
    ws.counts[static_cast<int64_t>(row) * ws.max_chunks + c] = int2{both & 0xFFFF, both >> 16};
}

// ---------------------------------------------------------------------------
// Shared memory of the refine pass.
struct RefineShared {
  uint2 cand[kCandCap];   // 64 KiB
  int digit_hist[256];
  int red[kRefineThreads / kWave + 4];
  int out_pos;
  uint32_t red_or, red_and;
  int bcast[4];
};

__device__ __forceinline__ void block_or_and(uint32_t o, uint32_t a, RefineShared& sh) {
  if (threadIdx.x == 0) {
    sh.red_or = 0u;
    sh.red_and = 0xFFFFFFFFu;
  }
  __syncthreads();
#pragma unroll
  for (int off = kWave / 2; off > 0; off >>= 1) {
    o |= __shfl_xor(o, off, kWave);
    a &= __shfl_xor(a, off, kWave);
  }
  if (__lane_id() == 0) {
    atomicOr(&sh.red_or, o);
    atomicAnd(&sh.red_and, a);
  }
  __syncthreads();
}

// Given digit_hist (256 counts), the digit d at which the running count taken
// from the largest digit (descending) or the smallest first reaches `need`;
// *before = the count strictly before d.
__device__ int pick_digit(RefineShared& sh, int need, bool descending, int* before) {
  if (threadIdx.x < kWave) {
    const int lane = threadIdx.x;
    int c[4], sum = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int pos = lane * 4 + i;
      c[i] = sh.digit_hist[descending ? 255 - pos : pos];
      sum += c[i];
    }
    const int inc = wave_inclusive_scan(sum);
    int run = inc - sum;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if (run < need && run + c[i] >= need) {
        const int pos = lane * 4 + i;
        sh.bcast[0] = descending ? 255 - pos : pos;
        sh.bcast[1] = run;
      }
      run += c[i];
    }
  }
  __syncthreads();
  const int d = sh.bcast[0];
  *before = sh.bcast[1];
  __syncthreads();
  return d;
}

__device__ __forceinline__ int top_bit(uint32_t x) { return 31 - __clz(x); }

// Radix select over the n LDS candidates: the key T of the need-th largest
// key; *above = how many keys exceed T.  Bits every key shares are skipped.
__device__ uint32_t select_key_lds(RefineShared& sh, int n, int need, int* above) {
  uint32_t o = 0u, a = 0xFFFFFFFFu;
  for (int i = threadIdx.x; i < n; i += kRefineThreads) {
    o |= sh.cand[i].x;
    a &= sh.cand[i].x;
  }
  block_or_and(o, a, sh);
  const uint32_t diff = sh.red_or ^ sh.red_and;
  uint32_t prefix = sh.red_and & ~diff;
  int gt = 0;
  if (diff) {
    uint32_t fixed = ~diff;
    int shift = top_bit(diff) - 7;
    if (shift < 0) shift = 0;
    while (true) {
      for (int i = threadIdx.x; i < 256; i += kRefineThreads) sh.digit_hist[i] = 0;
      __syncthreads();
      for (int i = threadIdx.x; i < n; i += kRefineThreads) {
        const uint32_t key = sh.cand[i].x;
        if (((key ^ prefix) & fixed) == 0u) atomicAdd(&sh.digit_hist[(key >> shift) & 0xFFu], 1);
      }
      __syncthreads();
      int before = 0;
      const int d = pick_digit(sh, need, true, &before);
      need -= before;
      gt += before;
      prefix |= static_cast<uint32_t>(d) << shift;
      fixed |= 0xFFu << shift;
      if (shift == 0) break;
      shift = shift >= 8 ? shift - 8 : 0;
    }
  }
  *above = gt;
  return prefix;
}

// Among LDS candidates with key == T, the need-th smallest column.
__device__ uint32_t select_col_lds(RefineShared& sh, int n, uint32_t T, int need) {
  uint32_t o = 0u, a = 0xFFFFFFFFu;
  for (int i = threadIdx.x; i < n; i += kRefineThreads) {
    const uint2 c = sh.cand[i];
    if (c.x == T) {
      o |= c.y;
      a &= c.y;
    }
  }
  block_or_and(o, a, sh);
  const uint32_t diff = sh.red_or ^ sh.red_and;
  uint32_t prefix = sh.red_and & ~diff;
  if (diff) {
    uint32_t fixed = ~diff;
    int shift = top_bit(diff) - 7;
    if (shift < 0) shift = 0;
    while (true) {
      for (int i = threadIdx.x; i < 256; i += kRefineThreads) sh.digit_hist[i] = 0;
      __syncthreads();
      for (int i = threadIdx.x; i < n; i += kRefineThreads) {
        const uint2 c = sh.cand[i];
        if (c.x == T && ((c.y ^ prefix) & fixed) == 0u) atomicAdd(&sh.digit_hist[(c.y >> shift) & 0xFFu], 1);
      }
      __syncthreads();
      int before = 0;
      const int d = pick_digit(sh, need, false, &before);
      need -= before;
      prefix |= static_cast<uint32_t>(d) << shift;
      fixed |= 0xFFu << shift;
      if (shift == 0) break;
      shift = shift >= 8 ? shift - 8 : 0;
    }
  }
  return prefix;
}

// Append this thread's column to the output through a block-wide LDS counter.
__device__ __forceinline__ void emit(RefineShared& sh, int32_t* out, int k, bool take, int col) {
  const uint64_t m = __ballot(take);
  if (!m) return;
  int pos = 0;
  if (__lane_id() == 0) pos = atomicAdd(&sh.out_pos, __popcll(m));
  pos = __shfl(pos, 0, kWave) + lanes_below(m);
  if (take && pos < k) out[pos] = col;
}

// Exact selection over the whole row: a stale histogram, or a threshold bin
// with more candidates than the capacity.
template <int KEY>
__device__ void whole_row_select(RefineShared& sh, const float* __restrict__ x, int len, int k,
                                 int32_t* __restrict__ out) {
  int cnt = 0;
  for (int s = threadIdx.x; s < len; s += kRefineThreads) cnt += (x[s] == x[s]) ? 1 : 0;
  const int n = block_sum<kRefineThreads>(cnt, sh.red);
  if (threadIdx.x == 0) sh.out_pos = 0;
  __syncthreads();
  if (n <= k) {
    for (int s0 = 0; s0 < len; s0 += kRefineThreads) {
      const int s = s0 + threadIdx.x;
      emit(sh, out, k, s < len && x[s] == x[s], s);
    }
    __syncthreads();
    for (int i = n + threadIdx.x; i < k; i += kRefineThreads) out[i] = -1;
    return;
  }
  constexpr int kKeyBits = KEY == IDX_KEY_FP32 ? 32 : 16;
  uint32_t prefix = 0u, fixed = 0u;
  int need = k;
  for (int shift = kKeyBits - 8; shift >= 0; shift -= 8) {
    for (int i = threadIdx.x; i < 256; i += kRefineThreads) sh.digit_hist[i] = 0;
    __syncthreads();
    for (int s = threadIdx.x; s < len; s += kRefineThreads) {
      const float v = x[s];
      if (v != v) continue;
      const uint32_t key = score_key<KEY>(v);
      if (((key ^ prefix) & fixed) == 0u) atomicAdd(&sh.digit_hist[(key >> shift) & 0xFFu], 1);
    }
    __syncthreads();
    int before = 0;
    const int d = pick_digit(sh, need, true, &before);
    need -= before;
    prefix |= static_cast<uint32_t>(d) << shift;
    fixed |= 0xFFu << shift;
  }
  const uint32_t T = prefix;
  // Keys above T, then the `need` lowest columns with key == T, in column order.
  int taken_ties = 0;
  for (int s0 = 0; s0 < len; s0 += kRefineThreads) {
    const int s = s0 + threadIdx.x;
    bool above = false, tie = false;
    if (s < len) {
      const float v = x[s];
      if (v == v) {
        const uint32_t key = score_key<KEY>(v);
        above = key > T;
        tie = key == T;
      }
    }
    int slice_ties = 0;
    const int rank = taken_ties + block_excl_scan<kRefineThreads>(tie ? 1 : 0, sh.red, &slice_ties);
    emit(sh, out, k, above || (tie && rank < need), s);
    taken_ties += slice_ties;
  }
}

template <int KEY>
__global__ __launch_bounds__(kThreads) void topk_write_kernel(const float* __restrict__ logits,
                                                              int64_t stride,
                                                              const int32_t* __restrict__ lens, int k,
                                                              int32_t* __restrict__ indices,
                                                              Workspace ws) {
  __shared__ int s_red[kWaves];
  const int row = blockIdx.y;
  const int c = blockIdx.x;
  const int len = clamp_len(lens, row, stride);
  const int nch = row_chunks(len);
  if (c >= nch) return;
  const int bstar = ws.meta[row].bstar;
  const int2* cnt = ws.counts + static_cast<int64_t>(row) * ws.max_chunks;
  const float* x = logits + static_cast<int64_t>(row) * stride;
  int32_t* out = indices + static_cast<int64_t>(row) * k;
  uint2* cand = ws.cand + static_cast<int64_t>(row) * kCandCap;

  // Positions of this chunk's columns: the counts of the chunks before it.
  int pg = 0, pe = 0;
  for (int i = threadIdx.x; i < c; i += kThreads) {
    const int2 v = cnt[i];
    pg += v.x;
    pe += v.y;
  }
  int run_g = block_sum(pg, s_red);
  int run_e = block_sum(pe, s_red);

  const int s0 = c * kChunk;
  const int s1 = min(len, s0 + kChunk);
  for (int base = s0; base < s1; base += kPerIter) {
    const int s = base + threadIdx.x * 4;
    f32x4 v = {0.f, 0.f, 0.f, 0.f};
    if (s < s1) v = *reinterpret_cast<const f32x4*>(x + s);
    bool gt[4], eq[4];
    classify4(v, s, s1, bstar, gt, eq);
    int tg = 0, te = 0;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      tg += gt[e];
      te += eq[e];
    }
    int tot = 0;
    const int pre = block_excl_scan(tg | (te << 16), s_red, &tot);
    int og = run_g + (pre & 0xFFFF), oe = run_e + (pre >> 16);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      if (gt[e]) {
        if (og < k) out[og] = s + e;
        ++og;
      }
      if (eq[e]) {
        if (oe < kCandCap) cand[oe] = uint2{score_key<KEY>(v[e]), static_cast<uint32_t>(s + e)};
        ++oe;
      }
    }
    run_g += tot & 0xFFFF;
    run_e += tot >> 16;
  }

}

// Finishes each row after the write pass: checks the real counts against b*
// and either refines the candidates or selects over the whole row.
template <int KEY>
__global__ __launch_bounds__(kRefineThreads) void topk_refine_kernel(const float* __restrict__ logits,
                                                                     int64_t stride,
                                                                     const int32_t* __restrict__ lens,
                                                                     int k, int32_t* __restrict__ indices,
                                                                     Workspace ws) {
  __shared__ RefineShared sh;
  const int row = blockIdx.x;
  const int len = clamp_len(lens, row, stride);
  const int nch = row_chunks(len);
  const int bstar = ws.meta[row].bstar;
  const int2* cnt = ws.counts + static_cast<int64_t>(row) * ws.max_chunks;
  const float* x = logits + static_cast<int64_t>(row) * stride;
  int32_t* out = indices + static_cast<int64_t>(row) * k;
  const uint2* cand = ws.cand + static_cast<int64_t>(row) * kCandCap;

  int tg = 0, te = 0;
  for (int i = threadIdx.x; i < nch; i += kRefineThreads) {
    const int2 v = cnt[i];
    tg += v.x;
    te += v.y;
  }
  const int n_gt = block_sum<kRefineThreads>(tg, sh.red);
  const int n_eq = block_sum<kRefineThreads>(te, sh.red);
  bool valid;
  if (bstar == kAllBins) valid = n_gt <= k && n_eq == 0;
  else valid = n_gt < k && n_gt + n_eq >= k && n_eq <= kCandCap;
  if (!valid) {
    whole_row_select<KEY>(sh, x, len, k, out);
    return;
  }
  if (bstar == kAllBins) {
    for (int i = n_gt + threadIdx.x; i < k; i += kRefineThreads) out[i] = -1;
    return;
  }
  const int need = k - n_gt;
  if (need == n_eq) {
    for (int i = threadIdx.x; i < n_eq; i += kRefineThreads) out[n_gt + i] = static_cast<int>(cand[i].y);
    return;
  }
  for (int i = threadIdx.x; i < n_eq; i += kRefineThreads) sh.cand[i] = cand[i];
  if (threadIdx.x == 0) sh.out_pos = n_gt;
  __syncthreads();
  int above = 0;
  const uint32_t T = select_key_lds(sh, n_eq, need, &above);
  const int ties_needed = need - above;
  int tc = 0;
  for (int i = threadIdx.x; i < n_eq; i += kRefineThreads) tc += sh.cand[i].x == T ? 1 : 0;
  const int ties = block_sum<kRefineThreads>(tc, sh.red);
  uint32_t col_cut = 0xFFFFFFFFu;
  if (ties > ties_needed) col_cut = select_col_lds(sh, n_eq, T, ties_needed);
  for (int i0 = 0; i0 < n_eq; i0 += kRefineThreads) {
    const int i = i0 + threadIdx.x;
    bool take = false;
    int col = 0;
    if (i < n_eq) {
      const uint2 cd = sh.cand[i];
      take = cd.x > T || (cd.x == T && cd.y <= col_cut);
      col = static_cast<int>(cd.y);
    }
    emit(sh, out, k, take, col);
  }
}

}  // namespace

size_t topk_workspace_size(int32_t rows, int64_t logits_stride) {
  if (rows <= 0 || logits_stride <= 0) return 0;
  return workspace_size(rows, chunks_for(logits_stride));
}

hipError_t launch_topk_rows(const TopkArgs& a, hipStream_t stream) {
  const int max_chunks = chunks_for(a.logits_stride);
  const Workspace ws = carve(a.workspace, a.rows, max_chunks);
  const dim3 grid(static_cast<unsigned>(max_chunks), static_cast<unsigned>(a.rows));
  const int32_t* hist = a.hist;
  if (hist == nullptr) {
    hipLaunchKernelGGL(topk_zero_hist_kernel, dim3(min(1024, (a.rows * kBins + 255) / 256)), dim3(256), 0,
                       stream, ws.hist, a.rows);
    hipLaunchKernelGGL(topk_hist_kernel, grid, dim3(kThreads), 0, stream, a.logits, a.logits_stride,
                       a.context_lens, ws.hist);
  }
  hipLaunchKernelGGL(topk_count_kernel, grid, dim3(kThreads), 0, stream, a.logits, a.logits_stride, hist,
                     a.context_lens, a.k, ws);
  if (a.key_dtype == IDX_KEY_FP32) {
    hipLaunchKernelGGL(topk_write_kernel<IDX_KEY_FP32>, grid, dim3(kThreads), 0, stream, a.logits,
                       a.logits_stride, a.context_lens, a.k, a.indices, ws);
    hipLaunchKernelGGL(topk_refine_kernel<IDX_KEY_FP32>, dim3(a.rows), dim3(kRefineThreads), 0, stream,
                       a.logits, a.logits_stride, a.context_lens, a.k, a.indices, ws);
  } else {
    hipLaunchKernelGGL(topk_write_kernel<IDX_KEY_FP16>, grid, dim3(kThreads), 0, stream, a.logits,
                       a.logits_stride, a.context_lens, a.k, a.indices, ws);
    hipLaunchKernelGGL(topk_refine_kernel<IDX_KEY_FP16>, dim3(a.rows), dim3(kRefineThreads), 0, stream,
                       a.logits, a.logits_stride, a.context_lens, a.k, a.indices, ws);
  }
  return hipGetLastError();
}

hipError_t launch_score_histogram(const float* scores, int64_t stride, const int32_t* lens,
                                  int32_t rows, int32_t* hist, hipStream_t stream) {
  const int64_t chunks64 = (stride + kChunk - 1) / kChunk;
  if (chunks64 > 0x7FFFFFFF) return hipErrorInvalidValue;
  hipLaunchKernelGGL(topk_hist_kernel, dim3(static_cast<unsigned>(chunks64), static_cast<unsigned>(rows)),
                     dim3(kThreads), 0, stream, scores, stride, lens, hist);
  return hipGetLastError();
}

}  // namespace pmqa
