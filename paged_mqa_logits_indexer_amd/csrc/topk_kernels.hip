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
//   topk_init      zero the per-row counters (and the row histograms when the
//                  caller passed none)
//   topk_hist      only when hist == NULL: build the row histograms (the first
//                  pass the fused producer histogram normally replaces)
//   topk_collect   many workgroups per row: threshold bin b* from the
//                  histogram; columns with bin < b* go straight to the output,
//                  columns with bin == b* are appended as (key, column)
//                  candidates; both are counted with the real scores
//   topk_refine    one workgroup per row: if the real counts confirm b*, radix
//                  select on the candidates' remaining key bits, ties by the
//                  lower column; otherwise an exact radix select over the row
//
// Why the result is exact whatever the histogram holds: bin() is
// non-increasing in the score and in its FP16 rounding, so every column of a
// lower bin has a strictly larger key than every column of a higher bin.  If
// the collect pass counts n_gt columns above b* and n_eq in it with
// n_gt < k <= n_gt + n_eq, the top-k is those n_gt columns plus the best
// k - n_gt of the candidates.  Any other count means the histogram was not the
// histogram of these scores, and the row is selected from scratch.
#include "indexer_common.h"

namespace pmqa {
namespace {

constexpr int kCollectThreads = 256;
constexpr int kChunk = 4096;  // scores per collect/hist workgroup
constexpr int kRefineThreads = 1024;
constexpr int kRefineWaves = kRefineThreads / kWave;
constexpr int kAllBins = kBins;  // threshold value meaning "every live score"

struct RowMeta {
  int n_gt;  // columns found above the threshold bin
  int n_eq;  // columns found in the threshold bin
  int pad0, pad1;
};

struct Workspace {
  RowMeta* meta;   // [rows]
  int* hist;       // [rows][1024] (used when the caller passes no histogram)
  uint2* cand;     // [rows][kCandCap] (key, column)
};

__host__ __device__ inline size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

__host__ __device__ inline Workspace carve(void* base, int rows) {
  char* p = static_cast<char*>(base);
  Workspace w;
  w.meta = reinterpret_cast<RowMeta*>(p);
  p += align256(sizeof(RowMeta) * rows);
  w.hist = reinterpret_cast<int*>(p);
  p += align256(sizeof(int) * kBins * static_cast<size_t>(rows));
  w.cand = reinterpret_cast<uint2*>(p);
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

// ---------------------------------------------------------------------------
__global__ void topk_init_kernel(Workspace ws, int rows, bool zero_hist) {
  const int row = blockIdx.x;
  if (row >= rows) return;
  if (threadIdx.x == 0) ws.meta[row] = RowMeta{0, 0, 0, 0};
  if (zero_hist) {
    for (int i = threadIdx.x; i < kBins; i += blockDim.x) ws.hist[static_cast<int64_t>(row) * kBins + i] = 0;
  }
}

// ---------------------------------------------------------------------------
// First pass over the scores when the producer supplied no histogram.
__global__ __launch_bounds__(kCollectThreads) void topk_hist_kernel(const float* __restrict__ logits,
                                                                    int64_t stride,
                                                                    const int32_t* __restrict__ lens,
                                                                    int* __restrict__ hist_out) {
  __shared__ int s_hist[kBins];
  const int row = blockIdx.y;
  const int len = clamp_len(lens, row, stride);
  const int s0 = blockIdx.x * kChunk;
  if (s0 >= len) return;
  for (int i = threadIdx.x; i < kBins; i += kCollectThreads) s_hist[i] = 0;
  __syncthreads();
  const float* x = logits + static_cast<int64_t>(row) * stride;
  const int s1 = min(len, s0 + kChunk);
  for (int s = s0 + threadIdx.x * 4; s < s1; s += kCollectThreads * 4) {
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
  for (int i = threadIdx.x; i < kBins / 2; i += kCollectThreads) {
    const uint2 v = sh[i];
    if (v.x | v.y) atomicAdd(gh + i, (static_cast<unsigned long long>(v.y) << 32) | v.x);
  }
}

// Threshold bin of a row: the first bin whose inclusive prefix count reaches
// k, or kAllBins when the histogram holds at most k scores.  Computed by all
// threads of the block; the histogram row is read from global memory.
template <int NT>
__device__ int threshold_bin(const int* __restrict__ h, int k, int* s_scan) {
  constexpr int per = kBins / NT;  // bins per thread
  constexpr int nw = NT / kWave;
  const int tid = threadIdx.x, lane = __lane_id(), wave = tid / kWave;
  int c[per > 0 ? per : 1];
  int sum = 0;
  if constexpr (per > 0) {
#pragma unroll
    for (int i = 0; i < per; ++i) {
      c[i] = h[tid * per + i];
      sum += c[i];
    }
  }
  const int inc = wave_inclusive_scan(sum);
  if (lane == kWave - 1) s_scan[wave] = inc;
  __syncthreads();
  int before = 0, total = 0;
#pragma unroll
  for (int w = 0; w < nw; ++w) {
    const int t = s_scan[w];
    before += (w < wave) ? t : 0;
    total += t;
  }
  __syncthreads();
  if (total <= k) return kAllBins;
  // Exactly one thread sees the crossing inside its bins.
  int run = before + inc - sum;
  if (tid == 0) s_scan[nw] = kAllBins;
  __syncthreads();
  if constexpr (per > 0) {
#pragma unroll
    for (int i = 0; i < per; ++i) {
      if (run < k && run + c[i] >= k) s_scan[nw] = tid * per + i;
      run += c[i];
    }
  }
  __syncthreads();
  const int bstar = s_scan[nw];
  __syncthreads();
  return bstar;
}

// ---------------------------------------------------------------------------
template <int KEY>
__global__ __launch_bounds__(kCollectThreads) void topk_collect_kernel(
    const float* __restrict__ logits, int64_t stride, const int32_t* __restrict__ hist,
    const int32_t* __restrict__ lens, int k, int32_t* __restrict__ indices, Workspace ws) {
  __shared__ int s_scan[kCollectThreads / kWave + 1];
  const int row = blockIdx.y;
  const int len = clamp_len(lens, row, stride);
  const int s0 = blockIdx.x * kChunk;
  if (s0 >= len) return;
  const int* h = hist ? hist + static_cast<int64_t>(row) * kBins : ws.hist + static_cast<int64_t>(row) * kBins;
  const int bstar = threshold_bin<kCollectThreads>(h, k, s_scan);

  const float* x = logits + static_cast<int64_t>(row) * stride;
  int32_t* out = indices + static_cast<int64_t>(row) * k;
  uint2* cand = ws.cand + static_cast<int64_t>(row) * kCandCap;
  RowMeta* meta = ws.meta + row;
  const int s1 = min(len, s0 + kChunk);
  for (int base = s0; base < s1; base += kCollectThreads * 4) {
    const int s = base + threadIdx.x * 4;
    f32x4 v = {0.f, 0.f, 0.f, 0.f};
    if (s < s1) v = *reinterpret_cast<const f32x4*>(x + s);
    bool gt[4], eq[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const uint32_t hb = f16_bits_rn(v[e]);
      const bool live = (s + e < s1) && !f16_is_nan(hb);
      const int bin = coarse_bin_f16(hb);
      gt[e] = live && bin < bstar;
      eq[e] = live && bin == bstar;
    }
    // Wave-aggregated appends: one atomic per wave and list.
    uint64_t mg[4], me[4];
    int ng = 0, ne = 0;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      mg[e] = __ballot(gt[e]);
      me[e] = __ballot(eq[e]);
      ng += __popcll(mg[e]);
      ne += __popcll(me[e]);
    }
    if (ng) {
      int pos = 0;
      if (__lane_id() == 0) pos = atomicAdd(&meta->n_gt, ng);
      pos = __shfl(pos, 0, kWave);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        if (gt[e]) {
          const int p = pos + lanes_below(mg[e]);
          if (p < k) out[p] = s + e;
        }
        pos += __popcll(mg[e]);
      }
    }
    if (ne) {
      int pos = 0;
      if (__lane_id() == 0) pos = atomicAdd(&meta->n_eq, ne);
      pos = __shfl(pos, 0, kWave);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        if (eq[e]) {
          const int p = pos + lanes_below(me[e]);
          if (p < kCandCap) cand[p] = uint2{score_key<KEY>(v[e]), static_cast<uint32_t>(s + e)};
        }
        pos += __popcll(me[e]);
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Refine / fallback: one 1024-thread workgroup per row.
struct RefineShared {
  uint2 cand[kCandCap];   // 64 KiB
  int digit_hist[256];
  int scan[kRefineWaves + 4];
  int out_pos;
  uint32_t red_or, red_and;
  int bcast[4];
};

__device__ __forceinline__ void block_or_and(uint32_t o, uint32_t a, RefineShared& sh) {
  if (threadIdx.x == 0) { sh.red_or = 0u; sh.red_and = 0xFFFFFFFFu; }
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

__device__ __forceinline__ int block_sum(int v, RefineShared& sh) {
  v = wave_sum(v);
  const int wave = threadIdx.x / kWave;
  if (__lane_id() == 0) sh.scan[wave] = v;
  __syncthreads();
  int t = 0;
#pragma unroll
  for (int w = 0; w < kRefineWaves; ++w) t += sh.scan[w];
  __syncthreads();
  return t;
}

// Given digit_hist (256 counts), find digit d (scanning from the largest for
// `descending`, else from the smallest) where the running count first reaches
// `need`; returns d and writes the count strictly before it to *before.
__device__ int pick_digit(RefineShared& sh, int need, bool descending, int* before) {
  if (threadIdx.x < kWave) {
    const int lane = threadIdx.x;
    int c[4], sum = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int pos = lane * 4 + i;
      const int d = descending ? 255 - pos : pos;
      c[i] = sh.digit_hist[d];
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

// Radix select over n (key, column) items held in LDS: returns the key T of
// the `need`-th largest key; *above = number of items with key > T.
__device__ uint32_t select_key_lds(RefineShared& sh, int n, int need, int* above) {
  uint32_t o = 0u, a = 0xFFFFFFFFu;
  for (int i = threadIdx.x; i < n; i += kRefineThreads) {
    o |= sh.cand[i].x;
    a &= sh.cand[i].x;
  }
  block_or_and(o, a, sh);
  const uint32_t diff = sh.red_or ^ sh.red_and;
  uint32_t prefix = sh.red_and & ~diff;  // the bits every key shares
  int gt = 0;
  if (diff) {
    uint32_t fixed = ~diff;  // bits already known
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

// Among LDS items with key == T, the `need`-th smallest column.
__device__ uint32_t select_col_lds(RefineShared& sh, int n, uint32_t T, int need) {
  uint32_t o = 0u, a = 0xFFFFFFFFu;
  for (int i = threadIdx.x; i < n; i += kRefineThreads) {
    const uint2 c = sh.cand[i];
    if (c.x == T) { o |= c.y; a &= c.y; }
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

// Append this thread's item to the output with a block-wide LDS counter.
__device__ __forceinline__ void emit(RefineShared& sh, int32_t* out, int k, bool take, int col) {
  const uint64_t m = __ballot(take);
  if (!m) return;
  int pos = 0;
  if (__lane_id() == 0) pos = atomicAdd(&sh.out_pos, __popcll(m));
  pos = __shfl(pos, 0, kWave) + lanes_below(m);
  if (take && pos < k) out[pos] = col;
}

// Exact selection over the whole row (stale histogram, overflow, or none).
template <int KEY>
__device__ void whole_row_select(RefineShared& sh, const float* __restrict__ x, int len, int k,
                                 int32_t* __restrict__ out) {
  // Selectable count.
  int cnt = 0;
  for (int s = threadIdx.x; s < len; s += kRefineThreads) cnt += (x[s] == x[s]) ? 1 : 0;
  const int n = block_sum(cnt, sh);
  if (threadIdx.x == 0) sh.out_pos = 0;
  __syncthreads();
  if (n <= k) {
    for (int s0 = 0; s0 < len; s0 += kRefineThreads) {
      const int s = s0 + threadIdx.x;
      const bool take = s < len && x[s] == x[s];
      emit(sh, out, k, take, s);
    }
    __syncthreads();
    for (int i = n + threadIdx.x; i < k; i += kRefineThreads) out[i] = -1;
    return;
  }
  // Radix select of the k-th largest key over the row, 8 bits a pass.
  constexpr int kKeyBits = KEY == IDX_KEY_FP32 ? 32 : 16;
  uint32_t prefix = 0u, fixed = 0u;
  int need = k, gt = 0;
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
    gt += before;
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
    // Rank of this tie among the ties of this slice (column order).
    const uint64_t mt = __ballot(tie);
    const int wave = threadIdx.x / kWave;
    if (__lane_id() == 0) sh.scan[wave] = __popcll(mt);
    __syncthreads();
    int before_w = 0, slice_ties = 0;
#pragma unroll
    for (int w = 0; w < kRefineWaves; ++w) {
      const int t = sh.scan[w];
      before_w += (w < wave) ? t : 0;
      slice_ties += t;
    }
    __syncthreads();
    const int rank = taken_ties + before_w + lanes_below(mt);
    emit(sh, out, k, above || (tie && rank < need), s);
    taken_ties += slice_ties;
  }
  (void)gt;
}

template <int KEY>
__global__ __launch_bounds__(kRefineThreads) void topk_refine_kernel(
    const float* __restrict__ logits, int64_t stride, const int32_t* __restrict__ hist,
    const int32_t* __restrict__ lens, int k, int32_t* __restrict__ indices, Workspace ws) {
  __shared__ RefineShared sh;
  const int row = blockIdx.x;
  const int len = clamp_len(lens, row, stride);
  const int* h = hist ? hist + static_cast<int64_t>(row) * kBins : ws.hist + static_cast<int64_t>(row) * kBins;
  const int bstar = threshold_bin<kRefineThreads>(h, k, sh.scan);
  const RowMeta meta = ws.meta[row];
  const float* x = logits + static_cast<int64_t>(row) * stride;
  int32_t* out = indices + static_cast<int64_t>(row) * k;

  bool valid;
  if (bstar == kAllBins) valid = meta.n_gt <= k && meta.n_eq == 0;
  else valid = meta.n_gt < k && meta.n_gt + meta.n_eq >= k && meta.n_eq <= kCandCap;

  if (!valid) {
    whole_row_select<KEY>(sh, x, len, k, out);
    return;
  }
  if (bstar == kAllBins) {
    for (int i = meta.n_gt + threadIdx.x; i < k; i += kRefineThreads) out[i] = -1;
    return;
  }
  const int n = meta.n_eq;
  const int need = k - meta.n_gt;
  const uint2* cand = ws.cand + static_cast<int64_t>(row) * kCandCap;
  if (need == n) {
    for (int i = threadIdx.x; i < n; i += kRefineThreads) out[meta.n_gt + i] = static_cast<int>(cand[i].y);
    return;
  }
  for (int i = threadIdx.x; i < n; i += kRefineThreads) sh.cand[i] = cand[i];
  if (threadIdx.x == 0) sh.out_pos = meta.n_gt;
  __syncthreads();
  int above = 0;
  const uint32_t T = select_key_lds(sh, n, need, &above);
  const int ties_needed = need - above;
  // Count of ties to decide whether the tie set must be cut by column.
  int tc = 0;
  for (int i = threadIdx.x; i < n; i += kRefineThreads) tc += sh.cand[i].x == T ? 1 : 0;
  const int ties = block_sum(tc, sh);
  uint32_t col_cut = 0xFFFFFFFFu;
  if (ties > ties_needed) col_cut = select_col_lds(sh, n, T, ties_needed);
  for (int i0 = 0; i0 < n; i0 += kRefineThreads) {
    const int i = i0 + threadIdx.x;
    bool take = false;
    int col = 0;
    if (i < n) {
      const uint2 c = sh.cand[i];
      take = c.x > T || (c.x == T && c.y <= col_cut);
      col = static_cast<int>(c.y);
    }
    emit(sh, out, k, take, col);
  }
}

}  // namespace

size_t topk_workspace_size(int32_t rows) {
  if (rows <= 0) return 0;
  return align256(sizeof(RowMeta) * rows) + align256(sizeof(int) * kBins * static_cast<size_t>(rows)) +
         sizeof(uint2) * kCandCap * static_cast<size_t>(rows);
}

hipError_t launch_topk_rows(const TopkArgs& a, hipStream_t stream) {
  const Workspace ws = carve(a.workspace, a.rows);
  const bool own_hist = a.hist == nullptr;
  const int64_t chunks64 = (a.logits_stride + kChunk - 1) / kChunk;
  if (chunks64 > 0x7FFFFFFF) return hipErrorInvalidValue;
  const dim3 grid_rows(static_cast<unsigned>(chunks64), static_cast<unsigned>(a.rows));
  hipLaunchKernelGGL(topk_init_kernel, dim3(a.rows), dim3(256), 0, stream, ws, a.rows, own_hist);
  if (own_hist) {
    hipLaunchKernelGGL(topk_hist_kernel, grid_rows, dim3(kCollectThreads), 0, stream, a.logits,
                       a.logits_stride, a.context_lens, ws.hist);
  }
  if (a.key_dtype == IDX_KEY_FP32) {
    hipLaunchKernelGGL(topk_collect_kernel<IDX_KEY_FP32>, grid_rows, dim3(kCollectThreads), 0, stream,
                       a.logits, a.logits_stride, a.hist, a.context_lens, a.k, a.indices, ws);
    hipLaunchKernelGGL(topk_refine_kernel<IDX_KEY_FP32>, dim3(a.rows), dim3(kRefineThreads), 0, stream,
                       a.logits, a.logits_stride, a.hist, a.context_lens, a.k, a.indices, ws);
  } else {
    hipLaunchKernelGGL(topk_collect_kernel<IDX_KEY_FP16>, grid_rows, dim3(kCollectThreads), 0, stream,
                       a.logits, a.logits_stride, a.hist, a.context_lens, a.k, a.indices, ws);
    hipLaunchKernelGGL(topk_refine_kernel<IDX_KEY_FP16>, dim3(a.rows), dim3(kRefineThreads), 0, stream,
                       a.logits, a.logits_stride, a.hist, a.context_lens, a.k, a.indices, ws);
  }
  return hipGetLastError();
}

hipError_t launch_score_histogram(const float* scores, int64_t stride, const int32_t* lens,
                                  int32_t rows, int32_t* hist, hipStream_t stream) {
  const int64_t chunks64 = (stride + kChunk - 1) / kChunk;
  if (chunks64 > 0x7FFFFFFF) return hipErrorInvalidValue;
  hipLaunchKernelGGL(topk_hist_kernel, dim3(static_cast<unsigned>(chunks64), static_cast<unsigned>(rows)),
                     dim3(kCollectThreads), 0, stream, scores, stride, lens, hist);
  return hipGetLastError();
}

}  // namespace pmqa
