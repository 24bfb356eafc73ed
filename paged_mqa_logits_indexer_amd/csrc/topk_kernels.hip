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
// Barriers here order LDS only (lds_barrier): no thread of a workgroup reads
// global memory that another thread of it wrote.
//
// Launch sequence of one topk_rows call (one stream, no host sync):
//   [hist == NULL only] topk_zero_hist + topk_hist: build the row histograms
//                  in the workspace (the first pass the producer's fused
//                  histogram normally replaces)
//   topk_scan      many workgroups per row, one 4096-score chunk each: the
//                  threshold bin b* from the histogram (requested together
//                  with the chunk's scores); the chunk's columns above b* and
//                  its (key, column) candidates of b* go, in column order, to
//                  the chunk's own slots in the workspace, and its two counts
//                  to counts[row][chunk] (plain stores, no atomics)
//   topk_refine    one workgroup per row adds up the chunk counts and checks
//                  them against b*: if they confirm it, the columns above b*
//                  are gathered into the output and the candidates into LDS,
//                  where a radix select on the remaining key bits finishes the
//                  row; otherwise an exact radix select over the whole row
//                  does.  Chunk slots rather than exact output positions keep
//                  the scan free of any cross-workgroup order: positions
//                  would need either a second pass over the scores or a
//                  device-scope handoff between workgroups, which on this
//                  multi-die part means L2 write-backs under the other dies.
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
constexpr int kPerThread = kChunk / kThreads;  // consecutive scores per thread in the scan
constexpr int kAllBins = kBins;             // threshold meaning "every live score"
constexpr int kRefineThreads = 512;         // one workgroup per row finishes it
static_assert(kBins == 4 * kThreads, "threshold_bin: four bins per thread");

struct RowMeta {
  int bstar;  // threshold bin the scan pass used
  int pad0, pad1, pad2;
};

// Scratch of one call.  Per (row, chunk) slot: up to gt_cap columns above b*
// (gt_cap = min(k, 4096): a chunk with k of them already makes the row's
// count contradict b*) and up to 4096 candidates of b*.
struct Workspace {
  RowMeta* meta;   // [rows]
  int2* counts;    // [rows][max_chunks]: (above b*, in b*) per chunk
  int* hist;       // [rows][1024]: histograms built when the caller has none
  int* gt;         // [rows][max_chunks][gt_cap]: columns above b*
  uint2* eq;       // [rows][max_chunks][kChunk]: (key, column) in b*
  int max_chunks;
  int gt_cap;
};

__host__ __device__ inline size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

__host__ __device__ inline int chunks_for(int64_t stride) {
  return static_cast<int>((stride + kChunk - 1) / kChunk);
}

__host__ __device__ inline int gt_cap_for(int k) { return k < kChunk ? k : kChunk; }

__host__ __device__ inline size_t workspace_size(int rows, int max_chunks, int k) {
  const size_t slots = static_cast<size_t>(rows) * max_chunks;
  return align256(sizeof(RowMeta) * rows) + align256(sizeof(int2) * slots) +
         align256(sizeof(int) * kBins * static_cast<size_t>(rows)) +
         align256(sizeof(int) * gt_cap_for(k) * slots) + sizeof(uint2) * kChunk * slots;
}

inline Workspace carve(void* base, int rows, int max_chunks, int k) {
  const size_t slots = static_cast<size_t>(rows) * max_chunks;
  char* p = static_cast<char*>(base);
  Workspace w;
  w.meta = reinterpret_cast<RowMeta*>(p);
  p += align256(sizeof(RowMeta) * rows);
  w.counts = reinterpret_cast<int2*>(p);
  p += align256(sizeof(int2) * slots);
  w.hist = reinterpret_cast<int*>(p);
  p += align256(sizeof(int) * kBins * static_cast<size_t>(rows));
  w.gt = reinterpret_cast<int*>(p);
  p += align256(sizeof(int) * gt_cap_for(k) * slots);
  w.eq = reinterpret_cast<uint2*>(p);
  w.max_chunks = max_chunks;
  w.gt_cap = gt_cap_for(k);
  return w;
}

template <int KEY>
__device__ __forceinline__ uint32_t score_key(float x) {
  if constexpr (KEY == IDX_KEY_FP32) return key_f32(x);
  else return key_f16(f16_bits_rn(x));
}

// Scores are float32, or (F16) the bits of IEEE binary16 values, whose key
// is always the FP16 key.
template <bool F16>
__device__ __forceinline__ const void* score_row(const void* scores, int row, int64_t stride) {
  return static_cast<const char*>(scores) + static_cast<int64_t>(row) * stride * (F16 ? 2 : 4);
}

// Key of score s of a row, and whether the score is selectable (not NaN).
template <int KEY, bool F16>
__device__ __forceinline__ bool score_at(const void* row, int s, uint32_t* key) {
  if constexpr (F16) {
    const uint32_t hb = static_cast<const uint16_t*>(row)[s];
    *key = key_f16(hb);
    return !f16_is_nan(hb);
  } else {
    const float v = static_cast<const float*>(row)[s];
    *key = score_key<KEY>(v);
    return v == v;
  }
}

// The FP16 bits of element e of a 16-byte vector of scores.
template <bool F16>
__device__ __forceinline__ uint32_t half_bits_of(const i32x4& v, int e) {
  if constexpr (F16) return (static_cast<uint32_t>(v[e >> 1]) >> (16 * (e & 1))) & 0xFFFFu;
  else return f16_bits_rn(__int_as_float(v[e]));
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
  lds_barrier();
  int t = 0;
#pragma unroll
  for (int w = 0; w < NT / kWave; ++w) t += s_red[w];
  lds_barrier();
  return t;
}

// Exclusive prefix of v in thread order; *total = block sum.
template <int NT = kThreads>
__device__ __forceinline__ int block_excl_scan(int v, int* s_red, int* total) {
  const int inc = wave_inclusive_scan(v);
  const int wave = threadIdx.x / kWave;
  if (__lane_id() == kWave - 1) s_red[wave] = inc;
  lds_barrier();
  int before = 0, all = 0;
#pragma unroll
  for (int w = 0; w < NT / kWave; ++w) {
    const int t = s_red[w];
    before += (w < wave) ? t : 0;
    all += t;
  }
  lds_barrier();
  *total = all;
  return before + inc - v;
}

// Exclusive prefixes of (a, b) in thread order from one pair of barriers;
// *total = the block sums.
template <int NT>
__device__ __forceinline__ int2 block_excl_scan2(int a, int b, int* s_red, int2* total) {
  const int ia = wave_inclusive_scan(a);
  const int ib = wave_inclusive_scan(b);
  const int wave = threadIdx.x / kWave;
  if (__lane_id() == kWave - 1) {
    s_red[2 * wave] = ia;
    s_red[2 * wave + 1] = ib;
  }
  lds_barrier();
  int ba = 0, bb = 0, ta = 0, tb = 0;
#pragma unroll
  for (int w = 0; w < NT / kWave; ++w) {
    const int u = s_red[2 * w], v = s_red[2 * w + 1];
    ba += w < wave ? u : 0;
    bb += w < wave ? v : 0;
    ta += u;
    tb += v;
  }
  lds_barrier();
  *total = int2{ta, tb};
  return int2{ba + ia - a, bb + ib - b};
}

// Threshold bin of a row: the first bin whose inclusive prefix count reaches
// k, or kAllBins when the histogram holds at most k scores.  Thread t holds
// the counts of bins 4t .. 4t+3.
__device__ int threshold_bin(const int (&c)[4], int k, int* s_red) {
  const int sum = c[0] + c[1] + c[2] + c[3];
  int total = 0;
  int run = block_excl_scan(sum, s_red, &total);
  if (total <= k) return kAllBins;
  // The crossing lies in exactly one thread's bins (counts are non-negative
  // in any histogram this call produced; for a foreign one any bin is fine,
  // the counts checked later decide).
  if (threadIdx.x == 0) s_red[kWaves] = kAllBins;
  lds_barrier();
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    if (run < k && run + c[i] >= k) s_red[kWaves] = threadIdx.x * 4 + i;
    run += c[i];
  }
  lds_barrier();
  const int bstar = s_red[kWaves];
  lds_barrier();
  return bstar;
}

// ---------------------------------------------------------------------------
__global__ void topk_zero_hist_kernel(int* hist, int rows) {
  const int64_t n = static_cast<int64_t>(rows) * kBins;
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; i < n;
       i += static_cast<int64_t>(gridDim.x) * blockDim.x)
    hist[i] = 0;
}

// Histogram of each row's live non-NaN scores, added to hist_out.
template <bool F16>
__global__ __launch_bounds__(kThreads) void topk_hist_kernel(const void* __restrict__ logits,
                                                             int64_t stride,
                                                             const int32_t* __restrict__ lens,
                                                             int* __restrict__ hist_out) {
  __shared__ int s_hist[kBins];
  const int row = blockIdx.y;
  const int len = clamp_len(lens, row, stride);
  const int s0 = blockIdx.x * kChunk;
  if (s0 >= len) return;
  for (int i = threadIdx.x; i < kBins; i += kThreads) s_hist[i] = 0;
  lds_barrier();
  const char* x = static_cast<const char*>(score_row<F16>(logits, row, stride));
  const int s1 = min(len, s0 + kChunk);
  constexpr int kPerVec = F16 ? 8 : 4;  // scores per 16-byte load
  for (int s = s0 + threadIdx.x * kPerVec; s < s1; s += kThreads * kPerVec) {
    // In bounds: s < len <= stride, s and the stride multiples of kPerVec.
    const i32x4 v = *reinterpret_cast<const i32x4*>(x + static_cast<int64_t>(s) * (F16 ? 2 : 4));
#pragma unroll
    for (int e = 0; e < kPerVec; ++e) {
      if (s + e < s1) {
        const uint32_t hb = half_bits_of<F16>(v, e);
        if (!f16_is_nan(hb)) atomicAdd(&s_hist[coarse_bin_f16(hb)], 1);
      }
    }
  }
  lds_barrier();
  unsigned long long* gh = reinterpret_cast<unsigned long long*>(hist_out + static_cast<int64_t>(row) * kBins);
  const uint2* sh = reinterpret_cast<const uint2*>(s_hist);
  for (int i = threadIdx.x; i < kBins / 2; i += kThreads) {
    const uint2 v = sh[i];
    if (v.x | v.y) atomicAdd(gh + i, (static_cast<unsigned long long>(v.y) << 32) | v.x);
  }
}

// ---------------------------------------------------------------------------
// Thread t of a chunk's workgroup takes 16 consecutive columns; a block scan
// of the per-thread counts gives every column its position in the chunk's
// slot, so each slot list is in column order.
template <int KEY, bool F16>
__global__ __launch_bounds__(kThreads) void topk_scan_kernel(const void* __restrict__ logits,
                                                             int64_t stride,
                                                             const int32_t* __restrict__ hist,
                                                             const int32_t* __restrict__ lens, int k,
                                                             Workspace ws) {
  __shared__ int s_red[kWaves + 1];
  const int row = blockIdx.y;
  const int c = blockIdx.x;
  const int len = clamp_len(lens, row, stride);
  if (c >= row_chunks(len)) return;

  // The histogram and the chunk's scores are requested together.
  const int* h = (hist ? hist : ws.hist) + static_cast<int64_t>(row) * kBins + threadIdx.x * 4;
  const int2 h01 = *reinterpret_cast<const int2*>(h);  // 8-B aligned
  const int2 h23 = *reinterpret_cast<const int2*>(h + 2);
  const char* x = static_cast<const char*>(score_row<F16>(logits, row, stride));
  const int s0 = c * kChunk + threadIdx.x * kPerThread;
  constexpr int kPerVec = F16 ? 8 : 4;  // scores per 16-byte load
  i32x4 v[kPerThread / kPerVec];
#pragma unroll
  for (int i = 0; i < kPerThread / kPerVec; ++i) {
    // In bounds: s0 + kPerVec*i < len <= stride, both multiples of kPerVec.
    const int s = s0 + kPerVec * i;
    v[i] = s < len ? *reinterpret_cast<const i32x4*>(x + static_cast<int64_t>(s) * (F16 ? 2 : 4))
                   : i32x4{0, 0, 0, 0};
  }
  const int hc[4] = {h01.x, h01.y, h23.x, h23.y};
  const int bstar = threshold_bin(hc, k, s_red);

  uint32_t gmask = 0u, emask = 0u;  // bit e: column s0 + e
#pragma unroll
  for (int e = 0; e < kPerThread; ++e) {
    const uint32_t hb = half_bits_of<F16>(v[e / kPerVec], e % kPerVec);
    const bool live = s0 + e < len && !f16_is_nan(hb);
    const int bin = coarse_bin_f16(hb);
    gmask |= static_cast<uint32_t>(live && bin < bstar) << e;
    emask |= static_cast<uint32_t>(live && bin == bstar) << e;
  }
  // Both counts in one scan: each is at most kChunk < 2^16.
  int tot = 0;
  const int pre = block_excl_scan(__popc(gmask) | (__popc(emask) << 16), s_red, &tot);
  const int64_t slot = static_cast<int64_t>(row) * ws.max_chunks + c;
  int* gt = ws.gt + slot * ws.gt_cap;
  uint2* eq = ws.eq + slot * kChunk;
  int og = pre & 0xFFFF, oe = pre >> 16;
#pragma unroll
  for (int e = 0; e < kPerThread; ++e) {
    if ((gmask >> e) & 1u) {
      if (og < ws.gt_cap) gt[og] = s0 + e;
      ++og;
    }
    if ((emask >> e) & 1u) {
      uint32_t key;
      if constexpr (F16) key = key_f16(half_bits_of<F16>(v[e / kPerVec], e % kPerVec));
      else key = score_key<KEY>(__int_as_float(v[e / kPerVec][e % kPerVec]));
      eq[oe++] = uint2{key, static_cast<uint32_t>(s0 + e)};
    }
  }
  if (threadIdx.x == 0) {
    ws.counts[slot] = int2{tot & 0xFFFF, tot >> 16};
    if (c == 0) ws.meta[row] = RowMeta{bstar, 0, 0, 0};
  }
}

// ---------------------------------------------------------------------------
// Shared memory of the refine pass.
struct RefineShared {
  uint2 cand[kCandCap];   // 64 KiB
  int pre_g[kRefineThreads];  // a block of chunks: offsets of their slot lists
  int pre_e[kRefineThreads];
  int cnt_g[kRefineThreads];  // and their lengths
  int cnt_e[kRefineThreads];
  int digit_hist[256];
  int red[2 * (kRefineThreads / kWave) + 4];
  uint32_t small[kWave];  // the few keys left after a radix pass
  int small_n;
  int out_pos;
  uint32_t red_or, red_and;
  int bcast[4];
};

__device__ __forceinline__ void block_or_and(uint32_t o, uint32_t a, RefineShared& sh) {
  if (threadIdx.x == 0) {
    sh.red_or = 0u;
    sh.red_and = 0xFFFFFFFFu;
  }
  lds_barrier();
  o = wave_or(o);
  a = wave_and(a);
  if (__lane_id() == 0) {
    atomicOr(&sh.red_or, o);
    atomicAnd(&sh.red_and, a);
  }
  lds_barrier();
}

// Given digit_hist (256 counts), the digit d at which the running count
// taken from the largest digit down first reaches `need`; *before = the count
// strictly above d, *in_bin = the count of d.
__device__ int pick_digit(RefineShared& sh, int need, int* before, int* in_bin) {
  if (threadIdx.x < kWave) {
    const int lane = threadIdx.x;
    int c[4], sum = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      c[i] = sh.digit_hist[255 - (lane * 4 + i)];
      sum += c[i];
    }
    const int inc = wave_inclusive_scan(sum);
    int run = inc - sum;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if (run < need && run + c[i] >= need) {
        sh.bcast[0] = 255 - (lane * 4 + i);
        sh.bcast[1] = run;
        sh.bcast[2] = c[i];
      }
      run += c[i];
    }
  }
  lds_barrier();
  const int d = sh.bcast[0];
  *before = sh.bcast[1];
  *in_bin = sh.bcast[2];
  lds_barrier();
  return d;
}

__device__ __forceinline__ int top_bit(uint32_t x) { return 31 - __clz(x); }

// The need-th largest of the m <= 64 candidate keys that match (prefix,
// fixed): the candidates are collected in LDS and wave 0 ranks each against
// all the others.  *above = how many of them exceed the result.
__device__ uint32_t rank_small(RefineShared& sh, int n, uint32_t prefix, uint32_t fixed, int need,
                               int* above) {
  for (int i = threadIdx.x; i < n; i += kRefineThreads) {
    const uint32_t key = sh.cand[i].x;
    if (((key ^ prefix) & fixed) == 0u) sh.small[atomicAdd(&sh.small_n, 1)] = key;
  }
  lds_barrier();
  if (threadIdx.x < kWave) {
    const int m = sh.small_n;
    const int lane = threadIdx.x;
    const uint32_t kj = lane < m ? sh.small[lane] : 0u;
    int gtc = 0, gec = 0;
    for (int i = 0; i < m; ++i) {
      const uint32_t ki = sh.small[i];
      gtc += ki > kj ? 1 : 0;
      gec += ki >= kj ? 1 : 0;
    }
    // Lanes holding the answer: fewer than `need` keys above, at least
    // `need` at or above (equal keys all qualify and agree).
    const uint64_t ok = __ballot(lane < m && gtc < need && need <= gec);
    const int src = first_lane(ok);
    if (lane == 0) {
      sh.bcast[0] = __builtin_amdgcn_readlane(static_cast<int>(kj), src);
      sh.bcast[1] = __builtin_amdgcn_readlane(gtc, src);
    }
  }
  lds_barrier();
  const uint32_t T = static_cast<uint32_t>(sh.bcast[0]);
  *above = sh.bcast[1];
  lds_barrier();
  return T;
}

// Radix select over the n LDS candidates: the key T of the need-th largest
// key; *above = how many keys exceed T.  Bits every key shares are skipped,
// and once a digit holds at most 64 keys they are ranked directly.
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
      if (threadIdx.x == 0) sh.small_n = 0;
      lds_barrier();
      for (int i = threadIdx.x; i < n; i += kRefineThreads) {
        const uint32_t key = sh.cand[i].x;
        if (((key ^ prefix) & fixed) == 0u) atomicAdd(&sh.digit_hist[(key >> shift) & 0xFFu], 1);
      }
      lds_barrier();
      int before = 0, in_bin = 0;
      const int d = pick_digit(sh, need, &before, &in_bin);
      need -= before;
      gt += before;
      prefix |= static_cast<uint32_t>(d) << shift;
      fixed |= 0xFFu << shift;
      if (shift == 0) break;
      if (in_bin <= kWave) {
        int over = 0;
        prefix = rank_small(sh, n, prefix, fixed, need, &over);
        gt += over;
        break;
      }
      shift = shift >= 8 ? shift - 8 : 0;
    }
  }
  *above = gt;
  return prefix;
}

// Append this thread's column to the output through a block-wide LDS counter.
__device__ __forceinline__ void emit(RefineShared& sh, int32_t* out, int k, bool take, int col) {
  const uint64_t m = __ballot(take);
  if (!m) return;
  int pos = 0;
  if (__lane_id() == 0) pos = atomicAdd(&sh.out_pos, __popcll(m));
  pos = __builtin_amdgcn_readlane(pos, 0) + lanes_below(m);
  if (take && pos < k) out[pos] = col;
}

// Exact selection over the whole row: a stale histogram, or a threshold bin
// with more candidates than the capacity.
template <int KEY, bool F16>
__device__ void whole_row_select(RefineShared& sh, const void* __restrict__ x, int len, int k,
                                 int32_t* __restrict__ out) {
  constexpr int kKey = F16 ? IDX_KEY_FP16 : KEY;
  int cnt = 0;
  for (int s = threadIdx.x; s < len; s += kRefineThreads) {
    uint32_t key;
    cnt += score_at<KEY, F16>(x, s, &key) ? 1 : 0;
  }
  const int n = block_sum<kRefineThreads>(cnt, sh.red);
  if (threadIdx.x == 0) sh.out_pos = 0;
  lds_barrier();
  if (n <= k) {
    for (int s0 = 0; s0 < len; s0 += kRefineThreads) {
      const int s = s0 + threadIdx.x;
      uint32_t key;
      emit(sh, out, k, s < len && score_at<KEY, F16>(x, s, &key), s);
    }
    lds_barrier();
    for (int i = n + threadIdx.x; i < k; i += kRefineThreads) out[i] = -1;
    return;
  }
  constexpr int kKeyBits = kKey == IDX_KEY_FP32 ? 32 : 16;
  uint32_t prefix = 0u, fixed = 0u;
  int need = k;
  for (int shift = kKeyBits - 8; shift >= 0; shift -= 8) {
    for (int i = threadIdx.x; i < 256; i += kRefineThreads) sh.digit_hist[i] = 0;
    lds_barrier();
    for (int s = threadIdx.x; s < len; s += kRefineThreads) {
      uint32_t key;
      if (!score_at<KEY, F16>(x, s, &key)) continue;
      if (((key ^ prefix) & fixed) == 0u) atomicAdd(&sh.digit_hist[(key >> shift) & 0xFFu], 1);
    }
    lds_barrier();
    int before = 0;
    int in_bin = 0;
    const int d = pick_digit(sh, need, &before, &in_bin);
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
    uint32_t key;
    if (s < len && score_at<KEY, F16>(x, s, &key)) {
      above = key > T;
      tie = key == T;
    }
    int slice_ties = 0;
    const int rank = taken_ties + block_excl_scan<kRefineThreads>(tie ? 1 : 0, sh.red, &slice_ties);
    emit(sh, out, k, above || (tie && rank < need), s);
    taken_ties += slice_ties;
  }
}

template <int NT>
__device__ __forceinline__ int block_max(int v, int* s_red) {
  v = wave_max(v);
  if (__lane_id() == 0) s_red[threadIdx.x / kWave] = v;
  lds_barrier();
  int m = s_red[0];
#pragma unroll
  for (int w = 1; w < NT / kWave; ++w) m = max(m, s_red[w]);
  lds_barrier();
  return m;
}

// The gather of a row's chunk slots, in chunk order: the columns above b*
// to out[0 .. n_gt), the candidates to sh.cand (or, when cand_out is given,
// only their columns to cand_out[0 .. n_eq)), so both lists stay in column
// order.  Each chunk's counts must fit its slot, which the caller's count
// check guarantees.
//
// Chunks are taken kRefineThreads at a time; each gets tpc threads (a power
// of two), and a thread's share of a round is kGatherPer consecutive entries
// of both of its chunk's lists.  Every load of a round is issued before its
// first store, so a round costs one memory round trip; loads are
// unconditional (clamped into the slot), because a load under a branch
// would make the compiler wait for every load issued before it.
constexpr int kGatherPer = 8;

struct GatherLane {
  int tpc;      // threads per chunk
  int cc;       // this thread's chunk in the block (clamped to the last one)
  bool active;  // the block has a chunk for this thread
  int l0;       // first entry of this thread's share of a round
};

__device__ __forceinline__ GatherLane gather_lane(int nb) {
  GatherLane g;
  g.tpc = 1 << (31 - __clz(kRefineThreads / nb));
  const int c = static_cast<int>(threadIdx.x) / g.tpc;
  g.active = c < nb;
  g.cc = g.active ? c : nb - 1;
  g.l0 = (static_cast<int>(threadIdx.x) % g.tpc) * kGatherPer;
  return g;
}

__device__ __forceinline__ void load_round(const int* gsrc, const uint2* esrc, int l, int glast, int elast,
                                           int (&gv)[kGatherPer], uint2 (&ev)[kGatherPer]) {
#pragma unroll
  for (int u = 0; u < kGatherPer; ++u) {
    gv[u] = gsrc[min(l + u, glast)];
    ev[u] = esrc[min(l + u, elast)];
  }
}

__device__ __forceinline__ void store_round(RefineShared& sh, bool active, int l, int cg, int ce, int og,
                                            int oe, const int (&gv)[kGatherPer],
                                            const uint2 (&ev)[kGatherPer], int32_t* __restrict__ out,
                                            int32_t* __restrict__ cand_out) {
#pragma unroll
  for (int u = 0; u < kGatherPer; ++u) {
    if (active && l + u < cg) out[og + l + u] = gv[u];
    if (active && l + u < ce) {
      if (cand_out) cand_out[oe + l + u] = static_cast<int32_t>(ev[u].y);
      else sh.cand[oe + l + u] = ev[u];
    }
  }
}

// The rounds of one block of chunks after any already done: entries from
// r_begin on.  cg/ce/og/oe: counts and list offsets of this thread's chunk.
__device__ __forceinline__ void gather_rest(RefineShared& sh, const GatherLane& g, const int* gsrc,
                                            const uint2* esrc, int r_begin, int cg, int ce, int og, int oe,
                                            int32_t* __restrict__ out, int32_t* __restrict__ cand_out) {
  const int step = g.tpc * kGatherPer;
  for (int r0 = r_begin; r0 < max(cg, ce); r0 += step) {  // per chunk; no barrier inside
    int gv[kGatherPer];
    uint2 ev[kGatherPer];
    load_round(gsrc, esrc, r0 + g.l0, max(cg - 1, 0), max(ce - 1, 0), gv, ev);
    store_round(sh, g.active, r0 + g.l0, cg, ce, og, oe, gv, ev, out, cand_out);
  }
}

// Blocks of chunks from cb0 on (rows of more than kRefineThreads chunks);
// base_g / base_e = the list entries of the chunks before cb0.
__device__ void gather_blocks(RefineShared& sh, const Workspace& ws, int64_t slot0, int nch, int cb0,
                              int base_g, int base_e, int32_t* __restrict__ out,
                              int32_t* __restrict__ cand_out) {
  for (int cb = cb0; cb < nch; cb += kRefineThreads) {
    const int j = cb + threadIdx.x;
    const int2 v = j < nch ? ws.counts[slot0 + j] : int2{0, 0};
    int2 tot;
    const int2 pre = block_excl_scan2<kRefineThreads>(v.x, v.y, sh.red, &tot);
    sh.pre_g[threadIdx.x] = pre.x;
    sh.pre_e[threadIdx.x] = pre.y;
    sh.cnt_g[threadIdx.x] = v.x;
    sh.cnt_e[threadIdx.x] = v.y;
    lds_barrier();
    const GatherLane g = gather_lane(min(kRefineThreads, nch - cb));
    gather_rest(sh, g, ws.gt + (slot0 + cb + g.cc) * ws.gt_cap, ws.eq + (slot0 + cb + g.cc) * kChunk, 0,
                sh.cnt_g[g.cc], sh.cnt_e[g.cc], base_g + sh.pre_g[g.cc], base_e + sh.pre_e[g.cc], out,
                cand_out);
    base_g += tot.x;
    base_e += tot.y;
    lds_barrier();
  }
}

// Finishes each row after the scan pass: checks the real counts against b*,
// then gathers the chunk slots and refines the candidates, or selects over
// the whole row.
template <int KEY, bool F16>
__global__ __launch_bounds__(kRefineThreads) void topk_refine_kernel(const void* __restrict__ logits,
                                                                     int64_t stride,
                                                                     const int32_t* __restrict__ lens,
                                                                     int k, int32_t* __restrict__ indices,
                                                                     Workspace ws) {
  __shared__ RefineShared sh;
  const int row = blockIdx.x;
  const int len = clamp_len(lens, row, stride);
  const int nch = row_chunks(len);
  const int bstar = ws.meta[row].bstar;
  const int64_t slot0 = static_cast<int64_t>(row) * ws.max_chunks;
  const void* x = score_row<F16>(logits, row, stride);
  int32_t* out = indices + static_cast<int64_t>(row) * k;

  // Slots have fixed addresses, so the first round of the gather is
  // requested together with the counts, before they are known (clamped into
  // the slot; entries past a chunk's count are never used).
  const GatherLane g = gather_lane(min(kRefineThreads, nch));
  const int2 first_raw = ws.counts[slot0 + min(static_cast<int>(threadIdx.x), nch - 1)];  // unconditional load
  const int2 first = static_cast<int>(threadIdx.x) < nch ? first_raw : int2{0, 0};
  const int* gsrc = ws.gt + (slot0 + g.cc) * ws.gt_cap;
  const uint2* esrc = ws.eq + (slot0 + g.cc) * kChunk;
  int gv[kGatherPer];
  uint2 ev[kGatherPer];
  load_round(gsrc, esrc, g.l0, ws.gt_cap - 1, kChunk - 1, gv, ev);

  // One block scan of both counts gives the first block's list offsets and
  // its totals; longer rows add the sums of the other chunks.
  int2 tot;
  const int2 pre = block_excl_scan2<kRefineThreads>(first.x, first.y, sh.red, &tot);
  int n_gt = tot.x, n_eq = tot.y;
  if (nch > kRefineThreads) {
    int tg = 0, te = 0;
    for (int i = kRefineThreads + threadIdx.x; i < nch; i += kRefineThreads) {
      const int2 v = ws.counts[slot0 + i];
      tg += v.x;
      te += v.y;
    }
    int2 rest;
    block_excl_scan2<kRefineThreads>(tg, te, sh.red, &rest);
    n_gt += rest.x;
    n_eq += rest.y;
  }
  bool valid;
  if (bstar == kAllBins) valid = n_gt <= k && n_eq == 0;
  else valid = n_gt < k && n_gt + n_eq >= k && n_eq <= kCandCap;
  if (!valid) {
    whole_row_select<KEY, F16>(sh, x, len, k, out);
    return;
  }
  const int need = k - n_gt;
  // When every candidate is taken (none exist below the all-bins threshold)
  // their columns go straight to the output.
  const bool direct = bstar == kAllBins || need == n_eq;
  int32_t* cand_out = direct ? out + n_gt : nullptr;
  sh.pre_g[threadIdx.x] = pre.x;
  sh.pre_e[threadIdx.x] = pre.y;
  sh.cnt_g[threadIdx.x] = first.x;
  sh.cnt_e[threadIdx.x] = first.y;
  lds_barrier();
  {
    const int cg = sh.cnt_g[g.cc], ce = sh.cnt_e[g.cc], og = sh.pre_g[g.cc], oe = sh.pre_e[g.cc];
    store_round(sh, g.active, g.l0, cg, ce, og, oe, gv, ev, out, cand_out);
    gather_rest(sh, g, gsrc, esrc, g.tpc * kGatherPer, cg, ce, og, oe, out, cand_out);
  }
  lds_barrier();
  if (nch > kRefineThreads) gather_blocks(sh, ws, slot0, nch, kRefineThreads, tot.x, tot.y, out, cand_out);
  if (direct) {
    for (int i = n_gt + n_eq + threadIdx.x; i < k; i += kRefineThreads) out[i] = -1;
    return;
  }
  if (threadIdx.x == 0) sh.out_pos = n_gt;
  lds_barrier();
  int above = 0;
  const uint32_t T = select_key_lds(sh, n_eq, need, &above);
  // Every key above T is taken, and of the keys equal to T the lowest
  // columns: the candidate list is in column order, so those are the first
  // need - above ties in list order.  Thread t ranks a run of consecutive
  // candidates.
  const int ties_needed = need - above;
  const int per = (n_eq + kRefineThreads - 1) / kRefineThreads;
  const int i_begin = min(n_eq, static_cast<int>(threadIdx.x) * per);
  const int i_end = min(n_eq, i_begin + per);
  int my_ties = 0;
  for (int i = i_begin; i < i_end; ++i) my_ties += sh.cand[i].x == T ? 1 : 0;
  int all_ties = 0;
  int rank = block_excl_scan<kRefineThreads>(my_ties, sh.red, &all_ties);
  for (int u = 0; u < per; ++u) {
    const int i = i_begin + u;
    bool take = false;
    int col = 0;
    if (i < i_end) {
      const uint2 cd = sh.cand[i];
      const bool tie = cd.x == T;
      take = cd.x > T || (tie && rank < ties_needed);
      rank += tie ? 1 : 0;
      col = static_cast<int>(cd.y);
    }
    emit(sh, out, k, take, col);
  }
}

}  // namespace

size_t topk_workspace_size(int32_t rows, int64_t logits_stride, int32_t k) {
  if (rows <= 0 || logits_stride <= 0 || k <= 0) return 0;
  return workspace_size(rows, chunks_for(logits_stride), k);
}

template <int KEY, bool F16>
void launch_select(const TopkArgs& a, const Workspace& ws, dim3 grid, hipStream_t stream,
                   hipEvent_t start, hipEvent_t stop) {
  launch_kernel(topk_scan_kernel<KEY, F16>, grid, dim3(kThreads), stream, start, nullptr, a.logits,
                a.logits_stride, a.hist, a.context_lens, a.k, ws);
  launch_kernel(topk_refine_kernel<KEY, F16>, dim3(a.rows), dim3(kRefineThreads), stream, nullptr, stop,
                a.logits, a.logits_stride, a.context_lens, a.k, a.indices, ws);
}

hipError_t launch_topk_rows(const TopkArgs& a, hipStream_t stream, LaunchEvents ev) {
  const int max_chunks = chunks_for(a.logits_stride);
  const Workspace ws = carve(a.workspace, a.rows, max_chunks, a.k);
  const dim3 grid(static_cast<unsigned>(max_chunks), static_cast<unsigned>(a.rows));
  hipEvent_t start = ev.start;  // recorded by the first kernel of the call
  if (a.hist == nullptr) {
    launch_kernel(topk_zero_hist_kernel, dim3(min(1024, (a.rows * kBins + 255) / 256)), dim3(256), stream,
                  start, nullptr, ws.hist, a.rows);
    start = nullptr;
    if (a.logits_f16)
      launch_kernel(topk_hist_kernel<true>, grid, dim3(kThreads), stream, nullptr, nullptr, a.logits,
                    a.logits_stride, a.context_lens, ws.hist);
    else
      launch_kernel(topk_hist_kernel<false>, grid, dim3(kThreads), stream, nullptr, nullptr, a.logits,
                    a.logits_stride, a.context_lens, ws.hist);
  }
  // FP16 scores are ranked by their FP16 keys.
  if (a.logits_f16) launch_select<IDX_KEY_FP16, true>(a, ws, grid, stream, start, ev.stop);
  else if (a.key_dtype == IDX_KEY_FP32) launch_select<IDX_KEY_FP32, false>(a, ws, grid, stream, start, ev.stop);
  else launch_select<IDX_KEY_FP16, false>(a, ws, grid, stream, start, ev.stop);
  return hipGetLastError();
}

hipError_t launch_score_histogram(const float* scores, int64_t stride, const int32_t* lens,
                                  int32_t rows, int32_t* hist, hipStream_t stream) {
  const int64_t chunks64 = (stride + kChunk - 1) / kChunk;
  if (chunks64 > 0x7FFFFFFF) return hipErrorInvalidValue;
  hipLaunchKernelGGL(topk_hist_kernel<false>, dim3(static_cast<unsigned>(chunks64), static_cast<unsigned>(rows)),
                     dim3(kThreads), 0, stream, scores, stride, lens, hist);
  return hipGetLastError();
}

}  // namespace pmqa
