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
//   rows of at most 16384 scores (stride <= 16384): topk_row, one 512-thread
//                  workgroup per row, whole row in registers: the threshold
//                  bin b* from the histogram (or from one it builds in LDS
//                  when there is none), the columns above b* straight to the
//                  output, the candidates of b* to LDS, where a radix select
//                  on the remaining key bits finishes the row (from
//                  registers, up to four candidates per thread, when the bin
//                  holds at most 2048).
//   longer rows:
//   [hist == NULL] topk_hist: build the row histograms in the workspace
//                  (the first pass the producer's fused histogram normally
//                  replaces); every call leaves them zero for the next one,
//                  as the finish pass clears the bins it reads
//   topk_collect   one 256-thread workgroup per 4096-score chunk: b* from the
//                  histogram (requested together with the chunk's scores),
//                  then one 64-bit atomic add on the row's counter pair
//                  (above b*, in b*) reserves the chunk's places: columns
//                  above b* go straight to the output (places below k), the
//                  (key, column) candidates of b* to the row's candidate
//                  buffer (places below 16384)
//   topk_finish    one 512-thread workgroup per row reads the counter pair
//                  (with b*, the slots and the first 1024 candidates from
//                  each end) and checks it against b*: if it confirms b*,
//                  the candidates are ranked -- from registers when those
//                  early loads hold them all, after a cut by sub-bins when
//                  the bin holds more than 2048, else in LDS as above;
//                  otherwise an exact radix select over the whole row
//                  rewrites the output.  It then clears the counter pair,
//                  sub-bins and built bins for the next call.
//
// Scores are classified against the FP16-key range of b* (bin_key_range),
// not by computing each score's bin.  Places taken by atomics put neither
// list in column order: ties at the final key are cut by a radix select on
// the column.
//
// Why the result is exact whatever the histogram holds: bin() is
// non-increasing in the score and in its FP16 rounding, so every column of a
// lower bin has a strictly larger key than every column of a higher bin.  If
// the scan counts n_gt columns above b* and n_eq in it with
// n_gt < k <= n_gt + n_eq, the top-k is those n_gt columns plus the best
// k - n_gt of the candidates.  Any other count means the histogram was not the
// histogram of these scores, and the row is selected from scratch.
#include <mutex>

#include "bin_key_range.h"
#include "indexer_common.h"
#include "launches.h"

namespace pmqa {
namespace {

constexpr int kThreads = 256;               // histogram and collect workgroups
constexpr int kWaves = kThreads / kWave;
constexpr int kPerThread = 16;              // consecutive scores per thread
constexpr int kChunk = kThreads * kPerThread;  // 4096 scores per collect workgroup
constexpr int kChunkShift = 12;
static_assert(kChunk == 1 << kChunkShift, "chunks are 2^kChunkShift scores");
constexpr int kRefineThreads = 512;         // row and finish workgroups
constexpr int kRowSpan = kRefineThreads * kPerThread;  // 8192: rows topk_row takes whole
constexpr int kAllBins = kBins;             // threshold meaning "every live score"
constexpr int kSparseBlock = 8;             // keys per block of the two-level candidate indexer
static_assert(kBins == 4 * kThreads, "collect: four bins per thread");
static_assert(kBins == 2 * kRefineThreads, "row and finish: two bins per thread");
// Candidates of the threshold bin the selector refines in LDS: twice the
// pages' capacity of 8192 (which stays the largest k), so that a threshold
// bin of up to 16384 scores -- one row of a verify batch whose scores mostly
// saturate holds about 16,000 -- is still refined from the collected
// candidates instead of by passes over the whole row; LDS holds 128 KiB of
// them beside the select's own arrays.
constexpr int kCandBuf = 2 * kCandCap;
static_assert(kRowSpan <= kCandBuf, "a whole row's candidates fit the LDS buffer");
constexpr int kRowSpanMax = 2 * kRowSpan;  // 16384: rows topk_row takes in two parts per thread

// Scratch of the chunked path, one fixed-size record per row, so a row's
// counters sit at the same place whatever the call's row count or stride:
//   counters  two (above b*) | (in b*) << 32 pairs.  Even collect workgroups
//             place their columns from the front of the output row and of
//             the candidate buffer, odd ones from the back, which halves the
//             atomics on each counter; the lists meet in the middle only when
//             the counts contradict b*.  The finish pass leaves them zero.
//             Then b* as the collect pass found it (the finish pass takes it
//             from here instead of scanning the histogram again); the
//             counters and b* are padded to 256 bytes.
//   sub       256 sub-bins of the threshold bin (its FP16-key range cut into
//             256 equal parts), added to by the collect workgroups from the
//             candidates they place; the finish pass cuts the threshold bin
//             once more with it and refines only the candidates of one
//             sub-bin (it checks the cut against the candidates' real counts
//             and, should they disagree, refines the whole bin), then leaves
//             it zero
//   hist      1024 bins, built here when the caller has no histogram (left
//             zero by the finish pass as well)
//   cand      16384 (key, column) candidates of b*
//   slots     the two counts of each collect workgroup, stored (not added),
//             so their sums are this call's true counts whatever the
//             counters held before it: a counter pair that did not start at
//             zero (a workspace never used before, or overwritten since) is
//             detected exactly, and its row is selected from scratch.
constexpr int kMaxCollectWgs = 1024;                 // per row: rows of up to 2^23 scores
constexpr int kSubBins = 256;
// Threshold bins of more than this many scores are cut once more by their
// sub-bins before the select; smaller ones are selected whole (two selects
// over a few hundred candidates cost more than one).
constexpr int kCutMin = 2048;
constexpr size_t kRecCount = 0;
constexpr size_t kRecSub = 256;
constexpr size_t kRecHist = kRecSub + sizeof(int) * kSubBins;
constexpr size_t kRecCand = kRecHist + sizeof(int) * kBins;
constexpr size_t kRecSlots = kRecCand + sizeof(uint2) * kCandBuf;
constexpr size_t kRowScratchBytes = kRecSlots + sizeof(int) * kMaxCollectWgs;  // 140,544
static_assert(kRowScratchBytes % 256 == 0, "records keep 256-byte alignment");
constexpr int64_t kRecHistStride = static_cast<int64_t>(kRowScratchBytes / sizeof(int));  // ints per record
constexpr int64_t kMaxChunkedStride = int64_t{2} * kMaxCollectWgs * kThreads * kPerThread;  // 2^23

struct Workspace {
  char* base;
  __device__ unsigned long long* count(int row) const {
    return reinterpret_cast<unsigned long long*>(base + static_cast<size_t>(row) * kRowScratchBytes + kRecCount);
  }
  // b* of the row's last collect pass (after the two counter pairs)
  __device__ int* bstar(int row) const {
    return reinterpret_cast<int*>(base + static_cast<size_t>(row) * kRowScratchBytes + kRecCount + 16);
  }
  __host__ __device__ int* hist(int row) const {
    return reinterpret_cast<int*>(base + static_cast<size_t>(row) * kRowScratchBytes + kRecHist);
  }
  __device__ uint2* cand(int row) const {
    return reinterpret_cast<uint2*>(base + static_cast<size_t>(row) * kRowScratchBytes + kRecCand);
  }
  __device__ int* sub(int row) const {
    return reinterpret_cast<int*>(base + static_cast<size_t>(row) * kRowScratchBytes + kRecSub);
  }
  __device__ int* slots(int row) const {
    return reinterpret_cast<int*>(base + static_cast<size_t>(row) * kRowScratchBytes + kRecSlots);
  }
};

__host__ __device__ inline int chunks_for(int64_t stride) {
  return static_cast<int>((stride + kChunk - 1) / kChunk);
}

__host__ __device__ inline size_t workspace_size(int rows) { return kRowScratchBytes * static_cast<size_t>(rows); }

inline Workspace carve(void* base) { return Workspace{static_cast<char*>(base)}; }

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

// Threshold bin of a row from NT threads holding B = 1024 / NT consecutive
// bins each: the first bin whose running count reaches k, or kAllBins when
// the histogram holds at most k scores; with it, the histogram's count before
// that bin and in it.  The least such bin is taken, so all workgroups of a
// row agree even on a foreign histogram with negative counts (whose crossing
// need not be unique); the counts checked later decide.  s_red holds
// NT / 64 + 3 entries.
struct Threshold {
  int bin, before, count;
};

template <int NT, int B>
__device__ __forceinline__ Threshold threshold_bin(const int (&c)[B], int k, int* s_red) {
  int sum = 0;
#pragma unroll
  for (int i = 0; i < B; ++i) sum += c[i];
  int total = 0;
  const int run0 = block_excl_scan<NT>(sum, s_red, &total);
  if (total <= k) return Threshold{kAllBins, total, 0};
  constexpr int kSlot = NT / kWave;
  if (threadIdx.x == 0) s_red[kSlot] = kAllBins;
  lds_barrier();
  int run = run0;
#pragma unroll
  for (int i = 0; i < B; ++i) {
    if (run < k && run + c[i] >= k) atomicMin(&s_red[kSlot], static_cast<int>(threadIdx.x) * B + i);
    run += c[i];
  }
  lds_barrier();
  const int bstar = s_red[kSlot];
  if (static_cast<int>(threadIdx.x) == bstar / B) {
    run = run0;
#pragma unroll
    for (int i = 0; i < B; ++i) {
      if (i == bstar % B) {
        s_red[kSlot + 1] = run;
        s_red[kSlot + 2] = c[i];
      }
      run += c[i];
    }
  }
  lds_barrier();
  const Threshold t{bstar, s_red[kSlot + 1], s_red[kSlot + 2]};
  lds_barrier();
  return t;
}

// The FP16 keys of the scores above b* lie in [hi, key(+inf)], those in b*
// in [lo, hi); NaNs fall outside both.  Unsigned differences test each range
// with one compare.
struct Classifier {
  uint32_t lo, eq_span, hi, gt_span;
  __device__ __forceinline__ explicit Classifier(int bstar) {
    const KeyRange r = bin_key_range(bstar);
    lo = r.lo;
    hi = r.hi;
    eq_span = r.hi - r.lo;
    gt_span = r.hi <= 0xFC00u ? 0xFC01u - r.hi : 0u;
  }
  __device__ bool above(uint32_t key16) const { return key16 - hi < gt_span; }
  __device__ bool in_bin(uint32_t key16) const { return key16 - lo < eq_span; }
};

// Sub-bin of a key of the threshold bin: its FP16 key's place in the bin's
// key range [lo, hi), cut into 256 equal parts (non-decreasing in the key, so
// every key of a higher sub-bin is larger).  Collect and finish compute it
// with this same arithmetic.
struct SubDigit {
  uint32_t lo, mult;
  __device__ __forceinline__ explicit SubDigit(int bstar) {
    const KeyRange r = bin_key_range(bstar);
    lo = r.lo;
    const uint32_t span = r.hi > r.lo ? r.hi - r.lo : 1u;  // <= 8457: the product below fits 32 bits
    mult = (static_cast<uint32_t>(kSubBins) << 16) / span;
  }
  __device__ __forceinline__ uint32_t of(uint32_t key16) const {
    return min(((key16 - lo) * mult) >> 16, static_cast<uint32_t>(kSubBins - 1));
  }
};

// The FP16 key of a stored selection key (FP32 keys hold the score itself).
template <int KEY>
__device__ __forceinline__ uint32_t key16_of(uint32_t key) {
  if constexpr (KEY == IDX_KEY_FP32) {
    const uint32_t u = (key & 0x80000000u) ? (key & 0x7FFFFFFFu) : ~key;
    return key_f16(f16_bits_rn(__uint_as_float(u)));
  } else {
    return key;
  }
}

// The 16 consecutive scores of a thread, from kPerThread / kPerVec 16-byte
// loads.  Loads past the row's last live vector are clamped to it (in
// bounds: the stride is a multiple of kPerVec) and their scores are masked
// off by the caller.
template <bool F16>
struct ThreadScores {
  static constexpr int kPerVec = F16 ? 8 : 4;
  static constexpr int kVecs = kPerThread / kPerVec;
  i32x4 v[kVecs];
  __device__ void load(const char* x, int s0, int len) {
    const int last_vec = len > 0 ? ((len - 1) / kPerVec) * kPerVec : 0;
#pragma unroll
    for (int u = 0; u < kVecs; ++u) {
      const int s = min(s0 + u * kPerVec, last_vec);
      v[u] = *reinterpret_cast<const i32x4*>(x + static_cast<int64_t>(s) * (F16 ? 2 : 4));
    }
  }
  __device__ uint32_t half_bits(int i) const { return half_bits_of<F16>(v[i / kPerVec], i % kPerVec); }
  // The selection key of score i (its FP16 key, or its FP32 key).
  template <int KEY>
  __device__ uint32_t key(int i) const {
    if constexpr (!F16 && KEY == IDX_KEY_FP32) return key_f32(__int_as_float(v[i / kPerVec][i % kPerVec]));
    else return key_f16(half_bits(i));
  }
  // Bit i of *gmask / *emask: score i is live and above b* / in b*.
  __device__ void classify(const Classifier& cl, int s0, int len, uint32_t* gmask, uint32_t* emask) const {
    uint32_t g = 0u, e = 0u;
#pragma unroll
    for (int i = 0; i < kPerThread; ++i) {
      const uint32_t k16 = key_f16(half_bits(i));
      const bool live = s0 + i < len;
      g |= static_cast<uint32_t>(live && cl.above(k16)) << i;
      e |= static_cast<uint32_t>(live && cl.in_bin(k16)) << i;
    }
    *gmask = g;
    *emask = e;
  }
};

// ---------------------------------------------------------------------------
// Histogram of each row's live non-NaN scores, added to hist_out.  One
// workgroup per M consecutive 4096-score chunks: the workgroup's bins are
// added to the row's with global atomics, and the memory side serves the
// atomics on one bin one after another, so long rows give each workgroup
// several chunks (fewer contributions per bin).
template <bool F16, int M>
__global__ __launch_bounds__(kThreads) void topk_hist_kernel(const void* __restrict__ logits,
                                                             int64_t stride,
                                                             const int32_t* __restrict__ lens,
                                                             int* __restrict__ hist_out,
                                                             int64_t hist_stride) {
  __shared__ int s_hist[kBins];
  const int row = blockIdx.y;
  const int len = clamp_len(lens, row, stride);
  const int64_t first = static_cast<int64_t>(blockIdx.x) * M * kChunk;
  if (first >= len) return;
  for (int i = threadIdx.x; i < kBins; i += kThreads) s_hist[i] = 0;
  const char* x = static_cast<const char*>(score_row<F16>(logits, row, stride));
  constexpr int kPerVec = F16 ? 8 : 4;  // scores per 16-byte load
  constexpr int kVecs = kChunk / (kThreads * kPerVec);
  // All of a thread's loads are requested before any is binned.  In bounds:
  // a vector starting at s < len <= stride ends inside the row (s and the
  // stride are multiples of kPerVec); vectors past the row's end read the
  // workgroup's first vector again and are not binned.
  const int f = static_cast<int>(first);  // first < len < 2^31
  i32x4 v[M][kVecs];
#pragma unroll
  for (int m = 0; m < M; ++m) {
#pragma unroll
    for (int u = 0; u < kVecs; ++u) {
      const int64_t s = first + m * kChunk + (u * kThreads + static_cast<int>(threadIdx.x)) * kPerVec;
      v[m][u] = *reinterpret_cast<const i32x4*>(x + (s < len ? s : f) * (F16 ? 2 : 4));
    }
  }
  lds_barrier();  // the bins are zero
#pragma unroll
  for (int m = 0; m < M; ++m) {
#pragma unroll
    for (int u = 0; u < kVecs; ++u) {
      const int64_t s = first + m * kChunk + (u * kThreads + static_cast<int>(threadIdx.x)) * kPerVec;
#pragma unroll
      for (int e = 0; e < kPerVec; ++e) {
        if (s + e < len) {
          const uint32_t hb = half_bits_of<F16>(v[m][u], e);
          if (!f16_is_nan(hb)) atomicAdd(&s_hist[coarse_bin_f16(hb)], 1);
        }
      }
    }
  }
  lds_barrier();
  unsigned long long* gh = reinterpret_cast<unsigned long long*>(hist_out + row * hist_stride);
  const uint2* sh = reinterpret_cast<const uint2*>(s_hist);
  for (int i = threadIdx.x; i < kBins / 2; i += kThreads) {
    const uint2 w = sh[i];
    if (w.x | w.y) atomicAdd(gh + i, (static_cast<unsigned long long>(w.y) << 32) | w.x);
  }
}

// ---------------------------------------------------------------------------
// One workgroup per M consecutive 4096-score chunks of a row; in chunk m
// thread t takes columns 16t .. 16t+15.  The workgroup's two counts, found by
// one block scan, are added to the row's counter pair in one atomic, whose old
// value gives the workgroup's first places in both lists.  The memory side
// serves the atomics on one counter one after another, so long rows give each
// workgroup two chunks.
template <int KEY, bool F16, int M>
// (Arguments in the order of first use: the leading 56 bytes arrive in scalar
// registers.)
__global__ __launch_bounds__(kThreads) void topk_collect_kernel(const void* __restrict__ logits,
                                                                int64_t stride,
                                                                const int32_t* hist,  // (see below)
                                                                const int32_t* __restrict__ lens,
                                                                char* __restrict__ ws_base,
                                                                int32_t* __restrict__ indices, int k,
                                                                int hist_stride) {
  const Workspace ws{ws_base};
  __shared__ int s_red[kWaves + 5];
  __shared__ int s_sub[kSubBins];
  const int row = blockIdx.y;
  const int tid = threadIdx.x;
  // The histogram is requested before the row's length arrives (a
  // workgroup past the row's end reads 4 KiB for nothing), so that the
  // threshold scan overlaps the round trip of the scores, which wait for
  // the length.  The compiler barrier keeps the loads here: through a
  // __restrict__ pointer they would count as invariant and be sunk past the
  // exit test.
  const int* h = hist + static_cast<int64_t>(row) * hist_stride + tid * 4;
  const int2 h01 = *reinterpret_cast<const int2*>(h);  // 8-B aligned
  const int2 h23 = *reinterpret_cast<const int2*>(h + 2);
  __asm__ volatile("" ::: "memory");
  const int len = clamp_len(lens, row, stride);
  const int64_t first = static_cast<int64_t>(blockIdx.x) * M * kChunk;  // first column of the workgroup
  if (first >= len) return;

  const char* x = static_cast<const char*>(score_row<F16>(logits, row, stride));
  int s0[M], live[M];  // live[m]: columns of chunk m below this length count
  ThreadScores<F16> sc[M];
#pragma unroll
  for (int m = 0; m < M; ++m) {
    // A chunk that starts below len <= stride < 2^31 starts at most at
    // 2^31 - 4096, so its columns fit an int; a chunk past the row end is
    // read at column 0 and takes no column.
    const int64_t c0 = first + m * kChunk;
    s0[m] = c0 < len ? static_cast<int>(c0) + tid * kPerThread : 0;
    live[m] = c0 < len ? len : 0;
    sc[m].load(x, s0[m], len);
  }
  const int hc[4] = {h01.x, h01.y, h23.x, h23.y};
  static_assert(kThreads == kSubBins, "one sub-bin per thread");
  s_sub[tid] = 0;  // published by the barriers of the scans below
  const Threshold th = threshold_bin<kThreads, 4>(hc, k, s_red);
  const int bstar = th.bin;
  const bool with_sub = th.count > kCutMin;  // uniform
  // Every workgroup of the row finds the same b*; the first (which runs
  // whenever the row has a live score) hands it to the finish pass.
  if (blockIdx.x == 0 && tid == 0) *ws.bstar(row) = bstar;

  const Classifier cl(bstar);
  uint32_t gmask[M], emask[M];
  int mine = 0;
#pragma unroll
  for (int m = 0; m < M; ++m) {
    sc[m].classify(cl, s0[m], live[m], &gmask[m], &emask[m]);
    mine += __popc(gmask[m]) | (__popc(emask[m]) << 16);
  }
  // Both counts in one scan: each is at most M * kChunk < 2^16.
  int tot = 0;
  const int pre = block_excl_scan<kThreads>(mine, s_red, &tot);
  // The workgroup's true counts, stored for the finish pass's check of the
  // counters (blockIdx.x < kMaxCollectWgs: the host limits the stride).
  if (tid == 0) ws.slots(row)[blockIdx.x] = tot;
  if (tot == 0) return;  // uniform
  if (tid == 0) {
    const unsigned long long add =
        static_cast<unsigned long long>(tot & 0xFFFF) | (static_cast<unsigned long long>(tot >> 16) << 32);
    const unsigned long long base = atomicAdd(ws.count(row) + (blockIdx.x & 1), add);
    s_red[kWaves + 3] = static_cast<int>(static_cast<uint32_t>(base));
    s_red[kWaves + 4] = static_cast<int>(static_cast<uint32_t>(base >> 32));
  }
  lds_barrier();
  // Places as unsigned: a row holds fewer than 2^31 columns.
  uint32_t og = static_cast<uint32_t>(s_red[kWaves + 3]) + static_cast<uint32_t>(pre & 0xFFFF);
  uint32_t oe = static_cast<uint32_t>(s_red[kWaves + 4]) + static_cast<uint32_t>(pre >> 16);
  // Place p counts from the front (even workgroups) or from the back (odd).
  const bool back = (blockIdx.x & 1) != 0;
  int32_t* out = indices + static_cast<int64_t>(row) * k;
  uint2* cand = ws.cand(row);
  const SubDigit sd(bstar);  // (no candidates when bstar is the all-bins threshold)
#pragma unroll
  for (int m = 0; m < M; ++m) {
#pragma unroll
    for (int i = 0; i < kPerThread; ++i) {
      if ((gmask[m] >> i) & 1u) {
        if (og < static_cast<uint32_t>(k)) out[back ? k - 1 - static_cast<int>(og) : static_cast<int>(og)] = s0[m] + i;
        ++og;
      }
      if ((emask[m] >> i) & 1u) {
        if (oe < static_cast<uint32_t>(kCandBuf))
          cand[back ? kCandBuf - 1 - static_cast<int>(oe) : static_cast<int>(oe)] =
              uint2{sc[m].template key<KEY>(i), static_cast<uint32_t>(s0[m] + i)};
        ++oe;
        if (with_sub) atomicAdd(&s_sub[sd.of(key_f16(sc[m].half_bits(i)))], 1);
      }
    }
  }
  if (!with_sub || (tot >> 16) == 0) return;  // uniform
  lds_barrier();
  const int v = s_sub[tid];
  if (v) atomicAdd(ws.sub(row) + tid, v);
}

// ---------------------------------------------------------------------------
// Shared memory of the row and finish passes.
struct RefineShared {
  uint2 cand[kCandBuf];   // 128 KiB
  int digit_hist[256];
  int red[2 * (kRefineThreads / kWave) + 4];
  uint32_t small[kWave];  // the few keys left after a radix pass, or the columns of few ties
  int small_n;
  int tie_n;
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
// taken from the largest digit down (or, ascending, from the smallest up)
// first reaches `need`; *before = the count strictly before d, *in_bin = the
// count of d.
__device__ __forceinline__ int pick_digit(RefineShared& sh, int need, int* before, int* in_bin,
                                          bool descending = true) {
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
__device__ __forceinline__ uint32_t rank_small(RefineShared& sh, int n, uint32_t prefix, uint32_t fixed, int need,
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
__device__ __forceinline__ uint32_t select_key_lds(RefineShared& sh, int n, int need, int* above) {
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

// Among the LDS candidates with key == T, the need-th smallest column C:
// taking the ties with column <= C takes exactly `need` of them (columns are
// distinct).  For candidate lists not in column order.
__device__ __forceinline__ uint32_t select_col_lds(RefineShared& sh, int n, uint32_t T, int need) {
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
      lds_barrier();
      for (int i = threadIdx.x; i < n; i += kRefineThreads) {
        const uint2 c = sh.cand[i];
        if (c.x == T && ((c.y ^ prefix) & fixed) == 0u) atomicAdd(&sh.digit_hist[(c.y >> shift) & 0xFFu], 1);
      }
      lds_barrier();
      int before = 0, in_bin = 0;
      const int d = pick_digit(sh, need, &before, &in_bin, false);
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
// Lanes of the wave that are not active (a per-thread loop that ended) take
// no part: the first active lane reserves the places.
__device__ __forceinline__ void emit(RefineShared& sh, int32_t* out, int k, bool take, int col) {
  const uint64_t m = __ballot(take);
  if (!m) return;
  const int leader = __builtin_amdgcn_readfirstlane(static_cast<int>(__lane_id()));
  int pos = 0;
  if (static_cast<int>(__lane_id()) == leader) pos = atomicAdd(&sh.out_pos, __popcll(m));
  pos = __builtin_amdgcn_readfirstlane(pos) + lanes_below(m);
  if (take && pos < k) out[pos] = col;
}

// Exact selection over the whole row: a stale histogram, or a threshold bin
// with more candidates than the capacity.  Thread t owns the contiguous
// columns [t * seg, (t + 1) * seg) (seg a multiple of 8, so its 16-byte
// vectors are aligned for float and half rows alike) and reads them with
// 16-byte loads, four in flight; after the digit passes one block scan of the
// threads' tie counts ranks the ties at the final key in column order.
template <bool F16>
struct SegmentReader {
  static constexpr int kPerVec = F16 ? 8 : 4;
#ifndef PMQA_TOPK_SEG_BATCH
#define PMQA_TOPK_SEG_BATCH 4
#endif
  static constexpr int kBatch = PMQA_TOPK_SEG_BATCH;  // vectors in flight per thread
  const char* x;
  int begin, end;  // this thread's columns
  __device__ SegmentReader(const void* row, int len) : x(static_cast<const char*>(row)) {
    const int seg = ((len + kRefineThreads - 1) / kRefineThreads + 7) / 8 * 8;
    begin = min(len, static_cast<int>(threadIdx.x) * seg);
    end = min(len, begin + seg);
  }
  // f(column, key, live) for every column of the segment, in column order.
  // A vector that starts below end starts below len <= stride and ends
  // inside the row (the stride is a multiple of kPerVec); vectors of a batch
  // past the segment read its first vector again and are not visited.
  template <int KEY, typename F>
  __device__ __forceinline__ void for_each(F&& f) const {
    for (int s0 = begin; s0 < end; s0 += kBatch * kPerVec) {
      i32x4 v[kBatch];
#pragma unroll
      for (int u = 0; u < kBatch; ++u) {
        const int s = s0 + u * kPerVec;
        v[u] = *reinterpret_cast<const i32x4*>(x + static_cast<int64_t>(s < end ? s : begin) * (F16 ? 2 : 4));
      }
#pragma unroll
      for (int u = 0; u < kBatch; ++u) {
#pragma unroll
        for (int e = 0; e < kPerVec; ++e) {
          const int s = s0 + u * kPerVec + e;
          if (s < end) {
            uint32_t key;
            bool live;
            if constexpr (F16) {
              const uint32_t hb = half_bits_of<true>(v[u], e);
              key = key_f16(hb);
              live = !f16_is_nan(hb);
            } else {
              const float val = __int_as_float(v[u][e]);
              key = score_key<KEY>(val);
              live = val == val;
            }
            f(s, key, live);
          }
        }
      }
    }
  }
};

// Digit counts of the whole-row passes.  FP32 keys: one copy of the 256
// bins per lane position, kept in the candidate buffer (unused until the
// gather) with bin d of lane l at word 64 d + l, so the 64 adds of one
// instruction fall on 64 different words and banks.  The top bytes of FP32
// keys are sign and exponent: with a single copy a wave whose scores share a
// few of them queues up to 64 increments of one word per instruction (a
// unit-regime verify row of 32K scores alone: 45.7 -> 39.2 us; aggregating
// the first lane's digit with ballots, the design before, gave 73 -> 64 us
// over plain adds).  FP16 keys add to digit_hist directly (measured faster).
static_assert(sizeof(uint2) * kCandBuf >= sizeof(int) * 256 * kWave, "lane bins fit the candidate buffer");

template <bool LANE_BINS>
__device__ __forceinline__ void digit_clear(RefineShared& sh) {
  if constexpr (LANE_BINS) {
    i32x4* p = reinterpret_cast<i32x4*>(sh.cand);
    for (int i = threadIdx.x; i < 256 * kWave / 4; i += kRefineThreads) p[i] = i32x4{0, 0, 0, 0};
  } else {
    for (int i = threadIdx.x; i < 256; i += kRefineThreads) sh.digit_hist[i] = 0;
  }
}

template <bool LANE_BINS>
__device__ __forceinline__ void digit_add(RefineShared& sh, bool act, uint32_t d) {
  if constexpr (LANE_BINS) {
    // every lane adds (0 when inactive): no exec-mask branch per score
    atomicAdd(&reinterpret_cast<int*>(sh.cand)[(d & 0xFFu) * kWave + __lane_id()], act ? 1 : 0);
  } else {
    if (act) atomicAdd(&sh.digit_hist[d], 1);
  }
}

// After a barrier that makes the adds visible: digit_hist[d] = the sum of
// bin d's copies (lane l reads copy (l + j) mod 64 at step j, 64 banks per
// instruction), published by a barrier.
template <bool LANE_BINS>
__device__ __forceinline__ void digit_publish(RefineShared& sh) {
  if constexpr (LANE_BINS) {
    const int* b = reinterpret_cast<const int*>(sh.cand);
    const int l = __lane_id();
    for (int d = threadIdx.x; d < 256; d += kRefineThreads) {
      int sum = 0;
#pragma unroll 8
      for (int j = 0; j < kWave; ++j) sum += b[d * kWave + ((l + j) & (kWave - 1))];
      sh.digit_hist[d] = sum;
    }
    lds_barrier();
  }
}

__device__ __forceinline__ void finish_candidates(RefineShared& sh, int32_t* __restrict__ out, int k, int n_gt,
                                                  int n_eq, int first_free, bool column_order);
__device__ __forceinline__ void finish_list(RefineShared& sh, int32_t* __restrict__ out, int k, int len,
                                            int n_gt, int n_eq, int first_free);

template <int KEY, bool F16>
__device__ __forceinline__ void whole_row_select(RefineShared& sh, const void* __restrict__ x, int len, int k,
                                                 int32_t* __restrict__ out) {
  constexpr int kKey = F16 ? IDX_KEY_FP16 : KEY;
  constexpr int kKeyBits = kKey == IDX_KEY_FP32 ? 32 : 16;
  const SegmentReader<F16> rd(x, len);
  constexpr bool kLaneBins = kKey == IDX_KEY_FP32;
  // Pass 1: the live count and the histogram of the top key digit.
  digit_clear<kLaneBins>(sh);
  if (threadIdx.x == 0) sh.out_pos = 0;
  lds_barrier();
  int cnt = 0;
  rd.template for_each<KEY>([&](int, uint32_t key, bool live) {
    cnt += live ? 1 : 0;
    digit_add<kLaneBins>(sh, live, key >> (kKeyBits - 8));
  });
  const int n = block_sum<kRefineThreads>(cnt, sh.red);  // its barriers also make the adds visible
  if (n <= k) {
    rd.template for_each<KEY>([&](int s, uint32_t, bool live) { emit(sh, out, k, live, s); });
    lds_barrier();
    for (int i = n + threadIdx.x; i < k; i += kRefineThreads) out[i] = -1;
    return;
  }
  uint32_t prefix = 0u, fixed = 0u;
  int need = k;
  for (int shift = kKeyBits - 8; shift >= 0; shift -= 8) {
    if (shift != kKeyBits - 8) {
      digit_clear<kLaneBins>(sh);  // the last pass's reads ended before pick_digit's barriers
      lds_barrier();
      rd.template for_each<KEY>([&](int, uint32_t key, bool live) {
        digit_add<kLaneBins>(sh, live && ((key ^ prefix) & fixed) == 0u, (key >> shift) & 0xFFu);
      });
      lds_barrier();
    }
    digit_publish<kLaneBins>(sh);
    int before = 0;
    int in_bin = 0;
    const int d = pick_digit(sh, need, &before, &in_bin);
    need -= before;
    prefix |= static_cast<uint32_t>(d) << shift;
    fixed |= 0xFFu << shift;
    if (shift > 0 && in_bin <= kCandBuf) {
      // The keys that share the prefix fit the LDS buffer: one pass emits the
      // keys above the prefix and gathers these candidates, and the row is
      // finished in LDS as for a confirmed threshold bin.
      if (threadIdx.x == 0) sh.small_n = 0;
      lds_barrier();
      rd.template for_each<KEY>([&](int s, uint32_t key, bool live) {
        emit(sh, out, k, live && (key & fixed) > prefix, s);
        const bool cand = live && (key & fixed) == prefix;
        const uint64_t m = __ballot(cand);
        if (m) {
          const int leader = __builtin_amdgcn_readfirstlane(static_cast<int>(__lane_id()));
          int pos = 0;
          if (static_cast<int>(__lane_id()) == leader) pos = atomicAdd(&sh.small_n, __popcll(m));
          pos = __builtin_amdgcn_readfirstlane(pos) + lanes_below(m);
          if (cand) sh.cand[pos] = uint2{key, static_cast<uint32_t>(s)};
        }
      });
      lds_barrier();
      const int n_above = k - need;
      finish_list(sh, out, k, len, n_above, in_bin, n_above);
      return;
    }
  }
  const uint32_t T = prefix;
  // Keys above T, then the `need` lowest columns with key == T: a thread's
  // ties come after those of every lower thread.
  int my_ties = 0;
  rd.template for_each<KEY>([&](int, uint32_t key, bool live) { my_ties += (live && key == T) ? 1 : 0; });
  int all_ties = 0;
  int rank = block_excl_scan<kRefineThreads>(my_ties, sh.red, &all_ties);
  rd.template for_each<KEY>([&](int s, uint32_t key, bool live) {
    const bool tie = live && key == T;
    emit(sh, out, k, (live && key > T) || (tie && rank < need), s);
    rank += tie ? 1 : 0;
  });
}

// Counts confirm b* when the columns above it fall short of k and those in it
// make up the difference (within the candidate capacity), or, for the
// all-bins threshold, when every live score is above it and they are at most
// k.
__device__ __forceinline__ bool counts_confirm(int bstar, int n_gt, int n_eq, int k) {
  if (bstar == kAllBins) return n_gt <= k && n_eq == 0;
  return n_gt < k && n_gt + n_eq >= k && n_eq <= kCandBuf;
}

// The n_eq candidates of b* are in sh.cand and the output row holds the n_gt
// columns above b* outside [first_free, first_free + k - n_gt): the best
// need = k - n_gt candidates fill that gap.  Every
// key above the need-th largest key T is taken, and of the keys equal to T
// the lowest columns: the first ones in list order when the list is in
// column order (thread t ranks a run of consecutive candidates), else those
// up to the column a radix select on the columns finds.
__device__ __forceinline__ void finish_candidates(RefineShared& sh, int32_t* __restrict__ out, int k, int n_gt,
                                                  int n_eq, int first_free, bool column_order) {
  const int need = k - n_gt;
  if (threadIdx.x == 0) {
    sh.out_pos = first_free;
    sh.tie_n = 0;
  }
  lds_barrier();
  int above = 0;
  const uint32_t T = select_key_lds(sh, n_eq, need, &above);
  const int ties_needed = need - above;
  if (column_order) {
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
    return;
  }
  // Count the ties at T; the columns of the first 64 are gathered as well
  // (select_key_lds is done with sh.small), so that few ties -- the usual
  // case -- are cut by ranking their columns directly.
  int tc = 0;
  for (int i0 = 0; i0 < n_eq; i0 += kRefineThreads) {
    const int i = i0 + static_cast<int>(threadIdx.x);
    const uint2 cd = i < n_eq ? sh.cand[i] : uint2{0u, 0u};
    const bool tie = i < n_eq && cd.x == T;
    tc += tie ? 1 : 0;
    const uint64_t m = __ballot(tie);
    if (m) {  // uniform in the wave
      int pos = 0;
      if (__lane_id() == 0) pos = atomicAdd(&sh.tie_n, __popcll(m));
      pos = __builtin_amdgcn_readfirstlane(pos) + lanes_below(m);
      if (tie && pos < kWave) sh.small[pos] = cd.y;
    }
  }
  const int ties = block_sum<kRefineThreads>(tc, sh.red);  // its barriers publish sh.small
  uint32_t col_cut = 0xFFFFFFFFu;
  if (ties > ties_needed) {
    if (ties <= kWave) {
      // The ties_needed-th smallest of the (distinct) tie columns.
      if (threadIdx.x < kWave) {
        const int lane = threadIdx.x;
        const uint32_t cj = lane < ties ? sh.small[lane] : 0xFFFFFFFFu;
        int below = 0;
        for (int i = 0; i < ties; ++i) below += sh.small[i] < cj ? 1 : 0;
        if (lane < ties && below == ties_needed - 1) sh.bcast[0] = static_cast<int>(cj);
      }
      lds_barrier();
      col_cut = static_cast<uint32_t>(sh.bcast[0]);
    } else {
      col_cut = select_col_lds(sh, n_eq, T, ties_needed);
    }
  }
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

// ---------------------------------------------------------------------------
// A threshold bin whose candidates all came with the early loads (at most
// 1024 from each end) is finished from registers: thread t holds front
// entries t and t + 512 and back entries t and t + 512.  The radix passes
// count into histograms of their own (zeroed once, up front), and after each
// pass's barrier every wave reads the counts and finds the digit itself, so
// a pass costs one barrier; the LDS candidate list is not used.
constexpr int kEarlyCand = 2;  // candidates per thread and end loaded with the counts
constexpr int kRegCand = 2 * kEarlyCand;
constexpr int kRegPasses = 4;  // 8-bit digits of a 32-bit value

// Radix select over the values v[i] (bit i of `valid`) of every thread of
// the block, `total` of them: the need-th largest value, *above = how many
// exceed it, *at = how many equal it.  hists: kRegPasses zeroed 256-bin
// histograms; o and a: bits that some valid value may have set, and bits
// that every valid value has set (the block-wide OR and AND, or looser
// bounds, which cost passes only).
// Block-uniform control flow: every wave finds the same digits.
__device__ __forceinline__ uint32_t select_regs(const uint32_t (&v)[kRegCand], uint32_t valid, uint32_t o,
                                                uint32_t a, int total, int need, int (*hists)[256], int* above,
                                                int* at) {
  const int lane = __lane_id();
  const uint32_t diff = o ^ a;
  uint32_t prefix = a & ~diff, fixed = ~diff;
  int gt = 0, eq = total;  // (every value the same when diff is 0)
  int shift = max(top_bit(diff | 1u) - 7, 0);
  for (int p = 0; diff != 0u && p < kRegPasses; ++p) {
    int* h = hists[p];
#pragma unroll
    for (int i = 0; i < kRegCand; ++i)
      if (((valid >> i) & 1u) && ((v[i] ^ prefix) & fixed) == 0u) atomicAdd(&h[(v[i] >> shift) & 0xFFu], 1);
    lds_barrier();
    // Lane l reads digits 255 - 4l down to 252 - 4l; every wave finds the same digit.
    const int4 q = reinterpret_cast<const int4*>(h)[kWave - 1 - lane];
    const int c[4] = {q.w, q.z, q.y, q.x};
    const int sum = c[0] + c[1] + c[2] + c[3];
    int run = wave_inclusive_scan(sum) - sum;
    int hit = -1, hit_before = 0, hit_in = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if (run < need && run + c[i] >= need) {
        hit = 255 - 4 * lane - i;
        hit_before = run;
        hit_in = c[i];
      }
      run += c[i];
    }
    const int src = first_lane(__ballot(hit >= 0));
    const int d = __builtin_amdgcn_readlane(hit, src) & 0xFF;
    const int before = __builtin_amdgcn_readlane(hit_before, src);
    eq = __builtin_amdgcn_readlane(hit_in, src);
    need -= before;
    gt += before;
    prefix |= static_cast<uint32_t>(d) << shift;
    fixed |= 0xFFu << shift;
    if (shift == 0) break;
    shift = max(shift - 8, 0);
  }
  *above = gt;
  *at = eq;
  return prefix;
}

// The block-wide OR and AND of the values v[i] with bit i of `valid`, through
// slots [0, 16) of s_red (one barrier).
__device__ __forceinline__ void or_and_regs(const uint32_t (&v)[kRegCand], uint32_t valid, int* s_red, uint32_t* o,
                                            uint32_t* a) {
  uint32_t x = 0u, y = 0xFFFFFFFFu;
#pragma unroll
  for (int i = 0; i < kRegCand; ++i) {
    if ((valid >> i) & 1u) {
      x |= v[i];
      y &= v[i];
    }
  }
  x = wave_or(x);
  y = wave_and(y);
  const int wave = threadIdx.x / kWave;
  if (__lane_id() == 0) {
    s_red[wave] = static_cast<int>(x);
    s_red[8 + wave] = static_cast<int>(y);
  }
  lds_barrier();
  x = 0u;
  y = 0xFFFFFFFFu;
#pragma unroll
  for (int w = 0; w < kRefineThreads / kWave; ++w) {
    x |= static_cast<uint32_t>(s_red[w]);
    y &= static_cast<uint32_t>(s_red[8 + w]);
  }
  *o = x;
  *a = y;
}

__device__ __forceinline__ void finish_regs(RefineShared& sh, int32_t* __restrict__ out, int k, int len,
                                            int need, int n_eq, int first_free, const uint2 (&c)[kRegCand],
                                            uint32_t valid) {
  // Eight zeroed histograms (keys, then columns) at the end of the LDS
  // candidate list: the candidates, when they were gathered there first (the
  // row pass), occupy at most its first 2048 entries.
  constexpr int kHistEntries = 2 * kRegPasses * 256 * 4 / static_cast<int>(sizeof(uint2));
  static_assert(kRefineThreads / kWave <= 8 && kHistEntries + kRegCand * kRefineThreads <= kCandBuf, "layout");
  int (*hists)[256] = reinterpret_cast<int (*)[256]>(&sh.cand[kCandBuf - kHistEntries]);
  reinterpret_cast<int4*>(&hists[0][0])[threadIdx.x] = make_int4(0, 0, 0, 0);
  if (threadIdx.x == 0) sh.out_pos = first_free;
  uint32_t key[kRegCand], ncol[kRegCand];
#pragma unroll
  for (int i = 0; i < kRegCand; ++i) {
    key[i] = c[i].x;
    ncol[i] = ~c[i].y;
  }
  uint32_t o, a;
  or_and_regs(key, valid, sh.red, &o, &a);  // its barrier also publishes the zeroed histograms
  int above = 0, ties = 0;
  const uint32_t T = select_regs(key, valid, o, a, n_eq, need, hists, &above, &ties);
  const int ties_needed = need - above;
  // Of more ties than needed, those up to the ties_needed-th smallest column
  // (columns are distinct): the ties_needed-th largest complemented column.
  uint32_t col_cut = 0xFFFFFFFFu;
  if (ties > ties_needed) {  // uniform
    uint32_t tie = 0u;
#pragma unroll
    for (int i = 0; i < kRegCand; ++i) tie |= (((valid >> i) & 1u) && key[i] == T ? 1u : 0u) << i;
    // The columns lie in [0, len): their complements differ at most in the
    // low bits that len - 1 spans, which bounds the passes without a
    // block-wide OR/AND of the tie columns.
    const uint32_t span = len > 1 ? (0xFFFFFFFFu >> __clz(static_cast<uint32_t>(len - 1))) : 1u;
    int unused0 = 0, unused1 = 0;
    col_cut = ~select_regs(ncol, tie, 0xFFFFFFFFu, ~span, ties, ties_needed, hists + kRegPasses, &unused0,
                           &unused1);
  }
#pragma unroll
  for (int i = 0; i < kRegCand; ++i) {
    const bool take = ((valid >> i) & 1u) && (key[i] > T || (key[i] == T && c[i].y <= col_cut));
    emit(sh, out, k, take, static_cast<int>(c[i].y));
  }
}

// The n_eq candidates just written to the LDS list (by any thread): selected
// from registers when they fit four per thread, else by the LDS select.
__device__ __forceinline__ void finish_list(RefineShared& sh, int32_t* __restrict__ out, int k, int len,
                                            int n_gt, int n_eq, int first_free) {
  if (n_eq <= kRegCand * kRefineThreads) {  // uniform
    lds_barrier();
    uint2 r[kRegCand];
    uint32_t valid = 0u;
#pragma unroll
    for (int j = 0; j < kRegCand; ++j) {
      const int i = j * kRefineThreads + static_cast<int>(threadIdx.x);
      r[j] = i < n_eq ? sh.cand[i] : make_uint2(0u, 0u);
      valid |= (i < n_eq ? 1u : 0u) << j;
    }
    finish_regs(sh, out, k, len, k - n_gt, n_eq, first_free, r, valid);
    return;
  }
  finish_candidates(sh, out, k, n_gt, n_eq, first_free, false);
}

// ---------------------------------------------------------------------------
// Rows of at most M * 8192 scores: one workgroup per row, thread t takes
// columns 8192m + 16t .. 8192m + 16t+15 of each part m, so block scans of the
// per-thread counts (part 0's places before part 1's) keep both lists in
// column order.  OWN_HIST: no histogram was given; the workgroup bins its row
// in LDS first.
// MAP (the sparse rows of the two-level candidate indexer): once the row's
// selection is written, each column c becomes the logical key
// 8 * table[row][c / 8] + c % 8 (-1 for padding, for columns past the table
// and for table padding), in place.
template <int KEY, bool F16, bool OWN_HIST, int M, bool MAP = false>
__global__ __launch_bounds__(kRefineThreads) void topk_row_kernel(const void* __restrict__ logits,
                                                                  int64_t stride,
                                                                  const int32_t* __restrict__ hist,
                                                                  const int32_t* __restrict__ lens, int k,
                                                                  int32_t* __restrict__ indices,
                                                                  const int32_t* __restrict__ table, int kb) {
  __shared__ RefineShared sh;
  __shared__ int s_hist[OWN_HIST ? kBins : 1];
  const int row = blockIdx.x;
  const int tid = threadIdx.x;
  const int len = clamp_len(lens, row, stride);
  const char* x = static_cast<const char*>(score_row<F16>(logits, row, stride));
  int32_t* out = indices + static_cast<int64_t>(row) * k;

  // The thread's two bins and its 16 scores of each 8192-column part are
  // requested together.
  int hv[2] = {0, 0};
  if constexpr (!OWN_HIST) {
    const int2 h = *reinterpret_cast<const int2*>(hist + static_cast<int64_t>(row) * kBins + 2 * tid);
    hv[0] = h.x;
    hv[1] = h.y;
  }
  int s0[M];
  ThreadScores<F16> sc[M];
#pragma unroll
  for (int m = 0; m < M; ++m) {
    s0[m] = m * kRowSpan + tid * kPerThread;
    sc[m].load(x, s0[m], len);
  }
  if constexpr (OWN_HIST) {
    s_hist[2 * tid] = 0;
    s_hist[2 * tid + 1] = 0;
    lds_barrier();
#pragma unroll
    for (int m = 0; m < M; ++m) {
#pragma unroll
      for (int i = 0; i < kPerThread; ++i) {
        const uint32_t hb = sc[m].half_bits(i);
        if (s0[m] + i < len && !f16_is_nan(hb)) atomicAdd(&s_hist[coarse_bin_f16(hb)], 1);
      }
    }
    lds_barrier();
    hv[0] = s_hist[2 * tid];
    hv[1] = s_hist[2 * tid + 1];
  }
  const int bstar = threshold_bin<kRefineThreads, 2>(hv, k, sh.red).bin;

  const Classifier cl(bstar);
  uint32_t gmask[M], emask[M];
#pragma unroll
  for (int m = 0; m < M; ++m) sc[m].classify(cl, s0[m], len, &gmask[m], &emask[m]);
  // Places in column order: every column of part 0 before any of part 1.
  int og[M], oe[M];
  int n_gt, n_eq;
  if constexpr (M == 1) {
    int tot = 0;
    const int pre = block_excl_scan<kRefineThreads>(__popc(gmask[0]) | (__popc(emask[0]) << 16), sh.red, &tot);
    n_gt = tot & 0xFFFF;
    n_eq = tot >> 16;
    og[0] = pre & 0xFFFF;
    oe[0] = pre >> 16;
  } else {
    int2 tot;
    const int2 pre = block_excl_scan2<kRefineThreads>(__popc(gmask[0]) | (__popc(emask[0]) << 16),
                                                      __popc(gmask[1]) | (__popc(emask[1]) << 16), sh.red, &tot);
    n_gt = (tot.x & 0xFFFF) + (tot.y & 0xFFFF);  // each at most 16384
    n_eq = (tot.x >> 16) + (tot.y >> 16);
    og[0] = pre.x & 0xFFFF;
    oe[0] = pre.x >> 16;
    og[1] = (tot.x & 0xFFFF) + (pre.y & 0xFFFF);
    oe[1] = (tot.x >> 16) + (pre.y >> 16);
  }
  if (!counts_confirm(bstar, n_gt, n_eq, k)) {
    whole_row_select<KEY, F16>(sh, x, len, k, out);
  } else {
    // When every candidate is taken (none exist below the all-bins
    // threshold) their columns go straight to the output.
    const bool direct = bstar == kAllBins || k - n_gt == n_eq;
#pragma unroll
    for (int m = 0; m < M; ++m) {
#pragma unroll
      for (int i = 0; i < kPerThread; ++i) {
        if ((gmask[m] >> i) & 1u) out[og[m]++] = s0[m] + i;  // og < n_gt <= k
        if ((emask[m] >> i) & 1u) {
          if (direct) out[n_gt + oe[m]] = s0[m] + i;
          else sh.cand[oe[m]] = uint2{sc[m].template key<KEY>(i), static_cast<uint32_t>(s0[m] + i)};
          ++oe[m];
        }
      }
    }
    if (direct) {
      for (int i = n_gt + n_eq + tid; i < k; i += kRefineThreads) out[i] = -1;
    } else {
      lds_barrier();
      if (M == 1 && n_eq <= kRefineThreads) {  // uniform
        // Few candidates: thread t takes list entries t, t + 512, ... into
        // registers and the select runs there (see finish_regs).  Measured
        // faster only for one-part rows with at most one candidate per
        // thread (tiny decode); rows of two parts (the candidate chain's
        // block top-k) and larger bins (its sparse rows) keep the LDS select.
        uint2 c[kRegCand];
        uint32_t valid = 0u;
#pragma unroll
        for (int j = 0; j < kRegCand; ++j) {
          const int i = j * kRefineThreads + tid;
          c[j] = i < n_eq ? sh.cand[i] : make_uint2(0u, 0u);
          valid |= (i < n_eq ? 1u : 0u) << j;
        }
        finish_regs(sh, out, k, len, k - n_gt, n_eq, n_gt, c, valid);
      } else {
        finish_candidates(sh, out, k, n_gt, n_eq, n_gt, true);
      }
    }
  }
  if constexpr (MAP) {
    // Every entry of the row is written by now (the barrier waits for the
    // workgroup's stores); they are read back from L2 (agent-scope loads
    // skip this CU's vector cache) and mapped in place.
    __syncthreads();
    const int32_t* trow = table + static_cast<int64_t>(row) * kb;
    for (int i = tid; i < k; i += kRefineThreads) {
      const int c = __hip_atomic_load(out + i, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      int v = -1;
      if (c >= 0 && c < kb * kSparseBlock) {
        const int b = trow[c / kSparseBlock];
        v = b == INT32_MAX ? -1 : b * kSparseBlock + (c % kSparseBlock);
      }
      out[i] = v;
    }
  }
}


// ---------------------------------------------------------------------------
// One workgroup per row after topk_collect: the two counter pairs, the
// collect workgroups' stored counts, the thread's two bins and the first 1024
// candidates from each end are requested together (the candidate buffer has a
// fixed address; entries past the counts are unused).

// The candidates past the early ones, front list then back list as one list
// of ef + eb: f(i, candidate) for i in [kEarlyCand * threads, ef) and
// [ef + kEarlyCand * threads, ef + eb).  Eight loads per thread are requested
// before any is used (a loop that waits for each load in turn costs a round
// trip per 512 candidates: about 20 us for a bin of 16,000).
template <typename F>
__device__ __forceinline__ void copy_rest(const uint2* __restrict__ cand, int ef, int eb, F&& f) {
  constexpr int kBatch = 8;
  const int tid = threadIdx.x;
  const int n_rest_f = max(ef - kEarlyCand * kRefineThreads, 0);
  const int n_rest = n_rest_f + max(eb - kEarlyCand * kRefineThreads, 0);
  for (int j0 = 0; j0 < n_rest; j0 += kBatch * kRefineThreads) {
    uint2 c[kBatch];
    int at[kBatch];
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
      const int j = j0 + u * kRefineThreads + tid;
      // j < n_rest_f: front entry i; else back entry; past the end: index 0
      // is read again (in bounds) and not used
      const int fi = kEarlyCand * kRefineThreads + j;
      const int bi = kEarlyCand * kRefineThreads + (j - n_rest_f);
      const bool front = j < n_rest_f;
      at[u] = j < n_rest ? (front ? fi : ef + bi) : -1;
      c[u] = cand[j < n_rest ? (front ? fi : kCandBuf - 1 - bi) : 0];
    }
#pragma unroll
    for (int u = 0; u < kBatch; ++u)
      if (at[u] >= 0) f(at[u], c[u]);
  }
}
constexpr int kSlotsPerThread = kMaxCollectWgs / kRefineThreads;
static_assert(kSlotsPerThread * kRefineThreads == kMaxCollectWgs && kRefineThreads % 2 == 0,
              "a thread's slots are all front or all back");

// Block sums of four counts (one pair of LDS barriers).
__device__ __forceinline__ i32x4 block_sum4(i32x4 v, int* s_red4) {
  const int wave = threadIdx.x / kWave;
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    v[c] = wave_sum(v[c]);
    if (__lane_id() == 0) s_red4[4 * wave + c] = v[c];
  }
  lds_barrier();
  i32x4 t{0, 0, 0, 0};
#pragma unroll
  for (int w = 0; w < kRefineThreads / kWave; ++w)
#pragma unroll
    for (int c = 0; c < 4; ++c) t[c] += s_red4[4 * w + c];
  lds_barrier();
  return t;
}

template <int KEY, bool F16>
// The arguments the first loads need come first (the leading ones are placed
// in scalar registers before the kernel starts).
__global__ __launch_bounds__(kRefineThreads) void topk_finish_kernel(char* __restrict__ ws_base,
                                                                     const int32_t* __restrict__ lens,
                                                                     int64_t stride, int32_t* __restrict__ indices,
                                                                     int collect_shift, int k, int own_hist,
                                                                     const void* __restrict__ logits) {
  const Workspace ws{ws_base};
  __shared__ RefineShared sh;
  __shared__ int s_red4[4 * (kRefineThreads / kWave)];
  const int row = blockIdx.x;
  const int tid = threadIdx.x;
  const uint2* cand = ws.cand(row);
  unsigned long long* count = ws.count(row);
  // What the collect pass left is requested first (none of it depends on the
  // row's length); the compiler barrier after these loads keeps them ahead
  // of the length's round trip.
  const unsigned long long front = count[0], back = count[1];
  // b* as the collect pass found it (the same for all of its workgroups).  A
  // row with no live score ran no collect workgroup and may read a stale
  // value: its counts (zero) then send it to the padding-only output, either
  // directly (b* = all bins) or through the whole-row select.
  const int bstar = *ws.bstar(row);
  int slot[kSlotsPerThread];
#pragma unroll
  for (int j = 0; j < kSlotsPerThread; ++j) slot[j] = ws.slots(row)[j * kRefineThreads + tid];
  const int sub = ws.sub(row)[tid < kSubBins ? tid : 0];
  uint2 early_f[kEarlyCand], early_b[kEarlyCand];
#pragma unroll
  for (int j = 0; j < kEarlyCand; ++j) {
    early_f[j] = cand[j * kRefineThreads + tid];
    early_b[j] = cand[kCandBuf - 1 - (j * kRefineThreads + tid)];
  }
  __asm__ volatile("" ::: "memory");
  const int len = clamp_len(lens, row, stride);
  const void* x = score_row<F16>(logits, row, stride);
  int32_t* out = indices + static_cast<int64_t>(row) * k;
  // Collect workgroups that took part: those whose first column is below len
  // (each took 2^collect_shift columns).
  const int n_wg = static_cast<int>((static_cast<uint32_t>(len) + (1u << collect_shift) - 1u) >> collect_shift);
  // This call's true counts: the sums of the slots of the workgroups that
  // ran, even ones (front pair) and odd ones (back pair) apart.
  i32x4 mine{0, 0, 0, 0};
#pragma unroll
  for (int j = 0; j < kSlotsPerThread; ++j) {
    const int v = j * kRefineThreads + tid < n_wg ? slot[j] : 0;
    mine[(tid & 1) * 2 + 0] += v & 0xFFFF;
    mine[(tid & 1) * 2 + 1] += v >> 16;
  }
  const i32x4 t = block_sum4(mine, s_red4);
  if (own_hist) {  // built by this call (no histogram given): the next call starts from zero
    *reinterpret_cast<int2*>(ws.hist(row) + 2 * tid) = make_int2(0, 0);
  }
  if (tid == 0) {  // the next call starts from zero
    count[0] = 0ull;
    count[1] = 0ull;
  }
  if (tid < kSubBins) ws.sub(row)[tid] = 0;
  // The counters must hold exactly this call's counts: a pair that did not
  // start at zero shifted every place its workgroups took, so the row is
  // selected from scratch rather than from places this call did not fill.
  const bool counters_ok = static_cast<uint32_t>(front) == static_cast<uint32_t>(t[0]) &&
                           static_cast<uint32_t>(front >> 32) == static_cast<uint32_t>(t[1]) &&
                           static_cast<uint32_t>(back) == static_cast<uint32_t>(t[2]) &&
                           static_cast<uint32_t>(back >> 32) == static_cast<uint32_t>(t[3]);
  const int gf = t[0], ef = t[1], gb = t[2], eb = t[3];
  const int n_gt = gf + gb, n_eq = ef + eb;
  if (!counters_ok || !counts_confirm(bstar, n_gt, n_eq, k)) {
    whole_row_select<KEY, F16>(sh, x, len, k, out);
    return;
  }
  // Columns above b* fill out[0 .. gf) and out[k - gb .. k); the selected
  // candidates go in between.
  if (bstar == kAllBins || k - n_gt == n_eq) {
    // Every candidate is taken: their columns go straight to the output.
#pragma unroll
    for (int j = 0; j < kEarlyCand; ++j) {
      const int i = j * kRefineThreads + tid;
      if (i < ef) out[gf + i] = static_cast<int32_t>(early_f[j].y);
      if (i < eb) out[gf + ef + i] = static_cast<int32_t>(early_b[j].y);
    }
    copy_rest(cand, ef, eb, [&](int i, uint2 c) { out[gf + i] = static_cast<int32_t>(c.y); });
    for (int i = gf + n_eq + tid; i < k - gb; i += kRefineThreads) out[i] = -1;
    return;
  }
  if (ef <= kEarlyCand * kRefineThreads && eb <= kEarlyCand * kRefineThreads) {  // uniform
    uint2 c[kRegCand];
    uint32_t valid = 0u;
#pragma unroll
    for (int j = 0; j < kEarlyCand; ++j) {
      const int i = j * kRefineThreads + tid;
      c[j] = early_f[j];
      c[kEarlyCand + j] = early_b[j];
      valid |= (i < ef ? 1u : 0u) << j;
      valid |= (i < eb ? 1u : 0u) << (kEarlyCand + j);
    }
    finish_regs(sh, out, k, len, k - n_gt, n_eq, gf, c, valid);
    return;
  }
  if (n_eq > kCutMin) {  // uniform
    // A large bin: cut once more by its sub-bins.  Candidate i of the list
    // (front entries [0, ef), then back entries) is taken by thread i % 512,
    // all of a thread's (at most 32) requested at once: one round trip for up
    // to 16384 candidates; indices past n_eq reread the last one, in bounds,
    // and are masked off.  They stay in registers: only the candidates that go
    // on are written to LDS.
    constexpr int kMaxPer = kCandBuf / kRefineThreads;
    static_assert(kMaxPer <= 32, "masks hold one bit per candidate");
    uint2 c[kMaxPer];
#pragma unroll
    for (int j = 0; j < kMaxPer; ++j) {
      const int i = min(j * kRefineThreads + tid, n_eq - 1);
      c[j] = make_uint2(0u, 0u);
      if (j * kRefineThreads < n_eq) c[j] = cand[i < ef ? i : kCandBuf - 1 - (i - ef)];  // uniform
    }
    // The sub-bin s* where the running count (largest sub-bins first)
    // reaches need; the candidates of higher sub-bins are taken, those of s*
    // refined.
    if (tid == 0) sh.bcast[0] = -1;
    if (tid < kSubBins) sh.digit_hist[tid] = sub;
    lds_barrier();
    const int need = k - n_gt;
    int sub_above = 0, sub_in = 0;
    const int sstar = pick_digit(sh, need, &sub_above, &sub_in);
    uint32_t m_live = 0u, m_above = 0u, m_in = 0u;
    const SubDigit sd(bstar);
    const uint32_t sstar_u = static_cast<uint32_t>(sstar);
#pragma unroll
    for (int j = 0; j < kMaxPer; ++j) {
      const bool live = j * kRefineThreads + tid < n_eq;
      const uint32_t d = sd.of(key16_of<F16 ? IDX_KEY_FP16 : KEY>(c[j].x));
      m_live |= (live ? 1u : 0u) << j;
      m_above |= (live && d > sstar_u ? 1u : 0u) << j;
      m_in |= (live && d == sstar_u ? 1u : 0u) << j;
    }
    int2 tot2;
    const int2 off = block_excl_scan2<kRefineThreads>(__popc(m_above), __popc(m_in), sh.red, &tot2);
    // The cut holds when the counts found confirm it: fewer than need above
    // s*, at least need with it (the sub-histogram is accumulated by atomics
    // on the workspace; a workspace that did not start zeroed shows here).
    // Otherwise, or when no sub-bin was found, the whole bin is refined.
    if (sstar >= 0 && tot2.x == sub_above && tot2.x < need && tot2.x + tot2.y >= need) {
      // A wave writes its entries at consecutive places from its first
      // lane's offset (the sum over the waves before it), candidate j of
      // every lane together, so that each store is contiguous.
      int pa = gf + __builtin_amdgcn_readfirstlane(off.x), pt = __builtin_amdgcn_readfirstlane(off.y);
#pragma unroll
      for (int j = 0; j < kMaxPer; ++j) {
        const bool a = (m_above >> j) & 1u, t = (m_in >> j) & 1u;
        const uint64_t ba = __ballot(a), bt = __ballot(t);
        if (a) out[pa + lanes_below(ba)] = static_cast<int32_t>(c[j].y);
        if (t) sh.cand[pt + lanes_below(bt)] = c[j];
        pa += __popcll(ba);
        pt += __popcll(bt);
      }
      lds_barrier();
      if (tot2.y <= kRegCand * kRefineThreads) {  // uniform: the kept sub-bin, from registers
        uint2 r[kRegCand];
        uint32_t valid = 0u;
#pragma unroll
        for (int j = 0; j < kRegCand; ++j) {
          const int i = j * kRefineThreads + tid;
          r[j] = i < tot2.y ? sh.cand[i] : make_uint2(0u, 0u);
          valid |= (i < tot2.y ? 1u : 0u) << j;
        }
        finish_regs(sh, out, k, len, need - tot2.x, tot2.y, gf + tot2.x, r, valid);
      } else {
        finish_candidates(sh, out, k, n_gt + tot2.x, tot2.y, gf + tot2.x, false);
      }
      return;
    }
#pragma unroll
    for (int j = 0; j < kMaxPer; ++j)
      if ((m_live >> j) & 1u) sh.cand[j * kRefineThreads + tid] = c[j];
    finish_candidates(sh, out, k, n_gt, n_eq, gf, false);
    return;
  }
#pragma unroll
  for (int j = 0; j < kEarlyCand; ++j) {
    const int i = j * kRefineThreads + tid;
    if (i < ef) sh.cand[i] = early_f[j];
    if (i < eb) sh.cand[ef + i] = early_b[j];
  }
  copy_rest(cand, ef, eb, [&](int i, uint2 c) { sh.cand[i] = c; });
  finish_list(sh, out, k, len, n_gt, n_eq, gf);
}

}  // namespace

size_t topk_workspace_size(int32_t rows, int64_t logits_stride, int32_t k) {
  if (rows <= 0 || logits_stride <= 0 || k <= 0) return 0;
  return workspace_size(rows);
}

template <int KEY, bool F16>
void launch_rows_whole(const TopkArgs& a, hipStream_t stream, LaunchEvents ev) {
  if (a.logits_stride > kRowSpan) {  // rows of up to 2 * kRowSpan: two parts per thread
    if (a.hist)
      launch_kernel(topk_row_kernel<KEY, F16, false, 2>, dim3(a.rows), dim3(kRefineThreads), stream, ev.start,
                    ev.stop, a.logits, a.logits_stride, a.hist, a.context_lens, a.k, a.indices, nullptr, 0);
    else
      launch_kernel(topk_row_kernel<KEY, F16, true, 2>, dim3(a.rows), dim3(kRefineThreads), stream, ev.start,
                    ev.stop, a.logits, a.logits_stride, a.hist, a.context_lens, a.k, a.indices, nullptr, 0);
    return;
  }
  if (a.hist)
    launch_kernel(topk_row_kernel<KEY, F16, false, 1>, dim3(a.rows), dim3(kRefineThreads), stream, ev.start, ev.stop,
                  a.logits, a.logits_stride, a.hist, a.context_lens, a.k, a.indices, nullptr, 0);
  else
    launch_kernel(topk_row_kernel<KEY, F16, true, 1>, dim3(a.rows), dim3(kRefineThreads), stream, ev.start, ev.stop,
                  a.logits, a.logits_stride, a.hist, a.context_lens, a.k, a.indices, nullptr, 0);
}

// Top-k inside the sparse rows (at most 16384 scores each) with the columns
// mapped to logical keys through the rows' block tables.
template <int KEY>
void launch_sparse_topk_rows(const TopkArgs& a, const int32_t* table, int kb, hipStream_t stream,
                             LaunchEvents ev) {
  if (a.logits_stride > kRowSpan) {
    if (a.hist)
      launch_kernel(topk_row_kernel<KEY, false, false, 2, true>, dim3(a.rows), dim3(kRefineThreads), stream,
                    ev.start, ev.stop, a.logits, a.logits_stride, a.hist, a.context_lens, a.k, a.indices, table, kb);
    else
      launch_kernel(topk_row_kernel<KEY, false, true, 2, true>, dim3(a.rows), dim3(kRefineThreads), stream,
                    ev.start, ev.stop, a.logits, a.logits_stride, a.hist, a.context_lens, a.k, a.indices, table, kb);
    return;
  }
  if (a.hist)
    launch_kernel(topk_row_kernel<KEY, false, false, 1, true>, dim3(a.rows), dim3(kRefineThreads), stream, ev.start,
                  ev.stop, a.logits, a.logits_stride, a.hist, a.context_lens, a.k, a.indices, table, kb);
  else
    launch_kernel(topk_row_kernel<KEY, false, true, 1, true>, dim3(a.rows), dim3(kRefineThreads), stream, ev.start,
                  ev.stop, a.logits, a.logits_stride, a.hist, a.context_lens, a.k, a.indices, table, kb);
}

// Chunks per collect workgroup: two for rows of more than 64 chunks, which
// halves the atomics on their counters.  (Four measured no faster on rows of
// 2^20 scores: the extra registers halve the waves per SIMD.)
inline int chunks_per_collect(int chunks) { return chunks > 64 ? 2 : 1; }

// Chunks per histogram workgroup for rows of more than 64 chunks.
#ifndef PMQA_TOPK_HIST_CHUNKS
#define PMQA_TOPK_HIST_CHUNKS 2
#endif
constexpr int kHistChunks = PMQA_TOPK_HIST_CHUNKS;

template <int KEY, bool F16, int M>
void launch_collect(const TopkArgs& a, const Workspace& ws, const int32_t* hist, int64_t hist_stride, int chunks,
                    hipStream_t stream, hipEvent_t start) {
  const dim3 grid(static_cast<unsigned>((chunks + M - 1) / M), static_cast<unsigned>(a.rows));
  launch_kernel(topk_collect_kernel<KEY, F16, M>, grid, dim3(kThreads), stream, start, nullptr, a.logits,
                a.logits_stride, hist, a.context_lens, ws.base, a.indices, a.k, static_cast<int>(hist_stride));
}

template <int KEY, bool F16>
void launch_chunked(const TopkArgs& a, const Workspace& ws, const int32_t* hist, int64_t hist_stride, bool own_hist,
                    int chunks, hipStream_t stream, hipEvent_t start, hipEvent_t stop) {
  const int m = chunks_per_collect(chunks);
  if (m == 2) launch_collect<KEY, F16, 2>(a, ws, hist, hist_stride, chunks, stream, start);
  else launch_collect<KEY, F16, 1>(a, ws, hist, hist_stride, chunks, stream, start);
  launch_kernel(topk_finish_kernel<KEY, F16>, dim3(a.rows), dim3(kRefineThreads), stream, nullptr, stop, ws.base,
                a.context_lens, a.logits_stride, a.indices, m == 2 ? kChunkShift + 1 : kChunkShift, a.k,
                own_hist ? 1 : 0, a.logits);
}

hipError_t launch_sparse_topk(const TopkArgs& a, const int32_t* table, int kb, hipStream_t stream,
                              LaunchEvents ev) {
  if (a.logits_stride > kRowSpanMax || a.logits_f16) return hipErrorInvalidValue;  // checked by the ABI first
  if (a.key_dtype == IDX_KEY_FP32) launch_sparse_topk_rows<IDX_KEY_FP32>(a, table, kb, stream, ev);
  else launch_sparse_topk_rows<IDX_KEY_FP16>(a, table, kb, stream, ev);
  return hipGetLastError();
}

hipError_t launch_topk_rows(const TopkArgs& a, hipStream_t stream, LaunchEvents ev) {
  // FP16 scores are ranked by their FP16 keys.
  if (a.logits_stride <= kRowSpanMax) {
    if (a.logits_f16) launch_rows_whole<IDX_KEY_FP16, true>(a, stream, ev);
    else if (a.key_dtype == IDX_KEY_FP32) launch_rows_whole<IDX_KEY_FP32, false>(a, stream, ev);
    else launch_rows_whole<IDX_KEY_FP16, false>(a, stream, ev);
    return hipGetLastError();
  }
  if (a.logits_stride > kMaxChunkedStride) return hipErrorInvalidValue;  // checked by the ABI first
  const Workspace ws = carve(a.workspace);
  const int chunks = chunks_for(a.logits_stride);
  const dim3 grid(static_cast<unsigned>(chunks), static_cast<unsigned>(a.rows));
  hipEvent_t start = ev.start;  // recorded by the first kernel of the call
  const int32_t* hist = a.hist;
  int64_t hist_stride = kBins;
  if (hist == nullptr) {
    // The workspace histograms are zero (left so by the finish pass); ones
    // that are not are a stale histogram, which the counts in the scores
    // overrule (the row is then selected from scratch).
    int* wh = ws.hist(0);
    if (chunks > 64) {
      const dim3 hgrid(static_cast<unsigned>((chunks + kHistChunks - 1) / kHistChunks), static_cast<unsigned>(a.rows));
      if (a.logits_f16)
        launch_kernel(topk_hist_kernel<true, kHistChunks>, hgrid, dim3(kThreads), stream, start, nullptr, a.logits,
                      a.logits_stride, a.context_lens, wh, kRecHistStride);
      else
        launch_kernel(topk_hist_kernel<false, kHistChunks>, hgrid, dim3(kThreads), stream, start, nullptr, a.logits,
                      a.logits_stride, a.context_lens, wh, kRecHistStride);
    } else if (a.logits_f16) {
      launch_kernel(topk_hist_kernel<true, 1>, grid, dim3(kThreads), stream, start, nullptr, a.logits,
                    a.logits_stride, a.context_lens, wh, kRecHistStride);
    } else {
      launch_kernel(topk_hist_kernel<false, 1>, grid, dim3(kThreads), stream, start, nullptr, a.logits,
                    a.logits_stride, a.context_lens, wh, kRecHistStride);
    }
    start = nullptr;
    hist = wh;
    hist_stride = kRecHistStride;
  }
  const bool own = a.hist == nullptr;
  if (a.logits_f16) launch_chunked<IDX_KEY_FP16, true>(a, ws, hist, hist_stride, own, chunks, stream, start, ev.stop);
  else if (a.key_dtype == IDX_KEY_FP32)
    launch_chunked<IDX_KEY_FP32, false>(a, ws, hist, hist_stride, own, chunks, stream, start, ev.stop);
  else launch_chunked<IDX_KEY_FP16, false>(a, ws, hist, hist_stride, own, chunks, stream, start, ev.stop);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// topk_rows_noalloc: the chunked path's per-row records for up to
// IDX_NOALLOC_MAX_ROWS rows live in this fixed device array instead of a
// caller's workspace.  Each GPU holds its own copy from the time the library
// is loaded until the process ends; host code reaches it only through the
// device address hipGetSymbolAddress returns for the current device (the
// array's name is a host-side stand-in, not a device address).  Nothing in
// it has to start at zero: the finish pass checks the counters against the
// stored per-workgroup counts and leaves counters and built histograms zero.
constexpr size_t kNoallocBytes = kRowScratchBytes * IDX_NOALLOC_MAX_ROWS;  // 17,989,632
static __device__ __align__(256) unsigned char scratch[kNoallocBytes];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// The device address of `scratch` on the current device, looked up once per
// device (on its first call) with that device current.
hipError_t scratch_address(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (p == nullptr) return hipErrorInvalidSymbol;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return hipSuccess;
}
}  // namespace

size_t topk_noalloc_scratch_bytes() { return kNoallocBytes; }

hipError_t launch_topk_rows_noalloc(const TopkArgs& a, hipStream_t stream, LaunchEvents ev) {
  TopkArgs b = a;
  if (a.logits_stride > kRowSpanMax) {  // only the chunked path uses scratch
    if (a.rows > IDX_NOALLOC_MAX_ROWS) return hipErrorInvalidValue;  // checked by the ABI first
    hipError_t e = scratch_address(&b.workspace);
    if (e != hipSuccess) return e;
  }
  return launch_topk_rows(b, stream, ev);
}

hipError_t launch_score_histogram(const float* scores, int64_t stride, const int32_t* lens,
                                  int32_t rows, int32_t* hist, hipStream_t stream) {
  const int64_t chunks64 = (stride + kChunk - 1) / kChunk;
  if (chunks64 > 0x7FFFFFFF) return hipErrorInvalidValue;
  hipLaunchKernelGGL((topk_hist_kernel<false, 1>), dim3(static_cast<unsigned>(chunks64), static_cast<unsigned>(rows)),
                     dim3(kThreads), 0, stream, scores, stride, lens, hist, static_cast<int64_t>(kBins));
  return hipGetLastError();
}

}  // namespace pmqa
