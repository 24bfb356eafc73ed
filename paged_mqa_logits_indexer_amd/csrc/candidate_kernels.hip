// Two-level candidate indexer, around the sparse logits (gfx950).
//
// SGLang PR #38944, "[DSV4.1] Enable the two-level candidate indexer on
// DeepGEMM's paged sparse MQA logits": the candidate-source layer publishes,
// per query row, an ascending table of 8-token logical blocks; the layers
// after it score those blocks only and select inside that sparse row.  The
// commit that replaces the source layer's torch pieces defines the two
// kernels here: amax8_varlen (block maxima, the newest block +inf) and
// sort_candidate_blocks (selected ids -> ascending INT32_MAX-padded table plus
// the same blocks as pool slots / 8, counting sort over a 16 KiB bitmap,
// identity table for rows with at most k blocks).  sparse_to_logical maps the
// selection inside a sparse row back to logical key positions.
#include <climits>

#include "indexer_common.h"
#include "launches.h"

namespace pmqa {
namespace {

constexpr int kBlk = 8;                  // tokens per candidate block
constexpr int kSortThreads = 256;
constexpr int kBitmapWords = kMaxCandidateBlocks / 32;  // 4096 words = 16 KiB
constexpr int kWordsPerThread = kBitmapWords / kSortThreads;

// One thread per (row, block): the NaN-ignoring maximum of the block's 8
// scores (v_max_f32 returns the other operand when one is NaN), +inf for the
// row's newest block; nothing is written at or past ceil(len / 8).  Every
// block before the newest lies wholly below len, so its two 16-byte loads
// read live scores only.  HIST: the maxima also go into the row's coarse
// histogram (per-workgroup LDS slots added with 64-bit atomics, as in the
// logits kernel), so the block top-k can skip its own first pass.  The first
// thread of each row writes the row's block count to block_lens (if given):
// the lengths the block top-k takes.
template <bool HIST>
__global__ __launch_bounds__(256) void block_amax8_kernel(const float* __restrict__ scores, int64_t stride,
                                                          const int32_t* __restrict__ lens,
                                                          float* __restrict__ out, int64_t out_stride,
                                                          int32_t* __restrict__ hist,
                                                          int32_t* __restrict__ block_lens) {
  __shared__ int s_hist[HIST ? kBins : 1];
  const int row = blockIdx.y;
  const int64_t j = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  const int64_t l = lens[row];
  const int64_t len = l < 0 ? 0 : (l > stride ? stride : l);
  const int64_t nb = (len + kBlk - 1) / kBlk;  // < 2^28: stride < 2^31
  if (block_lens && j == 0) block_lens[row] = static_cast<int32_t>(nb);
  if (static_cast<int64_t>(blockIdx.x) * 256 >= nb) return;  // uniform: no block of this row here
  if constexpr (HIST) {
    for (int i = threadIdx.x; i < kBins; i += 256) s_hist[i] = 0;
    __syncthreads();
  }
  if (j < nb) {
    float m = __int_as_float(0x7F800000);  // +inf: the newest block
    if (j < nb - 1) {
      const f32x4* p = reinterpret_cast<const f32x4*>(scores + static_cast<int64_t>(row) * stride + kBlk * j);
      const f32x4 a = p[0], b = p[1];
      m = fmaxf(fmaxf(fmaxf(a[0], a[1]), fmaxf(a[2], a[3])), fmaxf(fmaxf(b[0], b[1]), fmaxf(b[2], b[3])));
    }
    out[static_cast<int64_t>(row) * out_stride + j] = m;
    if constexpr (HIST) {
      const uint32_t hb = f16_bits_rn(m);
      if (!f16_is_nan(hb)) atomicAdd(&s_hist[coarse_bin_f16(hb)], 1);
    }
  }
  if constexpr (HIST) {
    __syncthreads();
    unsigned long long* gh = reinterpret_cast<unsigned long long*>(hist + static_cast<int64_t>(row) * kBins);
    const uint2* sh = reinterpret_cast<const uint2*>(s_hist);
    for (int i = threadIdx.x; i < kBins / 2; i += 256) {
      const uint2 v = sh[i];
      if (v.x | v.y) atomicAdd(gh + i, (static_cast<unsigned long long>(v.y) << 32) | v.x);
    }
  }
}

// One workgroup per row.  Rows with at most kb blocks get the identity table;
// otherwise the listed ids in [0, nb) set bits of an LDS bitmap (duplicates
// and out-of-range entries drop out), each thread counts the set bits of 16
// consecutive words, a block scan gives its first output place, and it emits
// its ids in ascending order.  All reads of `blocks` precede the first write
// of `table`, so the two may be the same buffer.
__global__ __launch_bounds__(kSortThreads) void sort_candidate_blocks_kernel(
    const int32_t* __restrict__ blocks, int kb, const int32_t* __restrict__ lens, int64_t max_len,
    const int32_t* __restrict__ block_table, int max_pages, int next_n, int32_t* table,
    int32_t* __restrict__ slots, int32_t* __restrict__ sparse_lens) {
  __shared__ uint32_t s_bits[kBitmapWords];
  __shared__ int s_red[kSortThreads / kWave];
  const int row = blockIdx.x;
  const int tid = threadIdx.x;
  const int64_t l = lens[row];
  const int len = static_cast<int>(l < 0 ? 0 : (l > max_len ? max_len : l));
  const int nb = (len + kBlk - 1) / kBlk;  // <= kMaxCandidateBlocks (host check on max_len)
  const int32_t* in = blocks + static_cast<int64_t>(row) * kb;
  int32_t* tout = table + static_cast<int64_t>(row) * kb;
  int32_t* sout = slots + static_cast<int64_t>(row) * kb;
  const int32_t* bt = block_table + static_cast<int64_t>(row / next_n) * max_pages;
  // pool slot / 8 of block b: page * 64 + (8 b) % 64, over 8
  auto slot8 = [&](int b) {
    const int page = bt[min((b * kBlk) / kPage, max_pages - 1)];
    return page * (kPage / kBlk) + (b & (kPage / kBlk - 1));
  };
  if (nb <= kb) {
    for (int i = tid; i < kb; i += kSortThreads) {
      tout[i] = i < nb ? i : INT_MAX;
      sout[i] = i < nb ? slot8(i) : INT_MAX;
    }
    if (tid == 0) sparse_lens[row] = len;
    return;
  }
  const int words = (nb + 31) / 32;
  for (int w = tid; w < words; w += kSortThreads) s_bits[w] = 0u;
  __syncthreads();
  for (int i = tid; i < kb; i += kSortThreads) {
    const int b = in[i];
    if (b >= 0 && b < nb) atomicOr(&s_bits[b >> 5], 1u << (b & 31));
  }
  __syncthreads();
  const int w0 = tid * kWordsPerThread;
  int cnt = 0;
#pragma unroll
  for (int u = 0; u < kWordsPerThread; ++u) cnt += w0 + u < words ? __popc(s_bits[w0 + u]) : 0;
  // exclusive scan of the counts over the workgroup
  const int inc = wave_inclusive_scan(cnt);
  if (__lane_id() == kWave - 1) s_red[tid / kWave] = inc;
  __syncthreads();
  int base = inc - cnt, total = 0;
#pragma unroll
  for (int w = 0; w < kSortThreads / kWave; ++w) {
    base += w < tid / kWave ? s_red[w] : 0;
    total += s_red[w];
  }
#pragma unroll
  for (int u = 0; u < kWordsPerThread; ++u) {
    uint32_t m = w0 + u < words ? s_bits[w0 + u] : 0u;
    while (m) {
      const int bit = __ffs(m) - 1;
      m &= m - 1u;
      tout[base++] = (w0 + u) * 32 + bit;  // base < total <= kb: at most kb bits were set
    }
  }
  for (int i = total + tid; i < kb; i += kSortThreads) {
    tout[i] = INT_MAX;
    sout[i] = INT_MAX;
  }
  // The page transform in a second pass over the written table (visible to
  // the whole workgroup after the barrier), so a thread's block-table loads
  // are independent of each other rather than one per emitted id in turn.
  __syncthreads();
  for (int i = tid; i < total; i += kSortThreads) sout[i] = slot8(tout[i]);
  if (tid == 0) {
    // every listed block is whole except the newest, which holds len - 8 (nb - 1) keys
    const bool newest = (s_bits[(nb - 1) >> 5] >> ((nb - 1) & 31)) & 1u;
    sparse_lens[row] = total * kBlk - (newest ? nb * kBlk - len : 0);
  }
}

// Column c of a sparse row is key 8 * table[c / 8] + c % 8; -1 stays -1 and
// so does a column past the table.
__global__ void sparse_to_logical_kernel(const int32_t* __restrict__ idx, int k,
                                         const int32_t* __restrict__ table, int kb, int rows,
                                         int32_t* __restrict__ out) {
  const int64_t n = static_cast<int64_t>(rows) * k;
  for (int64_t e = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; e < n;
       e += static_cast<int64_t>(gridDim.x) * blockDim.x) {
    const int row = static_cast<int>(e / k);
    const int c = idx[e];
    int v = -1;
    if (c >= 0 && c < kb * kBlk) {
      const int b = table[static_cast<int64_t>(row) * kb + c / kBlk];
      v = b == INT_MAX ? -1 : b * kBlk + (c & (kBlk - 1));
    }
    out[e] = v;
  }
}

}  // namespace

hipError_t launch_block_amax8(const float* scores, int64_t stride, const int32_t* lens, int32_t rows, float* out,
                              int64_t out_stride, int32_t* hist, int32_t* block_lens, hipStream_t stream,
                              LaunchEvents ev) {
  const int64_t nbmax = (stride + kBlk - 1) / kBlk;
  const int64_t gx = (nbmax + 255) / 256;
  if (gx > 0x7FFFFFFF) return hipErrorInvalidValue;
  const dim3 grid(static_cast<unsigned>(gx), static_cast<unsigned>(rows));
  if (hist)
    launch_kernel(block_amax8_kernel<true>, grid, dim3(256), stream, ev.start, ev.stop, scores, stride, lens, out,
                  out_stride, hist, block_lens);
  else
    launch_kernel(block_amax8_kernel<false>, grid, dim3(256), stream, ev.start, ev.stop, scores, stride, lens, out,
                  out_stride, hist, block_lens);
  return hipGetLastError();
}

hipError_t launch_sort_candidate_blocks(const int32_t* blocks, int32_t kb, const int32_t* lens, int32_t rows,
                                        int64_t max_len, const int32_t* block_table, int32_t max_pages,
                                        int32_t next_n, int32_t* table, int32_t* slots, int32_t* sparse_lens,
                                        hipStream_t stream, LaunchEvents ev) {
  launch_kernel(sort_candidate_blocks_kernel, dim3(rows), dim3(kSortThreads), stream, ev.start, ev.stop, blocks,
                kb, lens, max_len, block_table, max_pages, next_n, table, slots, sparse_lens);
  return hipGetLastError();
}

hipError_t launch_sparse_to_logical(const int32_t* idx, int32_t k, const int32_t* table, int32_t kb, int32_t rows,
                                    int32_t* out, hipStream_t stream, LaunchEvents ev) {
  const int64_t n = static_cast<int64_t>(rows) * k;
  const int64_t want = (n + 255) / 256;
  const int grid = static_cast<int>(want < 4096 ? (want > 0 ? want : 1) : 4096);
  launch_kernel(sparse_to_logical_kernel, dim3(grid), dim3(256), stream, ev.start, ev.stop, idx, k, table, kb,
                rows, out);
  return hipGetLastError();
}

}  // namespace pmqa
