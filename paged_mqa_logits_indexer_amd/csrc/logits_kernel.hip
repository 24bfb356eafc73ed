// Paged MQA logits with the fused coarse histogram, for gfx950 (CDNA4).
//
// DeepGEMM PR #94, "[SM100] Paged MQA logits: fused coarse score histogram
// for LiteTopK decode", sections "Motivation" and "What this adds":
//   logit[r, s] = scale_s * sum_h w[r, h] * ReLU(q[r, h, :] . k_s)
// over the live keys s < len_r of row r, FP8 E4M3 Q and K, H = 32, D = 128,
// and, while the scores are in registers, a 1024-bin descending histogram of
// the live non-NaN scores per row, kept in on-chip memory per token and added
// to the global histogram with packed 64-bit atomics when a workgroup leaves
// a request.  All next_n rows of a request share one read of each K page (the
// token Q tile of the same section).
//
// MI355X design:
//   * Work split: the K pages of all requests form one list; the persistent
//     grid (CUs x resident workgroups) takes equal contiguous shares of it, so
//     every workgroup streams the same number of pages whatever the length
//     mix.  A share that crosses into the next request flushes the histogram
//     of the request it leaves.
//   * K is read straight into registers in the operand layout of
//     v_mfma_f32_16x16x128_f8f6f4: lane (n, g) = (lane % 16, lane / 16) takes
//     key n of a 16-key block, bytes [16g, 16g+16) and [64+16g, 64+16g+16).
//     One 16-byte load instruction then covers 16 keys x 64 contiguous bytes,
//     and the two instructions of a block cover its 2 KiB exactly.  Q uses the
//     same byte-to-k assignment, so the contraction over d is complete.
//   * Heads are the MFMA rows (two 16-head blocks), keys the columns; a lane
//     holds 8 heads of one key per row, so ReLU and the head weights are
//     applied in-lane, and a two-step lane exchange finishes the head sum and
//     leaves lane l with the logit of key l of the page (coalesced stores).
//   * The next page of every wave is in flight while the current one is
//     computed.
#include "indexer_common.h"

namespace pmqa {
namespace {

constexpr int kWaves = 4;
constexpr int kThreads = kWaves * kWave;
constexpr int kReqPerThread = (IDX_MAX_REQUESTS + kThreads - 1) / kThreads;  // 16

struct PageRegs {
  i32x4 v[8];   // [key block kb][half]: K bytes in MFMA operand layout
  float scale;  // k_scales of key `lane` of the page
};

// ReLU as one integer max on the bit pattern: a set sign bit makes the int32
// negative, so negatives and -0 become +0 and everything else passes.
__device__ __forceinline__ float relu(float x) {
  return __int_as_float(max(__float_as_int(x), 0));
}

__device__ __forceinline__ i32x8 cat8(i32x4 a, i32x4 b) {
  return i32x8{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
}

__device__ __forceinline__ void load_page(const uint8_t* __restrict__ kv_pages,
                                          const float* __restrict__ k_scales,
                                          int page, int lane, PageRegs& r) {
  const int n = lane & 15, g = lane >> 4;
  const uint8_t* base = kv_pages + static_cast<int64_t>(page) * kPageBytes + n * kDim + g * 16;
#pragma unroll
  for (int kb = 0; kb < 4; ++kb) {
    r.v[2 * kb + 0] = *reinterpret_cast<const i32x4*>(base + kb * 16 * kDim);
    r.v[2 * kb + 1] = *reinterpret_cast<const i32x4*>(base + kb * 16 * kDim + 64);
  }
  r.scale = k_scales[static_cast<int64_t>(page) * kPage + lane];
}

// Sum over the four lane groups g of part[kb], leaving lane (n, g) with the
// total of key block g.  Two exchanges instead of one per key block.
__device__ __forceinline__ float reduce_scatter4(const float (&part)[4], int g) {
  const bool hi = g >= 2;
  const float s0 = hi ? part[0] : part[2];
  const float s1 = hi ? part[1] : part[3];
  const float r0 = __shfl_xor(s0, 32, kWave);
  const float r1 = __shfl_xor(s1, 32, kWave);
  const float k0 = (hi ? part[2] : part[0]) + r0;
  const float k1 = (hi ? part[3] : part[1]) + r1;
  const bool odd = g & 1;
  const float s = odd ? k0 : k1;
  const float r = __shfl_xor(s, 16, kWave);
  return (odd ? k1 : k0) + r;
}

template <int NN>
struct RequestRegs {
  i32x4 q[NN][2][2];  // [token][head block][half], operand layout
  f32x4 w[NN][2];     // weights of heads 16*mb + 4g + i
  int len[NN];
};

template <int NN, bool HIST>
__device__ __forceinline__ void compute_page(const PageRegs& pr, int lp, int lane,
                                             const RequestRegs<NN>& rq,
                                             float* __restrict__ logits,
                                             int64_t stride, int row0, int* s_hist) {
  const int g = lane >> 4;
  const int key = lp * kPage + lane;
#pragma unroll
  for (int j = 0; j < NN; ++j) {
    f32x4 acc[4][2];
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
      const i32x8 b = cat8(pr.v[2 * kb], pr.v[2 * kb + 1]);
#pragma unroll
      for (int mb = 0; mb < 2; ++mb) {
        const i32x8 a = cat8(rq.q[j][mb][0], rq.q[j][mb][1]);
        acc[kb][mb] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
            a, b, f32x4{0.f, 0.f, 0.f, 0.f}, 0, 0, 0, 127, 0, 127);
      }
    }
    float part[4];
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
      float s = 0.f;
#pragma unroll
      for (int mb = 0; mb < 2; ++mb) {
#pragma unroll
        for (int i = 0; i < 4; ++i) s = fmaf(rq.w[j][mb][i], relu(acc[kb][mb][i]), s);
      }
      part[kb] = s;
    }
    const float logit = reduce_scatter4(part, g) * pr.scale;
    if (key < rq.len[j]) {
      logits[static_cast<int64_t>(row0 + j) * stride + key] = logit;
      if constexpr (HIST) {
        const uint32_t hb = f16_bits_rn(logit);
        if (!f16_is_nan(hb)) atomicAdd(&s_hist[j * kBins + coarse_bin_f16(hb)], 1);
      }
    }
  }
}

__device__ __forceinline__ int block_exclusive_scan(int v, int* s_wave, int& total) {
  const int lane = __lane_id(), wave = threadIdx.x / kWave;
  const int inc = wave_inclusive_scan(v);
  if (lane == kWave - 1) s_wave[wave] = inc;
  __syncthreads();
  int before = 0, all = 0;
#pragma unroll
  for (int w = 0; w < kWaves; ++w) {
    const int t = s_wave[w];
    before += (w < wave) ? t : 0;
    all += t;
  }
  total = all;
  __syncthreads();
  return before + inc - v;
}

template <int NN, bool HIST>
__global__ __launch_bounds__(kThreads) void indexer_logits_kernel(LogitsArgs a) {
  __shared__ int s_start[IDX_MAX_REQUESTS + 1];  // first global page of request b
  __shared__ int s_wave[kWaves];
  __shared__ int s_hist[HIST ? NN * kBins : 1];

  const int tid = threadIdx.x;
  const int lane = __lane_id();
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int B = a.B;
  // No row reads past its block-table row or writes past its logits row.
  const int64_t mk = min(static_cast<int64_t>(a.max_pages) * kPage, a.logits_stride);
  const int max_keys = static_cast<int>(min(mk, static_cast<int64_t>(INT32_MAX)));

  // 1. Pages of each request (its longest row), exclusive prefix over requests.
  // Loads are unconditional (index clamped) so that all of them are in flight
  // together; requests past B count zero pages.
  int pages_local[kReqPerThread];
  int my_sum = 0;
#pragma unroll
  for (int i = 0; i < kReqPerThread; ++i) {
    const int b = tid * kReqPerThread + i;
    const int bc = min(b, B - 1);
    int mx = 0;
#pragma unroll
    for (int j = 0; j < NN; ++j) mx = max(mx, a.context_lens[bc * NN + j]);
    mx = min(max(mx, 0), max_keys);
    const int pg = b < B ? (mx >> 6) + ((mx & (kPage - 1)) != 0) : 0;
    pages_local[i] = pg;
    my_sum += pg;
  }
  int total = 0;
  int run = block_exclusive_scan(my_sum, s_wave, total);
#pragma unroll
  for (int i = 0; i < kReqPerThread; ++i) {
    const int b = tid * kReqPerThread + i;
    if (b < B) s_start[b] = run;
    run += pages_local[i];
  }
  if (tid == 0) s_start[B] = total;
  if constexpr (HIST) {
    for (int i = tid; i < NN * kBins; i += kThreads) s_hist[i] = 0;
  }
  __syncthreads();

  // 2. This workgroup's equal share [p0, p1) of the global page list.
  const int64_t G = gridDim.x;
  int p0 = static_cast<int>(static_cast<int64_t>(total) * blockIdx.x / G);
  const int p1 = static_cast<int>(static_cast<int64_t>(total) * (blockIdx.x + 1) / G);
  if (p0 >= p1) return;

  // Request holding page p0: the last b with s_start[b] <= p0.
  int lo = 0, hi = B;  // s_start[lo] <= p0 < s_start[hi]
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (s_start[mid] <= p0) lo = mid; else hi = mid;
  }
  int b = lo;

  while (p0 < p1) {
    while (s_start[b + 1] <= p0) ++b;  // skip requests without pages
    const int seg_begin = p0 - s_start[b];
    const int seg_end = min(p1, s_start[b + 1]) - s_start[b];
    const int row0 = b * NN;

    RequestRegs<NN> rq;
    {
      const int m = lane & 15, g = lane >> 4;
#pragma unroll
      for (int j = 0; j < NN; ++j) {
        rq.len[j] = min(max(a.context_lens[row0 + j], 0), max_keys);
#pragma unroll
        for (int mb = 0; mb < 2; ++mb) {
          const uint8_t* qp = a.q + (static_cast<int64_t>(row0 + j) * kHeads + mb * 16 + m) * kDim + g * 16;
          rq.q[j][mb][0] = *reinterpret_cast<const i32x4*>(qp);
          rq.q[j][mb][1] = *reinterpret_cast<const i32x4*>(qp + 64);
          rq.w[j][mb] = *reinterpret_cast<const f32x4*>(a.weights + static_cast<int64_t>(row0 + j) * kHeads + mb * 16 + 4 * g);
        }
      }
    }

    // Pages seg_begin + wave, + kWaves, ... of request b; up to 64 page ids
    // are fetched at once, lane i holding the id of the wave's i-th page.
    const int n_mine = seg_end - seg_begin > wave ? (seg_end - seg_begin - wave + kWaves - 1) / kWaves : 0;
    const int32_t* bt = a.block_table + static_cast<int64_t>(b) * a.max_pages;
    auto fetch_ids = [&](int it0) {
      const int it = it0 + lane;
      int id = 0;
      if (it < n_mine) id = bt[seg_begin + wave + it * kWaves];
      return min(max(id, 0), a.num_pages - 1);
    };
    int ids = fetch_ids(0);
    int ids_base = 0;

    if (n_mine > 0) {
      PageRegs cur, nxt;
      load_page(a.kv_pages, a.k_scales, __builtin_amdgcn_readlane(ids, 0), lane, cur);
      for (int it = 0; it < n_mine; it += 2) {
        // Issue the next page (the current one again at the end: it is cached).
        int it1 = it + 1 < n_mine ? it + 1 : it;
        if (it1 - ids_base >= kWave) { ids = fetch_ids(it1); ids_base = it1; }
        load_page(a.kv_pages, a.k_scales, __builtin_amdgcn_readlane(ids, it1 - ids_base), lane, nxt);
        compute_page<NN, HIST>(cur, seg_begin + wave + it * kWaves, lane, rq, a.logits,
                               a.logits_stride, row0, s_hist);
        if (it + 1 >= n_mine) break;
        int it2 = it + 2 < n_mine ? it + 2 : it + 1;
        if (it2 - ids_base >= kWave) { ids = fetch_ids(it2); ids_base = it2; }
        load_page(a.kv_pages, a.k_scales, __builtin_amdgcn_readlane(ids, it2 - ids_base), lane, cur);
        compute_page<NN, HIST>(nxt, seg_begin + wave + (it + 1) * kWaves, lane, rq, a.logits,
                               a.logits_stride, row0, s_hist);
      }
    }

    if constexpr (HIST) {
      // Flush the request's slots: pairs of bins with one 64-bit atomic each.
      __syncthreads();
      unsigned long long* gh = reinterpret_cast<unsigned long long*>(a.hist + static_cast<int64_t>(row0) * kBins);
      uint2* sh = reinterpret_cast<uint2*>(s_hist);
      for (int i = tid; i < NN * kBins / 2; i += kThreads) {
        const uint2 v = sh[i];
        if (v.x | v.y) {
          atomicAdd(gh + i, (static_cast<unsigned long long>(v.y) << 32) | v.x);
          sh[i] = uint2{0u, 0u};
        }
      }
      __syncthreads();
    }
    p0 = s_start[b] + seg_end;
    ++b;
  }
}

struct DeviceInfo {
  int cus = 0;
  int occ[4][2] = {};
};

DeviceInfo* device_info(int dev) {
  static DeviceInfo infos[64];
  static bool ready[64] = {};
  if (dev < 0 || dev >= 64) return nullptr;
  if (!ready[dev]) {
    DeviceInfo d;
    if (hipDeviceGetAttribute(&d.cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return nullptr;
    auto occ = [](const void* f) {
      int n = 0;
      if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, f, kThreads, 0) != hipSuccess) n = 1;
      return n > 0 ? n : 1;
    };
    d.occ[0][0] = occ(reinterpret_cast<const void*>(indexer_logits_kernel<1, false>));
    d.occ[0][1] = occ(reinterpret_cast<const void*>(indexer_logits_kernel<1, true>));
    d.occ[1][0] = occ(reinterpret_cast<const void*>(indexer_logits_kernel<2, false>));
    d.occ[1][1] = occ(reinterpret_cast<const void*>(indexer_logits_kernel<2, true>));
    d.occ[2][0] = occ(reinterpret_cast<const void*>(indexer_logits_kernel<3, false>));
    d.occ[2][1] = occ(reinterpret_cast<const void*>(indexer_logits_kernel<3, true>));
    d.occ[3][0] = occ(reinterpret_cast<const void*>(indexer_logits_kernel<4, false>));
    d.occ[3][1] = occ(reinterpret_cast<const void*>(indexer_logits_kernel<4, true>));
    infos[dev] = d;
    ready[dev] = true;  // benign race: every thread computes the same values
  }
  return &infos[dev];
}

template <int NN, bool HIST>
hipError_t launch(const LogitsArgs& a, int grid, hipStream_t stream) {
  hipLaunchKernelGGL((indexer_logits_kernel<NN, HIST>), dim3(grid), dim3(kThreads), 0, stream, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_indexer_logits(const LogitsArgs& a, hipStream_t stream) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  const DeviceInfo* info = device_info(dev);
  if (!info) return hipErrorInvalidDevice;
  const bool hist = a.hist != nullptr;
  const int64_t upper = static_cast<int64_t>(a.B) * a.max_pages;  // pages at most
  int64_t grid = static_cast<int64_t>(info->cus) * info->occ[a.next_n - 1][hist ? 1 : 0];
  if (upper < grid) grid = upper;
  if (grid < 1) grid = 1;
  const int g = static_cast<int>(grid);
  switch (a.next_n * 2 + (hist ? 1 : 0)) {
    case 2: return launch<1, false>(a, g, stream);
    case 3: return launch<1, true>(a, g, stream);
    case 4: return launch<2, false>(a, g, stream);
    case 5: return launch<2, true>(a, g, stream);
    case 6: return launch<3, false>(a, g, stream);
    case 7: return launch<3, true>(a, g, stream);
    case 8: return launch<4, false>(a, g, stream);
    case 9: return launch<4, true>(a, g, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace pmqa
