// Read probes: the practical HBM read ceilings the logits kernel is measured
// against.  Measurement aids, not part of the method.
#include "indexer_common.h"
#include "launches.h"

namespace pmqa {
namespace {

// Streaming read of a contiguous buffer, with ordinary (allocating) loads --
// the cache sweep that evicts K between timed calls -- or (NT) non-temporal
// ones, as the logits kernel's page loads into LDS: the read ceiling.  Each
// workgroup reads one contiguous 32 KiB chunk, 8 16-byte loads
// per thread in flight (a wave's load instruction covers 1 KiB of
// consecutive bytes).  Of the shapes swept on this GPU (16-128 KiB chunks,
// 256-1024 threads, one to four persistent workgroups per CU, loads straight
// to LDS), this one and four persistent workgroups per CU were fastest at
// 64-512 MB (138 MB: 23.0-23.4 us median, cold caches).
constexpr int kProbeThreads = 256;
constexpr int kProbeVecs = 8;
constexpr int64_t kProbeChunk = kProbeThreads * kProbeVecs;  // 16-byte vectors: 32 KiB per workgroup

template <bool NT>
__global__ __launch_bounds__(kProbeThreads) void hbm_read_probe_kernel(const i32x4* __restrict__ src,
                                                                        int64_t n_vec, uint32_t* sink) {
  const int64_t base = static_cast<int64_t>(blockIdx.x) * kProbeChunk + threadIdx.x;
  i32x4 v[kProbeVecs];
#pragma unroll
  for (int i = 0; i < kProbeVecs; ++i) {
    const int64_t j = base + static_cast<int64_t>(i) * kProbeThreads;
    if constexpr (NT) v[i] = j < n_vec ? __builtin_nontemporal_load(src + j) : i32x4{0, 0, 0, 0};
    else v[i] = j < n_vec ? src[j] : i32x4{0, 0, 0, 0};
  }
  uint32_t acc = 0u;
#pragma unroll
  for (int i = 0; i < kProbeVecs; ++i) acc ^= static_cast<uint32_t>(v[i][0] ^ v[i][1] ^ v[i][2] ^ v[i][3]);
#pragma unroll
  for (int off = kWave / 2; off > 0; off >>= 1) acc ^= __shfl_xor(acc, off, kWave);
  if (__lane_id() == 0 && acc == 0x9E3779B9u) atomicXor(sink, acc);  // keeps the loads live
}

// The gather probe reads with the non-temporal cache policy (`nt`), as the
// logits kernel's whole-line page loads do.
constexpr int kNtAux = 2;  // buffer-load cache-policy bits: nt

// Paged gather: the pages listed in `table` (8 KiB of FP8 keys each, plus
// the page's 64 fp32 scales), read the way a paged K stream must be read --
// page ids first, then whole-line 16-byte loads of each page -- with no
// arithmetic.  Workgroups of 8 waves take 64 consecutive table entries; wave
// w reads entries w, w + 8, ... with the next page in flight while the
// current one is folded into a checksum.  The fastest of the static shapes
// swept on a long-decode pool (4 or 8 waves, 8-64 pages per workgroup,
// strided or contiguous shares, operand-layout or whole-line loads).
constexpr int kGatherWaves = 8;
constexpr int kGatherPagesPerWg = 64;

struct GatherPage {
  i32x4 v[kPageBytes / 1024];
  int sc;
};

__device__ __forceinline__ void gather_load(const uint8_t* pool, const float* scales, int page, int lane,
                                            GatherPage& p) {
  const __amdgpu_buffer_rsrc_t kr = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint8_t*>(pool + static_cast<int64_t>(page) * kPageBytes), 0, kPageBytes, 0x00020000);
#pragma unroll
  for (int i = 0; i < kPageBytes / 1024; ++i)
    p.v[i] = __builtin_bit_cast(i32x4, __builtin_amdgcn_raw_buffer_load_b128(kr, i * 1024 + lane * 16, 0, kNtAux));
  const __amdgpu_buffer_rsrc_t sr = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<float*>(scales + static_cast<int64_t>(page) * kPage), 0, kPage * 4, 0x00020000);
  p.sc = __builtin_amdgcn_raw_buffer_load_b32(sr, lane * 4, 0, kNtAux);
}

__device__ __forceinline__ uint32_t gather_fold(const GatherPage& p) {
  uint32_t a = static_cast<uint32_t>(p.sc);
#pragma unroll
  for (int i = 0; i < kPageBytes / 1024; ++i) a ^= static_cast<uint32_t>(p.v[i][0] ^ p.v[i][1] ^ p.v[i][2] ^ p.v[i][3]);
  return a;
}

__global__ __launch_bounds__(kGatherWaves * kWave) void hbm_gather_probe_kernel(
    const uint8_t* __restrict__ pool, const float* __restrict__ scales, const int32_t* __restrict__ table,
    int32_t n_pages, int32_t pool_pages, uint32_t* sink) {
  const int lane = __lane_id();
  const int wave = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x) / kWave);
  const int first = static_cast<int>(blockIdx.x) * kGatherPagesPerWg + wave;
  const int last = min(static_cast<int>(blockIdx.x) * kGatherPagesPerWg + kGatherPagesPerWg, n_pages);
  const int count = last > first ? (last - first + kGatherWaves - 1) / kGatherWaves : 0;
  if (count == 0) return;
  // lane i holds the wave's i-th page id (at most 64 / 8 = 8 of them)
  const int ids = table[min(first + lane * kGatherWaves, n_pages - 1)];
  auto id = [&](int it) { return min(max(__builtin_amdgcn_readlane(ids, it), 0), pool_pages - 1); };
  GatherPage a, b;
  uint32_t acc = 0u;
  gather_load(pool, scales, id(0), lane, a);
  for (int it = 0;;) {
    gather_load(pool, scales, id(it + 1 < count ? it + 1 : it), lane, b);
    acc ^= gather_fold(a);
    if (++it >= count) break;
    gather_load(pool, scales, id(it + 1 < count ? it + 1 : it), lane, a);
    acc ^= gather_fold(b);
    if (++it >= count) break;
  }
  if (acc == 0x9E3779B9u) atomicXor(sink, acc);  // keeps the loads live
}

// MFMA / VALU co-issue: every wave runs `iters` rounds of four independent
// fp8 16x16x128 MFMAs (the logits kernels' instruction) and/or 32
// independent fp32 FMAs (eight per MFMA: the logits epilogue's two VALU
// operations on each of an MFMA's four outputs per lane), with no dependence
// between the two streams.  Timing the three modes shows how far the matrix
// and vector pipes of a SIMD overlap; the result per thread is stored so
// that nothing is dropped.
constexpr int kCoissueFmas = 32;

template <int MODE>
__global__ __launch_bounds__(256) void mfma_valu_probe_kernel(float* __restrict__ out, int iters, float c) {
  // e4m3 bytes 0x38 / 0x39 (1.0, 1.125) and 0x30 (0.5): finite products
  const int lo = 0x38383838 + static_cast<int>(threadIdx.x & 1u);
  const i32x8 a = {lo, lo, lo, lo, lo, lo, lo, lo};
  const i32x8 b = {0x30303030, 0x30303030, 0x30303030, 0x30303030,
                   0x30303030, 0x30303030, 0x30303030, 0x30303030};
  f32x4 acc0 = {0.f, 0.f, 0.f, 0.f}, acc1 = acc0, acc2 = acc0, acc3 = acc0;
  float v[kCoissueFmas];
#pragma unroll
  for (int i = 0; i < kCoissueFmas; ++i) v[i] = static_cast<float>(threadIdx.x) * 1e-3f + static_cast<float>(i);
  for (int it = 0; it < iters; ++it) {
    if constexpr (MODE != 1) {
      acc0 = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, acc0, 0, 0, 0, 127, 0, 127);
      acc1 = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, acc1, 0, 0, 0, 127, 0, 127);
      acc2 = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, acc2, 0, 0, 0, 127, 0, 127);
      acc3 = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, acc3, 0, 0, 0, 127, 0, 127);
    }
    if constexpr (MODE != 0) {
#pragma unroll
      for (int i = 0; i < kCoissueFmas; ++i) v[i] = fmaf(v[i], c, 0.5f);
    }
  }
  float s = acc0[0] + acc1[1] + acc2[2] + acc3[3];
#pragma unroll
  for (int i = 0; i < kCoissueFmas; ++i) s += v[i];
  out[static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x] = s;
}

}  // namespace

hipError_t launch_mfma_valu_probe(int mode, int workgroups, int iters, float* out, hipStream_t stream,
                                  LaunchEvents ev) {
  const dim3 grid(static_cast<unsigned>(workgroups)), block(256);
  if (mode == 0)
    launch_kernel(mfma_valu_probe_kernel<0>, grid, block, stream, ev.start, ev.stop, out, iters, 0.999f);
  else if (mode == 1)
    launch_kernel(mfma_valu_probe_kernel<1>, grid, block, stream, ev.start, ev.stop, out, iters, 0.999f);
  else
    launch_kernel(mfma_valu_probe_kernel<2>, grid, block, stream, ev.start, ev.stop, out, iters, 0.999f);
  return hipGetLastError();
}

hipError_t launch_hbm_read_probe(const void* src, size_t bytes, uint32_t* sink, bool nt, hipStream_t stream,
                                 LaunchEvents ev) {
  const int64_t n_vec = static_cast<int64_t>(bytes / 16);
  const int64_t grid = (n_vec + kProbeChunk - 1) / kProbeChunk;
  if (grid < 1 || grid > 0x7FFFFFFF) return hipErrorInvalidValue;
  launch_kernel(nt ? hbm_read_probe_kernel<true> : hbm_read_probe_kernel<false>, dim3(static_cast<unsigned>(grid)),
                dim3(kProbeThreads), stream, ev.start, ev.stop, static_cast<const i32x4*>(src), n_vec, sink);
  return hipGetLastError();
}

hipError_t launch_hbm_gather_probe(const uint8_t* pool, const float* scales, const int32_t* table,
                                   int32_t n_pages, int32_t pool_pages, uint32_t* sink, hipStream_t stream,
                                   LaunchEvents ev) {
  const int64_t grid = (static_cast<int64_t>(n_pages) + kGatherPagesPerWg - 1) / kGatherPagesPerWg;
  if (grid < 1 || grid > 0x7FFFFFFF) return hipErrorInvalidValue;
  launch_kernel(hbm_gather_probe_kernel, dim3(static_cast<unsigned>(grid)), dim3(kGatherWaves * kWave), stream,
                ev.start, ev.stop, pool, scales, table, n_pages, pool_pages, sink);
  return hipGetLastError();
}

}  // namespace pmqa
