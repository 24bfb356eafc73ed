// Streaming-read probe: the practical HBM read ceiling for 16-byte vector
// loads, measured beside the logits kernel.  Not part of the method.
#include "indexer_common.h"

namespace pmqa {
namespace {

constexpr int kProbeThreads = 256;
constexpr int kProbeVecs = 16;  // 16-byte loads per thread, all in flight together
constexpr int64_t kProbeChunk = kProbeThreads * kProbeVecs;  // 64 KiB per workgroup

// Each workgroup reads one contiguous 64 KiB chunk; a wave's load instruction
// covers 1 KiB of consecutive bytes.
__global__ __launch_bounds__(kProbeThreads) void hbm_read_probe_kernel(const i32x4* __restrict__ src,
                                                                        int64_t n_vec, uint32_t* sink) {
  const int64_t base = static_cast<int64_t>(blockIdx.x) * kProbeChunk + threadIdx.x;
  i32x4 v[kProbeVecs];
#pragma unroll
  for (int i = 0; i < kProbeVecs; ++i) {
    const int64_t j = base + static_cast<int64_t>(i) * kProbeThreads;
    v[i] = j < n_vec ? src[j] : i32x4{0, 0, 0, 0};
  }
  uint32_t acc = 0u;
#pragma unroll
  for (int i = 0; i < kProbeVecs; ++i) acc ^= static_cast<uint32_t>(v[i][0] ^ v[i][1] ^ v[i][2] ^ v[i][3]);
#pragma unroll
  for (int off = kWave / 2; off > 0; off >>= 1) acc ^= __shfl_xor(acc, off, kWave);
  if (__lane_id() == 0 && acc == 0x9E3779B9u) atomicXor(sink, acc);  // keeps the loads live
}

}  // namespace

hipError_t launch_hbm_read_probe(const void* src, size_t bytes, uint32_t* sink, hipStream_t stream,
                                 LaunchEvents ev) {
  const int64_t n_vec = static_cast<int64_t>(bytes / 16);
  const int64_t grid = (n_vec + kProbeChunk - 1) / kProbeChunk;
  if (grid < 1 || grid > 0x7FFFFFFF) return hipErrorInvalidValue;
  launch_kernel(hbm_read_probe_kernel, dim3(static_cast<unsigned>(grid)), dim3(kProbeThreads), stream,
                ev.start, ev.stop, static_cast<const i32x4*>(src), n_vec, sink);
  return hipGetLastError();
}

}  // namespace pmqa
