// Streaming-read probe: the practical HBM read ceiling for 16-byte vector
// loads, measured beside the logits kernel.  Not part of the method.
#include "indexer_common.h"

namespace pmqa {
namespace {

__global__ __launch_bounds__(256) void hbm_read_probe_kernel(const i32x4* __restrict__ src,
                                                              int64_t n_vec, uint32_t* sink) {
  uint32_t acc = 0u;
  const int64_t stride = static_cast<int64_t>(gridDim.x) * blockDim.x;
  int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  // Four independent loads in flight per thread per step.
  for (; i + 3 * stride < n_vec; i += 4 * stride) {
    const i32x4 a = src[i], b = src[i + stride], c = src[i + 2 * stride], d = src[i + 3 * stride];
    acc ^= static_cast<uint32_t>(a[0] ^ a[1] ^ a[2] ^ a[3] ^ b[0] ^ b[1] ^ b[2] ^ b[3] ^
                                 c[0] ^ c[1] ^ c[2] ^ c[3] ^ d[0] ^ d[1] ^ d[2] ^ d[3]);
  }
  for (; i < n_vec; i += stride) {
    const i32x4 a = src[i];
    acc ^= static_cast<uint32_t>(a[0] ^ a[1] ^ a[2] ^ a[3]);
  }
#pragma unroll
  for (int off = kWave / 2; off > 0; off >>= 1) acc ^= __shfl_xor(acc, off, kWave);
  if (__lane_id() == 0) atomicXor(sink, acc);
}

}  // namespace

hipError_t launch_hbm_read_probe(const void* src, size_t bytes, uint32_t* sink, hipStream_t stream) {
  int dev = 0, cus = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  if (e != hipSuccess) return e;
  const int64_t n_vec = static_cast<int64_t>(bytes / 16);
  int64_t grid = static_cast<int64_t>(cus) * 8;
  const int64_t need = (n_vec + 255) / 256;
  if (need < grid) grid = need > 0 ? need : 1;
  hipLaunchKernelGGL(hbm_read_probe_kernel, dim3(static_cast<unsigned>(grid)), dim3(256), 0, stream,
                     static_cast<const i32x4*>(src), n_vec, sink);
  return hipGetLastError();
}

}  // namespace pmqa
