// FP16-key ranges of the coarse histogram bins, for selecting against a
// threshold bin without computing each score's bin (gfx950 top-k).
#pragma once

#include "indexer_common.h"

namespace pmqa {

// The same bins as ranges of FP16 keys.  Since coarse_bin_f16 is
// non-increasing in key_f16, bin b holds exactly the non-NaN halves whose key
// lies in [lo, hi), and the bins before it exactly those with key in
// [hi, 0xFC00] (0xFC00 = key of +inf; larger keys are positive NaNs,
// keys below 0x03FF = key of -inf negative NaNs).  b == kBins (every score
// above the threshold) gives lo = hi = 0x03FF.
//
// mag_start(m): the least magnitude |h| (FP16 bits without sign) whose
// magnitude index in coarse_bin_f16 is at least m, for m in 0 .. 512.
__host__ __device__ __forceinline__ uint32_t mag_start(uint32_t m) {
  if (m <= 304u) return m << 6;          // below 16: |h| >> 6 (304 << 6 == 16.0)
  if (m >= 512u) return 0x7C01u;         // past infinity
  const uint32_t n = m - 288u;           // integer part 17 .. 223
  const uint32_t e = 31u - static_cast<uint32_t>(__builtin_clz(n));  // 4 .. 7
  return ((e + 15u) << 10) | ((n << (10u - e)) & 0x3FFu);             // FP16 bits of n
}

struct KeyRange {
  uint32_t lo, hi;
};

__host__ __device__ __forceinline__ KeyRange bin_key_range(int b) {
  if (b >= kBins) return KeyRange{0x03FFu, 0x03FFu};
  if (b < 512) {  // positive values, magnitude index 511 - b
    const uint32_t m = 511u - static_cast<uint32_t>(b);
    return KeyRange{0x8000u + mag_start(m), 0x8000u + mag_start(m + 1u)};
  }
  const uint32_t m = static_cast<uint32_t>(b) - 512u;  // negative values: key = 0x7FFF - |h|
  return KeyRange{0x8000u - mag_start(m + 1u), 0x8000u - mag_start(m)};
}

}  // namespace pmqa
