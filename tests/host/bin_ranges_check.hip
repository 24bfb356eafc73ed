// Host-side check of bin_key_range against coarse_bin_f16 and key_f16 over
// every FP16 encoding and every threshold bin (plus "all bins"): a half is in
// the key range [lo, hi) exactly when its bin is b, and in [hi, key(+inf)]
// exactly when its bin comes before b; NaNs are in neither.  Prints the
// number of mismatches and exits non-zero if there are any.  Also checks the
// branch-free bin (coarse_bin_f16_flat) against coarse_bin_f16 for every
// non-NaN half.
#include <cstdio>

#include "bin_key_range.h"
#include "indexer_common.h"

int main() {
  using namespace pmqa;
  long bad = 0, checked = 0;
  for (int b = 0; b <= kBins; ++b) {
    const KeyRange r = bin_key_range(b);
    for (uint32_t hb = 0; hb < 0x10000u; ++hb) {
      const uint32_t key = key_f16(hb);
      const bool in_eq = key >= r.lo && key < r.hi;
      const bool in_gt = key >= r.hi && key <= 0xFC00u;
      bool want_eq = false, want_gt = false;
      if (!f16_is_nan(hb)) {
        const int bin = coarse_bin_f16(hb);
        want_eq = bin == b;
        want_gt = bin < b;
      }
      if (in_eq != want_eq || in_gt != want_gt) {
        if (bad < 10) std::printf("bin %d half 0x%04x: eq %d/%d gt %d/%d\n", b, hb, in_eq, want_eq, in_gt, want_gt);
        ++bad;
      }
      ++checked;
    }
  }
  // the branch-free bin the logits kernel uses, against the reference form
  for (uint32_t hb = 0; hb < 0x10000u; ++hb) {
    if (f16_is_nan(hb)) continue;
    if (coarse_bin_f16_flat(hb) != coarse_bin_f16(hb)) {
      if (bad < 10) std::printf("flat bin of half 0x%04x: %d, want %d\n", hb, coarse_bin_f16_flat(hb), coarse_bin_f16(hb));
      ++bad;
    }
    ++checked;
  }
  std::printf("checked %ld, mismatches %ld\n", checked, bad);
  return bad == 0 ? 0 : 1;
}
