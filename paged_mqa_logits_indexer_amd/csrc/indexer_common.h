// Shared device definitions of the paged MQA indexer (gfx950 / CDNA4).
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <climits>

#include "paged_mqa_indexer.h"

namespace pmqa {

constexpr int kHeads = IDX_NUM_HEADS;          // 32
constexpr int kDim = IDX_HEAD_DIM;             // 128
constexpr int kPage = IDX_PAGE_TOKENS;         // 64 tokens per page
constexpr int kPageBytes = kPage * kDim;       // 8 KiB of FP8 K per page
constexpr int kBins = IDX_NUM_BINS;            // 1024
constexpr int kCandCap = IDX_CANDIDATE_CAPACITY;  // 8192
constexpr int kWave = 64;

typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

// ---------------------------------------------------------------------------
// Score -> FP16 (round to nearest even).  v_cvt_f16_f32 rounds with the mode
// register's default (nearest even), keeps FP16 subnormals and turns
// magnitudes >= 65520 into infinity, as IEEE binary16 requires.
// ---------------------------------------------------------------------------
__device__ __forceinline__ uint32_t f16_bits_rn(float x) {
  _Float16 h = static_cast<_Float16>(x);
  return static_cast<uint32_t>(__builtin_bit_cast(uint16_t, h));
}

// Coarse histogram bin of an FP16 bit pattern (not NaN).  DeepGEMM PR #94,
// "What this adds": 1024 descending bins; below 16 the bin is the exponent and
// top 4 mantissa bits; from 16 to 223 unit-width bins (the magnitude's integer
// part, the same for both signs); 223 and above, infinity included, one
// saturating bin per end.  All three regimes are decided on the FP16 value.
__host__ __device__ __forceinline__ int coarse_bin_f16(uint32_t hb) {
  const uint32_t a = hb & 0x7FFFu;
  uint32_t m;
  if (a < 0x4C00u) {            // |h| < 16
    m = a >> 6;                  // 0 .. 303
  } else if (a < 0x5AF8u) {     // 16 <= |h| < 223 (0x5AF8 == 223.0)
    const uint32_t e = (a >> 10) - 15u;             // 4 .. 7
    const uint32_t sig = 0x400u | (a & 0x3FFu);     // 1.mantissa * 2^10
    m = 288u + (sig >> (10u - e));                  // 288 + floor(|h|)
  } else {
    m = 511u;                    // saturating, includes infinity
  }
  return (hb & 0x8000u) ? static_cast<int>(512u + m) : static_cast<int>(511u - m);
}

__host__ __device__ __forceinline__ bool f16_is_nan(uint32_t hb) { return (hb & 0x7FFFu) > 0x7C00u; }

// The same bin without branches (a NaN gets the saturating bin; callers
// exclude NaNs): the fine regime from the bits, the unit regime from the
// exact float value of |h| -- truncated, it is floor(|h|), and clamping it at
// 223 first folds the saturating bin (infinity included) into the formula.
// Checked against coarse_bin_f16 for every non-NaN encoding on the host.
__host__ __device__ __forceinline__ int coarse_bin_f16_flat(uint32_t hb) {
  const uint32_t a = hb & 0x7FFFu;
  const float mag = static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(a)));
  const uint32_t unit = 288u + static_cast<uint32_t>(fminf(mag, 223.0f));
  const uint32_t m = a < 0x4C00u ? (a >> 6) : unit;
  return (hb & 0x8000u) ? static_cast<int>(512u + m) : static_cast<int>(511u - m);
}

// Order-preserving unsigned keys: larger score <=> larger key, -0 just below +0.
__device__ __forceinline__ uint32_t key_f32(float x) {
  const uint32_t u = __float_as_uint(x);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__host__ __device__ __forceinline__ uint32_t key_f16(uint32_t hb) {
  return (hb & 0x8000u) ? (~hb & 0xFFFFu) : (hb | 0x8000u);
}

// Wave-level helpers.
__device__ __forceinline__ int lane_id() { return __lane_id(); }

// Wave-wide scans and reductions on DPP lane moves (gfx9 family): within
// each row of 16 lanes, shifts by 1, 2, 4 and 8; then row_bcast:15 adds the
// last lane of rows 0 and 2 into rows 1 and 3, and row_bcast:31 the last
// lane of row 1 into rows 2 and 3.  A lane whose source lies outside the
// row (or outside the masked rows) receives `identity`.  No LDS traffic,
// unlike __shfl_up / __shfl_xor, which go through ds_bpermute.
template <int CTRL, int ROW_MASK = 0xF>
__device__ __forceinline__ int dpp_move(int v, int identity) {
  return __builtin_amdgcn_update_dpp(identity, v, CTRL, ROW_MASK, 0xF, false);
}

template <typename Op>
__device__ __forceinline__ int wave_inclusive_scan_op(int v, int identity, Op op) {
  v = op(v, dpp_move<0x111>(v, identity));  // row_shr:1
  v = op(v, dpp_move<0x112>(v, identity));  // row_shr:2
  v = op(v, dpp_move<0x114>(v, identity));  // row_shr:4
  v = op(v, dpp_move<0x118>(v, identity));  // row_shr:8
  v = op(v, dpp_move<0x142, 0xA>(v, identity));  // row_bcast:15 into rows 1, 3
  v = op(v, dpp_move<0x143, 0xC>(v, identity));  // row_bcast:31 into rows 2, 3
  return v;
}

__device__ __forceinline__ int wave_inclusive_scan(int v) {
  return wave_inclusive_scan_op(v, 0, [](int a, int b) { return a + b; });
}

// Reductions: the inclusive result of lane 63, the same in every lane.
__device__ __forceinline__ int wave_sum(int v) {
  return __builtin_amdgcn_readlane(wave_inclusive_scan(v), kWave - 1);
}
__device__ __forceinline__ int wave_max(int v) {
  return __builtin_amdgcn_readlane(
      wave_inclusive_scan_op(v, INT_MIN, [](int a, int b) { return a > b ? a : b; }), kWave - 1);
}
__device__ __forceinline__ uint32_t wave_or(uint32_t v) {
  return static_cast<uint32_t>(__builtin_amdgcn_readlane(
      wave_inclusive_scan_op(static_cast<int>(v), 0, [](int a, int b) { return a | b; }), kWave - 1));
}
__device__ __forceinline__ uint32_t wave_and(uint32_t v) {
  return static_cast<uint32_t>(__builtin_amdgcn_readlane(
      wave_inclusive_scan_op(static_cast<int>(v), -1, [](int a, int b) { return a & b; }), kWave - 1));
}

// Workgroup barrier that orders LDS accesses only.  __syncthreads() also
// waits until every global load and store the wave has issued is complete
// (vmcnt(0)), which costs a memory round trip right after global stores.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// Lowest set lane of a ballot (lane 0 for an empty one).
__device__ __forceinline__ int first_lane(uint64_t mask) {
  return mask ? static_cast<int>(__builtin_ctzll(mask)) : 0;
}

// Number of set bits of `mask` below this lane.
__device__ __forceinline__ int lanes_below(uint64_t mask) {
  return __builtin_amdgcn_mbcnt_hi(static_cast<uint32_t>(mask >> 32),
                                   __builtin_amdgcn_mbcnt_lo(static_cast<uint32_t>(mask), 0));
}

}  // namespace pmqa

// Host-side launch helpers and the argument blocks the kernels take (the
// launch entry points themselves are declared in launches.h).
namespace pmqa {
// Optional events recorded by a call's own dispatches (measurement only):
// `start` when its first kernel begins, `stop` when its last kernel ends.
struct LaunchEvents {
  hipEvent_t start = nullptr;
  hipEvent_t stop = nullptr;
};

// One kernel launch; with events it goes through hipExtLaunchKernel, which
// records them at the dispatch's own begin and end.
template <typename... KArgs, typename... Args>
inline void launch_kernel(void (*kernel)(KArgs...), dim3 grid, dim3 block, hipStream_t stream,
                          hipEvent_t start, hipEvent_t stop, Args... args) {
  if (start || stop)
    hipExtLaunchKernelGGL(kernel, grid, block, 0, stream, start, stop, 0, static_cast<KArgs>(args)...);
  else
    hipLaunchKernelGGL(kernel, grid, block, 0, stream, static_cast<KArgs>(args)...);
}

struct LogitsArgs {
  const uint8_t* q;
  const uint8_t* kv_pages;  // FP8 codes [pages][64][128], or packed MXFP4 tokens [pages][64][68]
  const float* k_scales;    // FP8 only
  const float* weights;
  const int32_t* block_table;
  const int32_t* context_lens;
  void* logits;      // float32, or IEEE binary16 bits with logits_f16
  int32_t* hist;
  int64_t logits_stride;
  int32_t logits_f16;
  int32_t k_mxfp4;   // K pages are packed MXFP4 tokens (float32 logits only)
  int32_t B;
  int32_t next_n;
  int32_t num_pages;
  int32_t max_pages;
};

// Two-level candidate indexer.  Candidate blocks are 8 tokens; a row's bitmap
// of them is 16 KiB, so rows hold at most 2^17 blocks (2^20 keys).
constexpr int kMaxCandidateBlocks = 1 << 17;

struct SparseLogitsArgs {
  const uint8_t* q;          // E4M3 [rows][32][128]
  const uint8_t* kv_pages;   // E4M3 [num_pages][64][128], or packed MXFP4 tokens [num_pages][64][68]
  const float* k_scales;     // [num_pages][64] (FP8 only)
  const float* weights;      // [rows][32]
  const int32_t* table;      // [rows][kb] ascending block ids, INT32_MAX padded
  const int32_t* slots;      // [rows][kb] the same blocks as pool slot / 8
  const int32_t* context_lens;  // [rows]
  float* logits;             // [rows][logits_stride], column 8 i + t = key 8 table[i] + t
  int64_t logits_stride;
  int32_t rows;
  int32_t kb;
  int32_t num_pages;
  int32_t k_mxfp4;
};

// Ragged prefill (extend) logits: request r owns rows cu_q[r] .. cu_q[r+1]-1,
// row t scores keys [0, row_lens[t]) of its request.
struct PrefillArgs {
  const uint8_t* q;            // E4M3 [tokens][32][128]
  const uint8_t* kv_pages;     // E4M3 [num_pages][64][128], or packed MXFP4 tokens [num_pages][64][68]
  const float* k_scales;       // [num_pages][64] (FP8 only)
  const float* weights;        // [tokens][32]
  const int32_t* block_table;  // [requests][max_pages]
  const int32_t* cu_q;         // [requests + 1]
  const int32_t* row_lens;     // [tokens]
  float* logits;               // [tokens][logits_stride]
  int64_t logits_stride;
  int32_t requests;
  int32_t tokens;
  int32_t num_pages;
  int32_t max_pages;
  int32_t k_mxfp4;
};

}  // namespace pmqa
