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
//   * Work split: a 2-D grid of (request, chunk of P pages); the workgroup of
//     a chunk past its request's last page exits at once.  Every workgroup
//     requests the rows' lengths, its page ids, Q and the head weights
//     together on entry, so its first K load waits for a single round trip,
//     and the grid holds a full round of resident workgroups or more, so the
//     start-up of later workgroups overlaps the streaming of earlier ones.
//   * K is read straight into registers in the operand layout of
//     v_mfma_f32_16x16x128_f8f6f4: lane (n, g) = (lane % 16, lane / 16) takes
//     key n of a 16-key block, bytes [16g, 16g+16) and [64+16g, 64+16g+16).
//     One 16-byte load instruction then covers 16 keys x 64 contiguous bytes,
//     and the two instructions of a block cover its 2 KiB exactly.  Q uses the
//     same byte-to-k assignment, so the contraction over d is complete.
//   * Heads are the MFMA rows (two 16-head blocks), keys the columns; a lane
//     holds 8 heads of one key per row, so ReLU and the head weights are
//     applied in-lane, and two permlane swaps (register exchanges between
//     16-lane rows, no LDS) finish the head sum and leave lane l with the
//     logit of key l of the page (coalesced stores).
//   * The next page of every wave is in flight while the current one is
//     computed.  Workgroups of requests with several rows fetch Q and the
//     weights once and hand them to their waves through LDS; three or four
//     rows get 8-wave workgroups.
//   * Scores are staged in LDS and leave with 16-byte stores after the
//     workgroup's last K load, as float32 or as their FP16 rounding (vLLM
//     PR #52696, "Summary").
//   * The histogram slots of the workgroup's rows live in LDS and are added
//     to the global histogram (two bins per 64-bit atomic) when it finishes.
#include <type_traits>

#include "indexer_common.h"
#include "launches.h"

namespace pmqa {
namespace {

#ifndef PMQA_LOGITS_PREFETCH
#define PMQA_LOGITS_PREFETCH 1
#endif
#ifndef PMQA_LOGITS_PAGES_PER_WG
#define PMQA_LOGITS_PAGES_PER_WG 0  // 0: chosen from the grid shape
#endif
#ifndef PMQA_LOGITS_PERSIST
#define PMQA_LOGITS_PERSIST 1
#endif
#ifndef PMQA_LOGITS_PERSIST_PPW
#define PMQA_LOGITS_PERSIST_PPW 64  // <= PMQA_LOGITS_MAX_PPW
#endif
#ifndef PMQA_LOGITS_PERSIST_WGS_PER_CU
#define PMQA_LOGITS_PERSIST_WGS_PER_CU 0  // 0: one per CU when the K pages go through LDS, else two
#endif
#ifndef PMQA_LOGITS_WAVES_MANY_ROWS
#define PMQA_LOGITS_WAVES_MANY_ROWS 8
#endif
// Waves per workgroup: 4 for one or two rows per request; 8 for three or
// four, whose waves hold two to a SIMD (register budget) -- one workgroup of
// 8 per CU rather than two of 4, so that every wave's start-up loads are
// issued before any of them streams K (a second workgroup's loads would queue
// behind the first one's pages in the CU's memory pipeline).
#ifndef PMQA_LOGITS_WAVES_ONE_ROW
#define PMQA_LOGITS_WAVES_ONE_ROW 4
#endif
template <int NN>
constexpr int kWavesOf = NN >= 3 ? PMQA_LOGITS_WAVES_MANY_ROWS : (NN == 1 ? PMQA_LOGITS_WAVES_ONE_ROW : 4);
constexpr int kPrefetch = PMQA_LOGITS_PREFETCH;  // pages in flight per wave
// MXFP4 pages are half the bytes: with one row per request a wave keeps two
// of them in flight (measured 18.6 -> 16.8 us at long decode; with more rows
// the larger Q operands leave no registers for it).
template <int NN, int KF>
constexpr int kPrefetchOf = (KF == 1 && NN == 1) ? 2 : kPrefetch;
#ifndef PMQA_LOGITS_MAX_PPW
#define PMQA_LOGITS_MAX_PPW 64
#endif
// Pages per share at most: 256 with one row per request, 64 with several
// (their staging is NN times larger).  With one row, longer shares mean
// fewer workgroups per long row: each bin receives fewer flush atomics
// (128 pages against 64: very_long 104.1 -> 103.3 us, histogram extra 2.1 ->
// 0.3 us), and at 256 a 4 x 1M-key call fits in one round of workgroups, one
// per CU, instead of two (very_long 96.0 -> 91.0 us).
constexpr int kMaxPagesPerWg = PMQA_LOGITS_MAX_PPW;
constexpr int kMaxPagesPerWgOneRow = 4 * kMaxPagesPerWg;
static_assert(kMaxPagesPerWgOneRow <= 4 * kWave, "page ids of a share must fit one fetch");
// LDS staging of a share's scores: next_n * pages_per_wg * 64 floats
// (64 KiB for one row, 16 KiB per row with several).
template <int NN>
constexpr int kStageFloats = NN * (NN == 1 ? kMaxPagesPerWgOneRow : kMaxPagesPerWg) * kPage;
// Staged score type: float32 logits, or the bits of their FP16 rounding.
template <bool F16>
using StageT = typename std::conditional<F16, uint16_t, float>::type;
template <int NN>
constexpr int kThreadsOf = kWavesOf<NN> * kWave;

// K page formats: FP8 E4M3 codes with a per-token fp32 scale (two arrays),
// or MXFP4 tokens -- 64 bytes of E2M1 codes (dimension 2i in the low nibble
// of byte i) and four E8M0 scale bytes, one per 32 dimensions, packed into 68
// bytes (SGLang PR #38944, block-scaled E2M1 index-K; vLLM PR #52696, the
// packed 68-byte cache layout).
constexpr int kKFp8 = 0;
constexpr int kKMxfp4 = 1;
constexpr int kMxTokenBytes = 68;
constexpr int kBlk8 = 8;                              // tokens per candidate block
constexpr int kBlocksPerChunk = kPage / kBlk8;        // 8 blocks = 64 sparse columns
constexpr int kMxPageBytes = kPage * kMxTokenBytes;  // 4352

template <int KF>
struct PageRegs;
template <>
struct PageRegs<kKFp8> {
  i32x4 v[8];   // [key block kb][half]: K bytes in MFMA operand layout
  float scale;  // k_scales of key `lane` of the page
};
template <>
struct PageRegs<kKMxfp4> {
  i32x4 v[4];   // [key block kb]: 32 E2M1 codes of key n, dimensions 32g .. 32g+31
  int sc[4];    // [key block kb]: the key's four E8M0 scale bytes
};

// ReLU as one integer max on the bit pattern: a set sign bit makes the int32
// negative, so negatives and -0 become +0 and everything else passes.
__device__ __forceinline__ float relu(float x) {
  return __int_as_float(max(__float_as_int(x), 0));
}

// The score exactly as it is stored.  Without the empty asm the compiler may
// fold "float32 multiply, then round to FP16" into one mixed-precision FMA
// that rounds the exact product straight to FP16, and the bin would then not
// always be the bin of the float32 value written to memory.
__device__ __forceinline__ float as_stored(float x) {
  __asm__ volatile("" : "+v"(x));
  return x;
}

__device__ __forceinline__ i32x8 cat8(i32x4 a, i32x4 b) {
  return i32x8{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
}

// Buffer resource of one contiguous range (gfx9-family descriptor word 3).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t range_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, static_cast<int>(bytes),
                                           0x00020000);
}

// FP8 pages of one-row requests go HBM -> LDS with buffer loads that write
// LDS directly (no VGPRs), each instruction a contiguous kilobyte -- 8 whole
// keys, full 128-byte lines -- with the 16-byte pieces permuted inside it, so
// that ds_read_b128 then fetches the MFMA operand layout (16 keys x 16 bytes
// per lane group) without LDS bank conflicts.  Read straight into registers
// in operand layout, every load instruction touches 16 half lines instead
// (measured on a paged-gather probe over the long-decode pool: 1.2-1.3 us
// slower at 138 MB).  Each wave keeps a ring of kRing page slots.
#ifndef PMQA_LOGITS_DMA
#define PMQA_LOGITS_DMA 1
#endif
#ifndef PMQA_LOGITS_DMA_RING
#define PMQA_LOGITS_DMA_RING 2
#endif
// One row per request, either K format (MXFP4: 16.3 -> 15.7 us at long
// decode against the register path, with an evicting cache sweep).
template <int NN, int KF>
constexpr bool kDmaOf = PMQA_LOGITS_DMA && NN == 1;
constexpr int kRing = PMQA_LOGITS_DMA_RING;
static_assert(kRing >= 2 && kRing <= 3, "ring depth: the waits below cover 2 or 3 slots");
// With the page ring, each wave stores its page's scores as soon as they are
// computed (the waits on the page loads count loads only, so stores in
// between cost them nothing) instead of staging the share's scores in LDS
// for stores after its last page.
#ifndef PMQA_LOGITS_DIRECT_STORE
#define PMQA_LOGITS_DIRECT_STORE 0
#endif
#ifndef PMQA_LOGITS_NT_STORE
#define PMQA_LOGITS_NT_STORE 0
#endif
template <int NN, int KF>
constexpr bool kDirectOf = kDmaOf<NN, KF> && PMQA_LOGITS_DIRECT_STORE;
// Page slot: FP8 codes then the 64 scales; or the MXFP4 page verbatim.
template <int KF>
constexpr int kSlotBytesOf = KF == kKFp8 ? kPageBytes + kPage * 4 : kMxPageBytes;
// Loads per page: 8 FP8 kilobytes + the scales; 4 MXFP4 kilobytes + 256 bytes.
template <int KF>
constexpr int kDmaInstrsOf = KF == kKFp8 ? kPageBytes / 1024 + 1 : kMxPageBytes / 1024 + 1;
static_assert(kMxPageBytes == 4 * 1024 + kPage * 4, "an MXFP4 page is four kilobytes and 64 words");
typedef __attribute__((address_space(3))) char lds_char;
typedef __attribute__((address_space(3))) void lds_void;

// LDS offset, inside a page slot, of 16-byte piece j (0..7) of key 8 i + kk:
// pieces of a key stay in its 128 bytes, exchanged by an XOR that differs
// between even and odd kilobytes, so the 16 keys an operand read touches
// (8 of an even and 8 of an odd kilobyte, one piece each) fall on 16
// different 16-byte bank groups.
__device__ __forceinline__ int dma_piece(int i, int kk, int j) {
  return i * 1024 + kk * 128 + ((j ^ ((kk >> 1) | ((i & 1) << 2))) * 16);
}

// Per-lane source offsets of the page loads: instruction i, lane l takes
// piece (l & 7) ^ f of key 8 i + (l >> 3), the piece dma_piece() puts in LDS
// slot l of kilobyte i.
struct DmaOffsets {
  uint32_t k[kPageBytes / 1024];
  uint32_t scale;
  __device__ explicit DmaOffsets(int lane) {
    const int kk = lane >> 3;
#pragma unroll
    for (int i = 0; i < kPageBytes / 1024; ++i)
      k[i] = static_cast<uint32_t>(i * 1024 + kk * 128 + (((lane & 7) ^ ((kk >> 1) | ((i & 1) << 2))) * 16));
    scale = static_cast<uint32_t>(lane * 4);
  }
};

// Issue one page into an LDS slot: eight kilobyte loads (keys 8i..8i+7, whole
// lines) and the 64 scales, each writing LDS at m0 + 16 (or 4) x lane.
// Written out in assembly so that the compiler, which cannot tell the ring's
// slots apart, does not drain every load in flight before each LDS access of
// the page loop; the caller waits for them itself (vmcnt, in issue order).
// A load that writes LDS must not directly follow the write of m0 that
// addresses it (one wait state on this GPU family): hence the s_nop after each.
// The loads carry the non-temporal cache policy (`nt`): every line of the K
// stream is read once, by one instruction, and streaming it through the
// caches as such measured faster (long decode 27.4 -> 25.6 us, very long
// 102.2 -> 97.1 us, varlen 129.8 -> 125.4 us; the sc0/sc1 bits add nothing).
// The operand-layout register loads of the other launches touch each line
// with two instructions, and there `nt` measured slower (spec verify 19.1 ->
// 21.4 us, also when only the line's second access carries it).
__device__ __forceinline__ void dma_page(const uint8_t* __restrict__ kv_pages, const float* __restrict__ k_scales,
                                         int page, const DmaOffsets& off, uint32_t slot) {
  const uint8_t* kp = kv_pages + static_cast<int64_t>(page) * kPageBytes;
  const float* sp = k_scales + static_cast<int64_t>(page) * kPage;
  __asm__ volatile(
      "s_mov_b32 m0, %[l0]\n"
      "s_nop 0\n"
      "global_load_lds_dwordx4 %[v0], %[kb] nt\n"
      "s_mov_b32 m0, %[l1]\n"
      "s_nop 0\n"
      "global_load_lds_dwordx4 %[v1], %[kb] nt\n"
      "s_mov_b32 m0, %[l2]\n"
      "s_nop 0\n"
      "global_load_lds_dwordx4 %[v2], %[kb] nt\n"
      "s_mov_b32 m0, %[l3]\n"
      "s_nop 0\n"
      "global_load_lds_dwordx4 %[v3], %[kb] nt\n"
      "s_mov_b32 m0, %[l4]\n"
      "s_nop 0\n"
      "global_load_lds_dwordx4 %[v4], %[kb] nt\n"
      "s_mov_b32 m0, %[l5]\n"
      "s_nop 0\n"
      "global_load_lds_dwordx4 %[v5], %[kb] nt\n"
      "s_mov_b32 m0, %[l6]\n"
      "s_nop 0\n"
      "global_load_lds_dwordx4 %[v6], %[kb] nt\n"
      "s_mov_b32 m0, %[l7]\n"
      "s_nop 0\n"
      "global_load_lds_dwordx4 %[v7], %[kb] nt\n"
      "s_mov_b32 m0, %[l8]\n"
      "s_nop 0\n"
      "global_load_lds_dword %[vs], %[sb] nt\n"
      :
      : [kb] "s"(kp), [sb] "s"(sp), [l0] "s"(slot), [l1] "s"(slot + 1024), [l2] "s"(slot + 2048),
        [l3] "s"(slot + 3072), [l4] "s"(slot + 4096), [l5] "s"(slot + 5120), [l6] "s"(slot + 6144),
        [l7] "s"(slot + 7168), [l8] "s"(slot + kPageBytes), [v0] "v"(off.k[0]), [v1] "v"(off.k[1]),
        [v2] "v"(off.k[2]), [v3] "v"(off.k[3]), [v4] "v"(off.k[4]), [v5] "v"(off.k[5]), [v6] "v"(off.k[6]),
        [v7] "v"(off.k[7]), [vs] "v"(off.scale)
      : "memory", "m0");
}

// The MFMA operands of a page slot: lane (n, g) reads pieces g and 4 + g of
// key 16 kb + n, and the scale of key `lane`.  The reads are written out with
// their own wait: the compiler would otherwise drain every page in flight
// before them (it cannot tell the ring's slots apart), and a load written in
// assembly must complete inside its own statement.
__device__ __forceinline__ void read_page(uint32_t base, int lane, PageRegs<kKFp8>& r) {
  const int n = lane & 15, g = lane >> 4;
  const uint32_t a0 = base + dma_piece(n >> 3, n & 7, g);      // half 0, key block 0
  const uint32_t a1 = base + dma_piece(n >> 3, n & 7, g + 4);  // half 1, key block 0
  const uint32_t as = base + kPageBytes + lane * 4;
  float sc;
  __asm__ volatile(
      "ds_read_b128 %0, %9\n"
      "ds_read_b128 %1, %10\n"
      "ds_read_b128 %2, %9 offset:2048\n"
      "ds_read_b128 %3, %10 offset:2048\n"
      "ds_read_b128 %4, %9 offset:4096\n"
      "ds_read_b128 %5, %10 offset:4096\n"
      "ds_read_b128 %6, %9 offset:6144\n"
      "ds_read_b128 %7, %10 offset:6144\n"
      "ds_read_b32 %8, %11\n"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(r.v[0]), "=&v"(r.v[1]), "=&v"(r.v[2]), "=&v"(r.v[3]), "=&v"(r.v[4]), "=&v"(r.v[5]),
        "=&v"(r.v[6]), "=&v"(r.v[7]), "=&v"(sc)
      : "v"(a0), "v"(a1), "v"(as)
      : "memory");
  r.scale = sc;
}

// MXFP4 pages go to LDS verbatim, in whole lines: instruction i (0..3) copies
// kilobyte i of the page (lane l: bytes 16 l .. 16 l + 15) and the fifth its
// last 256 bytes (lane l: one word), all non-temporal like the FP8 pages.
// Tokens are 68 bytes, so an operand piece -- bytes [16 g, 16 g + 16) of
// token 16 kb + n -- is only 4-byte aligned in LDS and is read as four words;
// consecutive tokens lie 17 words apart (17 is odd), so the 64 lanes of a
// read hit every bank twice, without conflicts.
struct DmaOffsetsMx {
  uint32_t k[4];
  uint32_t tail;
  __device__ explicit DmaOffsetsMx(int lane) {
#pragma unroll
    for (int i = 0; i < 4; ++i) k[i] = static_cast<uint32_t>(i * 1024 + lane * 16);
    tail = static_cast<uint32_t>(4 * 1024 + lane * 4);
  }
};

__device__ __forceinline__ void dma_page(const uint8_t* __restrict__ kv_pages, const float* __restrict__ /*k_scales*/,
                                         int page, const DmaOffsetsMx& off, uint32_t slot) {
  const uint8_t* kp = kv_pages + static_cast<int64_t>(page) * kMxPageBytes;
  __asm__ volatile(
      "s_mov_b32 m0, %[l0]\n"
      "s_nop 0\n"
      "global_load_lds_dwordx4 %[v0], %[kb] nt\n"
      "s_mov_b32 m0, %[l1]\n"
      "s_nop 0\n"
      "global_load_lds_dwordx4 %[v1], %[kb] nt\n"
      "s_mov_b32 m0, %[l2]\n"
      "s_nop 0\n"
      "global_load_lds_dwordx4 %[v2], %[kb] nt\n"
      "s_mov_b32 m0, %[l3]\n"
      "s_nop 0\n"
      "global_load_lds_dwordx4 %[v3], %[kb] nt\n"
      "s_mov_b32 m0, %[l4]\n"
      "s_nop 0\n"
      "global_load_lds_dword %[vt], %[kb] nt\n"
      :
      : [kb] "s"(kp), [l0] "s"(slot), [l1] "s"(slot + 1024), [l2] "s"(slot + 2048), [l3] "s"(slot + 3072),
        [l4] "s"(slot + 4096), [v0] "v"(off.k[0]), [v1] "v"(off.k[1]), [v2] "v"(off.k[2]), [v3] "v"(off.k[3]),
        [vt] "v"(off.tail)
      : "memory", "m0");
}

// The MFMA operands of an MXFP4 page slot: lane (n, g) reads bytes
// [16 g, 16 g + 16) of token 16 kb + n and the token's scale word, per key
// block kb; written out with its own wait, as read_page for FP8 pages.
__device__ __forceinline__ void read_page(uint32_t base, int lane, PageRegs<kKMxfp4>& r) {
  const int n = lane & 15, g = lane >> 4;
  const uint32_t a = base + static_cast<uint32_t>(n * kMxTokenBytes + g * 16);
  const uint32_t as = base + static_cast<uint32_t>(n * kMxTokenBytes + 64);
  static_assert(16 * kMxTokenBytes == 1088, "key blocks 1088 bytes apart (offsets below)");
  int w[16], sc[4];
  __asm__ volatile(
      "ds_read_b32 %0, %20\n"
      "ds_read_b32 %1, %20 offset:4\n"
      "ds_read_b32 %2, %20 offset:8\n"
      "ds_read_b32 %3, %20 offset:12\n"
      "ds_read_b32 %4, %20 offset:1088\n"
      "ds_read_b32 %5, %20 offset:1092\n"
      "ds_read_b32 %6, %20 offset:1096\n"
      "ds_read_b32 %7, %20 offset:1100\n"
      "ds_read_b32 %8, %20 offset:2176\n"
      "ds_read_b32 %9, %20 offset:2180\n"
      "ds_read_b32 %10, %20 offset:2184\n"
      "ds_read_b32 %11, %20 offset:2188\n"
      "ds_read_b32 %12, %20 offset:3264\n"
      "ds_read_b32 %13, %20 offset:3268\n"
      "ds_read_b32 %14, %20 offset:3272\n"
      "ds_read_b32 %15, %20 offset:3276\n"
      "ds_read_b32 %16, %21\n"
      "ds_read_b32 %17, %21 offset:1088\n"
      "ds_read_b32 %18, %21 offset:2176\n"
      "ds_read_b32 %19, %21 offset:3264\n"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(w[0]), "=&v"(w[1]), "=&v"(w[2]), "=&v"(w[3]), "=&v"(w[4]), "=&v"(w[5]), "=&v"(w[6]), "=&v"(w[7]),
        "=&v"(w[8]), "=&v"(w[9]), "=&v"(w[10]), "=&v"(w[11]), "=&v"(w[12]), "=&v"(w[13]), "=&v"(w[14]),
        "=&v"(w[15]), "=&v"(sc[0]), "=&v"(sc[1]), "=&v"(sc[2]), "=&v"(sc[3])
      : "v"(a), "v"(as)
      : "memory");
#pragma unroll
  for (int kb = 0; kb < 4; ++kb) {
    r.v[kb] = i32x4{w[4 * kb], w[4 * kb + 1], w[4 * kb + 2], w[4 * kb + 3]};
    r.sc[kb] = sc[kb];
  }
}

// One page of K in MFMA operand layout plus the scale of key `lane`.  Buffer
// loads take the page's base from scalar registers and a loop-invariant
// per-lane offset, so no address register is rewritten from one page to the
// next (a rewritten address register whose previous value feeds an
// outstanding load's destination would force a wait for all loads).
__device__ __forceinline__ void load_page(const uint8_t* __restrict__ kv_pages,
                                          const float* __restrict__ k_scales,
                                          int page, int lane_off, int lane, PageRegs<kKFp8>& r) {
  const __amdgpu_buffer_rsrc_t kr = range_rsrc(kv_pages + static_cast<int64_t>(page) * kPageBytes, kPageBytes);
#pragma unroll
  for (int kb = 0; kb < 4; ++kb) {
    r.v[2 * kb + 0] = __builtin_bit_cast(i32x4, __builtin_amdgcn_raw_buffer_load_b128(kr, lane_off + kb * 16 * kDim, 0, 0));
    r.v[2 * kb + 1] = __builtin_bit_cast(i32x4, __builtin_amdgcn_raw_buffer_load_b128(kr, lane_off + kb * 16 * kDim + 64, 0, 0));
  }
  const __amdgpu_buffer_rsrc_t sr = range_rsrc(k_scales + static_cast<int64_t>(page) * kPage, kPage * 4);
  r.scale = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(sr, lane * 4, 0, 0));
}

// One page of MXFP4 K.  For the fp8 x fp4 MFMA (16x16x128) lane (n, g) of
// the fp4 operand holds dimensions 32g .. 32g+31 of key n, element i in
// nibble i, and the E8M0 scale that lane passes covers those 32 dimensions
// (checked on the device with single-element operands); the fp8 Q operand
// keeps its layout.  So lane (n, g) reads bytes [16g, 16g+16) of token
// 16 kb + n -- one 16-byte load at a 4-byte-aligned offset -- and the token's
// scale word.  lane_off = 68 n + 16 g.
__device__ __forceinline__ void load_page(const uint8_t* __restrict__ kv_pages,
                                          const float* __restrict__ /*k_scales*/,
                                          int page, int lane_off, int lane, PageRegs<kKMxfp4>& r) {
  const __amdgpu_buffer_rsrc_t kr = range_rsrc(kv_pages + static_cast<int64_t>(page) * kMxPageBytes, kMxPageBytes);
  const int scale_off = (lane & 15) * kMxTokenBytes + 64;
#pragma unroll
  for (int kb = 0; kb < 4; ++kb) {
    r.v[kb] = __builtin_bit_cast(i32x4, __builtin_amdgcn_raw_buffer_load_b128(kr, lane_off + kb * 16 * kMxTokenBytes, 0, 0));
    r.sc[kb] = __builtin_amdgcn_raw_buffer_load_b32(kr, scale_off + kb * 16 * kMxTokenBytes, 0, 0);
  }
}

// Sum over the four lane groups g of part[kb], leaving lane (n, g) with the
// total of key block g.  Lane groups are rows of 16 lanes; gfx950's permlane
// swaps exchange registers between rows in the VALU (no LDS round trip):
// permlane32_swap(x, y) trades x of rows 2-3 for y of rows 0-1, so x + y is,
// in rows 0-1, the pair sum (row r, row r+2) of part[kb] and, in rows 2-3,
// that of part[kb+2]; permlane16_swap then trades the odd rows of k0 for the
// even rows of k1, and the same add finishes the four-row sum.
__device__ __forceinline__ float reduce_scatter4(const float (&part)[4]) {
  const auto x = __builtin_amdgcn_permlane32_swap(__float_as_uint(part[0]), __float_as_uint(part[2]), false, false);
  const auto y = __builtin_amdgcn_permlane32_swap(__float_as_uint(part[1]), __float_as_uint(part[3]), false, false);
  const float k0 = __uint_as_float(x[0]) + __uint_as_float(x[1]);  // block 0 (rows 0-1) / 2 (rows 2-3)
  const float k1 = __uint_as_float(y[0]) + __uint_as_float(y[1]);  // block 1 / 3
  const auto z = __builtin_amdgcn_permlane16_swap(__float_as_uint(k0), __float_as_uint(k1), false, false);
  return __uint_as_float(z[0]) + __uint_as_float(z[1]);
}

template <int NN>
struct RequestRegs {
  i32x4 q[NN][2][2];  // [token][head block][half], operand layout
  f32x4 w[NN][2];     // weights of heads 16*mb + 4g + i
  int len[NN];
};

// Scores of page `lp` (the `lpi`-th page of the workgroup's share) for the
// NN rows of the request.  Scores go to the workgroup's LDS staging area
// s_out[j][lpi][lane] -- float32, or with F16 the IEEE half the score rounds
// to (round to nearest even), the same half the histogram bins; they reach
// global memory after the share's last load (see the kernel), because a
// global store issued between this page and the next one's prefetch would
// have to complete before that page counts as arrived: the vector-memory
// counter covers loads and stores in issue order.
template <int NN, bool HIST, bool F16, int KF, bool DIRECT = false>
__device__ __forceinline__ void compute_page(const PageRegs<KF>& pr, int lp, int lpi, int ppw,
                                             int lane, const RequestRegs<NN>& rq,
                                             StageT<F16>* s_out, int* s_hist,
                                             StageT<F16>* __restrict__ out_row = nullptr) {
  const int key = lp * kPage + lane;
#pragma unroll
  for (int j = 0; j < NN; ++j) {
    f32x4 acc[4][2];
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
#pragma unroll
      for (int mb = 0; mb < 2; ++mb) {
        const i32x8 a = cat8(rq.q[j][mb][0], rq.q[j][mb][1]);
        if constexpr (KF == kKFp8) {
          const i32x8 b = cat8(pr.v[2 * kb], pr.v[2 * kb + 1]);
          acc[kb][mb] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
              a, b, f32x4{0.f, 0.f, 0.f, 0.f}, 0, 0, 0, 127, 0, 127);
        } else {
          // B in E2M1 (format 4): only its first four registers are read.
          const i32x8 b = cat8(pr.v[kb], i32x4{0, 0, 0, 0});
          const int scale = (pr.sc[kb] >> (8 * (lane >> 4))) & 0xFF;
          acc[kb][mb] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
              a, b, f32x4{0.f, 0.f, 0.f, 0.f}, 0, 4, 0, 127, 0, scale);
        }
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
    float head_sum = reduce_scatter4(part);
    if constexpr (KF == kKFp8) head_sum *= pr.scale;  // MXFP4 scales are in the products
    const float logit = as_stored(head_sum);
    uint32_t hb = 0u;
    if constexpr (HIST || F16) hb = f16_bits_rn(logit);
    if constexpr (DIRECT) {
      // one row (DIRECT is the one-row path): store the live score right away
      StageT<F16> v;
      if constexpr (F16) v = static_cast<uint16_t>(hb);
      else v = logit;
      if (key < rq.len[0]) {
        if constexpr (PMQA_LOGITS_NT_STORE) __builtin_nontemporal_store(v, out_row + key);
        else out_row[key] = v;
      }
    } else if constexpr (F16) {
      s_out[(j * ppw + lpi) * kPage + lane] = static_cast<uint16_t>(hb);
    } else {
      s_out[(j * ppw + lpi) * kPage + lane] = logit;
    }
    if constexpr (HIST && NN >= 2) {
      // Several rows: every lane adds, without a branch, so the binning
      // interleaves with the next row's MFMAs (spec verify 20.8 -> 19.1 us);
      // scores past the row's length and NaNs go to a spare slot after the
      // rows' bins, which is never read.
      const int bin = coarse_bin_f16_flat(hb);
      const bool counted = (key < rq.len[j]) & !f16_is_nan(hb);
      atomicAdd(&s_hist[counted ? j * kBins + bin : NN * kBins], 1);
    } else if constexpr (HIST) {
      // One row: the branch costs less than binning the few dead lanes
      // (long decode 27.9 vs 28.3 us branch-free).
      if (key < rq.len[j] && !f16_is_nan(hb)) atomicAdd(&s_hist[j * kBins + coarse_bin_f16(hb)], 1);
    }
  }
}

// Resident waves per SIMD the register budget is held to: 4 for one row per
// request (128 VGPRs), 3 for two rows, 2 for three or four.
// (One row with the LDS page ring: its LDS holds one workgroup per CU.)
template <int NN>
constexpr int kWavesPerSimd = NN == 1 ? (PMQA_LOGITS_DMA ? 1 : (kPrefetch == 1 ? 4 : (kPrefetch == 2 ? 3 : 2)))
                                      : (NN == 2 && kPrefetch == 1 ? 3 : 2);

// One share of the grid: pages [p0_64, p0_64 + pages_per_wg) of request b
// (the workgroup returns at once if that is past the request's last page).
template <int NN, bool HIST, bool F16, int KF>
__device__ __forceinline__ void logits_share(const LogitsArgs& a, int pages_per_wg, int b, int64_t p0_64,
                                             int* s_hist, StageT<F16>* s_out, i32x4* s_q, float* s_w,
                                             char* s_ring) {
  constexpr int kWaves = kWavesOf<NN>;
  constexpr int kThreads = kThreadsOf<NN>;
  const int tid = threadIdx.x;
  const int lane = __lane_id();
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int row0 = b * NN;
  // No row reads past its block-table row or writes past its logits row.
  const int64_t mk = min(static_cast<int64_t>(a.max_pages) * kPage, a.logits_stride);
  const int max_keys = static_cast<int>(min(mk, static_cast<int64_t>(INT32_MAX)));


  // Start-up loads: this wave's page ids (clamped into the block-table row,
  // so the read is in bounds even past the request's last page) and the
  // rows' lengths, which the first K loads depend on; then Q and the
  // weights.  With one row a wave loads its own Q operands (4 KiB, 3 % of
  // its share's K).  With several rows Q is read from global memory once per
  // workgroup, each wave fetching a slice into LDS: with four rows a wave's
  // operands are 16 KiB, as much as two K pages, and eight waves fetching
  // them each would hold up the CU's first K pages.
  const int32_t* bt = a.block_table + static_cast<int64_t>(b) * a.max_pages;
  const int64_t last_id = a.max_pages - 1;
  int ids = bt[min(p0_64 + wave + lane * kWaves, last_id)];
  RequestRegs<NN> rq;
  if constexpr (NN == 1) rq.len[0] = min(max(a.context_lens[row0], 0), max_keys);
  // Slice s = (row j, head block mb, half h) of Q: 64 lanes x 16 bytes.
  constexpr bool kQViaLds = NN >= 2;
  constexpr int kSlices = NN * 4;
  constexpr int kSlicesPerWave = kQViaLds ? (kSlices + kWaves - 1) / kWaves : kSlices;
  const int m = lane & 15, g = lane >> 4;
  i32x4 q_slice[kSlicesPerWave];
#pragma unroll
  for (int t = 0; t < kSlicesPerWave; ++t) {
    if constexpr (!kQViaLds) {
      const int j = t >> 2, mb = (t >> 1) & 1, h = t & 1;
      q_slice[t] = *reinterpret_cast<const i32x4*>(
          a.q + (static_cast<int64_t>(row0 + j) * kHeads + mb * 16 + m) * kDim + g * 16 + h * 64);
      continue;
    }
    const int sl = min(wave + t * kWaves, kSlices - 1);  // clamped: loads stay unconditional
    const int j = sl >> 2, mb = (sl >> 1) & 1, h = sl & 1;
    q_slice[t] = *reinterpret_cast<const i32x4*>(
        a.q + (static_cast<int64_t>(row0 + j) * kHeads + mb * 16 + m) * kDim + g * 16 + h * 64);
  }
  f32x4 w_direct[kQViaLds ? 1 : 2];
  float w_val = 0.f;
  if constexpr (kQViaLds) {
    w_val = a.weights[static_cast<int64_t>(row0) * kHeads + min(tid, NN * kHeads - 1)];
  } else {
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
      w_direct[mb] = *reinterpret_cast<const f32x4*>(a.weights + static_cast<int64_t>(row0) * kHeads + mb * 16 + 4 * g);
  }
  if constexpr (NN >= 2) {
    // Several rows: the page ids, Q and the weights are requested before the
    // rows' lengths and the exit test that needs them.  Without this compiler
    // barrier the loads are sunk past the branch, and a workgroup waits for
    // the lengths, then for its page ids and Q, then for K -- three round
    // trips before the first page instead of two (spec verify 21.7 ->
    // 20.9 us; with one row the order makes no measurable difference).
    __asm__ volatile("" ::: "memory");
#pragma unroll
    for (int j = 0; j < NN; ++j) rq.len[j] = min(max(a.context_lens[row0 + j], 0), max_keys);
  }
  int keys_b = 0;
#pragma unroll
  for (int j = 0; j < NN; ++j) keys_b = max(keys_b, rq.len[j]);
  const int pages_b = (keys_b >> 6) + ((keys_b & (kPage - 1)) != 0);
  // With many requests of varied length most workgroups of the grid lie past
  // their request's last page; they leave here, before any K is requested.
  if (p0_64 >= pages_b) return;  // uniform
  const int p0 = static_cast<int>(p0_64);
  const int p1 = static_cast<int>(min(p0_64 + pages_per_wg, static_cast<int64_t>(pages_b)));

  const int lpi0 = wave;  // share-local index of the wave's first page

  // Pages p0 + wave, + kWaves, ... < p1; lane i of `ids` holds the wave's
  // i-th page id.  A share has at most 4 * 64 pages, so one fetch
  // covers it, and the loop below has no conditional load: a load inside a
  // branch would make the compiler wait for every outstanding load (and, on
  // this architecture, store) before the next page could be issued.
  const int n_mine = p1 - p0 > wave ? (p1 - p0 - wave + kWaves - 1) / kWaves : 0;
  auto page_id = [&](int it) {
    const int id = __builtin_amdgcn_readlane(ids, it);
    return min(max(id, 0), a.num_pages - 1);
  };

  // Ring of kRg page buffers: while page `it` is computed, pages
  // it+1 .. it+kPf are in flight.  Past the last page the last one is
  // issued again (it is cached), which keeps every load unconditional; a wave
  // without pages issues its first prefetch all the same.
  const int lane_off = (lane & 15) * (KF == kKFp8 ? kDim : kMxTokenBytes) + (lane >> 4) * 16;  // key n, group g
  constexpr int kPf = kPrefetchOf<NN, KF>;
  constexpr int kRg = kPf + 1;
  PageRegs<KF> buf[kRg];
  const int n_last = max(n_mine, 1) - 1;
  auto prefetch = [&]() {
#pragma unroll
    for (int s = 0; s < kPf; ++s) {
      load_page(a.kv_pages, a.k_scales, page_id(s < n_last ? s : n_last), lane_off, lane, buf[s]);
    }
  };

  if constexpr (kQViaLds) {
    // Several rows: the first K pages are requested before Q is staged, so
    // they stream while Q arrives and goes through LDS.
    prefetch();
#pragma unroll
    for (int t = 0; t < kSlicesPerWave; ++t) {
      const int sl = wave + t * kWaves;
      if (sl < kSlices) s_q[sl * kWave + lane] = q_slice[t];
    }
    if (tid < NN * kHeads) s_w[tid] = w_val;
    if constexpr (HIST) {
      for (int i = tid; i < NN * kBins; i += kThreads) s_hist[i] = 0;
    }
    lds_barrier();  // LDS only: the prefetched K pages stay in flight
#pragma unroll
    for (int j = 0; j < NN; ++j) {
#pragma unroll
      for (int mb = 0; mb < 2; ++mb) {
        rq.q[j][mb][0] = s_q[((j * 2 + mb) * 2 + 0) * kWave + lane];
        rq.q[j][mb][1] = s_q[((j * 2 + mb) * 2 + 1) * kWave + lane];
        rq.w[j][mb] = *reinterpret_cast<const f32x4*>(&s_w[j * kHeads + mb * 16 + 4 * g]);
      }
    }
  } else {
    // One row: the workgroup waits for its start-up loads (Q included), then
    // all of its waves request K together; measured faster at this shape
    // than streaming K behind each wave's own Q loads.
    if constexpr (HIST) {
      for (int i = tid; i < NN * kBins; i += kThreads) s_hist[i] = 0;
      __syncthreads();
    }
#pragma unroll
    for (int mb = 0; mb < 2; ++mb) {
      rq.q[0][mb][0] = q_slice[mb * 2 + 0];
      rq.q[0][mb][1] = q_slice[mb * 2 + 1];
      rq.w[0][mb] = w_direct[mb];
    }
    if constexpr (!kDmaOf<NN, KF>) prefetch();
  }

  if constexpr (kDmaOf<NN, KF>) {
    // Ring of kRing LDS slots per wave: while page `it` is read and computed,
    // pages it+1 .. it+kRing-1 are in flight (those that exist: the last
    // pages are not issued again, which with non-temporal loads would read
    // them from HBM a second time).  The compiler does not order LDS reads
    // after these loads, so the waits are explicit: before a slot is
    // refilled, every LDS access issued so far has completed (its last reads
    // are a page old); before a page is read, at most the kDmaInstrsOf loads of
    // each page issued after it are outstanding -- the loop issues no other
    // vector memory operation, and loads complete in issue order.
    // The compiler does not see the page loads (assembly), so it would place
    // its waits for Q and the weights at their first use inside the loop,
    // where they would drain the loads in flight on every page; consuming
    // them here makes it wait once, before the first page is issued.
    __asm__ volatile("" ::"v"(rq.q[0][0][0]), "v"(rq.q[0][0][1]), "v"(rq.q[0][1][0]), "v"(rq.q[0][1][1]),
                     "v"(rq.w[0][0]), "v"(rq.w[0][1]));
    if (n_mine > 0) {
      const uint32_t ring = static_cast<uint32_t>(reinterpret_cast<uintptr_t>((lds_char*)(s_ring))) +
                            static_cast<uint32_t>(wave * (kRing * kSlotBytesOf<KF>));
      constexpr int kSlotBytes = kSlotBytesOf<KF>;
      const typename std::conditional<KF == kKFp8, DmaOffsets, DmaOffsetsMx>::type off(lane);
#pragma unroll
      for (int s = 0; s < kRing - 1; ++s)
        if (s < n_mine) dma_page(a.kv_pages, a.k_scales, page_id(s), off, ring + s * kSlotBytes);
      for (int it = 0; it < n_mine; ++it) {
        if (it + kRing - 1 < n_mine) {  // wave-uniform
          __asm__ volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
          dma_page(a.kv_pages, a.k_scales, page_id(it + kRing - 1), off,
                   ring + ((it + kRing - 1) % kRing) * kSlotBytes);
        }
        const int ahead = min(kRing - 1, n_mine - 1 - it);  // pages in flight issued after page `it`
        if constexpr (KF == kKFp8) {
          static_assert(kDmaInstrsOf<KF> == 9, "the waits below count 9 loads per page");
          if (kRing == 3 && ahead == 2) __asm__ volatile("s_waitcnt vmcnt(18)" ::: "memory");
          else if (ahead >= 1) __asm__ volatile("s_waitcnt vmcnt(9)" ::: "memory");
          else __asm__ volatile("s_waitcnt vmcnt(0)" ::: "memory");
        } else {
          static_assert(kDmaInstrsOf<KF> == 5, "the waits below count 5 loads per page");
          if (kRing == 3 && ahead == 2) __asm__ volatile("s_waitcnt vmcnt(10)" ::: "memory");
          else if (ahead >= 1) __asm__ volatile("s_waitcnt vmcnt(5)" ::: "memory");
          else __asm__ volatile("s_waitcnt vmcnt(0)" ::: "memory");
        }
        PageRegs<KF> pr;
        read_page(ring + (it % kRing) * kSlotBytes, lane, pr);
        compute_page<NN, HIST, F16, KF, kDirectOf<NN, KF>>(
            pr, p0 + lpi0 + it * kWaves, lpi0 + it * kWaves, pages_per_wg, lane, rq, s_out, s_hist,
            static_cast<StageT<F16>*>(a.logits) + static_cast<int64_t>(row0) * a.logits_stride);
      }
      // (every page issued has landed: the last iteration waited for all)
    }
  } else if (n_mine > 0) {
    for (int it0 = 0; it0 < n_mine; it0 += kRg) {
#pragma unroll
      for (int s = 0; s < kRg; ++s) {
        const int it = it0 + s;
        if (it >= n_mine) break;
        const int nx = it + kPf < n_mine ? it + kPf : n_mine - 1;
        load_page(a.kv_pages, a.k_scales, page_id(nx), lane_off, lane, buf[(s + kPf) % kRg]);
        compute_page<NN, HIST, F16, KF>(buf[s], p0 + lpi0 + it * kWaves, lpi0 + it * kWaves,
                                    pages_per_wg, lane, rq, s_out, s_hist);
      }
    }
  }

  __syncthreads();
  // Live scores of the share, row by row, with 16-byte stores (the row offset
  // p0 * 64 and the stride are multiples of 16 bytes: 4 floats, 8 halves).
  constexpr int kPerVec = 16 / static_cast<int>(sizeof(StageT<F16>));
#pragma unroll
  for (int j = 0; j < (kDirectOf<NN, KF> ? 0 : NN); ++j) {
    const int64_t k0 = static_cast<int64_t>(p0) * kPage;
    // Live scores of this share (none for a workgroup past the request's end).
    const int n = max(0, static_cast<int>(min(static_cast<int64_t>(p1) * kPage, static_cast<int64_t>(rq.len[j])) - k0));
    StageT<F16>* dst = static_cast<StageT<F16>*>(a.logits) + static_cast<int64_t>(row0 + j) * a.logits_stride + k0;
    const StageT<F16>* src = s_out + j * pages_per_wg * kPage;
    const int nv = n / kPerVec;
    for (int i = tid; i < nv; i += kThreads)
      reinterpret_cast<i32x4*>(dst)[i] = reinterpret_cast<const i32x4*>(src)[i];
    for (int i = nv * kPerVec + tid; i < n; i += kThreads) dst[i] = src[i];
  }
  if constexpr (HIST) {
    // Flush this workgroup's slots: pairs of bins with one 64-bit atomic each.
    unsigned long long* gh = reinterpret_cast<unsigned long long*>(a.hist + static_cast<int64_t>(row0) * kBins);
    const uint2* sh = reinterpret_cast<const uint2*>(s_hist);
    for (int i = tid; i < NN * kBins / 2; i += kThreads) {
      const uint2 v = sh[i];
      if (v.x | v.y) atomicAdd(gh + i, (static_cast<unsigned long long>(v.y) << 32) | v.x);
    }
  }
}

// Requests the persistent grid serves (their share counts are prefix-summed
// in LDS).
constexpr int kPersistMaxB = 256;

// Grid (chunks, B): workgroup (c, b) computes share c of request b.  With
// PERSIST the grid is a fixed number of workgroups instead, and the
// shares that exist -- ceil(pages_b / pages_per_wg) per request, from the
// rows' lengths -- are numbered request by request and dealt out round
// robin: with many requests of varied length a (chunks, B) grid is mostly
// workgroups past their request's end, which the dispatcher has to launch
// all the same.
template <int NN, bool HIST, bool F16, int KF, bool PERSIST>
__global__ __launch_bounds__(kThreadsOf<NN>) __attribute__((amdgpu_waves_per_eu(kWavesPerSimd<NN>)))
void indexer_logits_kernel(LogitsArgs a, int pages_per_wg) {
  __shared__ int s_hist[HIST ? NN * kBins + 1 : 1];  // the rows' bins and a spare slot
  // [NN][pages_per_wg][64] scores.  The persistent grid's shares are 64
  // pages: its staging stays at 16 KiB (the 32 KiB one-row staging measured
  // varlen 130.0 -> 135.3 us with the histogram on).
  __shared__ __align__(16) StageT<F16> s_out[PERSIST ? NN * kMaxPagesPerWg * kPage : kStageFloats<NN>];
  // Q in MFMA operand layout, [row][head block][half][lane], and the weights:
  // fetched once per workgroup and read by every wave from here.
  __shared__ __align__(16) i32x4 s_q[NN >= 2 ? NN * 4 * kWave : 1];
  __shared__ __align__(16) float s_w[NN >= 2 ? NN * kHeads : 1];
  __shared__ int s_pref[PERSIST ? kPersistMaxB + 1 : 1];  // shares of requests < b (persistent grid)
  // K page slots of each wave (one-row requests, FP8 K)
  __shared__ __align__(16) char s_ring[kDmaOf<NN, KF> ? kWavesOf<NN> * kRing * kSlotBytesOf<KF> : 16];

  if constexpr (!PERSIST) {
    logits_share<NN, HIST, F16, KF>(a, pages_per_wg, blockIdx.y, static_cast<int64_t>(blockIdx.x) * pages_per_wg,
                                    s_hist, s_out, s_q, s_w, s_ring);
    return;
  }
  constexpr int kThreads = kThreadsOf<NN>;
  const int tid = threadIdx.x;
  const int lane = __lane_id();
  const int64_t mk = min(static_cast<int64_t>(a.max_pages) * kPage, a.logits_stride);
  const int max_keys = static_cast<int>(min(mk, static_cast<int64_t>(INT32_MAX)));
  const int nb = min(a.B, kPersistMaxB);  // the host launches this mode only for B <= kPersistMaxB
  for (int r = tid; r < nb; r += kThreads) {
    int keys = 0;
#pragma unroll
    for (int j = 0; j < NN; ++j) keys = max(keys, min(max(a.context_lens[r * NN + j], 0), max_keys));
    const int pages = (keys + kPage - 1) / kPage;
    s_pref[r + 1] = (pages + pages_per_wg - 1) / pages_per_wg;
  }
  if (tid == 0) s_pref[0] = 0;
  __syncthreads();
  if (tid < kWave) {
    int base = 0;
    for (int c = 0; c < nb; c += kWave) {
      const int r = c + lane;
      int incl = r < nb ? s_pref[r + 1] : 0;
#pragma unroll
      for (int d = 1; d < kWave; d <<= 1) {
        const int v = __shfl_up(incl, d);
        if (lane >= d) incl += v;
      }
      if (r < nb) s_pref[r + 1] = base + incl;
      base += __shfl(incl, kWave - 1);
    }
  }
  __syncthreads();
  const int total = s_pref[nb];
  for (int item = blockIdx.x; item < total; item += gridDim.x) {
    // the request whose shares hold `item`: s_pref[b] <= item < s_pref[b + 1]
    int lo = 0, hi = nb;
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (s_pref[mid] <= item) lo = mid;
      else hi = mid;
    }
    logits_share<NN, HIST, F16, KF>(a, pages_per_wg, lo, static_cast<int64_t>(item - s_pref[lo]) * pages_per_wg,
                                    s_hist, s_out, s_q, s_w, s_ring);
    __syncthreads();  // LDS of this share is read to the end before the next one writes it
  }
}

// ---------------------------------------------------------------------------
// Paged sparse MQA logits: the consumer layers of the two-level candidate
// indexer (SGLang PR #38944) score only the 8-token blocks a source layer
// published.  Sparse column 8 i + t of a row is key 8 table[i] + t; the K row
// sits at pool slot 8 slots[i] + t (the published table carries the blocks as
// pool slots / 8, so no block-table lookup is needed here).  Each wave takes
// 64 columns (8 table entries) at a time: lane (n, g) of key block kb reads
// the K row of column 16 kb + n -- the dense kernel's operand layout with a
// gathered address per lane -- and the same MFMA + epilogue computes the 64
// logits.  Columns whose entry is padding, or whose key is at or past the
// row length, are not written.
constexpr int kSparseWaves = 4;
constexpr int kSparseChunksPerWg = kSparseWaves;  // one 64-column chunk per wave: tables are short

template <int KF>
__global__ __launch_bounds__(kSparseWaves * kWave) __attribute__((amdgpu_waves_per_eu(4)))
void indexer_sparse_logits_kernel(SparseLogitsArgs a) {
  __shared__ __align__(16) float s_out[kSparseChunksPerWg * kPage];
  __shared__ uint8_t s_live[kSparseChunksPerWg * kPage];
  const int tid = threadIdx.x;
  const int lane = __lane_id();
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int row = blockIdx.y;
  const int chunks = (a.kb + kBlocksPerChunk - 1) / kBlocksPerChunk;
  const int c0 = blockIdx.x * kSparseChunksPerWg;
  if (c0 >= chunks) return;
  const int c1 = min(c0 + kSparseChunksPerWg, chunks);
  const int len = max(a.context_lens[row], 0);
  const int m = lane & 15, g = lane >> 4;

  RequestRegs<1> rq;
  rq.len[0] = len;
#pragma unroll
  for (int mb = 0; mb < 2; ++mb) {
#pragma unroll
    for (int h = 0; h < 2; ++h)
      rq.q[0][mb][h] = *reinterpret_cast<const i32x4*>(
          a.q + (static_cast<int64_t>(row) * kHeads + mb * 16 + m) * kDim + g * 16 + h * 64);
    rq.w[0][mb] = *reinterpret_cast<const f32x4*>(a.weights + static_cast<int64_t>(row) * kHeads + mb * 16 + 4 * g);
  }
  const int32_t* tab = a.table + static_cast<int64_t>(row) * a.kb;
  const int32_t* slt = a.slots + static_cast<int64_t>(row) * a.kb;
  const int64_t pool_keys = static_cast<int64_t>(a.num_pages) * kPage;
  const int t = m & (kBlk8 - 1);  // token of the lane's key within its block

  for (int c = c0 + wave; c < c1; c += kSparseWaves) {
    // Table entries of this lane's four keys (clamped loads, masked below).
    int key_slot[4];
    bool live[4];
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
      const int i = c * kBlocksPerChunk + kb * 2 + (m >> 3);
      const int ic = min(i, a.kb - 1);
      const int blk = tab[ic];
      const int s8 = slt[ic];
      const int64_t ps = static_cast<int64_t>(s8) * kBlk8 + t;
      live[kb] = i < a.kb && blk != INT_MAX && static_cast<int64_t>(blk) * kBlk8 + t < len && s8 >= 0 &&
                 ps < pool_keys;
      key_slot[kb] = live[kb] ? static_cast<int>(ps) : 0;
    }
    PageRegs<KF> pr;
    // lane l's own column 64 c + l is key n = l % 16 of key block l / 16
    const int own = lane >> 4;
    const bool own_live = own == 0 ? live[0] : own == 1 ? live[1] : own == 2 ? live[2] : live[3];
    if constexpr (KF == kKFp8) {
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) {
        const i32x4* src = reinterpret_cast<const i32x4*>(a.kv_pages + static_cast<int64_t>(key_slot[kb]) * kDim + g * 16);
        pr.v[2 * kb + 0] = src[0];
        pr.v[2 * kb + 1] = src[4];  // + 64 bytes
      }
      const int own_slot = own == 0 ? key_slot[0] : own == 1 ? key_slot[1] : own == 2 ? key_slot[2] : key_slot[3];
      pr.scale = a.k_scales[own_slot];
    } else {
      // MXFP4 token: bytes [16g, 16g+16) of its 64 code bytes and its scale word
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) {
        const uint8_t* tok = a.kv_pages + static_cast<int64_t>(key_slot[kb]) * kMxTokenBytes;
        pr.v[kb] = *reinterpret_cast<const i32x4*>(tok + g * 16);  // 4-byte aligned
        pr.sc[kb] = *reinterpret_cast<const int*>(tok + 64);
      }
    }
    const int lpi = c - c0;
    compute_page<1, false, false, KF>(pr, 0, lpi, kSparseChunksPerWg, lane, rq, s_out, nullptr);
    s_live[lpi * kPage + lane] = own_live ? 1 : 0;
  }
  __syncthreads();
  float* dst = a.logits + static_cast<int64_t>(row) * a.logits_stride + static_cast<int64_t>(c0) * kPage;
  const int ncols = (c1 - c0) * kPage;
  for (int i = tid; i < ncols; i += kSparseWaves * kWave)
    if (s_live[i]) dst[i] = s_out[i];
}

// ---------------------------------------------------------------------------
// Ragged prefill (extend) logits (SGLang PR #38944, the commit adding an SM90
// FP8 prefill path): every query row of an extend batch against its own
// request's keys, scored request by request so one read of a K page serves
// many rows.  A workgroup takes a tile of kPfTile consecutive rows of one
// request; each wave keeps kPfRowsPerWave rows' Q operands and weights in
// registers and walks all of the workgroup's pages (FP8 pages reach the
// waves through an LDS ring the workgroup fills once per page; MXFP4 pages
// each wave loads itself, from the CU's cache after the first wave).  The
// contraction and epilogue are the decode kernel's (compute_page): a prefill
// logit is bitwise the decode logit of the same row and key.
//
// Grid (splits, tiles).  Tiles are numbered request by request,
// ceil(rows_r / kPfTile) each; the y extent bounds their count (tokens /
// kPfTile + requests) and each workgroup finds its request with a wave scan
// over cu_q.  The `splits` workgroups of a tile divide the tile's pages into
// contiguous ranges of equal length, so a workgroup's Q is fetched once for a
// long stream of pages and no workgroup of a short tile sits idle: a grid
// over (page chunk, tile) would hold mostly workgroups past their tile's last
// page, and the dispatcher, not the arithmetic, would set the pace.  Tiles are
// dispatched last to first (in a causal extend batch the longest rows come
// last), so the short tiles fill in at the end.  `splits` is a multiple of 8:
// workgroups go to the 8 XCDs in turn by linear id, so split s of every tile
// runs on XCD s % 8, and neighbouring tiles (whose ranges nearly coincide)
// read their pages from one L2.
#ifndef PMQA_PREFILL_WAVES
#define PMQA_PREFILL_WAVES 4
#endif
#ifndef PMQA_PREFILL_PAGES
#define PMQA_PREFILL_PAGES 16
#endif
constexpr int kPfWaves = PMQA_PREFILL_WAVES;
constexpr int kPfRowsPerWave = 4;
constexpr int kPfTile = kPfWaves * kPfRowsPerWave;
constexpr int kPfPages = PMQA_PREFILL_PAGES;  // pages staged in LDS between stores
constexpr int kXcds = 8;
static_assert(kPfTile <= kWave && (kPfTile & (kPfTile - 1)) == 0, "a tile's rows fit one wave");
static_assert(kPfPages <= kWave && (kWave % kPfPages) == 0, "staging groups tile a 64-page window");
constexpr int kRingSlot = kPageBytes / 16;  // 16-byte pieces of one FP8 page
static_assert(kPfWaves * kWave * 2 == kRingSlot, "two pieces per thread fill a page");

struct PrefillTile {
  int req;      // request of the tile; -1 past the last tile
  int row0;     // first row of the tile
  int row_end;  // one past the request's last row (at most tokens)
};

// Tile y -> request: an inclusive wave scan of ceil(rows_r / kPfTile) over
// the requests, 64 at a time.  Malformed offsets (decreasing) count as empty
// requests.  Uniform across the wave.
__device__ __forceinline__ PrefillTile find_prefill_tile(const int32_t* __restrict__ cu_q, int R, int tokens,
                                                         int y, int lane) {
  int base = 0;
  for (int c = 0; c < R; c += kWave) {
    const int r = c + lane;
    const int lo = cu_q[min(r, R)];
    const int hi = cu_q[min(r + 1, R)];
    const int t = r < R ? (max(hi - lo, 0) + kPfTile - 1) / kPfTile : 0;
    int incl = t;
#pragma unroll
    for (int d = 1; d < kWave; d <<= 1) {
      const int v = __shfl_up(incl, d);
      if (lane >= d) incl += v;
    }
    const int tot = __shfl(incl, kWave - 1);
    if (y < base + tot) {
      const unsigned long long hit = __ballot(base + incl > y);
      const int l = static_cast<int>(__builtin_ctzll(hit));
      PrefillTile pt;
      pt.req = c + l;
      pt.row0 = __shfl(lo, l) + (y - base - __shfl(incl - t, l)) * kPfTile;
      pt.row_end = min(__shfl(hi, l), tokens);
      return pt;
    }
    base += tot;
  }
  return PrefillTile{-1, 0, 0};
}

template <int KF>
__global__ __launch_bounds__(kPfWaves * kWave) __attribute__((amdgpu_waves_per_eu(2)))
void indexer_prefill_logits_kernel(PrefillArgs a) {
  __shared__ __align__(16) float s_out[kPfTile * kPfPages * kPage];  // [row of tile][page of group][64]
  __shared__ __align__(16) i32x4 s_ring[KF == kKFp8 ? 2 * kRingSlot : 1];  // two FP8 pages, swizzled
  const int tid = threadIdx.x;
  const int lane = __lane_id();
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int y = static_cast<int>(gridDim.y - 1 - blockIdx.y);  // last tile first
  const PrefillTile pt = find_prefill_tile(a.cu_q, a.requests, a.tokens, y, lane);
  if (pt.req < 0) return;
  // No row reads past its block-table row or writes past its logits row.
  const int64_t mk = min(static_cast<int64_t>(a.max_pages) * kPage, a.logits_stride);
  const int max_keys = static_cast<int>(min(mk, static_cast<int64_t>(INT32_MAX)));
  // Lane i of every kPfTile-lane group holds the visible length of tile row
  // i (0 past the request's last row); the tile's key extent is their maximum.
  const int ri = pt.row0 + (lane & (kPfTile - 1));
  const bool ri_live = ri >= 0 && ri < pt.row_end;
  const int ri_len = a.row_lens[min(max(ri, 0), a.tokens - 1)];
  const int li = ri_live ? min(max(ri_len, 0), max_keys) : 0;
  int keys_t = li;
#pragma unroll
  for (int d = 1; d < kPfTile; d <<= 1) keys_t = max(keys_t, __shfl_xor(keys_t, d));
  keys_t = __builtin_amdgcn_readfirstlane(keys_t);
  const int pages_t = (keys_t + kPage - 1) / kPage;
  // This workgroup's contiguous share [pb, pe) of the tile's pages.
  const int64_t sp = static_cast<int64_t>(blockIdx.x);
  const int pb = static_cast<int>(sp * pages_t / gridDim.x);
  const int pe = static_cast<int>((sp + 1) * pages_t / gridDim.x);
  if (pb >= pe) return;  // uniform over the workgroup
  const int32_t* bt = a.block_table + static_cast<int64_t>(pt.req) * a.max_pages;

  // This wave's rows: Q operands and head weights (clamped loads; rows past
  // the request have length 0 and are never written).
  const int m = lane & 15, g = lane >> 4;
  RequestRegs<kPfRowsPerWave> rq;
#pragma unroll
  for (int j = 0; j < kPfRowsPerWave; ++j) {
    const int row = pt.row0 + wave * kPfRowsPerWave + j;
    const bool live = row >= 0 && row < pt.row_end;
    const int lj = __shfl(li, wave * kPfRowsPerWave + j);
    rq.len[j] = live ? lj : 0;
    const int64_t qr = min(max(row, 0), a.tokens - 1);
#pragma unroll
    for (int mb = 0; mb < 2; ++mb) {
#pragma unroll
      for (int h = 0; h < 2; ++h)
        rq.q[j][mb][h] = *reinterpret_cast<const i32x4*>(a.q + (qr * kHeads + mb * 16 + m) * kDim + g * 16 + h * 64);
      rq.w[j][mb] = *reinterpret_cast<const f32x4*>(a.weights + qr * kHeads + mb * 16 + 4 * g);
    }
  }

  const int lane_off = (lane & 15) * (KF == kKFp8 ? kDim : kMxTokenBytes) + (lane >> 4) * 16;
  float* s_w = s_out + wave * kPfRowsPerWave * kPfPages * kPage;
  // Staged scores of pages [g0, g0 + np) leave with 16-byte stores (the
  // column offset g0 * 64 and the stride are multiples of 4 floats).  Only
  // this wave wrote them; its next writes to the staging area come after
  // these reads in the wave's own LDS order.
  auto flush = [&](int g0, int np) {
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
    __builtin_amdgcn_wave_barrier();
#pragma unroll
    for (int j = 0; j < kPfRowsPerWave; ++j) {
      const int n = max(0, min(rq.len[j] - g0 * kPage, np * kPage));
      if (n == 0) continue;
      const int row = pt.row0 + wave * kPfRowsPerWave + j;
      float* dst = a.logits + static_cast<int64_t>(row) * a.logits_stride + static_cast<int64_t>(g0) * kPage;
      const float* src = s_w + j * kPfPages * kPage;
      const int nv = n / 4;
      for (int i = lane; i < nv; i += kWave)
        reinterpret_cast<f32x4*>(dst)[i] = reinterpret_cast<const f32x4*>(src)[i];
      for (int i = nv * 4 + lane; i < n; i += kWave) dst[i] = src[i];
    }
  };

  // Windows of up to 64 pages: lane i of `ids` holds the id of the window's
  // i-th page.  Every kPfPages pages (and at the window's end) the staged
  // scores are stored.
  for (int w0 = pb; w0 < pe; w0 += kWave) {
    const int nw = min(kWave, pe - w0);
    const int ids = bt[min(w0 + lane, a.max_pages - 1)];
    auto page_id = [&](int it) {
      const int id = __builtin_amdgcn_readlane(ids, it);
      return min(max(id, 0), a.num_pages - 1);
    };
    if constexpr (KF == kKFp8) {
      // FP8 pages go through a two-slot LDS ring: the workgroup loads each
      // page once (two 16-byte pieces per thread, held in registers while
      // the previous page is computed) and every wave reads its MFMA
      // operands from LDS -- a quarter of the vector-memory traffic of four
      // waves loading the page each, and two pages in flight.  Piece q of a
      // page (key q / 8, 16-byte column q % 8) sits at column
      // (q % 8) ^ ((key / 2) % 8) of the key's 128-byte LDS row, so the 16
      // keys an operand read touches spread over all banks.
      i32x4 gk[2][2];
      float gs[2];
      auto gload = [&](int it, int set) {
        const int pid = page_id(it);
        const __amdgpu_buffer_rsrc_t kr = range_rsrc(a.kv_pages + static_cast<int64_t>(pid) * kPageBytes, kPageBytes);
        gk[set][0] = __builtin_bit_cast(i32x4, __builtin_amdgcn_raw_buffer_load_b128(kr, tid * 16, 0, 0));
        gk[set][1] = __builtin_bit_cast(i32x4, __builtin_amdgcn_raw_buffer_load_b128(kr, kPageBytes / 2 + tid * 16, 0, 0));
        const __amdgpu_buffer_rsrc_t sr = range_rsrc(a.k_scales + static_cast<int64_t>(pid) * kPage, kPage * 4);
        gs[set] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(sr, lane * 4, 0, 0));
      };
      auto lwrite = [&](int set, int slot) {
        i32x4* ring = s_ring + slot * kRingSlot;
#pragma unroll
        for (int ch = 0; ch < 2; ++ch) {
          const int q = tid + ch * kPfWaves * kWave;
          const int n = q >> 3;
          ring[n * 8 + ((q & 7) ^ ((n >> 1) & 7))] = gk[set][ch];
        }
      };
      gload(0, 0);
      gload(min(1, nw - 1), 1);
      lwrite(0, 0);
      lds_barrier();
      for (int it0 = 0; it0 < nw; it0 += 2) {
#pragma unroll
        for (int s = 0; s < 2; ++s) {
          const int it = it0 + s;
          if (it >= nw) break;
          PageRegs<kKFp8> pr;
          const i32x4* ring = s_ring + s * kRingSlot;
#pragma unroll
          for (int kb = 0; kb < 4; ++kb) {
            const int n = kb * 16 + m;
#pragma unroll
            for (int h = 0; h < 2; ++h) pr.v[2 * kb + h] = ring[n * 8 + ((g + 4 * h) ^ ((n >> 1) & 7))];
          }
          pr.scale = gs[s];
          gload(min(it + 2, nw - 1), s);
          const int slot = it % kPfPages;
          compute_page<kPfRowsPerWave, false, false, KF>(pr, w0 + it, slot, kPfPages, lane, rq, s_w, nullptr);
          if (slot == kPfPages - 1 || it == nw - 1) flush(w0 + it - slot, slot + 1);
          lwrite(s ^ 1, s ^ 1);
          lds_barrier();
        }
      }
    } else {
      // MXFP4 pages stay in registers: two page buffers, page it + 1 in
      // flight while page it is computed (past the window's last page the
      // last one is issued again, from cache).
      PageRegs<KF> buf[2];
      load_page(a.kv_pages, a.k_scales, page_id(0), lane_off, lane, buf[0]);
      for (int it0 = 0; it0 < nw; it0 += 2) {
#pragma unroll
        for (int s = 0; s < 2; ++s) {
          const int it = it0 + s;
          if (it >= nw) break;
          const int nx = it + 1 < nw ? it + 1 : nw - 1;
          load_page(a.kv_pages, a.k_scales, page_id(nx), lane_off, lane, buf[s ^ 1]);
          const int slot = it % kPfPages;
          compute_page<kPfRowsPerWave, false, false, KF>(buf[s], w0 + it, slot, kPfPages, lane, rq, s_w, nullptr);
          if (slot == kPfPages - 1 || it == nw - 1) flush(w0 + it - slot, slot + 1);
        }
      }
    }
  }
}

struct DeviceInfo {
  int cus = 0;
};

DeviceInfo* device_info(int dev) {
  static DeviceInfo infos[64];
  static bool ready[64] = {};
  if (dev < 0 || dev >= 64) return nullptr;
  if (!ready[dev]) {
    DeviceInfo d;
    if (hipDeviceGetAttribute(&d.cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return nullptr;
    infos[dev] = d;
    ready[dev] = true;  // benign race: every thread computes the same values
  }
  return &infos[dev];
}

// The persistent grid is built for one row per request (the decode shape
// with many requests) and FP8 K; other shapes take the (chunks, B) grid.
template <int NN, bool HIST, bool F16, int KF>
hipError_t launch(const LogitsArgs& a, dim3 grid, int pages_per_wg, int persistent, hipStream_t stream,
                  LaunchEvents ev) {
  if constexpr (NN == 1 && KF == kKFp8) {
    if (persistent) {
      launch_kernel(indexer_logits_kernel<NN, HIST, F16, KF, true>, grid, dim3(kThreadsOf<NN>), stream, ev.start,
                    ev.stop, a, pages_per_wg);
      return hipGetLastError();
    }
  }
  launch_kernel(indexer_logits_kernel<NN, HIST, F16, KF, false>, grid, dim3(kThreadsOf<NN>), stream, ev.start,
                ev.stop, a, pages_per_wg);
  return hipGetLastError();
}

// MXFP4 K is served with float32 logits only.
template <int NN, bool HIST>
hipError_t launch_fmt(const LogitsArgs& a, dim3 grid, int pages_per_wg, int persistent, hipStream_t stream,
                      LaunchEvents ev) {
  if (a.k_mxfp4) return launch<NN, HIST, false, kKMxfp4>(a, grid, pages_per_wg, persistent, stream, ev);
  if (a.logits_f16) return launch<NN, HIST, true, kKFp8>(a, grid, pages_per_wg, persistent, stream, ev);
  return launch<NN, HIST, false, kKFp8>(a, grid, pages_per_wg, persistent, stream, ev);
}

}  // namespace

hipError_t launch_indexer_logits(const LogitsArgs& a, hipStream_t stream, LaunchEvents ev) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  const DeviceInfo* info = device_info(dev);
  if (!info) return hipErrorInvalidDevice;
  const bool hist = a.hist != nullptr;
  // Pages per workgroup.  Long streams per wave amortise a workgroup's start
  // (one round trip for its page ids) and end (staged stores, histogram
  // flush), so a share is as long as the grid allows while every CU still
  // gets a workgroup: B * max_pages / CUs pages, 4..max_ppw.  The host
  // cannot read the lengths, so B * max_pages is an upper bound; with many
  // requests (B >= 32) the real lengths usually vary, and shorter shares
  // (16 pages) give the static grid enough rounds to even out.
  const int64_t pages_upper = static_cast<int64_t>(a.B) * a.max_pages;
  int64_t ppw = (pages_upper + info->cus - 1) / info->cus;
  if (a.B >= 32 && ppw > 16) ppw = 16;
#if PMQA_LOGITS_PAGES_PER_WG
  ppw = PMQA_LOGITS_PAGES_PER_WG;
#endif
  ppw = (ppw + 3) / 4 * 4;  // rounded up: the grid then holds at most one workgroup per CU
  const int64_t max_ppw = a.next_n == 1 ? kMaxPagesPerWgOneRow : kMaxPagesPerWg;
  ppw = ppw < 4 ? 4 : (ppw > max_ppw ? max_ppw : ppw);
  const int64_t chunks = (a.max_pages + ppw - 1) / ppw;
  if (chunks > 0x7FFFFFFF) return hipErrorInvalidValue;
  dim3 grid(static_cast<unsigned>(chunks), static_cast<unsigned>(a.B));
  // Many requests (lengths usually varied): a persistent grid of a few
  // workgroups per CU deals out the shares that exist.
  int persistent = 0;
#if PMQA_LOGITS_PERSIST
  if (a.next_n == 1 && !a.k_mxfp4 && a.B >= 32 && a.B <= kPersistMaxB) {
    ppw = PMQA_LOGITS_PERSIST_PPW;  // equal shares dealt round robin (at most kMaxPagesPerWg)
    const int64_t upper = (a.max_pages + ppw - 1) / ppw * a.B;
    // the LDS page ring leaves room for one workgroup per CU
    const int64_t per_cu = PMQA_LOGITS_PERSIST_WGS_PER_CU ? PMQA_LOGITS_PERSIST_WGS_PER_CU : (PMQA_LOGITS_DMA ? 1 : 2);
    const int64_t wgs = per_cu * info->cus;
    grid = dim3(static_cast<unsigned>(upper < wgs ? upper : wgs), 1);
    persistent = 1;
  }
#endif
  const int p = static_cast<int>(ppw);
  if (a.k_mxfp4 && a.logits_f16) return hipErrorInvalidValue;
  switch (a.next_n * 2 + (hist ? 1 : 0)) {
    case 2: return launch_fmt<1, false>(a, grid, p, persistent, stream, ev);
    case 3: return launch_fmt<1, true>(a, grid, p, persistent, stream, ev);
    case 4: return launch_fmt<2, false>(a, grid, p, persistent, stream, ev);
    case 5: return launch_fmt<2, true>(a, grid, p, persistent, stream, ev);
    case 6: return launch_fmt<3, false>(a, grid, p, persistent, stream, ev);
    case 7: return launch_fmt<3, true>(a, grid, p, persistent, stream, ev);
    case 8: return launch_fmt<4, false>(a, grid, p, persistent, stream, ev);
    case 9: return launch_fmt<4, true>(a, grid, p, persistent, stream, ev);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_indexer_prefill_logits(const PrefillArgs& a, hipStream_t stream, LaunchEvents ev) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  const DeviceInfo* info = device_info(dev);
  if (!info) return hipErrorInvalidDevice;
  const int64_t gy = (static_cast<int64_t>(a.tokens) + kPfTile - 1) / kPfTile + a.requests;
  if (gy > 65535) return hipErrorInvalidValue;
  // Workgroups per tile: 8 (one per XCD), more when there are too few tiles
  // to give every CU two workgroups; never more than a tile can have pages.
  int64_t splits = kXcds;
  while (splits * gy < 2 * info->cus && splits < kWave * kXcds) splits *= 2;
  const dim3 grid(static_cast<unsigned>(splits), static_cast<unsigned>(gy));
  if (a.k_mxfp4)
    launch_kernel(indexer_prefill_logits_kernel<kKMxfp4>, grid, dim3(kPfWaves * kWave), stream, ev.start, ev.stop,
                  a);
  else
    launch_kernel(indexer_prefill_logits_kernel<kKFp8>, grid, dim3(kPfWaves * kWave), stream, ev.start, ev.stop, a);
  return hipGetLastError();
}

hipError_t launch_indexer_sparse_logits(const SparseLogitsArgs& a, hipStream_t stream, LaunchEvents ev) {
  const int64_t chunks = (static_cast<int64_t>(a.kb) + kBlocksPerChunk - 1) / kBlocksPerChunk;
  const int64_t gx = (chunks + kSparseChunksPerWg - 1) / kSparseChunksPerWg;
  if (gx > 0x7FFFFFFF) return hipErrorInvalidValue;
  const dim3 grid(static_cast<unsigned>(gx), static_cast<unsigned>(a.rows));
  if (a.k_mxfp4)
    launch_kernel(indexer_sparse_logits_kernel<kKMxfp4>, grid, dim3(kSparseWaves * kWave), stream, ev.start,
                  ev.stop, a);
  else
    launch_kernel(indexer_sparse_logits_kernel<kKFp8>, grid, dim3(kSparseWaves * kWave), stream, ev.start,
                  ev.stop, a);
  return hipGetLastError();
}

}  // namespace pmqa
