// Host-side launch entry points implemented by the kernel files, called by
// the C ABI (abi.hip).
#pragma once

#include "indexer_common.h"

namespace pmqa {

hipError_t launch_indexer_logits(const LogitsArgs& a, hipStream_t stream, LaunchEvents ev = {});
hipError_t launch_indexer_sparse_logits(const SparseLogitsArgs& a, hipStream_t stream, LaunchEvents ev = {});
hipError_t launch_indexer_prefill_logits(const PrefillArgs& a, hipStream_t stream, LaunchEvents ev = {});
hipError_t launch_block_amax8(const float* scores, int64_t stride, const int32_t* lens, int32_t rows, float* out,
                              int64_t out_stride, int32_t* hist, int32_t* block_lens, hipStream_t stream,
                              LaunchEvents ev = {});
hipError_t launch_sort_candidate_blocks(const int32_t* blocks, int32_t kb, const int32_t* lens, int32_t rows,
                                        int64_t max_len, const int32_t* block_table, int32_t max_pages,
                                        int32_t next_n, int32_t* table, int32_t* slots, int32_t* sparse_lens,
                                        hipStream_t stream, LaunchEvents ev = {});
hipError_t launch_sparse_to_logical(const int32_t* idx, int32_t k, const int32_t* table, int32_t kb, int32_t rows,
                                    int32_t* out, hipStream_t stream, LaunchEvents ev = {});

struct TopkArgs {
  const void* logits;  // float32, or IEEE binary16 bits with logits_f16
  const int32_t* hist;
  const int32_t* context_lens;
  int32_t* indices;
  void* workspace;
  int64_t logits_stride;
  int32_t rows;
  int32_t k;
  int32_t key_dtype;
  int32_t logits_f16;
};
size_t topk_workspace_size(int32_t rows, int64_t logits_stride, int32_t k);
hipError_t launch_topk_rows(const TopkArgs& a, hipStream_t stream, LaunchEvents ev = {});
// topk_rows over sparse rows (stride <= 16384, float32) writing logical keys
// through the rows' block tables [rows][kb].
hipError_t launch_sparse_topk(const TopkArgs& a, const int32_t* table, int kb, hipStream_t stream,
                              LaunchEvents ev = {});
// topk_rows with the library's fixed per-device scratch (no workspace).
size_t topk_noalloc_scratch_bytes();
hipError_t launch_topk_rows_noalloc(const TopkArgs& a, hipStream_t stream, LaunchEvents ev = {});

hipError_t launch_score_histogram(const float* scores, int64_t stride, const int32_t* lens,
                                  int32_t rows, int32_t* hist, hipStream_t stream);

hipError_t launch_hbm_read_probe(const void* src, size_t bytes, uint32_t* sink, bool nt,
                                 hipStream_t stream, LaunchEvents ev = {});
hipError_t launch_hbm_gather_probe(const uint8_t* pool, const float* scales, const int32_t* table,
                                   int32_t n_pages, int32_t pool_pages, uint32_t* sink, hipStream_t stream,
                                   LaunchEvents ev = {});
hipError_t launch_mfma_valu_probe(int mode, int workgroups, int iters, float* out, hipStream_t stream,
                                  LaunchEvents ev = {});

}  // namespace pmqa
