// C ABI of the paged MQA indexer: host-side argument checks, then launches.
// Every check runs before anything is enqueued; see paged_mqa_indexer.h.
#include "indexer_common.h"
#include "launches.h"

namespace {

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

idx_status from_hip(hipError_t e) { return e == hipSuccess ? IDX_OK : IDX_ELAUNCH; }

// Events armed by indexer_time_next_call for this host thread's next call.
thread_local pmqa::LaunchEvents t_next_events;

// Every entry point takes (and so disarms) the armed events first, whether
// or not its checks pass.
pmqa::LaunchEvents take_events() {
  const pmqa::LaunchEvents ev = t_next_events;
  t_next_events = pmqa::LaunchEvents{};
  return ev;
}

idx_status logits_call(const uint8_t* q, const uint8_t* kv_pages, const float* k_scales,
                       const float* weights, const int32_t* block_table, const int32_t* context_lens,
                       int32_t B, int32_t next_n, int32_t num_pages, int32_t max_pages, void* logits,
                       int64_t logits_stride, bool f16, bool mxfp4, int32_t* hist, void* stream) {
  const pmqa::LaunchEvents ev = take_events();
  if (!q || !kv_pages || (!mxfp4 && !k_scales) || !weights || !block_table || !context_lens || !logits)
    return IDX_EINVAL;
  if (B <= 0 || num_pages <= 0 || max_pages <= 0 || logits_stride <= 0) return IDX_EINVAL;
  if (next_n < 1 || next_n > 4) return IDX_EUNSUPPORTED;
  if (B > IDX_MAX_REQUESTS || static_cast<int64_t>(B) * next_n > IDX_MAX_ROWS) return IDX_EUNSUPPORTED;
  // The page list of all requests is indexed with 32-bit integers.
  if (static_cast<int64_t>(B) * max_pages > INT32_MAX) return IDX_EUNSUPPORTED;
  // Rows are written with 16-byte stores: the stride is a multiple of 16 bytes.
  const int64_t per16 = f16 ? 8 : 4;
  if (!aligned(q, 16) || !aligned(kv_pages, 16) || !aligned(weights, 16) || (!mxfp4 && !aligned(k_scales, 4)) ||
      !aligned(block_table, 4) || !aligned(context_lens, 4) || !aligned(logits, 16) ||
      (logits_stride % per16) != 0 || (hist && !aligned(hist, 8)))
    return IDX_EALIGN;
  pmqa::LogitsArgs a;
  a.q = q;
  a.kv_pages = kv_pages;
  a.k_scales = k_scales;
  a.weights = weights;
  a.block_table = block_table;
  a.context_lens = context_lens;
  a.logits = logits;
  a.hist = hist;
  a.logits_stride = logits_stride;
  a.logits_f16 = f16 ? 1 : 0;
  a.k_mxfp4 = mxfp4 ? 1 : 0;
  a.B = B;
  a.next_n = next_n;
  a.num_pages = num_pages;
  a.max_pages = max_pages;
  return from_hip(pmqa::launch_indexer_logits(a, static_cast<hipStream_t>(stream), ev));
}

// noalloc: topk_rows_noalloc, whose scratch is the library's fixed array.
idx_status topk_call(const void* logits, int64_t logits_stride, bool f16, const int32_t* hist,
                     const int32_t* context_lens, int32_t rows, int32_t k, int32_t key_dtype,
                     int32_t* indices, void* workspace, size_t workspace_bytes, void* stream,
                     bool noalloc = false) {
  const pmqa::LaunchEvents ev = take_events();
  if (!logits || !context_lens || !indices || (!noalloc && !workspace)) return IDX_EINVAL;
  if (rows <= 0 || logits_stride <= 0 || k < 1 || k > IDX_CANDIDATE_CAPACITY) return IDX_EINVAL;
  if (key_dtype != IDX_KEY_FP32 && key_dtype != IDX_KEY_FP16) return IDX_EUNSUPPORTED;
  const int64_t per16 = f16 ? 8 : 4;  // rows are read with 16-byte loads
  if (rows > IDX_MAX_ROWS || logits_stride > IDX_TOPK_MAX_STRIDE) return IDX_EUNSUPPORTED;
  if (!aligned(logits, 16) || (logits_stride % per16) != 0 || !aligned(context_lens, 4) ||
      !aligned(indices, 4) || (!noalloc && !aligned(workspace, 256)) || (hist && !aligned(hist, 8)))
    return IDX_EALIGN;
  if (noalloc) {
    if (logits_stride > 16384 && rows > IDX_NOALLOC_MAX_ROWS) return IDX_ESCRATCH;
  } else if (workspace_bytes < pmqa::topk_workspace_size(rows, logits_stride, k)) {
    return IDX_EWORKSPACE;
  }
  pmqa::TopkArgs a;
  a.logits = logits;
  a.hist = hist;
  a.context_lens = context_lens;
  a.indices = indices;
  a.workspace = workspace;
  a.logits_stride = logits_stride;
  a.rows = rows;
  a.k = k;
  a.key_dtype = f16 ? IDX_KEY_FP16 : key_dtype;
  a.logits_f16 = f16 ? 1 : 0;
  if (noalloc) return from_hip(pmqa::launch_topk_rows_noalloc(a, static_cast<hipStream_t>(stream), ev));
  return from_hip(pmqa::launch_topk_rows(a, static_cast<hipStream_t>(stream), ev));
}

}  // namespace

extern "C" {

const char* indexer_status_str(int32_t s) {
  switch (s) {
    case IDX_OK: return "IDX_OK";
    case IDX_EINVAL: return "IDX_EINVAL: invalid argument";
    case IDX_EUNSUPPORTED: return "IDX_EUNSUPPORTED: unsupported configuration";
    case IDX_EALIGN: return "IDX_EALIGN: misaligned pointer or stride";
    case IDX_ELAUNCH: return "IDX_ELAUNCH: HIP launch or device query failed";
    case IDX_EWORKSPACE: return "IDX_EWORKSPACE: workspace too small";
    case IDX_ESCRATCH:
      return "IDX_ESCRATCH: more rows than the fixed scratch of topk_rows_noalloc holds (IDX_NOALLOC_MAX_ROWS)";
    default: return "unknown status";
  }
}

idx_status indexer_time_next_call(void* start_event, void* stop_event) {
  t_next_events.start = static_cast<hipEvent_t>(start_event);
  t_next_events.stop = static_cast<hipEvent_t>(stop_event);
  return IDX_OK;
}

idx_status indexer_logits(const uint8_t* q, const uint8_t* kv_pages, const float* k_scales,
                          const float* weights, const int32_t* block_table,
                          const int32_t* context_lens, int32_t B, int32_t next_n,
                          int32_t num_pages, int32_t max_pages, float* logits,
                          int64_t logits_stride, int32_t* hist, void* stream) {
  return logits_call(q, kv_pages, k_scales, weights, block_table, context_lens, B, next_n, num_pages,
                     max_pages, logits, logits_stride, false, false, hist, stream);
}

idx_status indexer_logits_f16(const uint8_t* q, const uint8_t* kv_pages, const float* k_scales,
                              const float* weights, const int32_t* block_table,
                              const int32_t* context_lens, int32_t B, int32_t next_n,
                              int32_t num_pages, int32_t max_pages, uint16_t* logits,
                              int64_t logits_stride, int32_t* hist, void* stream) {
  return logits_call(q, kv_pages, k_scales, weights, block_table, context_lens, B, next_n, num_pages,
                     max_pages, logits, logits_stride, true, false, hist, stream);
}

idx_status indexer_logits_mxfp4(const uint8_t* q, const uint8_t* kv_pages, const float* weights,
                                const int32_t* block_table, const int32_t* context_lens, int32_t B,
                                int32_t next_n, int32_t num_pages, int32_t max_pages, float* logits,
                                int64_t logits_stride, int32_t* hist, void* stream) {
  return logits_call(q, kv_pages, nullptr, weights, block_table, context_lens, B, next_n, num_pages,
                     max_pages, logits, logits_stride, false, true, hist, stream);
}

size_t topk_workspace_bytes(int32_t rows, int64_t logits_stride, int32_t k) {
  return pmqa::topk_workspace_size(rows, logits_stride, k);
}

idx_status topk_rows(const float* logits, int64_t logits_stride, const int32_t* hist,
                     const int32_t* context_lens, int32_t rows, int32_t k, int32_t key_dtype,
                     int32_t* indices, void* workspace, size_t workspace_bytes, void* stream) {
  return topk_call(logits, logits_stride, false, hist, context_lens, rows, k, key_dtype, indices,
                   workspace, workspace_bytes, stream);
}

idx_status topk_rows_noalloc(const float* logits, int64_t logits_stride, const int32_t* hist,
                             const int32_t* context_lens, int32_t rows, int32_t k, int32_t key_dtype,
                             int32_t* indices, void* stream) {
  return topk_call(logits, logits_stride, false, hist, context_lens, rows, k, key_dtype, indices, nullptr, 0,
                   stream, true);
}

idx_status topk_rows_f16(const uint16_t* logits, int64_t logits_stride, const int32_t* hist,
                         const int32_t* context_lens, int32_t rows, int32_t k, int32_t* indices,
                         void* workspace, size_t workspace_bytes, void* stream) {
  return topk_call(logits, logits_stride, true, hist, context_lens, rows, k, IDX_KEY_FP16, indices,
                   workspace, workspace_bytes, stream);
}

idx_status score_histogram(const float* scores, int64_t stride, const int32_t* context_lens,
                           int32_t rows, int32_t* hist, void* stream) {
  take_events();  // launches nothing timed; disarms like every call
  if (!scores || !context_lens || !hist) return IDX_EINVAL;
  if (rows <= 0 || stride <= 0) return IDX_EINVAL;
  if (rows > IDX_MAX_ROWS || stride > (int64_t{1} << 31) - 4) return IDX_EUNSUPPORTED;
  if (!aligned(scores, 16) || (stride % 4) != 0 || !aligned(context_lens, 4) || !aligned(hist, 8))
    return IDX_EALIGN;
  return from_hip(pmqa::launch_score_histogram(scores, stride, context_lens, rows, hist,
                                               static_cast<hipStream_t>(stream)));
}

idx_status block_amax8(const float* scores, int64_t stride, const int32_t* context_lens, int32_t rows,
                       float* out, int64_t out_stride, int32_t* hist, int32_t* block_lens, void* stream) {
  const pmqa::LaunchEvents ev = take_events();
  if (!scores || !context_lens || !out) return IDX_EINVAL;
  if (rows <= 0 || stride <= 0 || out_stride < (stride + 7) / 8) return IDX_EINVAL;
  if (rows > IDX_MAX_ROWS || stride > (int64_t{1} << 31) - 4) return IDX_EUNSUPPORTED;
  if (!aligned(scores, 16) || (stride % 4) != 0 || !aligned(context_lens, 4) || !aligned(out, 4) ||
      (hist && !aligned(hist, 8)) || (block_lens && !aligned(block_lens, 4)))
    return IDX_EALIGN;
  return from_hip(pmqa::launch_block_amax8(scores, stride, context_lens, rows, out, out_stride, hist, block_lens,
                                           static_cast<hipStream_t>(stream), ev));
}

idx_status sort_candidate_blocks(const int32_t* blocks, int32_t kb, const int32_t* context_lens,
                                 int32_t rows, int64_t max_len, const int32_t* block_table,
                                 int32_t max_pages, int32_t next_n, int32_t* table, int32_t* slots,
                                 int32_t* sparse_lens, void* stream) {
  const pmqa::LaunchEvents ev = take_events();
  if (!blocks || !context_lens || !block_table || !table || !slots || !sparse_lens) return IDX_EINVAL;
  if (rows <= 0 || kb <= 0 || max_len <= 0 || max_pages <= 0 || next_n < 1) return IDX_EINVAL;
  if (rows % next_n != 0) return IDX_EINVAL;
  if (rows > IDX_MAX_ROWS || kb > pmqa::kMaxCandidateBlocks ||
      max_len > static_cast<int64_t>(pmqa::kMaxCandidateBlocks) * 8)
    return IDX_EUNSUPPORTED;
  if (!aligned(blocks, 4) || !aligned(context_lens, 4) || !aligned(block_table, 4) || !aligned(table, 4) ||
      !aligned(slots, 4) || !aligned(sparse_lens, 4))
    return IDX_EALIGN;
  return from_hip(pmqa::launch_sort_candidate_blocks(blocks, kb, context_lens, rows, max_len, block_table,
                                                     max_pages, next_n, table, slots, sparse_lens,
                                                     static_cast<hipStream_t>(stream), ev));
}

static idx_status sparse_logits_call(const uint8_t* q, const uint8_t* kv_pages, const float* k_scales,
                              const float* weights, const int32_t* table, const int32_t* slots, int32_t kb,
                              const int32_t* context_lens, int32_t rows, int32_t num_pages, float* logits,
                              int64_t logits_stride, bool mxfp4, void* stream) {
  const pmqa::LaunchEvents ev = take_events();
  if (!q || !kv_pages || (!mxfp4 && !k_scales) || !weights || !table || !slots || !context_lens || !logits)
    return IDX_EINVAL;
  if (rows <= 0 || kb <= 0 || num_pages <= 0 || logits_stride < static_cast<int64_t>(kb) * 8) return IDX_EINVAL;
  if (rows > IDX_MAX_ROWS || kb > pmqa::kMaxCandidateBlocks) return IDX_EUNSUPPORTED;
  if (!aligned(q, 16) || !aligned(kv_pages, 16) || (!mxfp4 && !aligned(k_scales, 4)) || !aligned(weights, 16) ||
      !aligned(table, 4) || !aligned(slots, 4) || !aligned(context_lens, 4) || !aligned(logits, 4))
    return IDX_EALIGN;
  pmqa::SparseLogitsArgs a;
  a.k_mxfp4 = mxfp4 ? 1 : 0;
  a.q = q;
  a.kv_pages = kv_pages;
  a.k_scales = k_scales;
  a.weights = weights;
  a.table = table;
  a.slots = slots;
  a.context_lens = context_lens;
  a.logits = logits;
  a.logits_stride = logits_stride;
  a.rows = rows;
  a.kb = kb;
  a.num_pages = num_pages;
  return from_hip(pmqa::launch_indexer_sparse_logits(a, static_cast<hipStream_t>(stream), ev));
}

idx_status indexer_sparse_logits(const uint8_t* q, const uint8_t* kv_pages, const float* k_scales,
                                 const float* weights, const int32_t* table, const int32_t* slots,
                                 int32_t kb, const int32_t* context_lens, int32_t rows, int32_t num_pages,
                                 float* logits, int64_t logits_stride, void* stream) {
  return sparse_logits_call(q, kv_pages, k_scales, weights, table, slots, kb, context_lens, rows, num_pages,
                            logits, logits_stride, false, stream);
}

idx_status indexer_sparse_logits_mxfp4(const uint8_t* q, const uint8_t* kv_pages, const float* weights,
                                       const int32_t* table, const int32_t* slots, int32_t kb,
                                       const int32_t* context_lens, int32_t rows, int32_t num_pages,
                                       float* logits, int64_t logits_stride, void* stream) {
  return sparse_logits_call(q, kv_pages, nullptr, weights, table, slots, kb, context_lens, rows, num_pages,
                            logits, logits_stride, true, stream);
}

static idx_status prefill_call(const uint8_t* q, const uint8_t* kv_pages, const float* k_scales,
                               const float* weights, const int32_t* block_table, int32_t max_pages,
                               const int32_t* cu_q, int32_t requests, int32_t tokens, const int32_t* row_lens,
                               int32_t num_pages, float* logits, int64_t logits_stride, bool mxfp4, void* stream) {
  const pmqa::LaunchEvents ev = take_events();
  if (!q || !kv_pages || (!mxfp4 && !k_scales) || !weights || !block_table || !cu_q || !row_lens || !logits)
    return IDX_EINVAL;
  if (requests <= 0 || tokens <= 0 || num_pages <= 0 || max_pages <= 0 || logits_stride <= 0) return IDX_EINVAL;
  if (requests > IDX_MAX_REQUESTS || tokens > IDX_MAX_ROWS) return IDX_EUNSUPPORTED;
  if (static_cast<int64_t>(requests) * max_pages > INT32_MAX) return IDX_EUNSUPPORTED;
  if (!aligned(q, 16) || !aligned(kv_pages, 16) || (!mxfp4 && !aligned(k_scales, 4)) || !aligned(weights, 16) ||
      !aligned(block_table, 4) || !aligned(cu_q, 4) || !aligned(row_lens, 4) || !aligned(logits, 16) ||
      (logits_stride % 4) != 0)
    return IDX_EALIGN;
  pmqa::PrefillArgs a;
  a.q = q;
  a.kv_pages = kv_pages;
  a.k_scales = k_scales;
  a.weights = weights;
  a.block_table = block_table;
  a.cu_q = cu_q;
  a.row_lens = row_lens;
  a.logits = logits;
  a.logits_stride = logits_stride;
  a.requests = requests;
  a.tokens = tokens;
  a.num_pages = num_pages;
  a.max_pages = max_pages;
  a.k_mxfp4 = mxfp4 ? 1 : 0;
  return from_hip(pmqa::launch_indexer_prefill_logits(a, static_cast<hipStream_t>(stream), ev));
}

idx_status indexer_prefill_logits(const uint8_t* q, const uint8_t* kv_pages, const float* k_scales,
                                  const float* weights, const int32_t* block_table, int32_t max_pages,
                                  const int32_t* cu_q, int32_t requests, int32_t tokens, const int32_t* row_lens,
                                  int32_t num_pages, float* logits, int64_t logits_stride, void* stream) {
  return prefill_call(q, kv_pages, k_scales, weights, block_table, max_pages, cu_q, requests, tokens, row_lens,
                      num_pages, logits, logits_stride, false, stream);
}

idx_status indexer_prefill_logits_mxfp4(const uint8_t* q, const uint8_t* kv_pages, const float* weights,
                                        const int32_t* block_table, int32_t max_pages, const int32_t* cu_q,
                                        int32_t requests, int32_t tokens, const int32_t* row_lens,
                                        int32_t num_pages, float* logits, int64_t logits_stride, void* stream) {
  return prefill_call(q, kv_pages, nullptr, weights, block_table, max_pages, cu_q, requests, tokens, row_lens,
                      num_pages, logits, logits_stride, true, stream);
}

idx_status sparse_to_logical(const int32_t* indices, int32_t k, const int32_t* table, int32_t kb, int32_t rows,
                             int32_t* out, void* stream) {
  const pmqa::LaunchEvents ev = take_events();
  if (!indices || !table || !out) return IDX_EINVAL;
  if (rows <= 0 || k <= 0 || kb <= 0) return IDX_EINVAL;
  if (rows > IDX_MAX_ROWS || kb > pmqa::kMaxCandidateBlocks) return IDX_EUNSUPPORTED;
  if (!aligned(indices, 4) || !aligned(table, 4) || !aligned(out, 4)) return IDX_EALIGN;
  return from_hip(pmqa::launch_sparse_to_logical(indices, k, table, kb, rows, out,
                                                 static_cast<hipStream_t>(stream), ev));
}

idx_status sparse_topk(const float* scores, int64_t stride, const int32_t* hist, const int32_t* sparse_lens,
                       int32_t rows, int32_t k, int32_t key_dtype, const int32_t* table, int32_t kb,
                       int32_t* out, void* stream) {
  const pmqa::LaunchEvents ev = take_events();
  if (!scores || !sparse_lens || !table || !out) return IDX_EINVAL;
  if (rows <= 0 || stride <= 0 || kb <= 0 || k < 1 || k > IDX_CANDIDATE_CAPACITY) return IDX_EINVAL;
  if (key_dtype != IDX_KEY_FP32 && key_dtype != IDX_KEY_FP16) return IDX_EUNSUPPORTED;
  if (rows > IDX_MAX_ROWS || stride > 16384 || kb > pmqa::kMaxCandidateBlocks) return IDX_EUNSUPPORTED;
  if (!aligned(scores, 16) || (stride % 4) != 0 || !aligned(sparse_lens, 4) || !aligned(table, 4) ||
      !aligned(out, 4) || (hist && !aligned(hist, 8)))
    return IDX_EALIGN;
  pmqa::TopkArgs a;
  a.logits = scores;
  a.hist = hist;
  a.context_lens = sparse_lens;
  a.indices = out;
  a.workspace = nullptr;
  a.logits_stride = stride;
  a.rows = rows;
  a.k = k;
  a.key_dtype = key_dtype;
  a.logits_f16 = 0;
  return from_hip(pmqa::launch_sparse_topk(a, table, kb, static_cast<hipStream_t>(stream), ev));
}

idx_status hbm_gather_probe(const uint8_t* kv_pages, const float* k_scales, const int32_t* page_list,
                            int32_t n_pages, int32_t num_pages, uint32_t* sink, void* stream) {
  const pmqa::LaunchEvents ev = take_events();
  if (!kv_pages || !k_scales || !page_list || !sink || n_pages <= 0 || num_pages <= 0) return IDX_EINVAL;
  if (!aligned(kv_pages, 16) || !aligned(k_scales, 4) || !aligned(page_list, 4) || !aligned(sink, 4))
    return IDX_EALIGN;
  return from_hip(pmqa::launch_hbm_gather_probe(kv_pages, k_scales, page_list, n_pages, num_pages, sink,
                                                static_cast<hipStream_t>(stream), ev));
}

idx_status mfma_valu_probe(int32_t mode, int32_t waves_per_simd, int32_t iters, float* out, int64_t out_len,
                           void* stream) {
  const pmqa::LaunchEvents ev = take_events();
  if (!out || mode < 0 || mode > 2 || waves_per_simd < 1 || waves_per_simd > 8 || iters < 1 ||
      iters > (1 << 20))
    return IDX_EINVAL;
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
    return IDX_ELAUNCH;
  const int64_t workgroups = static_cast<int64_t>(cus) * waves_per_simd;  // 4 waves each: one per SIMD
  if (out_len < workgroups * 256) return IDX_EINVAL;
  if (!aligned(out, 4)) return IDX_EALIGN;
  return from_hip(pmqa::launch_mfma_valu_probe(mode, static_cast<int>(workgroups), iters, out,
                                               static_cast<hipStream_t>(stream), ev));
}

static idx_status read_probe(const void* src, size_t bytes, uint32_t* sink, bool nt, void* stream) {
  const pmqa::LaunchEvents ev = take_events();
  if (!src || !sink || bytes == 0) return IDX_EINVAL;
  if (!aligned(src, 16) || (bytes % 16) != 0 || !aligned(sink, 4)) return IDX_EALIGN;
  return from_hip(pmqa::launch_hbm_read_probe(src, bytes, sink, nt, static_cast<hipStream_t>(stream), ev));
}

idx_status hbm_read_probe(const void* src, size_t bytes, uint32_t* sink, void* stream) {
  return read_probe(src, bytes, sink, false, stream);
}

idx_status hbm_read_probe_nt(const void* src, size_t bytes, uint32_t* sink, void* stream) {
  return read_probe(src, bytes, sink, true, stream);
}

}  // extern "C"
