/*
 * paged_mqa_indexer.h -- C ABI of the MI355X (gfx950) paged MQA indexer.
 *
 * The decode-time sparse-attention indexer: for every query row it scores all
 * live keys of its request through a paged FP8 K cache, emits a 1024-bin
 * coarse histogram of those scores while they are still in registers, and a
 * selector then picks the top-k columns of each row from that histogram's
 * threshold bin plus a radix refine on the remaining key bits.
 *
 * Sources:
 *   [P1] DeepGEMM PR #94, "[SM100] Paged MQA logits: fused coarse score
 *        histogram for LiteTopK decode": "Motivation"; "What this adds"
 *        (histogram argument and contract, bin regimes, per-token slots
 *        flushed with packed 64-bit atomics, token Q tile); SGLang commit
 *        "Replace the CuTe DSL selector with a JIT CUDA selector; add verify"
 *        (exact top-2048 selector from the histogram, fallback, ties).
 *   [P2] SGLang PR #38944, "[DSV4.1] Enable the two-level candidate
 *        indexer": the sparse paged logits path, amax8_varlen and
 *        sort_candidate_blocks; the SM90 prefill commit (ragged extend
 *        batches scored per request; block-scaled E2M1 index-K).
 *   [P3] vLLM PR #52696, "[Performance][MLA] Use FP16 logits for sparse
 *        indexer": "Summary" and commits (selection on FP16 score keys,
 *        refining only the remaining key bits; FP16 logits; the MXFP4
 *        indexer cache's packed 68-byte layout).
 *
 * Conventions for every entry point:
 *   - Pointers marked (device) are device memory on the current HIP device;
 *     the library never dereferences them on the host and never copies them.
 *   - `stream` is a hipStream_t (NULL = the legacy default stream).  Every
 *     call only enqueues kernels on it and returns; nothing is synchronised,
 *     allocated or freed, and no pointer is kept after the call returns, so
 *     the calls can be captured into a HIP graph.
 *   - Arguments are checked on the host before anything is launched; a
 *     failed check returns its status and enqueues nothing.  Device-resident
 *     values (lengths, page ids, histogram counts) cannot be checked on the
 *     host; the kernels clamp them so that no access leaves its buffer, and
 *     the results for out-of-contract values are unspecified.
 *   - The buffers belong to the caller throughout.
 */
#ifndef PAGED_MQA_INDEXER_H
#define PAGED_MQA_INDEXER_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Status codes. */
typedef enum {
  IDX_OK = 0,
  IDX_EINVAL = 1,       /* null required pointer, non-positive size, k out of range   */
  IDX_EUNSUPPORTED = 2, /* next_n outside 1..4, unknown key dtype, size above limits  */
  IDX_EALIGN = 3,       /* a pointer or stride misses its required alignment          */
  IDX_ELAUNCH = 4,      /* the HIP runtime rejected a launch or the device query      */
  IDX_EWORKSPACE = 5,   /* workspace smaller than topk_workspace_bytes()              */
  IDX_ESCRATCH = 6      /* topk_rows_noalloc: more rows than its fixed scratch holds  */
} idx_status;

/* Score key used by topk_rows.  FP32: the float32 score itself.  FP16: the
 * score rounded to IEEE binary16 (round to nearest even), so scores that round
 * to the same FP16 value tie ([P3] Summary). */
typedef enum { IDX_KEY_FP32 = 0, IDX_KEY_FP16 = 1 } idx_key_dtype;

/* Fixed shape of the method ([P1] "What this adds": H = 32, D = 128). */
#define IDX_NUM_HEADS 32
#define IDX_HEAD_DIM 128
#define IDX_PAGE_TOKENS 64
#define IDX_NUM_BINS 1024
#define IDX_CANDIDATE_CAPACITY 8192 /* [P1] SGLang commit: candidate_capacity */
#define IDX_MAX_REQUESTS 4096
#define IDX_MAX_ROWS 65535
/* topk_rows: rows of more than 16384 scores go through the chunked path,
 * whose strides are limited to 2^23 (8x the longest context on the pages). */
#define IDX_TOPK_MAX_STRIDE (1 << 23)
/* topk_rows_noalloc: rows its fixed scratch holds (chunked path only). */
#define IDX_NOALLOC_MAX_ROWS 128

/*
 * indexer_logits -- paged MQA logits with an optional fused coarse histogram.
 * [P1] "Motivation", "What this adds".
 *
 * Rows: r = b * next_n + j for request b in [0, B) and token j in [0, next_n).
 * Row r sees keys s in [0, len_r), len_r = context_lens[r] (speculative verify:
 * token j of a request usually sees L + j keys).  Key s of request b lives in
 * physical page block_table[b * max_pages + s / 64], slot s % 64.
 *
 *   logits[r * logits_stride + s] =
 *       k_scales[page][slot] * sum_h weights[r*32 + h] * max(0, sum_d Q[r,h,d] * K[page,slot,d])
 *
 * with Q and K decoded from OCP FP8 E4M3FN, products summed in fp32.  Columns
 * s >= len_r are not written (padding stays as the caller left it).  All
 * next_n rows of a request are computed from one read of its K pages.
 *
 * q            (device) uint8 [B*next_n][32][128], E4M3FN codes, 16-B aligned
 * kv_pages     (device) uint8 [num_pages][64][128], E4M3FN codes, 16-B aligned
 * k_scales     (device) float [num_pages][64], one scale per token, 4-B aligned
 * weights      (device) float [B*next_n][32], 16-B aligned
 * block_table  (device) int32 [B][max_pages]; ids in [0, num_pages)
 * context_lens (device) int32 [B*next_n]; 0 <= len_r <= min(max_pages*64, logits_stride)
 * B            1 .. IDX_MAX_REQUESTS; next_n 1..4; B*next_n <= IDX_MAX_ROWS;
 *              B*max_pages < 2^31
 * logits       (device) float [B*next_n][logits_stride], 16-B aligned,
 *              logits_stride > 0 and a multiple of 4
 * hist         (device) int32 [B*next_n][1024] or NULL.  When given, every
 *              live (s < len_r), non-NaN score adds 1 to bin(score) of its row;
 *              counts accumulate across calls, so the caller zeroes the buffer
 *              before the first call and resets it after consuming it.  Must
 *              be 8-B aligned (pairs of bins are added with 64-bit atomics,
 *              exact while every count stays below 2^31).  With hist == NULL
 *              no histogram work runs, and the logits are bit-identical either way.
 *
 * bin(x), [P1] "What this adds" (descending, bin 0 = largest): h = fp16_RN(x),
 *   a = |h|; m = (bits(h) & 0x7FFF) >> 6 if a < 16 (exponent + 4 mantissa bits),
 *   m = 288 + floor(a) if 16 <= a < 223 (unit bins, same for both signs),
 *   m = 511 if a >= 223 or inf (saturating); bin = 511 - m for a clear sign bit,
 *   512 + m for a set one.
 */
idx_status indexer_logits(const uint8_t* q, const uint8_t* kv_pages,
                          const float* k_scales, const float* weights,
                          const int32_t* block_table, const int32_t* context_lens,
                          int32_t B, int32_t next_n, int32_t num_pages,
                          int32_t max_pages, float* logits, int64_t logits_stride,
                          int32_t* hist, void* stream);

/*
 * topk_workspace_bytes -- size of the scratch buffer topk_rows needs for
 * `rows` rows (host-only query, no device work): one 140,544-byte record per
 * row -- two 8-byte counter pairs and the threshold bin (padded to 256
 * bytes), a 1 KiB histogram of the threshold bin's sub-bins, a 4 KiB
 * histogram, 128 KiB of candidates and 4 KiB of per-workgroup counts --
 * whatever the stride and k, so a row's record sits at the same place for
 * every call.
 * Rows of at most 16384 scores (logits_stride <= 16384) leave the workspace
 * untouched.  Returns 0 for rows <= 0, logits_stride <= 0 or k <= 0.
 */
size_t topk_workspace_bytes(int32_t rows, int64_t logits_stride, int32_t k);

/*
 * topk_rows -- exact per-row top-k of a score matrix.  [P1] SGLang commit
 * (histogram-driven exact selector, fallback, lower index wins ties), [P1]
 * "Motivation" (the selector's own first pass builds the histogram when the
 * producer did not), [P3] Summary (FP16 keys, refining the remaining bits).
 *
 * For row r, the selectable columns are s < context_lens[r] whose score is not
 * NaN.  The selected set is the first min(k, n_selectable) of them in the
 * order (key descending, column ascending), where key is the score as FP32 or
 * its fp16_RN value (key_dtype).  indices[r*k + 0 .. n-1] receive the set in
 * unspecified order; indices[r*k + n .. k-1] receive -1.
 *
 * With hist != NULL (the producer's histogram of exactly these scores), the
 * threshold bin is read from it: columns in higher bins are emitted directly,
 * columns of the threshold bin become candidates (at most 16384 per row) that
 * a radix select on the remaining key bits ranks.  The real counts found in
 * the scores are checked against the threshold; a stale histogram, or a
 * threshold bin with more than 16384 scores, makes that row fall back to an
 * exact whole-row radix select -- the result is exact in every case.  With
 * hist == NULL the histogram is first built from the scores.
 *
 * logits      (device) float [rows][logits_stride], 16-B aligned, stride % 4 == 0,
 *             logits_stride <= IDX_TOPK_MAX_STRIDE
 * hist        (device) int32 [rows][1024] or NULL; read only
 * context_lens(device) int32 [rows]; 0 <= len_r <= logits_stride
 * rows        1 .. IDX_MAX_ROWS;  k in 1 .. IDX_CANDIDATE_CAPACITY
 * key_dtype   IDX_KEY_FP32 or IDX_KEY_FP16
 * indices     (device) int32 [rows][k]
 * workspace   (device) scratch of at least topk_workspace_bytes(rows, ...) bytes,
 *             256-B aligned, owned by the caller; it needs no initialisation.
 *             Results are exact whatever it holds: the collect workgroups
 *             store their counts beside the atomic counters they add to, and
 *             a row whose counters did not start at zero (or whose workspace
 *             histogram, hist == NULL, did not) is selected from scratch.
 *             Every call leaves its rows' counters and built histograms zero
 *             (also when a captured graph replays it), so only the first call
 *             on a fresh or overwritten workspace takes that slower path.
 *             Calls that share a workspace must be ordered on one stream.
 */
idx_status topk_rows(const float* logits, int64_t logits_stride,
                     const int32_t* hist, const int32_t* context_lens,
                     int32_t rows, int32_t k, int32_t key_dtype, int32_t* indices,
                     void* workspace, size_t workspace_bytes, void* stream);

/*
 * topk_rows_noalloc -- topk_rows without a workspace, for callers that cannot
 * allocate device memory (code under HIP graph capture, serving loops and
 * harnesses that forbid hipMalloc).  The chunked path's per-row records
 * (rows of more than 16384 scores) live in a fixed array of the library,
 * IDX_NOALLOC_MAX_ROWS records = 17,989,632 bytes per GPU, held from the
 * time the library is loaded until the process ends; its device address is
 * looked up once per GPU, on the first call there.  The call allocates and
 * frees nothing.  Every call on a GPU shares that GPU's array: calls that
 * overlap on one GPU (other streams, other host threads) race and must not
 * be issued; calls ordered on one stream are fine.  Nothing in the array has
 * to start at zero (see topk_rows' workspace).  Arguments as for topk_rows;
 * rows > IDX_NOALLOC_MAX_ROWS with logits_stride > 16384 returns
 * IDX_ESCRATCH before anything is launched.
 */
idx_status topk_rows_noalloc(const float* logits, int64_t logits_stride,
                             const int32_t* hist, const int32_t* context_lens,
                             int32_t rows, int32_t k, int32_t key_dtype, int32_t* indices,
                             void* stream);

/*
 * score_histogram -- the selector's own first pass ([P1] "Motivation": the
 * pass that builds the coarse histogram from the scores when the producer did
 * not): adds bin(x) of every live (s < len_r), non-NaN score of each row to
 * hist[r][*], with the same bin function as indexer_logits.
 *
 * scores       (device) float [rows][stride], 16-B aligned, stride % 4 == 0
 * context_lens (device) int32 [rows]; 0 <= len_r <= stride
 * rows         1 .. IDX_MAX_ROWS
 * hist         (device) int32 [rows][1024], 8-B aligned; accumulated (+=)
 */
idx_status score_histogram(const float* scores, int64_t stride, const int32_t* context_lens,
                           int32_t rows, int32_t* hist, void* stream);

/*
 * indexer_logits_f16 -- indexer_logits writing each score as the IEEE binary16
 * value it rounds to (round to nearest even; magnitudes at or above 65520
 * become infinities): [P3] "Summary" (FP16 logits for the sparse indexer).
 * Everything else -- arguments, rows, lengths, histogram -- is as for
 * indexer_logits; the histogram bins the same FP16 values (bin() already
 * rounds to FP16), so it is identical to indexer_logits' histogram.
 *
 * logits        (device) uint16 [B*next_n][logits_stride], binary16 bits,
 *               16-B aligned, logits_stride > 0 and a multiple of 8
 */
idx_status indexer_logits_f16(const uint8_t* q, const uint8_t* kv_pages,
                              const float* k_scales, const float* weights,
                              const int32_t* block_table, const int32_t* context_lens,
                              int32_t B, int32_t next_n, int32_t num_pages,
                              int32_t max_pages, uint16_t* logits, int64_t logits_stride,
                              int32_t* hist, void* stream);

/*
 * indexer_logits_mxfp4 -- indexer_logits with MXFP4 keys: block-scaled E2M1
 * index-K ([P2] SGLang PR #38944, the SM90 prefill commit) in the packed
 * 68-byte token layout of the MXFP4 indexer cache ([P3] vLLM PR #52696),
 * the fp8 x fp4 variant that [P1] "What this adds" names.  Per token: bytes 0..63 hold the 128 E2M1
 * codes (dimension 2i in the low nibble of byte i, 2i+1 in the high nibble),
 * bytes 64..67 the E8M0 scales of dimensions 0-31, 32-63, 64-95, 96-127.
 * The key is code value * 2^(scale - 127); there is no per-token fp32 scale:
 *   logit[r, s] = sum_h w[r, h] * ReLU(q[r, h, :] . k_s).
 * Q stays E4M3.  The histogram (optional) is the same as for indexer_logits
 * ([P1] supports it for FP8 only; here the same fused code serves both).
 *
 * kv_pages      (device) uint8 [num_pages][64][68], 16-B aligned
 * logits        (device) float [B*next_n][logits_stride], stride % 4 == 0
 * other arguments as for indexer_logits (no k_scales)
 */
idx_status indexer_logits_mxfp4(const uint8_t* q, const uint8_t* kv_pages,
                                const float* weights, const int32_t* block_table,
                                const int32_t* context_lens, int32_t B, int32_t next_n,
                                int32_t num_pages, int32_t max_pages, float* logits,
                                int64_t logits_stride, int32_t* hist, void* stream);

/*
 * Two-level candidate indexer ([P2] SGLang PR #38944: the candidate-source
 * layer publishes an ascending table of 8-token logical blocks per query
 * row; the layers after it score those blocks only -- paged sparse MQA
 * logits -- and select inside that sparse row).  Block b holds keys
 * 8b .. 8b+7 of the row; only keys below the row's length are live.
 *
 * block_amax8 -- [P2] amax8_varlen: out[r][j] = maximum of the live scores
 * 8j .. 8j+7 of row r (NaN ignored; NaN if all are NaN) for j < ceil(len_r/8),
 * except the newest block, written as +inf so it is always selected; nothing
 * is written at or past ceil(len_r / 8).  The block top-k is topk_rows over
 * these rows with lengths ceil(len_r / 8), which the call writes to
 * block_lens when it is not NULL.  With hist != NULL the maxima are also
 * added to the row's 1024-bin coarse histogram ([P1] contract: zero at
 * entry, accumulating), so that top-k needs no first pass.
 *
 * scores       (device) float [rows][stride], 16-B aligned, stride % 4 == 0
 * context_lens (device) int32 [rows]; clamped to [0, stride]
 * out          (device) float [rows][out_stride], out_stride >= ceil(stride/8)
 * hist         (device) int32 [rows][1024], 8-B aligned, or NULL
 * block_lens   (device) int32 [rows] (overwritten), 4-B aligned, or NULL
 */
idx_status block_amax8(const float* scores, int64_t stride, const int32_t* context_lens,
                       int32_t rows, float* out, int64_t out_stride, int32_t* hist,
                       int32_t* block_lens, void* stream);

/*
 * sort_candidate_blocks -- [P2] sort_candidate_blocks: the selected block ids
 * of each row (any order, -1 padded; ids outside [0, ceil(len/8)) and
 * repeats are ignored) become the ascending table padded with INT32_MAX,
 * and the same blocks as pool slots / 8 through the row's page table:
 * (page * 64 + (8b) % 64) / 8 with page = block_table[row / next_n][8b / 64].
 * Rows with at most kb blocks get the identity table 0 .. ceil(len/8)-1.
 * sparse_lens[r] receives the live keys of the listed blocks (the sparse row
 * length).  A counting sort over a 16 KiB bitmap: rows hold at most 2^17
 * blocks, so max_len (an upper bound of every length) is at most 2^20.
 * `table` may be `blocks` itself (every read precedes the first write).
 *
 * blocks       (device) int32 [rows][kb]
 * block_table  (device) int32 [rows / next_n][max_pages]
 * table, slots (device) int32 [rows][kb];  sparse_lens (device) int32 [rows]
 */
idx_status sort_candidate_blocks(const int32_t* blocks, int32_t kb, const int32_t* context_lens,
                                 int32_t rows, int64_t max_len, const int32_t* block_table,
                                 int32_t max_pages, int32_t next_n, int32_t* table, int32_t* slots,
                                 int32_t* sparse_lens, void* stream);

/*
 * indexer_sparse_logits -- [P2] paged sparse MQA logits: for row r and table
 * entry i (block b = table[r][i] != INT32_MAX) and t in 0..7 with key
 * 8b + t < len_r, logits[r][8i + t] = the indexer logit of that key
 * (indexer_logits' formula, FP8 K), its K row read at pool slot
 * 8 * slots[r][i] + t of kv_pages / k_scales.  Other columns are not
 * written.  Each row has its own table, Q and weights (next_n rows of a
 * request are independent rows here).
 *
 * q, kv_pages, k_scales, weights as for indexer_logits (per row)
 * table, slots  (device) int32 [rows][kb] from sort_candidate_blocks
 * logits        (device) float [rows][logits_stride], logits_stride >= 8 kb
 */
idx_status indexer_sparse_logits(const uint8_t* q, const uint8_t* kv_pages, const float* k_scales,
                                 const float* weights, const int32_t* table, const int32_t* slots,
                                 int32_t kb, const int32_t* context_lens, int32_t rows,
                                 int32_t num_pages, float* logits, int64_t logits_stride,
                                 void* stream);

/*
 * indexer_sparse_logits_mxfp4 -- indexer_sparse_logits over packed MXFP4
 * pages (the fp8 x fp4 sparse logits [P2] routes the paged fp4 decode path
 * through; the keys as in indexer_logits_mxfp4).  kv_pages uint8
 * [num_pages][64][68], no k_scales; other arguments as above.
 */
idx_status indexer_sparse_logits_mxfp4(const uint8_t* q, const uint8_t* kv_pages,
                                       const float* weights, const int32_t* table,
                                       const int32_t* slots, int32_t kb,
                                       const int32_t* context_lens, int32_t rows,
                                       int32_t num_pages, float* logits,
                                       int64_t logits_stride, void* stream);

/*
 * indexer_prefill_logits -- [P2] the SM90 FP8 prefill commit: indexer
 * logits of a ragged prefill (extend) batch.  Request r owns rows
 * cu_q[r] .. cu_q[r+1]-1 (cu_q ascending, cu_q[0] = 0, cu_q[requests] =
 * tokens; a request may own none).  Row t of request r scores the keys
 * s < row_lens[t] of r through block_table[r]:
 *   logits[t][s] = k_scales[page][slot] * sum_h w[t][h] * ReLU(q[t][h] . k_s)
 * with indexer_logits' formula, FP32 accumulation and output.  For an extend
 * chunk of n rows appended to a context of L keys (prefix included), causal
 * visibility is row_lens = L - n + 1 + i for its row i (the decode path's
 * next_n convention, so a batch of next_n-row requests is a decode call).
 * Columns >= row_lens[t] are not written; rows feed topk_rows with
 * context_lens = row_lens.
 *
 * q            (device) uint8 [tokens][32][128] E4M3FN, 16-byte aligned
 * kv_pages     (device) uint8 [num_pages][64][128] E4M3FN, 16-byte aligned
 * k_scales     (device) float [num_pages][64]
 * weights      (device) float [tokens][32], 16-byte aligned
 * block_table  (device) int32 [requests][max_pages]
 * cu_q         (device) int32 [requests + 1]
 * row_lens     (device) int32 [tokens], clamped to [0, min(64 max_pages,
 *              logits_stride)]
 * logits       (device) float [tokens][logits_stride], 16-byte aligned,
 *              logits_stride a multiple of 4
 * requests     1 .. IDX_MAX_REQUESTS;  tokens 1 .. IDX_MAX_ROWS
 * Errors: IDX_EINVAL (NULL pointer, non-positive size), IDX_EUNSUPPORTED
 * (limits above), IDX_EALIGN (alignment, stride), IDX_ELAUNCH.
 */
idx_status indexer_prefill_logits(const uint8_t* q, const uint8_t* kv_pages, const float* k_scales,
                                  const float* weights, const int32_t* block_table,
                                  int32_t max_pages, const int32_t* cu_q, int32_t requests,
                                  int32_t tokens, const int32_t* row_lens, int32_t num_pages,
                                  float* logits, int64_t logits_stride, void* stream);

/*
 * indexer_prefill_logits_mxfp4 -- indexer_prefill_logits over packed MXFP4
 * pages (the block-scaled E2M1 index-K of [P2]'s prefill commit, consumed
 * by the fp8 x fp4 MFMA directly instead of being unpacked to E4M3 first;
 * the keys as in indexer_logits_mxfp4).  kv_pages uint8 [num_pages][64][68],
 * no k_scales; other arguments as above.
 */
idx_status indexer_prefill_logits_mxfp4(const uint8_t* q, const uint8_t* kv_pages,
                                        const float* weights, const int32_t* block_table,
                                        int32_t max_pages, const int32_t* cu_q,
                                        int32_t requests, int32_t tokens,
                                        const int32_t* row_lens, int32_t num_pages,
                                        float* logits, int64_t logits_stride, void* stream);

/*
 * sparse_to_logical -- the selection inside a sparse row as logical key
 * positions: out[r][j] = 8 * table[r][c / 8] + c % 8 for c = indices[r][j];
 * -1 (and columns past the table or on padding) give -1.
 *
 * indices, out  (device) int32 [rows][k];  table (device) int32 [rows][kb]
 */
idx_status sparse_to_logical(const int32_t* indices, int32_t k, const int32_t* table,
                             int32_t kb, int32_t rows, int32_t* out, void* stream);

/*
 * sparse_topk -- [P2] the top-k inside the sparse rows and the map back to
 * logical keys in one call: topk_rows over the sparse logits (rows of at most
 * 16384 scores, lengths sparse_lens, float32, FP32 or FP16 keys, hist
 * optional as for topk_rows), each selected column c written as
 * 8 * table[r][c / 8] + c % 8 -- what sparse_to_logical does to topk_rows'
 * output, without its launch -- and -1 for padding, for columns past the
 * table and for table padding (INT32_MAX).  No workspace: rows this short
 * are selected by one workgroup each.
 *
 * scores       (device) float [rows][stride], 16-B aligned, stride % 4 == 0,
 *              stride <= 16384 (else IDX_EUNSUPPORTED)
 * sparse_lens  (device) int32 [rows]
 * table        (device) int32 [rows][kb], kb <= 131072 blocks
 * out          (device) int32 [rows][k], overwritten
 */
idx_status sparse_topk(const float* scores, int64_t stride, const int32_t* hist, const int32_t* sparse_lens,
                       int32_t rows, int32_t k, int32_t key_dtype, const int32_t* table, int32_t kb,
                       int32_t* out, void* stream);

/*
 * topk_rows_f16 -- topk_rows over binary16 scores ([P3] "Summary": selection
 * on FP16 logits).  The key is the FP16 value itself (scores that are the
 * same half tie, and the lower column wins), the same order as topk_rows
 * with IDX_KEY_FP16 on the float32 scores these halves round from.
 *
 * logits        (device) uint16 [rows][logits_stride], binary16 bits, 16-B
 *               aligned, logits_stride a multiple of 8
 * other arguments as for topk_rows; the workspace size is
 * topk_workspace_bytes(rows, logits_stride, k)
 */
idx_status topk_rows_f16(const uint16_t* logits, int64_t logits_stride,
                         const int32_t* hist, const int32_t* context_lens,
                         int32_t rows, int32_t k, int32_t* indices,
                         void* workspace, size_t workspace_bytes, void* stream);

/*
 * indexer_time_next_call -- measurement aid.  Arms the calling host thread:
 * its next call of this library records start_event when that call's first
 * kernel begins and stop_event when its last kernel ends (the dispatches
 * record them themselves, hipExtLaunchKernel), so the elapsed time between
 * them is the call's device time without the stream's dispatch gaps around
 * it.  Either event may be NULL; events are hipEvent_t created by the
 * caller.  The next call disarms it whatever its outcome (a call that fails
 * a check records nothing).  Not meant for graph capture.
 */
idx_status indexer_time_next_call(void* start_event, void* stop_event);

/* Human-readable name of a status code (static string). */
const char* indexer_status_str(int32_t status);

/*
 * hbm_read_probe -- measurement aid, not part of the method: streams `bytes`
 * bytes (a multiple of 16) from `src` (device, 16-B aligned) with ordinary
 * 16-B vector loads (they allocate in the caches, so a large buffer read this
 * way is a cache sweep) and writes one checksum word to *sink (device).
 * Errors: IDX_EINVAL for a null pointer or bytes == 0, IDX_EALIGN for a
 * misaligned src/sink or bytes not a multiple of 16.
 */
idx_status hbm_read_probe(const void* src, size_t bytes, uint32_t* sink, void* stream);

/*
 * hbm_read_probe_nt -- as hbm_read_probe with non-temporal loads, the cache
 * policy of the logits kernel's page loads: its duration is the practical
 * contiguous HBM read ceiling that kernel is compared with.  Same arguments
 * and errors.
 */
idx_status hbm_read_probe_nt(const void* src, size_t bytes, uint32_t* sink, void* stream);

/*
 * hbm_gather_probe -- measurement aid, not part of the method: reads the
 * FP8 K pages listed in page_list (n_pages ids into kv_pages [num_pages][64]
 * [128] and k_scales [num_pages][64]; ids are clamped into [0, num_pages))
 * the way a paged K stream must be read -- page ids first, then whole-line
 * 16-byte loads of each page and its scales -- with no arithmetic, and writes
 * one checksum word to *sink.  Over the pages a logits call reads (each
 * request's block-table row up to its last live page), its duration is the
 * practical ceiling for that call's K stream.
 */
idx_status hbm_gather_probe(const uint8_t* kv_pages, const float* k_scales, const int32_t* page_list,
                            int32_t n_pages, int32_t num_pages, uint32_t* sink, void* stream);

/*
 * mfma_valu_probe -- measurement aid, not part of the method: how far a
 * SIMD's matrix and vector pipes overlap.  Launches waves_per_simd (1..8)
 * 256-thread workgroups per CU (one wave per SIMD each); every wave runs
 * `iters` (1..2^20) rounds of four independent fp8 16x16x128 MFMAs (mode 0),
 * 32 independent fp32 FMAs (mode 1) or both, interleaved and independent
 * (mode 2) -- eight FMAs per MFMA, the logits epilogue's ratio -- and stores
 * one float per thread to out (device, 4-B aligned, out_len >= CUs *
 * waves_per_simd * 256 floats).  IDX_EINVAL for a mode, count or out_len out
 * of range, before anything is launched.
 */
idx_status mfma_valu_probe(int32_t mode, int32_t waves_per_simd, int32_t iters, float* out, int64_t out_len,
                           void* stream);

#ifdef __cplusplus
}
#endif

#endif /* PAGED_MQA_INDEXER_H */
