"""Python binding of the MI355X paged MQA indexer C ABI (include/paged_mqa_indexer.h).

Argument marshalling only: tensors are checked for dtype, device, shape and
layout, their device pointers and the current HIP stream are handed to the C
entry points of ``libpaged_mqa_indexer.so``, and a non-zero status raises
``IndexerError``.  Every step of the computation runs in the library's HIP
kernels; there is no fallback path.  PyTorch only supplies device memory and
streams.

Entry points (same names as the C ABI):
  indexer_logits(q, kv_pages, k_scales, weights, block_table, context_lens,
                 next_n, logits, hist=None, events=None)        float32 logits
  indexer_logits_f16(... same ..., logits, hist=None, events=None) float16 logits
  indexer_logits_mxfp4(q, kv_pages, weights, block_table, context_lens, next_n,
                       logits, hist=None, events=None)  packed MXFP4 K, float32 logits
  topk_workspace_bytes(rows, logits_stride, k)
  topk_rows(logits, hist, context_lens, k, key_dtype, indices, workspace=None,
            events=None)                                          float32 scores
  topk_rows_f16(logits, hist, context_lens, k, indices, workspace=None,
                events=None)                                      float16 scores
  topk_rows_noalloc(logits, hist, context_lens, k, key_dtype, indices,
                    events=None)          float32 scores, the library's fixed scratch
  score_histogram(scores, context_lens, hist)
  block_amax8(scores, context_lens, out)                       two-level candidate indexer:
  sort_candidate_blocks(blocks, context_lens, max_len, block_table, next_n,
                        table, slots, sparse_lens)
  indexer_sparse_logits(q, kv_pages, k_scales, weights, table, slots,
                        context_lens, logits)
  sparse_to_logical(indices, table, out)
  sparse_topk(scores, hist, sparse_lens, k, key_dtype, table, out)
  indexer_status_str(status)
  indexer_time_next_call(start, stop)
  hbm_read_probe(src, sink, events=None)
  hbm_read_probe_nt(src, sink, events=None)
  hbm_gather_probe(kv_pages, k_scales, page_list, sink, events=None)
  mfma_valu_probe(mode, waves_per_simd, iters, out, events=None)
With ``events=(start, stop)`` (torch.cuda.Event with timing enabled, either
may be None) the call is preceded by indexer_time_next_call, so its own
kernel dispatches record the events: start when its first kernel begins,
stop when its last kernel ends.
"""

from __future__ import annotations

import ctypes
import os

import torch

__all__ = [
    "IndexerError", "KEY_FP32", "KEY_FP16", "NUM_BINS", "CANDIDATE_CAPACITY",
    "EXPORTED_SYMBOLS", "load_library", "library_path", "indexer_logits", "indexer_logits_f16",
    "indexer_logits_mxfp4", "block_amax8", "sort_candidate_blocks", "indexer_sparse_logits",
    "indexer_sparse_logits_mxfp4", "indexer_prefill_logits", "indexer_prefill_logits_mxfp4",
    "sparse_to_logical", "sparse_topk",
    "topk_workspace_bytes", "topk_rows", "topk_rows_f16", "topk_rows_noalloc", "score_histogram",
    "indexer_status_str", "indexer_time_next_call", "hbm_read_probe", "hbm_read_probe_nt",
    "hbm_gather_probe", "mfma_valu_probe",
]

KEY_FP32 = 0
KEY_FP16 = 1
NUM_BINS = 1024
CANDIDATE_CAPACITY = 8192
HEADS = 32
HEAD_DIM = 128
PAGE_TOKENS = 64
MXFP4_TOKEN_BYTES = 68

EXPORTED_SYMBOLS = ("indexer_logits", "indexer_logits_f16", "indexer_logits_mxfp4", "block_amax8",
                    "sort_candidate_blocks", "indexer_sparse_logits", "indexer_sparse_logits_mxfp4",
                    "indexer_prefill_logits", "indexer_prefill_logits_mxfp4", "sparse_to_logical", "sparse_topk",
                    "topk_workspace_bytes", "topk_rows", "topk_rows_noalloc",
                    "topk_rows_f16", "score_histogram", "indexer_status_str",
                    "indexer_time_next_call", "hbm_read_probe", "hbm_read_probe_nt", "hbm_gather_probe",
                    "mfma_valu_probe")

_PKG_DIR = os.path.dirname(os.path.abspath(__file__))
_LIB_NAME = "libpaged_mqa_indexer.so"
_lib = None


class IndexerError(RuntimeError):
    """A C entry point returned a non-zero idx_status."""

    def __init__(self, func: str, status: int, msg: str):
        super().__init__(f"{func} failed: {msg} (status {status})")
        self.status = status


def library_path() -> str:
    return os.environ.get("PMQA_INDEXER_LIB", os.path.join(_PKG_DIR, _LIB_NAME))


def load_library() -> ctypes.CDLL:
    """Load the HIP library (once).  Raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    path = library_path()
    if not os.path.exists(path):
        raise RuntimeError(
            f"HIP library {path} is missing: build it with "
            "`python -m paged_mqa_logits_indexer_amd.build` (or __graft_entry__.build())")
    lib = ctypes.CDLL(path)
    vp, i32, i64, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
    lib.indexer_logits.argtypes = [vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, vp, i64, vp, vp]
    lib.indexer_logits.restype = ctypes.c_int
    lib.topk_workspace_bytes.argtypes = [i32, i64, i32]
    lib.topk_workspace_bytes.restype = sz
    lib.topk_rows.argtypes = [vp, i64, vp, vp, i32, i32, i32, vp, vp, sz, vp]
    lib.topk_rows.restype = ctypes.c_int
    lib.score_histogram.argtypes = [vp, i64, vp, i32, vp, vp]
    lib.score_histogram.restype = ctypes.c_int
    lib.indexer_status_str.argtypes = [i32]
    lib.indexer_status_str.restype = ctypes.c_char_p
    lib.hbm_read_probe.argtypes = [vp, sz, vp, vp]
    lib.hbm_read_probe.restype = ctypes.c_int
    lib.hbm_read_probe_nt.argtypes = [vp, sz, vp, vp]
    lib.hbm_read_probe_nt.restype = ctypes.c_int
    lib.hbm_gather_probe.argtypes = [vp, vp, vp, i32, i32, vp, vp]
    lib.hbm_gather_probe.restype = ctypes.c_int
    lib.mfma_valu_probe.argtypes = [i32, i32, i32, vp, i64, vp]
    lib.mfma_valu_probe.restype = ctypes.c_int
    lib.indexer_logits_f16.argtypes = lib.indexer_logits.argtypes
    lib.indexer_logits_f16.restype = ctypes.c_int
    lib.indexer_logits_mxfp4.argtypes = [vp, vp, vp, vp, vp, i32, i32, i32, i32, vp, i64, vp, vp]
    lib.indexer_logits_mxfp4.restype = ctypes.c_int
    lib.block_amax8.argtypes = [vp, i64, vp, i32, vp, i64, vp, vp, vp]
    lib.block_amax8.restype = ctypes.c_int
    lib.sort_candidate_blocks.argtypes = [vp, i32, vp, i32, i64, vp, i32, i32, vp, vp, vp, vp]
    lib.sort_candidate_blocks.restype = ctypes.c_int
    lib.indexer_sparse_logits.argtypes = [vp, vp, vp, vp, vp, vp, i32, vp, i32, i32, vp, i64, vp]
    lib.indexer_sparse_logits.restype = ctypes.c_int
    lib.indexer_sparse_logits_mxfp4.argtypes = [vp, vp, vp, vp, vp, i32, vp, i32, i32, vp, i64, vp]
    lib.indexer_sparse_logits_mxfp4.restype = ctypes.c_int
    lib.indexer_prefill_logits.argtypes = [vp, vp, vp, vp, vp, i32, vp, i32, i32, vp, i32, vp, i64, vp]
    lib.indexer_prefill_logits.restype = ctypes.c_int
    lib.indexer_prefill_logits_mxfp4.argtypes = [vp, vp, vp, vp, i32, vp, i32, i32, vp, i32, vp, i64, vp]
    lib.indexer_prefill_logits_mxfp4.restype = ctypes.c_int
    lib.sparse_to_logical.argtypes = [vp, i32, vp, i32, i32, vp, vp]
    lib.sparse_topk.argtypes = [vp, i64, vp, vp, i32, i32, i32, vp, i32, vp, vp]
    lib.sparse_topk.restype = ctypes.c_int
    lib.sparse_to_logical.restype = ctypes.c_int
    lib.topk_rows_f16.argtypes = [vp, i64, vp, vp, i32, i32, vp, vp, sz, vp]
    lib.topk_rows_f16.restype = ctypes.c_int
    lib.topk_rows_noalloc.argtypes = [vp, i64, vp, vp, i32, i32, i32, vp, vp]
    lib.topk_rows_noalloc.restype = ctypes.c_int
    lib.indexer_time_next_call.argtypes = [vp, vp]
    lib.indexer_time_next_call.restype = ctypes.c_int
    _lib = lib
    return lib


def indexer_status_str(status: int) -> str:
    return load_library().indexer_status_str(int(status)).decode()


def _check(func: str, status: int) -> None:
    if status != 0:
        raise IndexerError(func, status, indexer_status_str(status))


def _stream_ptr(device: torch.device) -> int:
    return torch.cuda.current_stream(device).cuda_stream


def _need(t: torch.Tensor, name: str, dtype, device=None, ndim=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be a GPU tensor")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if ndim is not None and t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dims, got {tuple(t.shape)}")


def _ptr(t):
    return None if t is None else t.data_ptr()


def _event_handles(events, device: torch.device):
    """hipEvent_t handles of (start, stop), either of which may be None; a
    torch event that was never recorded has no HIP event yet, so it is
    recorded once to create it."""
    start, stop = events
    handles = []
    for ev in (start, stop):
        if ev is None:
            handles.append(None)
            continue
        if not isinstance(ev, torch.cuda.Event):
            raise TypeError("events must be a pair of torch.cuda.Event (or None)")
        if not ev.cuda_event:
            ev.record(torch.cuda.current_stream(device))
        handles.append(ev.cuda_event)
    return handles


def indexer_time_next_call(start, stop, device=None) -> None:
    """Arm this host thread's next library call to record (start, stop)
    from its own kernel dispatches (torch.cuda.Event, or None)."""
    dev = device if device is not None else torch.device("cuda", torch.cuda.current_device())
    h = _event_handles((start, stop), dev)
    _check("indexer_time_next_call", load_library().indexer_time_next_call(*h))


def _arm(events, device) -> None:
    if events is not None:
        indexer_time_next_call(events[0], events[1], device)


def _logits_call(name, dtype, q, kv_pages, k_scales, weights, block_table, context_lens, next_n,
                 logits, hist, events):
    """k_scales None: MXFP4 pages [P, 64, 68] (indexer_logits_mxfp4)."""
    dev = q.device
    mx = k_scales is None
    _need(q, "q", torch.uint8, dev, 3)
    _need(kv_pages, "kv_pages", torch.uint8, dev, 3)
    if not mx:
        _need(k_scales, "k_scales", torch.float32, dev, 2)
    _need(weights, "weights", torch.float32, dev, 2)
    _need(block_table, "block_table", torch.int32, dev, 2)
    _need(context_lens, "context_lens", torch.int32, dev, 1)
    _need(logits, "logits", dtype, dev, 2)
    B, max_pages = block_table.shape
    rows = B * next_n
    if tuple(q.shape) != (rows, HEADS, HEAD_DIM) or not q.is_contiguous():
        raise ValueError(f"q must be contiguous [{rows}, 32, 128]")
    P = kv_pages.shape[0]
    tok = MXFP4_TOKEN_BYTES if mx else HEAD_DIM
    if tuple(kv_pages.shape) != (P, PAGE_TOKENS, tok) or not kv_pages.is_contiguous():
        raise ValueError(f"kv_pages must be contiguous [P, 64, {tok}]")
    if not mx and (tuple(k_scales.shape) != (P, PAGE_TOKENS) or not k_scales.is_contiguous()):
        raise ValueError("k_scales must be contiguous [P, 64]")
    if tuple(weights.shape) != (rows, HEADS) or not weights.is_contiguous():
        raise ValueError(f"weights must be contiguous [{rows}, 32]")
    if not block_table.is_contiguous():
        raise ValueError("block_table must be contiguous")
    if tuple(context_lens.shape) != (rows,) or not context_lens.is_contiguous():
        raise ValueError(f"context_lens must be contiguous [{rows}]")
    if logits.shape[0] != rows or logits.stride(1) != 1:
        raise ValueError(f"logits must be [{rows}, stride] with unit column stride")
    if hist is not None:
        _need(hist, "hist", torch.int32, dev, 2)
        if tuple(hist.shape) != (rows, NUM_BINS) or not hist.is_contiguous():
            raise ValueError(f"hist must be contiguous [{rows}, 1024]")
    lib = load_library()
    with torch.cuda.device(dev):
        _arm(events, dev)
        tail = (_ptr(weights), _ptr(block_table), _ptr(context_lens), int(B), int(next_n), int(P),
                int(max_pages), _ptr(logits), int(logits.stride(0)), _ptr(hist), _stream_ptr(dev))
        if mx:
            st = getattr(lib, name)(_ptr(q), _ptr(kv_pages), *tail)
        else:
            st = getattr(lib, name)(_ptr(q), _ptr(kv_pages), _ptr(k_scales), *tail)
    _check(name, st)


def indexer_logits(q, kv_pages, k_scales, weights, block_table, context_lens, next_n,
                   logits, hist=None, events=None):
    """Paged MQA logits (and histogram) on the current stream of q's device.

    q [B*next_n, 32, 128] uint8 (e4m3fn codes); kv_pages [P, 64, 128] uint8;
    k_scales [P, 64] float32; weights [B*next_n, 32] float32;
    block_table [B, max_pages] int32; context_lens [B*next_n] int32;
    logits [B*next_n, stride] float32 with unit column stride;
    hist [B*next_n, 1024] int32 or None (accumulated into).
    """
    _logits_call("indexer_logits", torch.float32, q, kv_pages, k_scales, weights, block_table,
                 context_lens, next_n, logits, hist, events)


def indexer_logits_f16(q, kv_pages, k_scales, weights, block_table, context_lens, next_n,
                       logits, hist=None, events=None):
    """indexer_logits writing float16 logits [B*next_n, stride] (stride % 8 == 0)."""
    _logits_call("indexer_logits_f16", torch.float16, q, kv_pages, k_scales, weights, block_table,
                 context_lens, next_n, logits, hist, events)


def indexer_logits_mxfp4(q, kv_pages, weights, block_table, context_lens, next_n, logits,
                         hist=None, events=None):
    """indexer_logits with packed MXFP4 keys: kv_pages [P, 64, 68] uint8 (64 bytes
    of E2M1 codes, then four E8M0 block scales per token); float32 logits."""
    _logits_call("indexer_logits_mxfp4", torch.float32, q, kv_pages, None, weights, block_table,
                 context_lens, next_n, logits, hist, events)


def _rows2(t, name, dtype, dev, rows=None):
    _need(t, name, dtype, dev, 2)
    if not t.is_contiguous() or (rows is not None and t.shape[0] != rows):
        raise ValueError(f"{name} must be contiguous [{rows if rows is not None else 'rows'}, n]")


def block_amax8(scores, context_lens, out, hist=None, block_lens=None, events=None):
    """Block maxima of 8 scores per row (newest block +inf) into out [rows, >= ceil(stride/8)];
    with ``hist`` [rows, 1024] int32 their coarse histogram is accumulated too, and
    ``block_lens`` [rows] int32 receives each row's block count ceil(len / 8) (the
    lengths the block top-k takes)."""
    dev = scores.device
    _need(scores, "scores", torch.float32, dev, 2)
    rows = scores.shape[0]
    _rows2(out, "out", torch.float32, dev, rows)
    _need(context_lens, "context_lens", torch.int32, dev, 1)
    if scores.stride(1) != 1 or tuple(context_lens.shape) != (rows,):
        raise ValueError("scores must have unit column stride; context_lens [rows]")
    lib = load_library()
    with torch.cuda.device(dev):
        _arm(events, dev)
        if hist is not None:
            _rows2(hist, "hist", torch.int32, dev, rows)
        if block_lens is not None:
            _need(block_lens, "block_lens", torch.int32, dev, 1)
            if tuple(block_lens.shape) != (rows,) or not block_lens.is_contiguous():
                raise ValueError("block_lens must be a contiguous int32 [rows]")
        st = lib.block_amax8(_ptr(scores), int(scores.stride(0)), _ptr(context_lens), int(rows), _ptr(out),
                             int(out.stride(0)), _ptr(hist), _ptr(block_lens), _stream_ptr(dev))
    _check("block_amax8", st)


def sort_candidate_blocks(blocks, context_lens, max_len, block_table, next_n, table, slots, sparse_lens,
                          events=None):
    """Ascending INT32_MAX-padded block tables, pool slots / 8 and sparse row lengths."""
    dev = blocks.device
    _rows2(blocks, "blocks", torch.int32, dev)
    rows, kb = blocks.shape
    _rows2(table, "table", torch.int32, dev, rows)
    _rows2(slots, "slots", torch.int32, dev, rows)
    _rows2(block_table, "block_table", torch.int32, dev)
    _need(context_lens, "context_lens", torch.int32, dev, 1)
    _need(sparse_lens, "sparse_lens", torch.int32, dev, 1)
    if table.shape[1] != kb or slots.shape[1] != kb:
        raise ValueError("table and slots must be [rows, kb] like blocks")
    lib = load_library()
    with torch.cuda.device(dev):
        _arm(events, dev)
        st = lib.sort_candidate_blocks(_ptr(blocks), int(kb), _ptr(context_lens), int(rows), int(max_len),
                                       _ptr(block_table), int(block_table.shape[1]), int(next_n),
                                       _ptr(table), _ptr(slots), _ptr(sparse_lens), _stream_ptr(dev))
    _check("sort_candidate_blocks", st)


def indexer_sparse_logits(q, kv_pages, k_scales, weights, table, slots, context_lens, logits,
                          events=None):
    """Logits of the listed 8-token blocks only: logits [rows, >= 8 kb].  With
    k_scales None, kv_pages are packed MXFP4 tokens [P, 64, 68]
    (indexer_sparse_logits_mxfp4)."""
    dev = q.device
    mx = k_scales is None
    _need(q, "q", torch.uint8, dev, 3)
    _need(kv_pages, "kv_pages", torch.uint8, dev, 3)
    if kv_pages.shape[1:] != ((PAGE_TOKENS, MXFP4_TOKEN_BYTES) if mx else (PAGE_TOKENS, HEAD_DIM)):
        raise ValueError("kv_pages must be [P, 64, 68] (MXFP4) or [P, 64, 128] with k_scales")
    if not mx:
        _need(k_scales, "k_scales", torch.float32, dev, 2)
    _need(weights, "weights", torch.float32, dev, 2)
    _rows2(table, "table", torch.int32, dev)
    rows, kb = table.shape
    _rows2(slots, "slots", torch.int32, dev, rows)
    _need(context_lens, "context_lens", torch.int32, dev, 1)
    _need(logits, "logits", torch.float32, dev, 2)
    if tuple(q.shape) != (rows, HEADS, HEAD_DIM) or tuple(weights.shape) != (rows, HEADS):
        raise ValueError(f"q [{rows}, 32, 128] and weights [{rows}, 32] (one per row)")
    if logits.shape[0] != rows or logits.stride(1) != 1:
        raise ValueError("logits must be [rows, stride] with unit column stride")
    lib = load_library()
    with torch.cuda.device(dev):
        _arm(events, dev)
        tail = (_ptr(weights), _ptr(table), _ptr(slots), int(kb), _ptr(context_lens), int(rows),
                int(kv_pages.shape[0]), _ptr(logits), int(logits.stride(0)), _stream_ptr(dev))
        if mx:
            st = lib.indexer_sparse_logits_mxfp4(_ptr(q), _ptr(kv_pages), *tail)
        else:
            st = lib.indexer_sparse_logits(_ptr(q), _ptr(kv_pages), _ptr(k_scales), *tail)
    _check("indexer_sparse_logits_mxfp4" if mx else "indexer_sparse_logits", st)


def indexer_prefill_logits(q, kv_pages, k_scales, weights, block_table, cu_q, row_lens, logits,
                           events=None):
    """Ragged prefill logits: request r owns rows cu_q[r] .. cu_q[r+1]-1; row t
    scores keys [0, row_lens[t]) of its request into logits [tokens, stride].
    With k_scales None, kv_pages are packed MXFP4 tokens
    (indexer_prefill_logits_mxfp4)."""
    dev = q.device
    mx = k_scales is None
    _need(q, "q", torch.uint8, dev, 3)
    _need(kv_pages, "kv_pages", torch.uint8, dev, 3)
    if kv_pages.shape[1:] != ((PAGE_TOKENS, MXFP4_TOKEN_BYTES) if mx else (PAGE_TOKENS, HEAD_DIM)):
        raise ValueError("kv_pages must be [P, 64, 68] (MXFP4) or [P, 64, 128] with k_scales")
    if not mx:
        _need(k_scales, "k_scales", torch.float32, dev, 2)
    _need(weights, "weights", torch.float32, dev, 2)
    _rows2(block_table, "block_table", torch.int32, dev)
    _need(cu_q, "cu_q", torch.int32, dev, 1)
    _need(row_lens, "row_lens", torch.int32, dev, 1)
    _need(logits, "logits", torch.float32, dev, 2)
    tokens = q.shape[0]
    requests = block_table.shape[0]
    if tuple(q.shape) != (tokens, HEADS, HEAD_DIM) or tuple(weights.shape) != (tokens, HEADS):
        raise ValueError(f"q [{tokens}, 32, 128] and weights [{tokens}, 32] (one per row)")
    if cu_q.shape[0] != requests + 1 or row_lens.shape[0] != tokens:
        raise ValueError("cu_q must be [requests + 1] and row_lens [tokens]")
    if logits.shape[0] != tokens or logits.stride(1) != 1:
        raise ValueError("logits must be [tokens, stride] with unit column stride")
    lib = load_library()
    with torch.cuda.device(dev):
        _arm(events, dev)
        tail = (_ptr(weights), _ptr(block_table), int(block_table.shape[1]), _ptr(cu_q), int(requests),
                int(tokens), _ptr(row_lens), int(kv_pages.shape[0]), _ptr(logits), int(logits.stride(0)),
                _stream_ptr(dev))
        if mx:
            st = lib.indexer_prefill_logits_mxfp4(_ptr(q), _ptr(kv_pages), *tail)
        else:
            st = lib.indexer_prefill_logits(_ptr(q), _ptr(kv_pages), _ptr(k_scales), *tail)
    _check("indexer_prefill_logits_mxfp4" if mx else "indexer_prefill_logits", st)


def sparse_to_logical(indices, table, out, events=None):
    """Sparse-row columns -> logical key positions (-1 stays -1)."""
    dev = indices.device
    _rows2(indices, "indices", torch.int32, dev)
    rows, k = indices.shape
    _rows2(table, "table", torch.int32, dev, rows)
    _rows2(out, "out", torch.int32, dev, rows)
    lib = load_library()
    with torch.cuda.device(dev):
        _arm(events, dev)
        st = lib.sparse_to_logical(_ptr(indices), int(k), _ptr(table), int(table.shape[1]), int(rows),
                                   _ptr(out), _stream_ptr(dev))
    _check("sparse_to_logical", st)


def sparse_topk(scores, hist, sparse_lens, k, key_dtype, table, out, events=None):
    """Top-k inside the sparse rows (float32 [rows, stride <= 16384]) written
    as logical key positions through ``table`` [rows, kb]: topk_rows followed
    by sparse_to_logical in one launch."""
    dev = scores.device
    _need(scores, "scores", torch.float32, dev, 2)
    rows = scores.shape[0]
    _need(sparse_lens, "sparse_lens", torch.int32, dev, 1)
    _rows2(table, "table", torch.int32, dev, rows)
    _rows2(out, "out", torch.int32, dev, rows)
    if scores.stride(1) != 1 or tuple(sparse_lens.shape) != (rows,) or out.shape[1] != k:
        raise ValueError("scores must have unit column stride; sparse_lens [rows]; out [rows, k]")
    if hist is not None:
        _rows2(hist, "hist", torch.int32, dev, rows)
    lib = load_library()
    with torch.cuda.device(dev):
        _arm(events, dev)
        st = lib.sparse_topk(_ptr(scores), int(scores.stride(0)), _ptr(hist), _ptr(sparse_lens), int(rows),
                             int(k), int(key_dtype), _ptr(table), int(table.shape[1]), _ptr(out),
                             _stream_ptr(dev))
    _check("sparse_topk", st)


def topk_workspace_bytes(rows: int, logits_stride: int, k: int) -> int:
    return int(load_library().topk_workspace_bytes(int(rows), int(logits_stride), int(k)))


def _topk_call(name, dtype, logits, hist, context_lens, k, key_dtype, indices, workspace, events):
    dev = logits.device
    _need(logits, "logits", dtype, dev, 2)
    _need(context_lens, "context_lens", torch.int32, dev, 1)
    _need(indices, "indices", torch.int32, dev, 2)
    rows = logits.shape[0]
    if logits.stride(1) != 1:
        raise ValueError("logits must have unit column stride")
    if tuple(context_lens.shape) != (rows,) or not context_lens.is_contiguous():
        raise ValueError(f"context_lens must be contiguous [{rows}]")
    if tuple(indices.shape) != (rows, k) or not indices.is_contiguous():
        raise ValueError(f"indices must be contiguous [{rows}, {k}]")
    if hist is not None:
        _need(hist, "hist", torch.int32, dev, 2)
        if tuple(hist.shape) != (rows, NUM_BINS) or not hist.is_contiguous():
            raise ValueError(f"hist must be contiguous [{rows}, 1024]")
    if name == "topk_rows_noalloc":
        workspace = None
    elif workspace is None:
        workspace = _device_workspace(dev, topk_workspace_bytes(rows, logits.stride(0), k))
    else:
        _need(workspace, "workspace", torch.uint8, dev)
    lib = load_library()
    with torch.cuda.device(dev):
        _arm(events, dev)
        head = (_ptr(logits), int(logits.stride(0)), _ptr(hist), _ptr(context_lens), int(rows), int(k))
        if workspace is None:
            tail = (_ptr(indices), _stream_ptr(dev))
        else:
            tail = (_ptr(indices), _ptr(workspace), int(workspace.numel()), _stream_ptr(dev))
        if key_dtype is None:
            st = getattr(lib, name)(*head, *tail)
        else:
            st = getattr(lib, name)(*head, int(key_dtype), *tail)
    _check(name, st)


# One workspace per device for calls that pass none, allocated the first time
# a call needs more than the current one holds and reused after that.
_workspaces: dict = {}


def _device_workspace(dev: torch.device, need: int) -> torch.Tensor:
    key = dev.index if dev.index is not None else torch.cuda.current_device()
    ws = _workspaces.get(key)
    if ws is None or ws.numel() < need:
        ws = torch.zeros(max(need, 256), dtype=torch.uint8, device=dev)
        _workspaces[key] = ws
    return ws


def topk_rows(logits, hist, context_lens, k, key_dtype, indices, workspace=None, events=None):
    """Exact per-row top-k indices of float32 scores into ``indices`` [rows, k].

    ``workspace`` is a uint8 GPU tensor of at least topk_workspace_bytes()
    bytes (no initialisation needed).  When None, the device's shared
    workspace of this module is used (allocated, or grown, only when a call
    needs more than it holds); calls that use it must be ordered on one
    stream.
    """
    _topk_call("topk_rows", torch.float32, logits, hist, context_lens, k, key_dtype, indices,
               workspace, events)


def topk_rows_f16(logits, hist, context_lens, k, indices, workspace=None, events=None):
    """topk_rows over float16 scores [rows, stride] (stride % 8 == 0), FP16 keys."""
    _topk_call("topk_rows_f16", torch.float16, logits, hist, context_lens, k, None, indices,
               workspace, events)


def topk_rows_noalloc(logits, hist, context_lens, k, key_dtype, indices, events=None):
    """topk_rows with the library's fixed per-GPU scratch instead of a workspace
    (at most 128 rows when rows hold more than 16384 scores); allocates
    nothing.  Calls that overlap on one GPU race on that scratch."""
    _topk_call("topk_rows_noalloc", torch.float32, logits, hist, context_lens, k, key_dtype, indices,
               None, events)


def score_histogram(scores, context_lens, hist):
    """Add the coarse bins of every live non-NaN score of each row to ``hist``."""
    dev = scores.device
    _need(scores, "scores", torch.float32, dev, 2)
    _need(context_lens, "context_lens", torch.int32, dev, 1)
    _need(hist, "hist", torch.int32, dev, 2)
    rows = scores.shape[0]
    if scores.stride(1) != 1:
        raise ValueError("scores must have unit column stride")
    if tuple(context_lens.shape) != (rows,) or not context_lens.is_contiguous():
        raise ValueError(f"context_lens must be contiguous [{rows}]")
    if tuple(hist.shape) != (rows, NUM_BINS) or not hist.is_contiguous():
        raise ValueError(f"hist must be contiguous [{rows}, 1024]")
    lib = load_library()
    with torch.cuda.device(dev):
        st = lib.score_histogram(_ptr(scores), int(scores.stride(0)), _ptr(context_lens),
                                 int(rows), _ptr(hist), _stream_ptr(dev))
    _check("score_histogram", st)


def _read_probe(name: str, src: torch.Tensor, sink: torch.Tensor, events) -> None:
    if src.device.type != "cuda" or not src.is_contiguous():
        raise ValueError("src must be a contiguous GPU tensor")
    _need(sink, "sink", torch.int32, src.device)
    lib = load_library()
    nbytes = src.numel() * src.element_size()
    with torch.cuda.device(src.device):
        _arm(events, src.device)
        st = getattr(lib, name)(_ptr(src), nbytes - nbytes % 16, _ptr(sink), _stream_ptr(src.device))
    _check(name, st)


def hbm_read_probe(src: torch.Tensor, sink: torch.Tensor, events=None) -> None:
    """Stream all bytes of ``src`` (contiguous GPU tensor) once with ordinary
    loads (a cache sweep for large buffers); checksum to sink."""
    _read_probe("hbm_read_probe", src, sink, events)


def hbm_read_probe_nt(src: torch.Tensor, sink: torch.Tensor, events=None) -> None:
    """hbm_read_probe with non-temporal loads: the contiguous read ceiling."""
    _read_probe("hbm_read_probe_nt", src, sink, events)


def hbm_gather_probe(kv_pages: torch.Tensor, k_scales: torch.Tensor, page_list: torch.Tensor,
                     sink: torch.Tensor, events=None) -> None:
    """Read the FP8 K pages (and their scales) listed in ``page_list`` once,
    the way the paged K stream is read; checksum to ``sink``."""
    dev = kv_pages.device
    _need(kv_pages, "kv_pages", torch.uint8, dev, 3)
    _need(k_scales, "k_scales", torch.float32, dev, 2)
    _need(page_list, "page_list", torch.int32, dev, 1)
    _need(sink, "sink", torch.int32, dev)
    if not (kv_pages.is_contiguous() and k_scales.is_contiguous() and page_list.is_contiguous()):
        raise ValueError("kv_pages, k_scales and page_list must be contiguous")
    if tuple(kv_pages.shape[1:]) != (PAGE_TOKENS, HEAD_DIM):
        raise ValueError("kv_pages must be [num_pages, 64, 128]")
    lib = load_library()
    with torch.cuda.device(dev):
        _arm(events, dev)
        st = lib.hbm_gather_probe(_ptr(kv_pages), _ptr(k_scales), _ptr(page_list), int(page_list.numel()),
                                  int(kv_pages.shape[0]), _ptr(sink), _stream_ptr(dev))
    _check("hbm_gather_probe", st)


def mfma_valu_probe(mode: int, waves_per_simd: int, iters: int, out: torch.Tensor, events=None) -> None:
    """MFMA / VALU co-issue probe: mode 0 fp8 MFMAs only, 1 fp32 FMAs only,
    2 both (independent, eight FMAs per MFMA); ``out`` float32 with at least
    CUs * waves_per_simd * 256 elements."""
    dev = out.device
    _need(out, "out", torch.float32, dev)
    if not out.is_contiguous():
        raise ValueError("out must be contiguous")
    lib = load_library()
    with torch.cuda.device(dev):
        _arm(events, dev)
        st = lib.mfma_valu_probe(int(mode), int(waves_per_simd), int(iters), _ptr(out), int(out.numel()),
                                 _stream_ptr(dev))
    _check("mfma_valu_probe", st)
