"""Plain CPU oracle of the ragged prefill (extend) indexer logits.

TEST INFRASTRUCTURE ONLY, like indexer_oracle: only ``tests/``,
``__graft_entry__.smoke()`` and ``bench.py``'s cpu_baseline leg may use it.

Source: [P2] SGLang PR #38944, "[DSV4.1] Enable the two-level candidate
indexer on DeepGEMM's paged sparse MQA logits", the commit that adds an SM90
FP8 prefill path for ragged extend batches: the prefill logits are the
indexer logits of every query row of the batch -- E4M3 products accumulated
in FP32 with the ReLU, the head weighting and the head sum fused, FP32 output
rows padded to a multiple of 4 -- scored request by request so that each K
row of a request serves all of that request's query rows, then handed to the
ragged top-k.

* ``request_of_rows``      -- the request each row belongs to;
* ``prefill_logits``       -- dense logits of every row over its visible keys;
* ``prefill_logits_at``, ``prefill_error_bound_at``, ``prefill_head_sum_at``
                           -- one row at chosen key positions (for checks at
                              sizes the dense oracle is too slow for).

Readings taken where the page is silent:

* A ragged batch is given by row offsets cu_q (request r owns rows
  cu_q[r] .. cu_q[r+1]-1) and a visible length per row: row t scores keys
  [0, row_lens[t]) of its own request, gathered through that request's
  block-table row.  For an extend chunk of n rows appended to a context of
  L keys (prefix included), row i sees L - n + 1 + i keys (causal) -- the
  decode path's convention for next_n rows -- so a batch whose requests all
  have next_n rows is exactly a decode call.
* The per-token K scale multiplies the head-reduced sum and Q is E4M3 with
  no query scale, as in the decode path.
"""

from __future__ import annotations

import numpy as np

from .indexer_oracle import _request_keys_at, _row_logits, head_sum_at, logits_error_bound_at


def request_of_rows(cu_q) -> np.ndarray:
    """int64 [rows]: request r for every row in [cu_q[r], cu_q[r+1])."""
    cu = np.asarray(cu_q, dtype=np.int64)
    counts = np.diff(cu)
    return np.repeat(np.arange(counts.size, dtype=np.int64), counts)


def prefill_logits(q, kv_pages, k_scales, weights, block_table, cu_q, row_lens,
                   logits_stride=None, fill=np.nan, keys_per_chunk=8192):
    """float32 [rows, logits_stride]: row t holds its logits over keys
    [0, row_lens[t]) of its request; ``fill`` elsewhere."""
    q = np.asarray(q)
    lens = np.asarray(row_lens, dtype=np.int64)
    rows = q.shape[0]
    if logits_stride is None:
        logits_stride = int(lens.max()) if rows else 0
    out = np.full((rows, logits_stride), fill, dtype=np.float32)
    cu = np.asarray(cu_q, dtype=np.int64)
    for r in range(cu.size - 1):
        t0, t1 = int(cu[r]), int(cu[r + 1])
        if t1 <= t0:
            continue
        n_keys = int(lens[t0:t1].max())
        for s0 in range(0, n_keys, keys_per_chunk):
            s1 = min(n_keys, s0 + keys_per_chunk)
            keys, sc = _request_keys_at(kv_pages, k_scales, block_table[r], np.arange(s0, s1))
            for t in range(t0, t1):
                e = min(s1, int(lens[t]))
                if e > s0:
                    out[t, s0:e] = _row_logits(q[t], weights[t], keys[:e - s0], sc[:e - s0])
    return out


def _one_row(q, weights, block_table, cu_q, row):
    """The row's own arrays as a one-row, one-request call."""
    r = int(request_of_rows(cu_q)[row])
    return q[row:row + 1], weights[row:row + 1], block_table[r:r + 1]


def prefill_logits_at(q, kv_pages, k_scales, weights, block_table, cu_q, row, cols):
    """Logits of row ``row`` at the given key positions of its request."""
    q1, w1, bt1 = _one_row(q, weights, block_table, cu_q, row)
    keys, sc = _request_keys_at(kv_pages, k_scales, bt1[0], cols)
    return _row_logits(q1[0], w1[0], keys, sc)


def prefill_error_bound_at(q, kv_pages, k_scales, weights, block_table, cu_q, row, cols,
                           rel=1e-5, unscaled=False):
    """rel * sc_s * sum_h |w_h| * sum_d |q_hd * k_sd| for row ``row``."""
    q1, w1, bt1 = _one_row(q, weights, block_table, cu_q, row)
    return logits_error_bound_at(q1, kv_pages, k_scales, w1, bt1, 1, 0, cols, rel=rel,
                                 unscaled=unscaled)


def prefill_head_sum_at(q, kv_pages, k_scales, weights, block_table, cu_q, row, cols):
    """sum_h w_h * ReLU(q_h . k_s) of row ``row`` before the scale."""
    q1, w1, bt1 = _one_row(q, weights, block_table, cu_q, row)
    return head_sum_at(q1, kv_pages, k_scales, w1, bt1, 1, 0, cols)
