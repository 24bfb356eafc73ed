"""Plain CPU oracle for the paged MQA indexer: logits, coarse histogram, top-k.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path imports this module:
only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may use it.  It shares no code with the HIP library.

Sources (the three pages this method is described on):

* [P1] DeepGEMM PR #94, "[SM100] Paged MQA logits: fused coarse score
  histogram for LiteTopK decode" -- sections "Motivation", "What this adds"
  (histogram contract and bin regimes), and the SGLang commit "Replace the
  CuTe DSL selector with a JIT CUDA selector; add verify" (exact top-2048
  selector, ties to the lower slot, fallback).
* [P3] vLLM PR #52696, "[Performance][MLA] Use FP16 logits for sparse
  indexer" -- "Summary" and commit messages (FP16 score keys).

Everything here is the plain definition written out, in float64 where
floating point is involved:

* ``e4m3fn_decode_table``  -- OCP FP8 E4M3FN from its bit definition.
* ``indexer_logits``       -- logit[r, s] = sc_s * sum_h w[r,h] * ReLU(q[r,h] . k_s)
                              over the live keys of row r, gathered through the
                              block table (P1 "What this adds": FP8 Q/K, H=32,
                              D=128, FP32 weights and logits).  The dot products
                              of e4m3 values are exact in float64 (each product
                              is a multiple of 2^-18 below 2^18 in magnitude, a
                              sum of 128 such stays below 2^25, so 43 of the 53
                              bits suffice).
* ``coarse_bin``           -- the 1024-bin descending coarse histogram bin of
                              P1 "What this adds" (three regimes).
* ``coarse_histogram``     -- counts of live, non-NaN scores, added to the
                              incoming counts (counts accumulate across calls).
* ``score_keys``           -- order-preserving unsigned keys for FP32 scores
                              and for FP16-RN scores (P3 Summary: FP16 keys).
* ``topk_rows``            -- exact top-k by a full sort, key descending, ties to
                              the lower column index (P1 SGLang commit: ties go
                              to the lower slot).
* ``e2m1_decode_table``, ``decode_e8m0``, ``dequant_mxfp4_tokens`` -- block-scaled
                              E2M1 (MXFP4) index keys in the packed 68-byte token
                              layout (P2 "unpack_fp4_index_keys_to_fp8": block-scaled
                              E2M1 index-K; P3 "the packed 68-byte cache layout",
                              dequantized MXFP4 references).  The logits functions
                              take such pages in place of FP8 pages + scales.

Readings taken where the pages leave a step open (each is justified in the
design notes of the repository):

* The per-token K scale multiplies the head-reduced sum.
* Q is cast straight to e4m3 with no query scale.
* All three bin regimes are decided on h = fp16_RN(x) (round to nearest even,
  subnormals kept, |x| >= 65520 becomes inf), so the bin is a function of h.
* A unit bin of magnitude k holds k <= |h| < k + 1 for either sign (for a
  negative score the bin is (-(k+1), -k]).
* Live means column < context_len of that row; NaN is never counted or
  selected; +-inf are counted in the saturating bins and are selectable.
* FP16 keys order scores by fp16_RN(x); equal fp16 values are ties.
* Fewer selectable scores than k: all of them, then -1 padding.
* MXFP4 keys: a token is 64 bytes of E2M1 codes (dimension 2i in the low
  nibble of byte i, 2i+1 in the high nibble) followed by four E8M0 scale
  bytes, one per 32 consecutive dimensions; the key is code value times
  2^(scale - 127), with no further per-token scale; Q stays E4M3.
"""

from __future__ import annotations

import math

import numpy as np

NUM_HEADS = 32
HEAD_DIM = 128
PAGE_SIZE = 64
NUM_BINS = 1024

KEY_FP32 = 0
KEY_FP16 = 1


# ---------------------------------------------------------------------------
# O1  FP8 E4M3FN decode (OCP 8-bit floating point specification):
#     sign bit, 4 exponent bits with bias 7, 3 mantissa bits; exponent field 0
#     encodes subnormals m/8 * 2^-6; S.1111.111 is NaN; there is no infinity.
# ---------------------------------------------------------------------------
def e4m3fn_decode_table() -> np.ndarray:
    """All 256 E4M3FN codes decoded to float64 from the bit definition."""
    table = np.empty(256, dtype=np.float64)
    for code in range(256):
        sign = -1.0 if (code >> 7) & 1 else 1.0
        exp_field = (code >> 3) & 0xF
        mant = code & 0x7
        if exp_field == 0xF and mant == 0x7:
            value = math.nan
        elif exp_field == 0:
            value = sign * (mant / 8.0) * 2.0 ** (1 - 7)
        else:
            value = sign * (1.0 + mant / 8.0) * 2.0 ** (exp_field - 7)
        table[code] = value
    return table


E4M3FN = e4m3fn_decode_table()


def decode_e4m3fn(codes: np.ndarray) -> np.ndarray:
    """Decode a uint8 array of E4M3FN codes to float64."""
    return E4M3FN[np.asarray(codes, dtype=np.uint8)]


# ---------------------------------------------------------------------------
# MXFP4 keys (OCP microscaling formats: E2M1 elements, E8M0 block scales)
#     E2M1: sign bit, 2 exponent bits with bias 1, 1 mantissa bit; exponent
#     field 0 encodes subnormals m/2; no infinity or NaN.
#     E8M0: an unsigned biased exponent, 2^(e - 127); 0xFF is NaN.
# ---------------------------------------------------------------------------
MXFP4_TOKEN_BYTES = 68  # 64 bytes of codes for 128 dimensions + 4 scale bytes
MXFP4_BLOCK = 32        # dimensions per scale


def e2m1_decode_table() -> np.ndarray:
    """All 16 E2M1 codes decoded to float64 from the bit definition."""
    table = np.empty(16, dtype=np.float64)
    for code in range(16):
        sign = -1.0 if (code >> 3) & 1 else 1.0
        exp_field = (code >> 1) & 0x3
        mant = code & 0x1
        if exp_field == 0:
            value = sign * (mant / 2.0) * 2.0 ** (1 - 1)
        else:
            value = sign * (1.0 + mant / 2.0) * 2.0 ** (exp_field - 1)
        table[code] = value
    return table


E2M1 = e2m1_decode_table()


def decode_e8m0(codes: np.ndarray) -> np.ndarray:
    """E8M0 scale bytes to float64 powers of two (0xFF -> NaN)."""
    e = np.asarray(codes, dtype=np.int64)
    return np.where(e == 255, np.nan, np.ldexp(1.0, e - 127))


def dequant_mxfp4_tokens(tokens: np.ndarray) -> np.ndarray:
    """uint8 [..., 68] packed MXFP4 tokens -> float64 [..., 128] keys."""
    tokens = np.asarray(tokens, dtype=np.uint8)
    data = tokens[..., :HEAD_DIM // 2]
    codes = np.empty(data.shape[:-1] + (HEAD_DIM,), dtype=np.uint8)
    codes[..., 0::2] = data & 0x0F
    codes[..., 1::2] = data >> 4
    scales = decode_e8m0(tokens[..., HEAD_DIM // 2:MXFP4_TOKEN_BYTES])  # [..., 4]
    per_dim = np.repeat(scales, MXFP4_BLOCK, axis=-1)                  # [..., 128]
    with np.errstate(invalid="ignore", over="ignore"):
        return E2M1[codes] * per_dim


def is_mxfp4_pages(kv_pages) -> bool:
    """MXFP4 pages are [num_pages, 64, 68]; FP8 pages [num_pages, 64, 128]."""
    return np.asarray(kv_pages).shape[-1] == MXFP4_TOKEN_BYTES


# ---------------------------------------------------------------------------
# O2-O4  logits
# ---------------------------------------------------------------------------
def _request_keys_at(kv_pages, k_scales, block_table_row, cols):
    """Gather the keys at logical positions ``cols`` of one request: FP8
    codes and their per-token scales, or MXFP4 tokens (scale 1)."""
    cols = np.asarray(cols, dtype=np.int64)
    pages = np.asarray(block_table_row, dtype=np.int64)[cols // PAGE_SIZE]
    slots = cols % PAGE_SIZE
    if is_mxfp4_pages(kv_pages):
        return dequant_mxfp4_tokens(kv_pages[pages, slots]), np.ones(len(cols))
    k8 = kv_pages[pages, slots]
    sc = k_scales[pages, slots]
    return decode_e4m3fn(k8), sc.astype(np.float64)


def _row_logits(q_row, w_row, keys, scales):
    """logit_s = sc_s * sum_h w_h * max(q_h . k_s, 0), float64, one rounding.

    q_row: uint8 [32, 128]; w_row: float32 [32]; keys float64 [n, 128];
    scales float64 [n].  The float64 dot products are exact (module doc).
    """
    qd = decode_e4m3fn(q_row)  # [32, 128]
    dots = qd @ keys.T  # [32, n], exact
    relu = np.maximum(dots, 0.0)
    head_sum = w_row.astype(np.float64) @ relu  # [n]
    with np.errstate(invalid="ignore", over="ignore"):
        return (scales * head_sum).astype(np.float32)


def indexer_logits(q, kv_pages, k_scales, weights, block_table, context_lens,
                   next_n, logits_stride=None, pages_per_chunk=2048,
                   fill=np.nan):
    """Dense logits of every live key of every row.

    q            uint8  [B*next_n, 32, 128]  (E4M3FN codes)
    kv_pages     uint8  [num_pages, 64, 128] (E4M3FN codes), or
                 uint8  [num_pages, 64, 68]  (packed MXFP4 tokens)
    k_scales     f32    [num_pages, 64] (None with MXFP4 pages)
    weights      f32    [B*next_n, 32]
    block_table  int32  [B, max_pages]       (shared by the next_n rows of b)
    context_lens int32  [B*next_n]           (row r sees keys [0, len_r))

    Returns float32 [B*next_n, logits_stride]; columns >= len_r hold ``fill``.
    """
    q = np.asarray(q)
    rows = q.shape[0]
    B = rows // next_n
    lens = np.asarray(context_lens, dtype=np.int64)
    if logits_stride is None:
        logits_stride = int(lens.max()) if rows else 0
    out = np.full((rows, logits_stride), fill, dtype=np.float32)
    chunk = pages_per_chunk * PAGE_SIZE
    for b in range(B):
        r0 = b * next_n
        n_keys = int(lens[r0:r0 + next_n].max())
        for s0 in range(0, n_keys, chunk):
            s1 = min(n_keys, s0 + chunk)
            keys, sc = _request_keys_at(kv_pages, k_scales, block_table[b],
                                        np.arange(s0, s1))
            for j in range(next_n):
                r = r0 + j
                e = min(s1, int(lens[r]))
                if e <= s0:
                    continue
                out[r, s0:e] = _row_logits(q[r], weights[r], keys[:e - s0],
                                           sc[:e - s0])
    return out


def indexer_logits_at(q, kv_pages, k_scales, weights, block_table, next_n, row,
                      cols):
    """Logits of row ``row`` at the given logical key positions only."""
    b = row // next_n
    keys, sc = _request_keys_at(kv_pages, k_scales, block_table[b], cols)
    return _row_logits(q[row], weights[row], keys, sc)


def logits_error_bound_at(q, kv_pages, k_scales, weights, block_table, next_n,
                          row, cols, rel=1e-5, unscaled=False):
    """Tolerance rel * sc_s * sum_h |w_h| * sum_d |q_hd * k_sd| (float64).

    The nested absolute sums bound every rounding a fp32 implementation of
    the same formula makes, whatever its summation order.  ``unscaled`` leaves
    out sc_s (the tolerance of the head sum itself).
    """
    b = row // next_n
    keys, sc = _request_keys_at(kv_pages, k_scales, block_table[b], cols)
    qd = np.abs(decode_e4m3fn(q[row]))
    abs_dots = qd @ np.abs(keys).T
    head = np.abs(weights[row].astype(np.float64)) @ abs_dots
    if unscaled:
        return rel * head
    with np.errstate(invalid="ignore", over="ignore"):
        return rel * np.abs(sc) * head


def head_sum_at(q, kv_pages, k_scales, weights, block_table, next_n, row, cols):
    """sum_h w_h * ReLU(q_h . k_s) before the scale (float64)."""
    b = row // next_n
    keys, _ = _request_keys_at(kv_pages, k_scales, block_table[b], cols)
    qd = decode_e4m3fn(q[row])
    return weights[row].astype(np.float64) @ np.maximum(qd @ keys.T, 0.0)


def logits_terms_at(q, kv_pages, k_scales, weights, block_table, next_n, rows, cols,
                    rel=1e-5):
    """For rows of one request at the key positions ``cols``: the expected
    logits and the three acceptance terms, from one gather of the keys.

    Returns (want, bound, head_sum, head_bound), each float [len(rows), n]:
    row by row the values of indexer_logits_at, logits_error_bound_at (with
    and without the scale) and head_sum_at -- the same expressions, so the
    same numbers (the dot products are exact in float64; the head sums are
    the same vector-matrix products as there).
    """
    b = rows[0] // next_n
    if any(r // next_n != b for r in rows):
        raise ValueError("rows of one request only")
    keys, sc = _request_keys_at(kv_pages, k_scales, block_table[b], cols)
    abs_keys_t = np.abs(keys).T
    out = [np.empty((len(rows), len(cols)), dtype) for dtype in
           (np.float32, np.float64, np.float64, np.float64)]
    for i, r in enumerate(rows):
        qd = decode_e4m3fn(q[r])
        dots = qd @ keys.T
        w = weights[r].astype(np.float64)
        head_sum = w @ np.maximum(dots, 0.0)
        head = np.abs(w) @ (np.abs(qd) @ abs_keys_t)
        with np.errstate(invalid="ignore", over="ignore"):
            out[0][i] = (sc * head_sum).astype(np.float32)
            out[1][i] = rel * np.abs(sc) * head
        out[2][i] = head_sum
        out[3][i] = rel * head
    return tuple(out)


def check_logits(got, want, bound, head_sum=None, head_bound=None):
    """Element-wise acceptance of GPU logits against the oracle.

    Finite expected values: |got - want| <= bound.  Non-finite expected values
    (an infinite scale) are checked by class: NaN matches NaN, and +-inf
    matches the same infinity; when the unscaled head sum is within its own
    tolerance of zero either sign, or NaN, is accepted because the sign of a
    sum that is zero up to rounding is not determined by the formula.
    Returns a boolean array, True where the element is accepted.
    """
    got = np.asarray(got, dtype=np.float64)
    want = np.asarray(want, dtype=np.float64)
    bound = np.asarray(bound, dtype=np.float64)
    ok = np.zeros(got.shape, dtype=bool)
    fin = np.isfinite(want) & np.isfinite(bound)
    with np.errstate(invalid="ignore"):
        ok[fin] = np.abs(got[fin] - want[fin]) <= bound[fin]
    nf = ~fin
    if np.any(nf):
        same_nan = np.isnan(got) & np.isnan(want)
        same_inf = np.isinf(got) & np.isinf(want) & (np.sign(got) == np.sign(want))
        ok[nf] = (same_nan | same_inf)[nf]
        if head_sum is not None and head_bound is not None:
            near_zero = np.abs(np.asarray(head_sum)) <= np.asarray(head_bound)
            ok[nf] |= (near_zero & (np.isinf(got) | np.isnan(got)))[nf]
    return ok


# ---------------------------------------------------------------------------
# O5  coarse histogram bins (P1 "What this adds")
# ---------------------------------------------------------------------------
def fp16_rne(x) -> np.ndarray:
    """IEEE binary16 round-to-nearest-even of float32 values (numpy's cast)."""
    with np.errstate(over="ignore"):
        return np.asarray(x, dtype=np.float32).astype(np.float16)


def check_logits_f16(got, want, bound, head_sum=None, head_bound=None):
    """Element-wise acceptance of FP16 logits (vLLM PR #52696 "Summary": the
    indexer stores its logits as FP16).

    A finite expected value accepts exactly the halves that are fp16_RN(y)
    of some float32 y with |y - want| <= bound, i.e. the float32 values the
    float32 check accepts, rounded: rounding is monotone, so these are the
    halves between fp16_RN(ylo) and fp16_RN(yhi), ylo / yhi the least / the
    greatest float32 in [want - bound, want + bound].  Non-finite expected
    values are checked by class as in check_logits (an infinity rounds to
    the same infinity, NaN stays NaN).  ``got`` is float16 (or its bits as
    uint16).  Returns a boolean array, True where the element is accepted.
    """
    got = np.asarray(got)
    if got.dtype == np.uint16:
        got = got.view(np.float16)
    g = got.astype(np.float64)
    want = np.asarray(want, dtype=np.float64)
    bound = np.asarray(bound, dtype=np.float64)
    ok = np.zeros(g.shape, dtype=bool)
    fin = np.isfinite(want) & np.isfinite(bound)
    if np.any(fin):
        lo64, hi64 = want[fin] - bound[fin], want[fin] + bound[fin]
        with np.errstate(over="ignore"):
            lo32, hi32 = lo64.astype(np.float32), hi64.astype(np.float32)
        lo32 = np.where(lo32.astype(np.float64) < lo64, np.nextafter(lo32, np.float32(np.inf)), lo32)
        hi32 = np.where(hi32.astype(np.float64) > hi64, np.nextafter(hi32, np.float32(-np.inf)), hi32)
        lo16 = fp16_rne(lo32).astype(np.float64)
        hi16 = fp16_rne(hi32).astype(np.float64)
        with np.errstate(invalid="ignore"):
            ok[fin] = (lo16 <= g[fin]) & (g[fin] <= hi16)
    nf = ~fin
    if np.any(nf):
        ok[nf] = check_logits(g[nf], want[nf], bound[nf],
                              None if head_sum is None else np.asarray(head_sum)[nf],
                              None if head_bound is None else np.asarray(head_bound)[nf])
    return ok


def coarse_bin(x) -> np.ndarray:
    """Bin 0..1023 of each float32 score; -1 for NaN (never counted).

    h = fp16_RN(x), a = |h|, then the magnitude code m:
      a < 16          m = exponent and top 4 mantissa bits of h   (0..303)
      16 <= a < 223   m = 288 + floor(a)                           (304..510)
      a >= 223, inf   m = 511                                      (saturating)
    and bin = 511 - m for a positive sign bit, 512 + m for a negative one, so
    bin 0 holds the largest scores.
    """
    x = np.asarray(x, dtype=np.float32)
    h = fp16_rne(x)
    bits = h.view(np.uint16).astype(np.int64)
    negative = (bits >> 15) == 1
    mag = np.abs(h.astype(np.float64))
    fine = (bits & 0x7FFF) >> 6
    with np.errstate(invalid="ignore"):
        unit = 288 + np.floor(np.where(np.isfinite(mag), mag, 0.0)).astype(np.int64)
        m = np.where(mag < 16.0, fine, np.where(mag < 223.0, unit, 511))
    b = np.where(negative, 512 + m, 511 - m)
    return np.where(np.isnan(x), -1, b).astype(np.int64)


def coarse_histogram(logits, context_lens, hist_in=None) -> np.ndarray:
    """int32 [rows, 1024]: counts of live non-NaN scores added to ``hist_in``."""
    logits = np.asarray(logits)
    rows = logits.shape[0]
    hist = np.zeros((rows, NUM_BINS), dtype=np.int64)
    if hist_in is not None:
        hist += np.asarray(hist_in, dtype=np.int64)
    for r in range(rows):
        n = int(context_lens[r])
        b = coarse_bin(logits[r, :n])
        b = b[b >= 0]
        hist[r] += np.bincount(b, minlength=NUM_BINS)
    return hist.astype(np.int32)


# ---------------------------------------------------------------------------
# O6  order-preserving keys; O7  exact top-k
# ---------------------------------------------------------------------------
def score_keys(x, key_dtype) -> np.ndarray:
    """Unsigned keys whose integer order is the score order (-inf .. +inf).

    FP32: the float32 bits with the sign bit set for a positive sign and all
    bits inverted for a negative sign.  FP16: the same on fp16_RN(x).  -0 sorts
    just below +0.
    """
    x = np.asarray(x, dtype=np.float32)
    if key_dtype == KEY_FP32:
        u = x.view(np.uint32).astype(np.uint64)
        k = np.where(u >> 31 == 1, (~u) & 0xFFFFFFFF, u | 0x80000000)
    elif key_dtype == KEY_FP16:
        u = fp16_rne(x).view(np.uint16).astype(np.uint64)
        k = np.where(u >> 15 == 1, (~u) & 0xFFFF, u | 0x8000)
    else:
        raise ValueError("unknown key dtype")
    return k.astype(np.uint64)


def topk_row(x, length, k, key_dtype) -> np.ndarray:
    """Sorted column indices of the top-k of one row (without padding).

    Candidates are the live (< length), non-NaN columns.  Full sort by key
    descending, then column ascending; the first min(k, n) are returned in
    ascending column order.
    """
    x = np.asarray(x, dtype=np.float32)[:length]
    cols = np.nonzero(~np.isnan(x))[0]
    keys = score_keys(x[cols], key_dtype)
    order = np.lexsort((cols, -keys.astype(np.float64)))  # key desc, col asc
    # float64 holds every 32-bit key exactly, so the negation is exact.
    take = cols[order[:min(k, cols.size)]]
    return np.sort(take)


def topk_rows(logits, context_lens, k, key_dtype) -> np.ndarray:
    """int32 [rows, k]: each row's selected set in ascending order, -1 padded."""
    logits = np.asarray(logits)
    rows = logits.shape[0]
    out = np.full((rows, k), -1, dtype=np.int32)
    for r in range(rows):
        sel = topk_row(logits[r], int(context_lens[r]), k, key_dtype)
        out[r, :sel.size] = sel
    return out
