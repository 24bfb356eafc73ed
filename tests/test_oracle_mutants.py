"""Plant one plausible mistake at a time in a copy of the oracle (on the CPU)
and require the pins to catch it, so that passing pins mean something."""
import importlib.util
import math
import os

import numpy as np
import pytest

import oracle.indexer_oracle as base
from tests import oracle_pins as P


def fresh_oracle():
    spec = importlib.util.spec_from_file_location("oracle_mutant", base.__file__)
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    # a fresh copy of the candidate-indexer oracle too (inside the package, so
    # its relative import of the logits oracle resolves)
    cspec = importlib.util.spec_from_file_location(
        "oracle.candidates_mutant", os.path.join(os.path.dirname(base.__file__), "candidates.py"))
    cmod = importlib.util.module_from_spec(cspec)
    cspec.loader.exec_module(cmod)
    mod.candidates = cmod
    pspec = importlib.util.spec_from_file_location(
        "oracle.prefill_mutant", os.path.join(os.path.dirname(base.__file__), "prefill.py"))
    pmod = importlib.util.module_from_spec(pspec)
    pspec.loader.exec_module(pmod)
    mod.prefill = pmod
    return mod


# ---- mutations: each takes a fresh oracle module and breaks one thing ----
def m_e4m3_bias(O):
    t = O.E4M3FN.copy()
    t[np.isfinite(t)] *= 0.5  # exponent bias 8 instead of 7
    O.decode_e4m3fn = lambda c: t[np.asarray(c, dtype=np.uint8)]


def m_e4m3_subnormal(O):
    t = O.E4M3FN.copy()
    for c in range(256):
        if (c >> 3) & 0xF == 0 and c & 7:
            s = -1 if c >> 7 else 1
            t[c] = s * (1 + (c & 7) / 8) * 2.0 ** -7
    O.decode_e4m3fn = lambda c: t[np.asarray(c, dtype=np.uint8)]


def _wrap_bin(O, fn):
    orig = O.coarse_bin
    O.coarse_bin = lambda x: fn(np.asarray(x, np.float32), orig(x))


def m_bin_sign_swapped(O):
    _wrap_bin(O, lambda x, b: np.where(b >= 0, 1023 - b, b))


def m_bin_unit_off_by_one(O):
    def f(x, b):
        a = np.abs(O.fp16_rne(x).astype(np.float64))
        unit = (a >= 16) & (a < 223)
        return np.where(unit, np.where(b < 512, b + 1, b - 1), b)
    _wrap_bin(O, f)


def m_bin_fine_shift7(O):
    def f(x, b):
        h = O.fp16_rne(x)
        bits = h.view(np.uint16).astype(np.int64)
        a = np.abs(h.astype(np.float64))
        m = (bits & 0x7FFF) >> 7
        alt = np.where(bits >> 15 == 1, 512 + m, 511 - m)
        return np.where((a < 16) & (b >= 0), alt, b)
    _wrap_bin(O, f)


def m_bin_saturate_224(O):
    def f(x, b):
        a = np.abs(O.fp16_rne(x).astype(np.float64))
        edge = (a >= 223) & (a < 224)
        return np.where(edge, np.where(b < 512, 1, 1022), b)
    _wrap_bin(O, f)


def m_bin_regimes_on_fp32(O):
    def f(x, b):
        a = np.abs(x.astype(np.float64))
        with np.errstate(invalid="ignore"):
            lit = (a >= 16) & (a < 223)
            m = 288 + np.floor(np.where(lit, a, 0)).astype(np.int64)
        alt = np.where(np.signbit(x), 512 + m, 511 - m)
        return np.where(lit & (b >= 0), alt, b)
    _wrap_bin(O, f)


def m_fp16_truncate(O):
    def trunc(x):
        x = np.asarray(x, dtype=np.float32)
        h = x.astype(np.float16)
        hv = h.astype(np.float32)
        over = np.abs(hv) > np.abs(x)  # rounded away from zero
        bits = h.view(np.uint16).astype(np.int32)
        bits = np.where(over & np.isfinite(x), bits - 1, bits)  # one step back
        return bits.astype(np.uint16).view(np.float16)
    O.fp16_rne = trunc


def m_logits_no_relu(O):
    def row(q_row, w_row, keys, scales):
        qd = O.decode_e4m3fn(q_row)
        with np.errstate(invalid="ignore", over="ignore"):
            return (scales * (w_row.astype(np.float64) @ (qd @ keys.T))).astype(np.float32)
    O._row_logits = row


def m_logits_no_scale(O):
    orig = O._row_logits
    O._row_logits = lambda q, w, k, s: orig(q, w, k, np.ones_like(s))


def m_logits_heads_reversed(O):
    orig = O._row_logits
    O._row_logits = lambda q, w, k, s: orig(q, w[::-1].copy(), k, s)


def m_gather_page_slot_swapped(O):
    def keys_at(kv_pages, k_scales, bt_row, cols):
        cols = np.asarray(cols, dtype=np.int64)
        pages = np.asarray(bt_row, dtype=np.int64)[cols % 64]
        slots = cols // 64
        return O.decode_e4m3fn(kv_pages[pages, slots % 64]), \
            k_scales[pages, slots % 64].astype(np.float64)
    O._request_keys_at = keys_at


def m_gather_logical_page(O):
    def keys_at(kv_pages, k_scales, bt_row, cols):
        cols = np.asarray(cols, dtype=np.int64)
        pages = cols // 64  # ignores the block table
        return O.decode_e4m3fn(kv_pages[pages, cols % 64]), \
            k_scales[pages, cols % 64].astype(np.float64)
    O._request_keys_at = keys_at


def m_topk_ties_high(O):
    def row(x, length, k, key_dtype):
        x = np.asarray(x, dtype=np.float32)[:length]
        cols = np.nonzero(~np.isnan(x))[0]
        keys = O.score_keys(x[cols], key_dtype)
        order = np.lexsort((-cols, -keys.astype(np.float64)))
        return np.sort(cols[order[:min(k, cols.size)]])
    O.topk_row = row


def m_topk_keeps_nan(O):
    def row(x, length, k, key_dtype):
        x = np.asarray(x, dtype=np.float32)[:length]
        cols = np.arange(x.size)
        keys = O.score_keys(x, key_dtype)
        order = np.lexsort((cols, -keys.astype(np.float64)))
        return np.sort(cols[order[:min(k, cols.size)]])
    O.topk_row = row


def m_topk_ignores_length(O):
    orig = O.topk_row
    O.topk_row = lambda x, length, k, kd: orig(x, len(x), k, kd)


def m_hist_counts_padding(O):
    orig = O.coarse_histogram
    O.coarse_histogram = lambda lg, lens, hist_in=None: orig(
        lg, np.full(len(lens), np.asarray(lg).shape[1]), hist_in)


def m_hist_drops_incoming(O):
    orig = O.coarse_histogram
    O.coarse_histogram = lambda lg, lens, hist_in=None: orig(lg, lens)


def m_keys_negatives_not_inverted(O):
    orig = O.score_keys

    def keys(x, kd):
        x = np.asarray(x, dtype=np.float32)
        if kd == O.KEY_FP32:
            return (x.view(np.uint32).astype(np.uint64) | 0x80000000)
        return orig(x, kd)
    O.score_keys = keys


def m_keys_zero_signs_equal(O):
    orig = O.score_keys

    def keys(x, kd):
        x = np.asarray(x, dtype=np.float32).copy()
        x[x == 0] = 0.0
        return orig(x, kd)
    O.score_keys = keys


def m_e2m1_subnormal(O):
    t = O.E2M1.copy()
    t[1], t[9] = 1.0, -1.0  # subnormal read as 1.0 * 2^0
    O.E2M1 = t


def _wrap_dequant(O, fn):
    O.dequant_mxfp4_tokens = lambda tok: fn(np.asarray(tok, dtype=np.uint8))


def m_mxfp4_nibbles_swapped(O):
    def deq(tok):
        data = tok[..., :64]
        codes = np.empty(data.shape[:-1] + (128,), dtype=np.uint8)
        codes[..., 0::2] = data >> 4
        codes[..., 1::2] = data & 0x0F
        sc = np.repeat(O.decode_e8m0(tok[..., 64:68]), 32, axis=-1)
        return O.E2M1[codes] * sc
    _wrap_dequant(O, deq)


def m_mxfp4_scale_blocks_reversed(O):
    orig = O.dequant_mxfp4_tokens

    def deq(tok):
        t = tok.copy()
        t[..., 64:68] = tok[..., 64:68][..., ::-1]
        return orig(t)
    _wrap_dequant(O, deq)


def m_mxfp4_scale_ignored(O):
    orig = O.dequant_mxfp4_tokens

    def deq(tok):
        t = tok.copy()
        t[..., 64:68] = 127
        return orig(t)
    _wrap_dequant(O, deq)


def m_e8m0_bias_128(O):
    O.decode_e8m0 = lambda c: np.where(np.asarray(c, np.int64) == 255, np.nan,
                                       np.ldexp(1.0, np.asarray(c, np.int64) - 128))


def m_amax8_block_count(O):
    # floor(len / 8) + 1 blocks: one too many when len is a multiple of 8
    orig = O.candidates.block_amax8

    def amax(sc, lens, fill=np.nan):
        lens = np.asarray(lens, np.int64)
        sc = np.asarray(sc, np.float32)
        wide = np.full((sc.shape[0], sc.shape[1] + 8), np.nan, np.float32)
        wide[:, :sc.shape[1]] = sc
        out = orig(wide, np.where(lens % 8 == 0, lens + 1, lens), fill)
        return out[:, :max(out.shape[1], 1)]
    O.candidates.block_amax8 = amax


def m_amax8_newest_not_inf(O):
    def amax(sc, lens, fill=np.nan):
        sc = np.asarray(sc, np.float32)
        lens = np.asarray(lens, np.int64)
        nb = -(-lens // 8)
        out = np.full((sc.shape[0], max(int(nb.max()), 1)), fill, np.float32)
        for r in range(sc.shape[0]):
            for j in range(int(nb[r])):
                with np.errstate(invalid="ignore"):
                    out[r, j] = np.fmax.reduce(sc[r, 8 * j:min(int(lens[r]), 8 * j + 8)])
        return out
    O.candidates.block_amax8 = amax


def m_s2l_padding_mapped(O):
    # table padding (INT32_MAX) treated as a block id
    B = O.candidates.BLOCK

    def s2l(table, cols):
        table = np.asarray(table, np.int64)
        cols = np.asarray(cols, np.int64)
        out = np.full(cols.shape, -1, np.int64)
        ok = (cols >= 0) & (cols < B * table.shape[1])
        r = np.nonzero(ok)
        out[ok] = B * table[r[0], cols[ok] // B] + cols[ok] % B
        return out
    O.candidates.sparse_to_logical = s2l


def m_s2l_past_table_clamped(O):
    # columns past the table read the last entry instead of giving -1
    B = O.candidates.BLOCK
    big = O.candidates.INT32_MAX

    def s2l(table, cols):
        table = np.asarray(table, np.int64)
        cols = np.asarray(cols, np.int64)
        out = np.full(cols.shape, -1, np.int64)
        ok = cols >= 0
        r = np.nonzero(ok)
        blocks = table[r[0], np.minimum(cols[ok] // B, table.shape[1] - 1)]
        out[ok] = np.where(blocks == big, -1, B * blocks + cols[ok] % B)
        return out
    O.candidates.sparse_to_logical = s2l


def m_sort_no_identity(O):
    orig = O.candidates.sort_candidate_blocks
    O.candidates.sort_candidate_blocks = lambda b, n, bt, nn: orig(
        b, np.full(len(n), 1 << 30), bt, nn)


def m_sort_slot_transform(O):
    orig = O.candidates.sort_candidate_blocks

    def sort(b, n, bt, nn):
        t, s = orig(b, n, bt, nn)
        s = np.where(t != 2 ** 31 - 1, s - (t % 8) + (t // 8) % 8, s).astype(np.int32)
        return t, s
    O.candidates.sort_candidate_blocks = sort


def m_sparse_block_offset(O):
    def sp(q, kv, ks, w, bt, table, lens, nn, fill=np.nan):
        t = np.asarray(table, np.int64)
        t = np.where(t != 2 ** 31 - 1, t + 1, t)
        return orig(q, kv, ks, w, bt, t, lens, nn, fill)
    orig = O.candidates.sparse_logits
    O.candidates.sparse_logits = sp


def _wrap_prefill(O, fn):
    orig = O.prefill.prefill_logits
    O.prefill.prefill_logits = lambda q, kv, ks, w, bt, cu, lens, *a, **k: fn(orig, q, kv, ks, w, bt,
                                                                               np.asarray(cu), np.asarray(lens),
                                                                               *a, **k)


def m_prefill_tables_reversed(O):
    # every row reads the pages of the mirror-image request
    _wrap_prefill(O, lambda f, q, kv, ks, w, bt, cu, lens, *a, **k: f(q, kv, ks, w, bt[::-1], cu, lens,
                                                                       *a, **k))


def m_prefill_request_max_len(O):
    # every row of a request scores the request's longest visible range
    def f(orig, q, kv, ks, w, bt, cu, lens, *a, **k):
        l2 = lens.copy()
        for r in range(cu.size - 1):
            if cu[r + 1] > cu[r]:
                l2[cu[r]:cu[r + 1]] = lens[cu[r]:cu[r + 1]].max()
        return orig(q, kv, ks, w, bt, cu, l2, *a, **k)
    _wrap_prefill(O, f)


def m_prefill_boundary_row(O):
    # the first row of every request after the first goes to the request before
    def f(orig, q, kv, ks, w, bt, cu, lens, *a, **k):
        c2 = cu.copy()
        c2[1:-1] += 1
        return orig(q, kv, ks, w, bt, np.minimum(c2, cu[-1]), lens, *a, **k)
    _wrap_prefill(O, f)


# ---- the acceptance helpers (head sum, error bound, class check) ----
def m_head_sum_no_relu(O):
    def hs(q, kv_pages, k_scales, weights, block_table, next_n, row, cols):
        keys, _ = O._request_keys_at(kv_pages, k_scales, block_table[row // next_n], cols)
        return weights[row].astype(np.float64) @ (O.decode_e4m3fn(q[row]) @ keys.T)
    O.head_sum_at = hs


def m_head_sum_scaled(O):
    orig = O.head_sum_at

    def hs(q, kv_pages, k_scales, weights, block_table, next_n, row, cols):
        _, sc = O._request_keys_at(kv_pages, k_scales, block_table[row // next_n], cols)
        with np.errstate(invalid="ignore", over="ignore"):
            return sc * orig(q, kv_pages, k_scales, weights, block_table, next_n, row, cols)
    O.head_sum_at = hs


def m_bound_unscaled_keeps_scale(O):
    orig = O.logits_error_bound_at
    O.logits_error_bound_at = lambda *a, rel=1e-5, unscaled=False: orig(*a, rel=rel)


def m_bound_signed_dots(O):
    def bound(q, kv_pages, k_scales, weights, block_table, next_n, row, cols, rel=1e-5,
              unscaled=False):
        keys, sc = O._request_keys_at(kv_pages, k_scales, block_table[row // next_n], cols)
        head = np.abs(weights[row].astype(np.float64)) @ np.abs(O.decode_e4m3fn(q[row]) @ keys.T)
        with np.errstate(invalid="ignore", over="ignore"):
            return rel * head if unscaled else rel * np.abs(sc) * head
    O.logits_error_bound_at = bound


def m_waiver_on_finite(O):
    orig = O.check_logits

    def check(got, want, bound, head_sum=None, head_bound=None):
        ok = orig(got, want, bound, head_sum, head_bound)
        if head_sum is not None and head_bound is not None:
            ok |= np.abs(np.asarray(head_sum)) <= np.asarray(head_bound)
        return ok
    O.check_logits = check


def m_inf_sign_ignored(O):
    orig = O.check_logits

    def check(got, want, bound, head_sum=None, head_bound=None):
        ok = orig(got, want, bound, head_sum, head_bound)
        return ok | (np.isinf(np.asarray(got, np.float64)) & np.isinf(np.asarray(want, np.float64)))
    O.check_logits = check


def m_nan_matches_any_nonfinite(O):
    orig = O.check_logits

    def check(got, want, bound, head_sum=None, head_bound=None):
        g, w = np.asarray(got, np.float64), np.asarray(want, np.float64)
        ok = orig(got, want, bound, head_sum, head_bound)
        return ok | (np.isnan(w) & ~np.isfinite(g)) | (np.isnan(g) & ~np.isfinite(w))
    O.check_logits = check


def m_waiver_accepts_finite(O):
    orig = O.check_logits

    def check(got, want, bound, head_sum=None, head_bound=None):
        ok = orig(got, want, bound, head_sum, head_bound)
        if head_sum is not None and head_bound is not None:
            nf = ~np.isfinite(np.asarray(want, np.float64))
            ok |= nf & (np.abs(np.asarray(head_sum)) <= np.asarray(head_bound))
        return ok
    O.check_logits = check


MUTANTS = [
    (m_e4m3_bias, [P.pin_e4m3]),
    (m_e4m3_subnormal, [P.pin_e4m3]),
    (m_bin_sign_swapped, [P.pin_bins_golden]),
    (m_bin_unit_off_by_one, [P.pin_bins_golden, P.pin_bins_exhaustive]),
    (m_bin_fine_shift7, [P.pin_bins_golden, P.pin_bins_exhaustive]),
    (m_bin_saturate_224, [P.pin_bins_golden, P.pin_bins_exhaustive]),
    (m_bin_regimes_on_fp32, [P.pin_bins_golden]),
    (m_fp16_truncate, [P.pin_fp16_rne]),
    (m_logits_no_relu, [P.pin_logits_exact, P.pin_logits_library]),
    (m_logits_no_scale, [P.pin_logits_exact]),
    (m_logits_heads_reversed, [P.pin_logits_exact]),
    (m_gather_page_slot_swapped, [P.pin_logits_exact, P.pin_logits_paging]),
    (m_gather_logical_page, [P.pin_logits_exact, P.pin_logits_paging]),
    (m_topk_ties_high, [P.pin_topk, P.pin_topk_invariants]),
    (m_topk_keeps_nan, [P.pin_topk]),
    (m_topk_ignores_length, [P.pin_topk]),
    (m_hist_counts_padding, [P.pin_histogram]),
    (m_hist_drops_incoming, [P.pin_histogram]),
    (m_keys_negatives_not_inverted, [P.pin_keys]),
    (m_keys_zero_signs_equal, [P.pin_keys]),
    (m_e2m1_subnormal, [P.pin_e2m1, P.pin_mxfp4_matches_fp8_path]),
    (m_mxfp4_nibbles_swapped, [P.pin_mxfp4_layout, P.pin_mxfp4_exact]),
    (m_mxfp4_scale_blocks_reversed, [P.pin_mxfp4_layout, P.pin_mxfp4_exact]),
    (m_mxfp4_scale_ignored, [P.pin_mxfp4_layout, P.pin_mxfp4_matches_fp8_path]),
    (m_e8m0_bias_128, [P.pin_e8m0, P.pin_mxfp4_exact]),
    (m_amax8_block_count, [P.pin_block_amax8]),
    (m_s2l_padding_mapped, [P.pin_sparse_to_logical_edges]),
    (m_s2l_past_table_clamped, [P.pin_sparse_to_logical_edges]),
    (m_amax8_newest_not_inf, [P.pin_block_amax8]),
    (m_sort_no_identity, [P.pin_sort_candidate_blocks]),
    (m_sort_slot_transform, [P.pin_sort_candidate_blocks]),
    (m_sparse_block_offset, [P.pin_sparse_logits]),
    (m_prefill_tables_reversed, [P.pin_prefill_decode_case, P.pin_prefill_exact]),
    (m_prefill_request_max_len, [P.pin_prefill_decode_case, P.pin_prefill_exact]),
    (m_prefill_boundary_row, [P.pin_prefill_decode_case, P.pin_prefill_exact]),
    (m_head_sum_no_relu, [P.pin_head_sum_exact]),
    (m_head_sum_scaled, [P.pin_head_sum_exact]),
    (m_bound_unscaled_keeps_scale, [P.pin_error_bound_exact]),
    (m_bound_signed_dots, [P.pin_error_bound_exact]),
    (m_waiver_on_finite, [P.pin_check_logits_classes]),
    (m_inf_sign_ignored, [P.pin_check_logits_classes]),
    (m_nan_matches_any_nonfinite, [P.pin_check_logits_classes]),
    (m_waiver_accepts_finite, [P.pin_check_logits_classes]),
]


@pytest.mark.parametrize("mutate,pins", MUTANTS, ids=[m.__name__ for m, _ in MUTANTS])
def test_pins_catch_planted_mistake(mutate, pins):
    O = fresh_oracle()
    mutate(O)
    fails = []
    for pin in pins:
        with np.errstate(all="ignore"):
            try:
                fails += pin(O)
            except Exception as e:  # a crash is also a caught mistake
                fails.append(f"{pin.__name__} raised {type(e).__name__}: {e}")
    assert fails, f"no pin caught {mutate.__name__}"


def test_fresh_copy_passes():
    O = fresh_oracle()
    assert not P.pin_bins_golden(O)
    assert math.isnan(O.E4M3FN[0x7F])
