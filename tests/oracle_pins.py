"""Checks that pin the CPU oracle to facts outside itself.

Each ``pin_*`` function takes the oracle module and returns a list of failure
messages (empty when the oracle passes).  ``test_oracle_pins.py`` runs them on
the real oracle; ``test_oracle_mutants.py`` runs them on copies of the oracle
with a planted mistake and requires at least one to fail.

What the pins lean on, none of which is the oracle's own code:
  * the OCP E4M3FN bit definition and PyTorch's float8_e4m3fn cast;
  * the E2M1 value table of the OCP MX specification (tests/golden/) and
    PyTorch's float8_e8m0fnu cast; hand-built MXFP4 tokens; the FP8 path on
    MXFP4 keys with one scale per token;
  * exact rational arithmetic (fractions.Fraction) for fp16 rounding, for the
    dot products and for the whole logit formula on tiny inputs;
  * hand-derived bins and keys in tests/golden/ (DeepGEMM PR #94 "What this
    adds" bin definition; vLLM PR #52696 FP16 keys);
  * closed-form bin populations over all 65,536 FP16 encodings;
  * histogram invariants (total = live non-NaN count; additivity; padding);
  * brute-force top-k with Python's sorted() and an explicit comparator;
  * for the candidate indexer: explicit loops for the block maxima, sorted()
    and the page transform per block, and the dense logits at the listed
    positions.
"""

from __future__ import annotations

import bisect
import math
import os
from fractions import Fraction

import numpy as np
import torch

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


# ---------------------------------------------------------------- helpers --
def load_golden_bins():
    vals, bins = [], []
    with open(os.path.join(GOLDEN, "coarse_bins_by_hand.txt")) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if not line:
                continue
            v, b = line.split()
            vals.append(float(v))
            bins.append(int(b))
    return np.array(vals, dtype=np.float32), np.array(bins, dtype=np.int64)


def load_golden_keys():
    out = []
    with open(os.path.join(GOLDEN, "score_keys_by_hand.txt")) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if not line:
                continue
            dt, v, k = line.split()
            out.append((dt, np.float32(float(v)), int(k, 16)))
    return out


def torch_e4m3_decode(codes) -> np.ndarray:
    t = torch.from_numpy(np.ascontiguousarray(codes, dtype=np.uint8))
    return t.view(torch.float8_e4m3fn).float().numpy().astype(np.float64)


_FP16_POS = None


def _fp16_positive_values():
    """Exact values of all finite non-negative fp16 encodings 0x0000..0x7BFF."""
    global _FP16_POS
    if _FP16_POS is None:
        vals = []
        for bits in range(0x7C00):
            e, m = bits >> 10, bits & 0x3FF
            if e == 0:
                vals.append(Fraction(m, 1 << 24))
            else:
                vals.append(Fraction(1024 + m, 1024) * Fraction(2) ** (e - 15))
        _FP16_POS = vals
    return _FP16_POS


def fraction_rne_fp16_bits(x: float) -> int:
    """IEEE binary16 round-to-nearest-even of a finite double, by exact search."""
    vals = _fp16_positive_values()
    sign = 0x8000 if math.copysign(1.0, x) < 0 else 0
    a = abs(Fraction(x))
    if a >= Fraction(65520):
        return sign | 0x7C00
    i = bisect.bisect_left(vals, a)
    if i < len(vals) and vals[i] == a:
        return sign | i
    lo, hi = i - 1, i
    if hi >= len(vals):
        return sign | lo
    dlo, dhi = a - vals[lo], vals[hi] - a
    if dlo < dhi:
        return sign | lo
    if dhi < dlo:
        return sign | hi
    return sign | (lo if lo % 2 == 0 else hi)


# ------------------------------------------------------------------- pins --
def pin_e4m3(O):
    fails = []
    codes = np.arange(256, dtype=np.uint8)
    got = O.decode_e4m3fn(codes)
    ref = torch_e4m3_decode(codes)
    nan_g, nan_r = np.isnan(got), np.isnan(ref)
    if not np.array_equal(nan_g, nan_r):
        fails.append("e4m3 NaN codes differ from torch float8_e4m3fn")
    ok = ~nan_r
    if not np.array_equal(got[ok], ref[ok]):
        fails.append("e4m3 values differ from torch float8_e4m3fn")
    spot = {0x7E: 448.0, 0x08: 2.0 ** -6, 0x01: 2.0 ** -9, 0x38: 1.0,
            0xFE: -448.0, 0x07: 7 * 2.0 ** -9}
    for c, v in spot.items():
        if got[c] != v:
            fails.append(f"e4m3 code {c:#x} -> {got[c]}, spec says {v}")
    if not (np.isnan(got[0x7F]) and np.isnan(got[0xFF])):
        fails.append("e4m3 0x7F/0xFF must be NaN")
    if not (got[0x80] == 0 and math.copysign(1, got[0x80]) < 0):
        fails.append("e4m3 0x80 must be -0")
    return fails


def pin_fp16_rne(O, n_random=20000, seed=7):
    fails = []
    # every fp16 value round-trips
    allh = np.arange(65536, dtype=np.uint32).astype(np.uint16).view(np.float16)
    fin = ~np.isnan(allh)
    back = O.fp16_rne(allh[fin].astype(np.float32)).view(np.uint16)
    if not np.array_equal(back, allh[fin].view(np.uint16)):
        fails.append("fp16_rne does not round-trip fp16 values")
    # midpoints between adjacent non-negative fp16 values, and +-1 fp32 ulp
    vals = _fp16_positive_values()
    mids = np.array([float((vals[i] + vals[i + 1]) / 2) for i in range(len(vals) - 1)]
                    + [65520.0], dtype=np.float32)
    up = np.nextafter(mids, np.float32(np.inf))
    dn = np.nextafter(mids, np.float32(0))
    rng = np.random.default_rng(seed)
    rnd = rng.integers(0, 0x7F800000, n_random, dtype=np.uint32).view(np.float32)
    probe = np.concatenate([mids, up, dn, rnd, -mids[::97], -rnd[::7]])
    got = O.fp16_rne(probe).view(np.uint16).astype(np.int64)
    want = np.array([fraction_rne_fp16_bits(float(v)) for v in probe], dtype=np.int64)
    bad = np.nonzero(got != want)[0]
    if bad.size:
        v = probe[bad[0]]
        fails.append(f"fp16_rne({v!r}) = {got[bad[0]]:#06x}, exact RNE {want[bad[0]]:#06x}"
                     f" ({bad.size} mismatches)")
    return fails


def pin_bins_golden(O):
    vals, bins = load_golden_bins()
    got = O.coarse_bin(vals)
    bad = np.nonzero(got != bins)[0]
    return [f"bin({vals[i]!r}) = {got[i]}, hand-derived {bins[i]}" for i in bad]


def pin_bins_exhaustive(O):
    """All 65,536 fp16 encodings: NaN excluded, order, closed-form populations."""
    fails = []
    enc = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    x = enc.view(np.float16).astype(np.float32)
    b = O.coarse_bin(x)
    nan = np.isnan(x)
    if not np.all(b[nan] == -1):
        fails.append("NaN encodings must get no bin")
    if np.any((b[~nan] < 0) | (b[~nan] > 1023)):
        fails.append("bins outside 0..1023")
    # non-increasing in value; -0 sorts below +0
    v = x[~nan].astype(np.float64)
    neg = np.signbit(x[~nan])
    order = np.lexsort((~neg, v))
    bs = b[~nan][order]
    if np.any(np.diff(bs) > 0):
        fails.append("bin is not non-increasing in the score")
    counts = np.bincount(b[~nan], minlength=1024)
    expect = np.zeros(1024, dtype=np.int64)
    for m in range(512):
        if m < 304:
            c = 64
        elif m < 511:
            k = m - 288
            c = 2 ** (10 - int(math.floor(math.log2(k))))
        else:
            c = 0x7C00 - 0x5AF8 + 1  # encodings of 223.0 .. +inf
        expect[511 - m] = c
        expect[512 + m] = c
    if not np.array_equal(counts, expect):
        d = np.nonzero(counts != expect)[0]
        fails.append(f"bin populations differ from closed form at bins {d[:8]}")
    # fine regime equals the reversed 10-bit fp16 coarse key
    mag = np.abs(x)
    fine = (~nan) & (mag < 16)
    k16 = np.where(enc >> 15 == 1, (~enc.astype(np.uint32)) & 0xFFFF,
                   enc.astype(np.uint32) | 0x8000)
    if not np.array_equal(b[fine], 1023 - (k16[fine] >> 6)):
        fails.append("fine regime is not the reversed 10-bit fp16 coarse key")
    return fails


def pin_keys(O):
    with np.errstate(over="ignore", invalid="ignore"):
        return _pin_keys(O)


def _pin_keys(O):
    fails = []
    for dt, v, k in load_golden_keys():
        kd = O.KEY_FP32 if dt == "fp32" else O.KEY_FP16
        got = int(O.score_keys(np.array([v], np.float32), kd)[0])
        if got != k:
            fails.append(f"{dt} key({v!r}) = {got:#x}, hand-derived {k:#x}")
    # integer order of keys is the value order (-0 below +0), both dtypes
    rng = np.random.default_rng(11)
    x = np.concatenate([rng.standard_normal(3000).astype(np.float32) * 50,
                        np.array([0.0, -0.0, np.inf, -np.inf, 1e-30, -1e-30,
                                  65519.0, 65521.0, -65521.0], np.float32)])
    for kd, val in ((O.KEY_FP32, x.astype(np.float64)),
                    (O.KEY_FP16, x.astype(np.float16).astype(np.float64))):
        keys = O.score_keys(x, kd).astype(np.float64)
        neg = np.signbit(x if kd == O.KEY_FP32 else x.astype(np.float16))
        order = np.lexsort((~neg, val))
        ks = keys[order]
        if np.any(np.diff(ks) < 0):
            fails.append(f"keys (dtype {kd}) do not follow the value order")
        same = (np.diff(val[order]) == 0) & (np.diff(neg[order].astype(int)) == 0)
        if np.any(np.diff(ks)[same] != 0):
            fails.append(f"equal values get different keys (dtype {kd})")
    return fails


def pin_bins_coarsen_keys(O, seed=5):
    """bin(x) < bin(y) implies key(x) > key(y), for FP32 and FP16 keys."""
    rng = np.random.default_rng(seed)
    vals, _ = load_golden_bins()
    x = np.concatenate([vals[~np.isnan(vals)],
                        (rng.standard_normal(4000) * 80).astype(np.float32),
                        (rng.standard_normal(2000) * 4).astype(np.float32)])
    b = O.coarse_bin(x)
    fails = []
    for kd in (O.KEY_FP32, O.KEY_FP16):
        k = O.score_keys(x, kd).astype(np.float64)
        # within increasing bins, max key of a later bin < min key of an earlier
        ub = np.unique(b)
        mins = np.array([k[b == u].min() for u in ub])
        maxs = np.array([k[b == u].max() for u in ub])
        if np.any(maxs[1:] >= mins[:-1]):
            fails.append(f"bins do not coarsen the key order (dtype {kd})")
    return fails


def pin_histogram(O, seed=3):
    fails = []
    rng = np.random.default_rng(seed)
    rows, n = 5, 3000
    x = (rng.standard_normal((rows, n)) * rng.choice([0.5, 8, 90], (rows, 1))
         ).astype(np.float32)
    x[0, 10:20] = np.nan
    x[1, :5] = [np.inf, -np.inf, 0.0, -0.0, np.nan]
    lens = np.array([n, n - 7, 100, 0, 2999], dtype=np.int32)
    pad_val = np.float32(1e30)  # would land in bin 0
    for r in range(rows):
        x[r, lens[r]:] = pad_val
    h = O.coarse_histogram(x, lens)
    live = np.array([np.sum(~np.isnan(x[r, :lens[r]])) for r in range(rows)])
    if not np.array_equal(h.sum(axis=1), live):
        fails.append("histogram total != live non-NaN count")
    h2 = O.coarse_histogram(x, lens, hist_in=h)
    if not np.array_equal(h2, 2 * h):
        fails.append("histogram does not accumulate onto the incoming counts")
    x2 = x.copy()
    for r in range(rows):
        x2[r, lens[r]:] = -pad_val
    if not np.array_equal(O.coarse_histogram(x2, lens), h):
        fails.append("padding columns change the histogram")
    # brute force on one short row with the hand-checked bin values
    vals, bins = load_golden_bins()
    hv = O.coarse_histogram(vals[None, :], np.array([vals.size], np.int32))[0]
    want = np.zeros(1024, np.int64)
    for bb in bins:
        if bb >= 0:
            want[bb] += 1
    if not np.array_equal(hv, want):
        fails.append("histogram of the hand-derived values is wrong")
    return fails


def _brute_topk(x, length, k, key_dtype):
    """Top-k by sorted() with an explicit comparator, no oracle code."""
    items = []
    for i in range(length):
        v = float(x[i])
        if math.isnan(v):
            continue
        if key_dtype == 1:
            v = float(np.float16(np.float32(x[i])))
        positive_zero_first = 0 if math.copysign(1.0, v) > 0 else 1
        items.append((-v, positive_zero_first, i))
    items.sort()
    return sorted(i for _, _, i in items[:k])


def pin_topk(O, seed=9):
    fails = []
    rng = np.random.default_rng(seed)
    cases = []
    for n, k in ((50, 7), (300, 64), (1000, 1000), (257, 300), (2048, 100)):
        x = (rng.standard_normal(n) * 3).astype(np.float32)
        x[rng.integers(0, n, n // 10)] = np.float32(1.5)  # fp32 ties
        x[rng.integers(0, n, 3)] = np.nan
        x[rng.integers(0, n, 2)] = np.inf
        x[rng.integers(0, n, 2)] = -0.0
        x[rng.integers(0, n, 2)] = 0.0
        cases.append((x, n - 3, k))
    # many fp32 values sharing one fp16 value
    y = (np.float32(20.0) + rng.integers(0, 8, 600).astype(np.float32)
         * np.float32(2.0 ** -10)).astype(np.float32)
    cases.append((y, 600, 37))
    for x, length, k in cases:
        for kd in (O.KEY_FP32, O.KEY_FP16):
            got = list(O.topk_row(x, length, k, kd))
            want = _brute_topk(x, length, k, kd)
            if got != want:
                fails.append(f"top-{k} of a length-{length} row (dtype {kd}) "
                             f"differs from brute force")
    # special cases with known answers
    n, k = 500, 64
    const = np.full(n, 2.5, np.float32)
    if list(O.topk_row(const, n, k, O.KEY_FP32)) != list(range(k)):
        fails.append("constant row must select the lowest k indices")
    inc = np.arange(n, dtype=np.float32)
    if list(O.topk_row(inc, n, k, O.KEY_FP32)) != list(range(n - k, n)):
        fails.append("increasing row must select the last k indices")
    nan = np.full(n, np.nan, np.float32)
    out = O.topk_rows(nan[None, :], np.array([n], np.int32), k, O.KEY_FP32)
    if not np.all(out == -1):
        fails.append("all-NaN row must give only -1")
    short = O.topk_rows(inc[None, :], np.array([10], np.int32), k, O.KEY_FP32)[0]
    if list(short[:10]) != list(range(10)) or not np.all(short[10:] == -1):
        fails.append("a row with fewer live scores than k selects all, then -1")
    return fails


def pin_topk_invariants(O, seed=13):
    fails = []
    rng = np.random.default_rng(seed)
    for _ in range(6):
        n = int(rng.integers(3000, 9000))
        k = int(rng.integers(1, 2500))
        x = (rng.standard_normal(n) * rng.choice([1, 30, 300])).astype(np.float32)
        x[rng.integers(0, n, 50)] = np.float32(x[0])
        for kd in (O.KEY_FP32, O.KEY_FP16):
            sel = O.topk_row(x, n, k, kd)
            keys = O.score_keys(x, kd).astype(np.int64)
            mask = np.zeros(n, bool)
            mask[sel] = True
            if sel.size != min(k, n) or np.unique(sel).size != sel.size:
                fails.append("selected set has the wrong size")
                continue
            if mask.all():
                continue
            t = keys[mask].min()
            if keys[~mask].max() > t:
                fails.append("an unselected score outranks a selected one")
            tie_out = np.nonzero((~mask) & (keys == t))[0]
            tie_in = np.nonzero(mask & (keys == t))[0]
            if tie_out.size and tie_in.size and tie_out.min() < tie_in.max():
                fails.append("ties not broken by the lower index")
    return fails


def _tiny_logit_inputs(seed=21, B=2, next_n=2, base=70, weight_scale=1.0):
    import gen
    return gen.make_indexer_inputs("tiny", B, next_n, [base + 3 * b for b in range(B)],
                                   seed, weight_scale=weight_scale)


def pin_logits_exact(O, n_cols=6):
    """The whole formula in exact rationals, rounded once to float32."""
    fails = []
    x = _tiny_logit_inputs()
    got = O.indexer_logits(x.q, x.kv_pages, x.k_scales, x.weights, x.block_table,
                           x.context_lens, x.next_n, x.logits_stride)
    rng = np.random.default_rng(1)
    for r in range(x.rows):
        b = r // x.next_n
        n = int(x.context_lens[r])
        qd = torch_e4m3_decode(x.q[r])
        cols = sorted(set(rng.integers(0, n, n_cols).tolist()) | {0, n - 1})
        for s in cols:
            page = int(x.block_table[b, s // 64])
            slot = s % 64
            kd = torch_e4m3_decode(x.kv_pages[page, slot])
            sc = Fraction(float(x.k_scales[page, slot]))
            total = Fraction(0)
            for h in range(32):
                dot = sum((Fraction(float(qd[h, d])) * Fraction(float(kd[d]))
                           for d in range(128)), Fraction(0))
                if dot > 0:
                    total += Fraction(float(x.weights[r, h])) * dot
            want = np.float32(float(sc * total))
            g = got[r, s]
            ulp = np.spacing(np.float32(abs(want))) if want != 0 else np.float32(1e-45)
            if not abs(float(g) - float(want)) <= float(ulp):
                fails.append(f"logit[{r},{s}] = {g}, exact {want}")
        if not np.all(np.isnan(got[r, n:])):
            fails.append(f"row {r}: columns past the length were written")
    return fails


def pin_logits_library(O):
    """Unit weights and scales, one page: sum_h ReLU(Q K^T) by a numpy matmul."""
    import gen
    x = gen.make_indexer_inputs("lib", 1, 1, [64], 31)
    x.weights[:] = 1.0
    x.k_scales[:] = 1.0
    got = O.indexer_logits(x.q, x.kv_pages, x.k_scales, x.weights, x.block_table,
                           x.context_lens, 1, 64)
    page = int(x.block_table[0, 0])
    qd = torch_e4m3_decode(x.q[0])
    kd = torch_e4m3_decode(x.kv_pages[page])
    want = np.maximum(np.matmul(qd, kd.T), 0).sum(axis=0).astype(np.float32)
    if not np.array_equal(got[0], want):
        return ["unit-weight one-page logits differ from sum_h ReLU(Q K^T)"]
    return []


def pin_logits_paging(O):
    """Permuting physical pages together with the block table changes nothing."""
    x = _tiny_logit_inputs(seed=23, B=3, next_n=2, base=150)
    a = O.indexer_logits(x.q, x.kv_pages, x.k_scales, x.weights, x.block_table,
                         x.context_lens, x.next_n, x.logits_stride)
    perm = np.random.default_rng(2).permutation(x.num_pages)
    inv = np.argsort(perm)
    kv2 = x.kv_pages[perm]
    sc2 = x.k_scales[perm]
    bt2 = inv[x.block_table].astype(np.int32)
    bt2[x.block_table < 0] = 0
    b = O.indexer_logits(x.q, kv2, sc2, x.weights, bt2, x.context_lens,
                         x.next_n, x.logits_stride)
    if not np.array_equal(a, b, equal_nan=True):
        return ["logits change when pages are permuted with the block table"]
    return []


def pin_error_bound(O):
    """An fp32 evaluation of the formula sits inside the bound; 3x bound fails."""
    fails = []
    x = _tiny_logit_inputs(seed=25, B=1, next_n=1, base=200, weight_scale=3.0)
    want = O.indexer_logits(x.q, x.kv_pages, x.k_scales, x.weights, x.block_table,
                            x.context_lens, 1, x.logits_stride)[0]
    cols = np.arange(200)
    bound = O.logits_error_bound_at(x.q, x.kv_pages, x.k_scales, x.weights,
                                    x.block_table, 1, 0, cols)
    qd = torch_e4m3_decode(x.q[0]).astype(np.float32)
    pages = x.block_table[0, cols // 64]
    kd = torch_e4m3_decode(x.kv_pages[pages, cols % 64]).astype(np.float32)
    sc = x.k_scales[pages, cols % 64]
    # sequential float32 accumulation, vectorised over the 200 keys
    acc = np.zeros(200, np.float32)
    for h in range(32):
        dot = np.zeros(200, np.float32)
        for d in range(128):
            dot = (dot + qd[h, d] * kd[:, d]).astype(np.float32)
        acc = (acc + x.weights[0, h] * np.maximum(dot, np.float32(0))).astype(np.float32)
    f32 = (acc * sc).astype(np.float32)
    if not np.all(O.check_logits(f32, want, bound)):
        fails.append("a plain fp32 evaluation falls outside the tolerance")
    bad = want + 3 * bound.astype(np.float32)
    moved = 3 * bound > np.spacing(np.abs(want))
    if np.any(O.check_logits(bad, want, bound)[moved]):
        fails.append("a 3x-bound error is accepted")
    return fails



# ------------------------------------------------- acceptance helpers --
def _exact_dots(qd, kd):
    """Exact rational q_h . k for the 32 heads (qd [32,128], kd [128])."""
    return [sum((Fraction(float(qd[h, d])) * Fraction(float(kd[d])) for d in range(128)),
                Fraction(0)) for h in range(32)]


def _exact_abs_dots(qd, kd):
    return [sum((abs(Fraction(float(qd[h, d])) * Fraction(float(kd[d]))) for d in range(128)),
                Fraction(0)) for h in range(32)]


def _acceptance_inputs():
    """Tiny inputs with an infinite K scale on some slots, so that the head
    sum and the scaled logit part ways (the mixed verify workload's case)."""
    import gen
    x = gen.make_indexer_inputs("acc", 1, 2, [130], 41, weight_scale=2.0)
    # scales spread over several binades so that scaled and unscaled differ
    rng = np.random.default_rng(3)
    x.k_scales[:] = (2.0 ** rng.integers(-12, 6, size=x.k_scales.shape)).astype(np.float32)
    x.k_scales[x.block_table[0, 0], [3, 17]] = np.inf
    x.k_scales[x.block_table[0, 1], 5] = np.inf
    return x


def pin_head_sum_exact(O):
    """head_sum_at = sum_h w_h * ReLU(q_h . k_s) in exact rationals, before
    any K scale (also where the scale is infinite), within the float64
    rounding of a 32-term sum (gamma_32 of the absolute terms)."""
    fails = []
    x = _acceptance_inputs()
    cols = np.array([0, 3, 17, 40, 64 + 5, 64 + 30, 129])
    for r in range(x.rows):
        got = O.head_sum_at(x.q, x.kv_pages, x.k_scales, x.weights, x.block_table,
                            x.next_n, r, cols)
        qd = torch_e4m3_decode(x.q[r])
        for i, s in enumerate(cols.tolist()):
            page = int(x.block_table[r // x.next_n, s // 64])
            kd = torch_e4m3_decode(x.kv_pages[page, s % 64])
            terms = [Fraction(float(x.weights[r, h])) * d
                     for h, d in enumerate(_exact_dots(qd, kd)) if d > 0]
            exact = sum(terms, Fraction(0))
            tol = 32 * 2.0 ** -53 * float(sum((abs(t) for t in terms), Fraction(0)))
            if not (math.isfinite(float(got[i])) and abs(Fraction(float(got[i])) - exact) <= Fraction(tol)):
                fails.append(f"head_sum row {r} col {s}: {got[i]!r}, exact {float(exact)!r}")
    return fails


def pin_error_bound_exact(O):
    """logits_error_bound_at = rel * |sc_s| * sum_h |w_h| * sum_d |q_hd k_sd|
    (and without |sc_s| when unscaled) in exact rationals, to float64
    rounding; scales spread over 2^-12 .. 2^5 so the two modes differ."""
    fails = []
    x = _acceptance_inputs()
    cols = np.array([1, 3, 20, 64 + 5, 64 + 63, 128])
    rel = 1e-5
    for r in range(x.rows):
        scaled = O.logits_error_bound_at(x.q, x.kv_pages, x.k_scales, x.weights,
                                         x.block_table, x.next_n, r, cols, rel=rel)
        unscaled = O.logits_error_bound_at(x.q, x.kv_pages, x.k_scales, x.weights,
                                           x.block_table, x.next_n, r, cols, rel=rel,
                                           unscaled=True)
        qd = torch_e4m3_decode(x.q[r])
        for i, s in enumerate(cols.tolist()):
            page = int(x.block_table[r // x.next_n, s // 64])
            kd = torch_e4m3_decode(x.kv_pages[page, s % 64])
            head = sum((abs(Fraction(float(x.weights[r, h]))) * a
                        for h, a in enumerate(_exact_abs_dots(qd, kd))), Fraction(0))
            want_u = Fraction(rel) * head
            if abs(Fraction(float(unscaled[i])) - want_u) > want_u * Fraction(1, 2 ** 40):
                fails.append(f"unscaled bound row {r} col {s}: {unscaled[i]!r} vs {float(want_u)!r}")
            sc = float(x.k_scales[page, s % 64])
            if math.isinf(sc):
                if not np.isinf(scaled[i]):
                    fails.append(f"scaled bound at an infinite scale is {scaled[i]!r}")
                continue
            want_s = want_u * abs(Fraction(sc))
            if abs(Fraction(float(scaled[i])) - want_s) > want_s * Fraction(1, 2 ** 40):
                fails.append(f"scaled bound row {r} col {s}: {scaled[i]!r} vs {float(want_s)!r}")
    return fails


def pin_check_logits_classes(O):
    """check_logits on hand-built cases.  A finite expected value is judged by
    |got - want| <= bound alone (the near-zero waiver never widens it).  A
    non-finite expected value (an infinite K scale) is judged by class: NaN
    matches NaN, an infinity the same infinity; the waiver -- the unscaled
    head sum within its own tolerance of zero, so its sign is rounding --
    accepts any infinity or NaN, never a finite value, and a wrong-signed
    infinity with a large head sum is refused."""
    inf, nan = np.inf, np.nan
    # got, want, bound, head_sum, head_bound, accepted
    cases = [
        (1.0, 1.0, 0.0, 0.0, 1.0, True),
        (1.5, 1.0, 0.5, 0.0, 1.0, True),
        (1.5, 1.0, 0.25, 0.0, 1.0, False),      # waiver not for finite values
        (5.0, 1.0, 1.0, 1e-9, 1.0, False),
        (-1.0, 1.0, 1.0, 0.0, 1.0, False),
        (inf, 1.0, 1.0, 0.0, 1.0, False),
        (nan, 1.0, 1.0, 0.0, 1.0, False),
        (nan, nan, inf, 0.0, 1e-5, True),        # NaN <-> NaN
        (nan, nan, inf, 3.0, 1e-5, True),
        (inf, nan, inf, 0.0, 1e-5, True),        # head sum zero: either class
        (-inf, nan, inf, 0.0, 1e-5, True),
        (inf, nan, inf, 3.0, 1e-5, False),
        (inf, inf, inf, 5.0, 1e-4, True),
        (-inf, -inf, inf, -5.0, 1e-4, True),
        (-inf, inf, inf, 5.0, 1e-4, False),      # wrong sign, large head sum
        (inf, -inf, inf, -5.0, 1e-4, False),
        (nan, inf, inf, 5.0, 1e-4, False),
        (-inf, inf, inf, 5e-5, 1e-4, True),      # head sum within rounding of 0
        (nan, -inf, inf, -1e-4, 1e-4, True),
        (-inf, inf, inf, 1.0001e-4, 1e-4, False),
        (1e30, inf, inf, 1e-6, 1e-4, False),     # a finite value is never an inf
        (0.0, nan, inf, 0.0, 1e-5, False),
    ]
    fails = []
    g, w, b, hs, hb, acc = (np.array(c, dtype=np.float64) for c in zip(*cases))
    got = O.check_logits(g, w, b, hs, hb)
    for i, case in enumerate(cases):
        if bool(got[i]) != case[-1]:
            fails.append(f"check_logits{case[:-1]} = {bool(got[i])}, expected {case[-1]}")
    # without head sums, no waiver at all
    got = O.check_logits(np.array([inf, -inf, nan]), np.array([nan, inf, -inf]),
                         np.array([inf, inf, inf]))
    if got.any():
        fails.append(f"class mismatches accepted without a waiver: {got.tolist()}")
    # from the formula: at an infinite scale the logit is the head sum's sign
    # times infinity (NaN for a zero sum); flipping that sign is refused
    # wherever the head sum is clear of its tolerance
    x = _acceptance_inputs()
    cols = np.arange(130)
    for r in range(x.rows):
        want = O.indexer_logits_at(x.q, x.kv_pages, x.k_scales, x.weights, x.block_table,
                                   x.next_n, r, cols)
        bound = O.logits_error_bound_at(x.q, x.kv_pages, x.k_scales, x.weights,
                                        x.block_table, x.next_n, r, cols)
        hs = O.head_sum_at(x.q, x.kv_pages, x.k_scales, x.weights, x.block_table,
                           x.next_n, r, cols)
        hb = O.logits_error_bound_at(x.q, x.kv_pages, x.k_scales, x.weights,
                                     x.block_table, x.next_n, r, cols, unscaled=True)
        nf = ~np.isfinite(want)
        if nf.sum() != 3:
            fails.append(f"row {r}: expected 3 infinite-scale logits, got {int(nf.sum())}")
        for c in np.nonzero(nf)[0]:
            sign = np.sign(hs[c])
            expect = np.nan if sign == 0 else sign * np.inf
            if not (np.isnan(want[c]) if sign == 0 else want[c] == expect):
                fails.append(f"row {r} col {c}: logit {want[c]} vs head sum {hs[c]}")
            if abs(hs[c]) > hb[c] and sign != 0:
                if O.check_logits(np.array([-expect]), want[c:c + 1], bound[c:c + 1],
                                  hs[c:c + 1], hb[c:c + 1])[0]:
                    fails.append(f"row {r} col {c}: the wrong-signed infinity is accepted")
            if not O.check_logits(want[c:c + 1], want[c:c + 1], bound[c:c + 1],
                                  hs[c:c + 1], hb[c:c + 1])[0]:
                fails.append(f"row {r} col {c}: the oracle's own value is refused")
    return fails


def pin_logits_terms_match(O):
    """logits_terms_at (one gather for all four terms) gives, row for row,
    exactly what indexer_logits_at, logits_error_bound_at (both modes) and
    head_sum_at give -- on FP8 keys with infinite scales and on MXFP4 keys."""
    import gen
    fails = []
    xs = [_acceptance_inputs(),
          gen.make_indexer_inputs("terms_mx", 2, 3, [200, 77], 43, kfmt="mxfp4")]
    for x in xs:
        for b in range(x.B):
            rows = list(range(b * x.next_n, (b + 1) * x.next_n))
            cols = np.arange(int(x.context_lens[rows].max()))
            want, bound, hs, hb = O.logits_terms_at(x.q, x.kv_pages, x.k_scales, x.weights,
                                                    x.block_table, x.next_n, rows, cols)
            for i, r in enumerate(rows):
                ref = (O.indexer_logits_at(x.q, x.kv_pages, x.k_scales, x.weights, x.block_table,
                                           x.next_n, r, cols),
                       O.logits_error_bound_at(x.q, x.kv_pages, x.k_scales, x.weights,
                                               x.block_table, x.next_n, r, cols),
                       O.head_sum_at(x.q, x.kv_pages, x.k_scales, x.weights, x.block_table,
                                     x.next_n, r, cols),
                       O.logits_error_bound_at(x.q, x.kv_pages, x.k_scales, x.weights,
                                               x.block_table, x.next_n, r, cols, unscaled=True))
                for name, got, want_ in zip(("logits", "bound", "head_sum", "head_bound"),
                                            (want[i], bound[i], hs[i], hb[i]), ref):
                    if not np.array_equal(got, want_, equal_nan=True):
                        fails.append(f"{x.name} row {r}: {name} differs from the separate helper")
    return fails


def _f32_between(lo, hi):
    """Every float32 in [lo, hi] (float64 bounds), by bit pattern."""
    a = np.float32(lo)
    if float(a) < lo:
        a = np.nextafter(a, np.float32(np.inf))
    b = np.float32(hi)
    if float(b) > hi:
        b = np.nextafter(b, np.float32(-np.inf))
    if float(a) > float(b):
        return np.zeros(0, np.float32)
    ia, ib = int(np.array(a).view(np.int32)), int(np.array(b).view(np.int32))
    if float(a) >= 0:  # both non-negative: bit order = value order
        return np.arange(ia, ib + 1, dtype=np.int64).astype(np.int32).view(np.float32)
    if float(b) < 0:   # both negative: bit order reversed
        return np.arange(ib, ia + 1, dtype=np.int64).astype(np.int32).view(np.float32)
    neg = np.arange(0x80000000, ia + (1 << 32) + 1, dtype=np.int64) & 0xFFFFFFFF
    pos = np.arange(0, ib + 1, dtype=np.int64)
    return np.concatenate([neg, pos]).astype(np.uint32).view(np.float32)


def pin_logits_f16_check(O, seed=31):
    """check_logits_f16 accepts exactly the halves that some float32 within the
    bound rounds to: brute force over every such float32 (the definition),
    against all halves near them; plus hand cases at a rounding tie."""
    fails = []
    rng = np.random.default_rng(seed)
    cases = [(1.0, 2.0 ** -12), (1.0, 2.0 ** -11), (-3.0, 2.0 ** -9), (0.0, 1e-7), (65504.0, 16.0),
             (65519.0, 1.0), (1e-6, 1e-8), (-2.0 ** -14, 2.0 ** -26)]
    for _ in range(40):
        mag = 10.0 ** rng.uniform(-6, 4.5)
        want = float(np.float32(rng.choice([-1, 1]) * mag))
        cases.append((want, abs(want) * 10.0 ** rng.uniform(-7, -3)))
    halves = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16).view(np.float16)
    finite_halves = halves[np.isfinite(halves)]
    for want, bound in cases:
        ys = _f32_between(want - bound, want + bound)
        if ys.size == 0 or ys.size > 3_000_000:
            continue
        reach = np.unique(O.fp16_rne(ys).view(np.uint16))
        got = O.check_logits_f16(finite_halves, np.full(finite_halves.shape, want),
                                 np.full(finite_halves.shape, bound))
        accepted = np.unique(finite_halves[got].view(np.uint16))
        reach_f = reach[np.isfinite(reach.view(np.float16))]
        if not np.array_equal(np.sort(accepted), np.sort(reach_f)):
            fails.append(f"want {want!r} bound {bound!r}: accepted "
                         f"{finite_halves[got][:4].tolist()} vs reachable {reach.view(np.float16)[:4].tolist()}")
    # 1 - 2^-12 is the tie between the halves 1 - 2^-11 and 1: even -> 1.0
    one = O.check_logits_f16(np.array([1.0, 1 - 2 ** -11, 1 + 2 ** -10], np.float16),
                             np.array([1.0] * 3), np.array([2.0 ** -12] * 3))
    if one.tolist() != [True, False, False]:
        fails.append(f"tie case: {one.tolist()}")
    # infinities by class; an overflowing finite value rounds to infinity
    cls = O.check_logits_f16(np.array([np.inf, -np.inf, np.inf], np.float16),
                             np.array([np.inf, -np.inf, 70000.0]), np.array([1.0, 1.0, 1.0]))
    if cls.tolist() != [True, True, True]:
        fails.append(f"non-finite classes: {cls.tolist()}")
    return fails

# ---------------------------------------------------------- MXFP4 keys --
def load_golden_e2m1():
    vals = {}
    with open(os.path.join(GOLDEN, "e2m1_values_by_hand.txt")) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if line:
                c, v = line.split()
                vals[int(c)] = float(v)
    return vals


def pin_e2m1(O):
    """The 16 E2M1 values against the hand-written table from the MX spec,
    signed zeros included."""
    fails = []
    want = load_golden_e2m1()
    for c in range(16):
        got = float(O.E2M1[c])
        if got != want[c] or math.copysign(1.0, got) != math.copysign(1.0, want[c]):
            fails.append(f"E2M1 code {c}: {got}, want {want[c]}")
    return fails


def pin_e8m0(O):
    """All 256 E8M0 scale bytes against PyTorch's float8_e8m0fnu cast."""
    codes = np.arange(256, dtype=np.uint8)
    with np.errstate(invalid="ignore"):
        want = torch.from_numpy(codes).view(torch.float8_e8m0fnu).float().numpy().astype(np.float64)
    got = O.decode_e8m0(codes)
    if not np.array_equal(got, want, equal_nan=True):
        bad = np.nonzero(~((got == want) | (np.isnan(got) & np.isnan(want))))[0][:5]
        return [f"E8M0 codes {bad.tolist()} differ from torch"]
    return []


def pin_mxfp4_layout(O):
    """Hand-built tokens: dimension 2i in the low nibble of byte i, 2i+1 in the
    high nibble; scale byte j covers dimensions 32j .. 32j+31."""
    fails = []
    tok = np.zeros((2, 68), dtype=np.uint8)
    tok[0, 0] = 0x2B      # dim 0: code 0xB = -1.5, dim 1: code 2 = 1.0
    tok[0, 20] = 0x70     # dim 40: 0, dim 41: code 7 = 6.0
    tok[0, 63] = 0x0D     # dim 126: code 0xD = -3.0, dim 127: 0
    tok[0, 64:68] = [127, 128, 125, 130]   # 1, 2, 1/4, 8
    tok[1, :64] = 0x11    # every dimension 0.5
    tok[1, 64:68] = [0, 254, 255, 127]     # 2^-127, 2^127, NaN, 1
    want0 = np.zeros(128)
    want0[0], want0[1], want0[41], want0[126] = -1.5, 1.0, 6.0 * 2, -3.0 * 8
    got = O.dequant_mxfp4_tokens(tok)
    if not np.array_equal(got[0], want0):
        fails.append(f"token 0: nonzero dims {np.nonzero(got[0])[0].tolist()} "
                     f"values {got[0][np.nonzero(got[0])[0]].tolist()}")
    want1 = np.concatenate([np.full(32, 0.5 * 2.0 ** -127), np.full(32, 0.5 * 2.0 ** 127),
                            np.full(32, np.nan), np.full(32, 0.5)])
    if not np.array_equal(got[1], want1, equal_nan=True):
        fails.append("token 1: block scales misapplied")
    return fails


def _mxfp4_as_fp8(x, scale_bytes):
    """FP8 pages + per-token scales holding exactly the keys of MXFP4 pages
    whose four block scales are all equal (every E2M1 value is an E4M3 value)."""
    codes = np.empty(x.kv_pages.shape[:2] + (128,), dtype=np.uint8)
    codes[..., 0::2] = x.kv_pages[..., :64] & 0x0F
    codes[..., 1::2] = x.kv_pages[..., :64] >> 4
    vals = load_golden_e2m1()
    table = np.array([vals[c] for c in range(16)], dtype=np.float32)
    kv8 = torch.from_numpy(table[codes]).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    sc = np.ldexp(np.float32(1.0), scale_bytes.astype(np.int64) - 127).astype(np.float32)
    return kv8, sc


def pin_mxfp4_matches_fp8_path(O):
    """With one scale per token, MXFP4 logits equal the FP8-path logits of the
    same keys written as E4M3 codes with that scale (bitwise)."""
    import gen
    x = gen.make_indexer_inputs("mx", 2, 2, [150, 131], 41, kfmt="mxfp4")
    rng = np.random.default_rng(4)
    per_tok = rng.integers(120, 134, size=x.kv_pages.shape[:2]).astype(np.uint8)
    x.kv_pages[..., 64:68] = per_tok[..., None]
    got = O.indexer_logits(x.q, x.kv_pages, None, x.weights, x.block_table,
                           x.context_lens, x.next_n, x.logits_stride)
    kv8, sc = _mxfp4_as_fp8(x, per_tok)
    want = O.indexer_logits(x.q, kv8, sc, x.weights, x.block_table,
                            x.context_lens, x.next_n, x.logits_stride)
    if not np.array_equal(got, want, equal_nan=True):
        return ["MXFP4 logits differ from the FP8 path on equal block scales"]
    return []


def pin_mxfp4_exact(O, n_cols=4):
    """Different scales per block: the formula in exact rationals, rounded once."""
    import gen
    fails = []
    x = gen.make_indexer_inputs("mx", 1, 2, [90], 43, kfmt="mxfp4")
    rng = np.random.default_rng(6)
    x.kv_pages[..., 64:68] = rng.integers(118, 138, size=x.kv_pages.shape[:2] + (4,)).astype(np.uint8)
    got = O.indexer_logits(x.q, x.kv_pages, None, x.weights, x.block_table,
                           x.context_lens, x.next_n, x.logits_stride)
    vals = load_golden_e2m1()
    for r in range(x.rows):
        n = int(x.context_lens[r])
        qd = torch_e4m3_decode(x.q[r])
        for s in sorted(set(rng.integers(0, n, n_cols).tolist()) | {n - 1}):
            tok = x.kv_pages[int(x.block_table[0, s // 64]), s % 64]
            kd = []
            for d in range(128):
                byte = int(tok[d // 2])
                code = (byte >> 4) if d % 2 else (byte & 0xF)
                kd.append(Fraction(vals[code]) * Fraction(2) ** (int(tok[64 + d // 32]) - 127))
            total = Fraction(0)
            for h in range(32):
                dot = sum((Fraction(float(qd[h, d])) * kd[d] for d in range(128)), Fraction(0))
                if dot > 0:
                    total += Fraction(float(x.weights[r, h])) * dot
            want = np.float32(float(total))
            g = got[r, s]
            ulp = np.spacing(np.float32(abs(want))) if want != 0 else np.float32(1e-45)
            if not abs(float(g) - float(want)) <= float(ulp):
                fails.append(f"MXFP4 logit[{r},{s}] = {g}, exact {want}")
    return fails


# ------------------------------------------------- candidate indexer --
def pin_block_amax8(O, seed=61):
    """Brute force with explicit comparisons: live scores only, NaN skipped,
    the newest block +inf, nothing past ceil(len / 8)."""
    fails = []
    rng = np.random.default_rng(seed)
    rows, width = 6, 70
    sc = rng.standard_normal((rows, width)).astype(np.float32)
    sc[rng.random((rows, width)) < 0.1] = np.nan
    sc[0, 3] = np.inf
    sc[1, 8:16] = np.nan          # a block of NaNs only
    sc[2, 10] = -np.inf
    lens = np.array([70, 23, 8, 1, 0, 57])
    got = O.candidates.block_amax8(sc, lens)
    for r in range(rows):
        n = int(lens[r])
        nb = -(-n // 8)
        for j in range(got.shape[1]):
            if j >= nb:
                if not np.isnan(got[r, j]):
                    fails.append(f"amax8[{r},{j}] written past the count")
                continue
            if j == nb - 1:
                want = np.float32(np.inf)
            else:
                best = None
                for i in range(8 * j, min(n, 8 * j + 8)):
                    v = float(sc[r, i])
                    if v != v:
                        continue
                    if best is None or v > best:
                        best = v
                want = np.float32(np.nan if best is None else best)
            g = got[r, j]
            if not ((np.isnan(want) and np.isnan(g)) or g == want):
                fails.append(f"amax8[{r},{j}] = {g}, want {want}")
    return fails


def pin_sort_candidate_blocks(O, seed=63):
    """Python sorted() and the page transform written out per block."""
    import gen
    fails = []
    rng = np.random.default_rng(seed)
    # rows of the last request have at most kb blocks: the identity table,
    # whatever subset the input lists
    x = gen.make_indexer_inputs("blk", 3, 2, [700, 900, 60], 7)
    rows, kb = x.rows, 12
    n_blocks = -(-x.context_lens.astype(np.int64) // 8)
    blocks = np.full((rows, kb), -1, dtype=np.int32)
    for r in range(rows):
        pick = rng.choice(int(n_blocks[r]), size=min(kb - r % 3, int(n_blocks[r]) - 2), replace=False)
        blocks[r, :len(pick)] = pick
        if r % 2 and len(pick) > 3:  # a repeat and an id past the row: both dropped
            blocks[r, 1] = blocks[r, 0]
            blocks[r, 2] = int(n_blocks[r]) + 3
    table, slots = O.candidates.sort_candidate_blocks(blocks, n_blocks, x.block_table, x.next_n)
    big = 2 ** 31 - 1
    for r in range(rows):
        if n_blocks[r] <= kb:
            ids = list(range(int(n_blocks[r])))
        else:
            ids = sorted(set(int(b) for b in blocks[r] if 0 <= b < int(n_blocks[r])))
        want_t = ids + [big] * (kb - len(ids))
        want_s = []
        for b in ids:
            page = int(x.block_table[r // x.next_n, (b * 8) // 64])
            want_s.append(page * 8 + b % 8)
        want_s += [big] * (kb - len(ids))
        if table[r].tolist() != want_t:
            fails.append(f"row {r}: table {table[r].tolist()} want {want_t}")
        if slots[r].tolist() != want_s:
            fails.append(f"row {r}: slots {slots[r].tolist()} want {want_s}")
    return fails


def pin_sparse_logits(O, seed=65):
    """Sparse logits are the dense logits at the listed blocks' live keys, in
    table order; sparse_to_logical and sparse_row_lens agree."""
    import gen
    fails = []
    rng = np.random.default_rng(seed)
    x = gen.make_indexer_inputs("sp", 2, 2, [300, 451], 9)
    dense = O.indexer_logits(x.q, x.kv_pages, x.k_scales, x.weights, x.block_table,
                             x.context_lens, x.next_n, x.logits_stride)
    kb = 9
    big = 2 ** 31 - 1
    table = np.full((x.rows, kb), big, dtype=np.int32)
    for r in range(x.rows):
        nb = -(-int(x.context_lens[r]) // 8)
        ids = np.sort(rng.choice(nb - 1, size=kb - 1 - r % 2, replace=False))
        ids = np.concatenate([ids, [nb - 1]])  # the newest block, partly live
        table[r, :len(ids)] = ids
    got = O.candidates.sparse_logits(x.q, x.kv_pages, x.k_scales, x.weights, x.block_table,
                                     table, x.context_lens, x.next_n)
    lens = O.candidates.sparse_row_lens(table, x.context_lens)
    for r in range(x.rows):
        col = 0
        for i in range(kb):
            b = int(table[r, i])
            for t in range(8):
                c = 8 * i + t
                key = 8 * b + t
                live = b != big and key < int(x.context_lens[r])
                if live:
                    if got[r, c] != dense[r, key]:
                        fails.append(f"sparse[{r},{c}] != dense[{r},{key}]")
                    if int(O.candidates.sparse_to_logical(table[r:r + 1], np.array([[c]]))[0, 0]) != key:
                        fails.append(f"sparse column {c} of row {r} maps elsewhere")
                    col += 1
                elif not np.isnan(got[r, c]):
                    fails.append(f"sparse[{r},{c}] written though not live")
        if int(lens[r]) != col:
            fails.append(f"row {r}: sparse length {int(lens[r])}, live {col}")
    return fails


def pin_sparse_to_logical_edges(O):
    """sparse_to_logical written out by hand on a two-block table whose second
    entry is padding: columns of the first block map to 8 * 3 + c, columns of
    the padding entry and past the table (c >= 16) and -1 give -1."""
    big = 2 ** 31 - 1
    table = np.array([[3, big], [0, 7]], dtype=np.int32)
    cols = np.array([[0, 7, 8, 15, 16, -1, 23, 5],
                     [8, 15, 0, 16, 9, -1, 2, 14]], dtype=np.int32)
    want = [[24, 31, -1, -1, -1, -1, -1, 29],
            [56, 63, 0, -1, 57, -1, 2, 62]]
    got = O.candidates.sparse_to_logical(table, cols)
    return [] if got.tolist() == want else [f"got {got.tolist()} want {want}"]


def pin_prefill_decode_case(O):
    """A ragged batch whose requests all have next_n rows is a decode call:
    the prefill oracle equals the decode oracle bit for bit (fill included)."""
    import gen
    x = gen.make_indexer_inputs("pd", 3, 2, [300, 451, 17], 9)
    cu = np.arange(x.B + 1, dtype=np.int32) * x.next_n
    want = O.indexer_logits(x.q, x.kv_pages, x.k_scales, x.weights, x.block_table,
                            x.context_lens, x.next_n, x.logits_stride)
    got = O.prefill.prefill_logits(x.q, x.kv_pages, x.k_scales, x.weights, x.block_table, cu,
                                   x.context_lens, x.logits_stride)
    if not np.array_equal(got, want, equal_nan=True):
        return ["prefill logits of a decode-shaped batch differ from the decode logits"]
    return []


def pin_prefill_exact(O, n_cols=3):
    """Ragged rows (an empty request included) in exact rationals: row t of
    request r (found by walking cu_q) scores keys [0, len_t) of r's pages."""
    import gen
    fails = []
    x = gen.make_prefill_inputs("pe", [3, 0, 2, 1], [70, 5, 0, 130], 41)
    got = O.prefill.prefill_logits(x.q, x.kv_pages, x.k_scales, x.weights, x.block_table,
                                   x.cu_q, x.context_lens, x.logits_stride)
    rng = np.random.default_rng(3)
    for t in range(x.rows):
        r = next(i for i in range(x.B) if x.cu_q[i] <= t < x.cu_q[i + 1])
        n = int(x.context_lens[t])
        qd = torch_e4m3_decode(x.q[t])
        cols = sorted(set(rng.integers(0, n, n_cols).tolist()) | {n - 1})
        for s in cols:
            page = int(x.block_table[r, s // 64])
            kd = torch_e4m3_decode(x.kv_pages[page, s % 64])
            total = Fraction(0)
            for h in range(32):
                dot = sum((Fraction(float(qd[h, d])) * Fraction(float(kd[d])) for d in range(128)),
                          Fraction(0))
                if dot > 0:
                    total += Fraction(float(x.weights[t, h])) * dot
            want = np.float32(float(Fraction(float(x.k_scales[page, s % 64])) * total))
            ulp = np.spacing(np.float32(abs(want))) if want != 0 else np.float32(1e-45)
            if not abs(float(got[t, s]) - float(want)) <= float(ulp):
                fails.append(f"prefill logit[{t},{s}] = {got[t, s]}, exact {want}")
        if not np.all(np.isnan(got[t, n:])):
            fails.append(f"prefill row {t}: columns past its length were written")
        at = O.prefill.prefill_logits_at(x.q, x.kv_pages, x.k_scales, x.weights, x.block_table,
                                         x.cu_q, t, np.array(cols))
        if not np.array_equal(at, got[t, cols]):
            fails.append(f"prefill_logits_at row {t} differs from prefill_logits")
    return fails


ALL_PINS = (pin_e4m3, pin_fp16_rne, pin_logits_f16_check, pin_bins_golden, pin_bins_exhaustive,
            pin_keys, pin_bins_coarsen_keys, pin_histogram, pin_topk,
            pin_topk_invariants, pin_logits_exact, pin_logits_library,
            pin_logits_paging, pin_error_bound, pin_head_sum_exact,
            pin_error_bound_exact, pin_check_logits_classes, pin_logits_terms_match, pin_e2m1, pin_e8m0, pin_mxfp4_layout,
            pin_mxfp4_matches_fp8_path, pin_mxfp4_exact, pin_block_amax8,
            pin_sort_candidate_blocks, pin_sparse_logits, pin_sparse_to_logical_edges,
            pin_prefill_decode_case,
            pin_prefill_exact)
