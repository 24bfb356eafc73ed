"""Shared GPU-test plumbing: upload seeded inputs, run the HIP library through
its C ABI, and compare element by element with the CPU oracle."""

from __future__ import annotations

import sys

import numpy as np
import torch

import oracle as O
import paged_mqa_logits_indexer_amd as pmqa

DEV = "cuda:0"


def announce(msg: str) -> None:
    """Name the case on the real stderr before each GPU step."""
    sys.__stderr__.write(f"[gpu] {msg}\n")
    sys.__stderr__.flush()


class DevInputs:
    """One indexer call's inputs in device memory."""

    def __init__(self, x, device=DEV):
        self.x = x
        self.device = device
        self.q = torch.from_numpy(np.ascontiguousarray(x.q)).to(device)
        self.kv = torch.from_numpy(np.ascontiguousarray(x.kv_pages)).to(device)
        # MXFP4 pages ([P, 64, 68] packed tokens) carry their scales inside
        self.sc = None if x.k_scales is None else torch.from_numpy(np.ascontiguousarray(x.k_scales)).to(device)
        self.w = torch.from_numpy(np.ascontiguousarray(x.weights)).to(device)
        self.bt = torch.from_numpy(np.ascontiguousarray(x.block_table)).to(device)
        self.lens = torch.from_numpy(np.ascontiguousarray(x.context_lens)).to(device)

    def new_logits(self, fill=float("inf")):
        return torch.full((self.x.rows, self.x.logits_stride), fill, dtype=torch.float32,
                          device=self.device)

    def new_hist(self):
        return torch.zeros((self.x.rows, 1024), dtype=torch.int32, device=self.device)

    def logits(self, logits, hist=None):
        if self.sc is None:
            pmqa.indexer_logits_mxfp4(self.q, self.kv, self.w, self.bt, self.lens,
                                      self.x.next_n, logits, hist)
            return
        pmqa.indexer_logits(self.q, self.kv, self.sc, self.w, self.bt, self.lens,
                            self.x.next_n, logits, hist)

    def f16_stride(self):
        """The workload's stride rounded up to 8 halves (16-byte rows)."""
        return -(-self.x.logits_stride // 8) * 8

    def run_f16(self, with_hist=True, fill=float("inf")):
        lg = torch.full((self.x.rows, self.f16_stride()), fill, dtype=torch.float16,
                        device=self.device)
        h = self.new_hist() if with_hist else None
        pmqa.indexer_logits_f16(self.q, self.kv, self.sc, self.w, self.bt, self.lens,
                                self.x.next_n, lg, h)
        torch.cuda.synchronize()
        return lg, h

    def run(self, with_hist=True, fill=float("inf")):
        lg = self.new_logits(fill)
        h = self.new_hist() if with_hist else None
        self.logits(lg, h)
        torch.cuda.synchronize()
        return lg, h


# The selector gives each 8192-score chunk of a row its own workgroup; a row
# of one chunk is finished by that workgroup alone, longer rows by the last
# of their workgroups to arrive.  Edge-case tests run both: "one_chunk" keeps
# the first 8192 columns of every row (stride 8192), "as_is" keeps the rows
# (several chunks), and "wide" also pads the stride past 2^18 scores, so most
# workgroups of the grid find no chunk.
CHUNK = 8192
WIDE_STRIDE = (1 << 18) + 8
PATHS = ["one_chunk", "as_is", "wide"]


def on_path(scores, lens, path):
    """(scores, lens) as device tensors laid out for ``path``."""
    if path == "as_is":
        return scores, lens
    if path == "one_chunk":
        n = min(CHUNK, scores.shape[1])
        return scores[:, :n].contiguous(), torch.clamp(lens, max=n)
    w = torch.full((scores.shape[0], WIDE_STRIDE), float("inf"), dtype=scores.dtype,
                   device=scores.device)
    w[:, :scores.shape[1]] = scores
    return w, lens


def topk_f16(logits, hist, lens, k, workspace=None):
    idx = torch.full((logits.shape[0], k), -7, dtype=torch.int32, device=logits.device)
    pmqa.topk_rows_f16(logits, hist, lens, k, idx, workspace)
    torch.cuda.synchronize()
    return idx


def topk(logits, hist, lens, k, key_dtype, workspace=None):
    idx = torch.full((logits.shape[0], k), -7, dtype=torch.int32, device=logits.device)
    pmqa.topk_rows(logits, hist, lens, k, key_dtype, idx, workspace)
    torch.cuda.synchronize()
    return idx


def sample_cols(n, sample, rng):
    if sample is None or n <= sample + 128:
        return np.arange(n)
    pick = rng.choice(n, sample, replace=False)
    edge = np.concatenate([np.arange(min(64, n)), np.arange(max(0, n - 64), n)])
    return np.unique(np.concatenate([pick, edge]))


def check_logits(x, got, sample=None, seed=0, rows=None):
    """GPU logits within the tolerance of the oracle; returns max |err|/bound.
    float16 logits are checked with the oracle's FP16 rule (the halves that
    float32 values within the bound round to)."""
    rng = np.random.default_rng(seed)
    worst = 0.0
    rows = range(x.rows) if rows is None else rows
    for r in rows:
        n = int(x.context_lens[r])
        if n == 0:
            continue
        cols = sample_cols(n, sample, rng)
        want = O.indexer_logits_at(x.q, x.kv_pages, x.k_scales, x.weights, x.block_table,
                                   x.next_n, r, cols)
        bound = O.logits_error_bound_at(x.q, x.kv_pages, x.k_scales, x.weights,
                                        x.block_table, x.next_n, r, cols)
        hsum = O.head_sum_at(x.q, x.kv_pages, x.k_scales, x.weights, x.block_table,
                             x.next_n, r, cols)
        hbound = O.logits_error_bound_at(x.q, x.kv_pages, x.k_scales, x.weights,
                                         x.block_table, x.next_n, r, cols, unscaled=True)
        g = got[r, cols]
        check = O.check_logits_f16 if g.dtype == np.float16 else O.check_logits
        ok = check(g, want, bound, hsum, hbound)
        if not ok.all():
            bad = np.nonzero(~ok)[0][:5]
            raise AssertionError(
                f"row {r}: {int((~ok).sum())} logits outside tolerance, e.g. cols "
                f"{cols[bad].tolist()} got {g[bad].tolist()} want {want[bad].tolist()} "
                f"bound {bound[bad].tolist()}")
        fin = np.isfinite(want) & (bound > 0)
        if fin.any():
            worst = max(worst, float(np.max(np.abs(g[fin].astype(np.float64) - want[fin])
                                            / bound[fin])))
    return worst


def check_logits_full(x, got, chunk=32768):
    """Every live logit of every row within the tolerance of the oracle (the
    keys of a request gathered once per chunk for all of its rows); returns
    (max |err|/bound over finite expected values, logits checked)."""
    worst, checked = 0.0, 0
    next_n = x.next_n
    for b in range(x.B):
        rows = list(range(b * next_n, (b + 1) * next_n))
        n_max = int(max(int(x.context_lens[r]) for r in rows))
        for c0 in range(0, n_max, chunk):
            cols = np.arange(c0, min(n_max, c0 + chunk))
            want, bound, hs, hb = O.logits_terms_at(x.q, x.kv_pages, x.k_scales, x.weights,
                                                    x.block_table, next_n, rows, cols)
            for i, r in enumerate(rows):
                n = min(int(x.context_lens[r]) - c0, cols.size)
                if n <= 0:
                    continue
                g = got[r, c0:c0 + n]
                w_, bd = want[i, :n], bound[i, :n]
                check = O.check_logits_f16 if g.dtype == np.float16 else O.check_logits
                ok = check(g, w_, bd, hs[i, :n], hb[i, :n])
                if not ok.all():
                    bad = np.nonzero(~ok)[0][:5]
                    raise AssertionError(
                        f"row {r}: {int((~ok).sum())} logits outside tolerance, e.g. cols "
                        f"{(bad + c0).tolist()} got {g[bad].tolist()} want {w_[bad].tolist()} "
                        f"bound {bd[bad].tolist()}")
                fin = np.isfinite(w_) & (bd > 0)
                if fin.any():
                    worst = max(worst, float(np.max(np.abs(g[fin].astype(np.float64) - w_[fin])
                                                    / bd[fin])))
                checked += n
    return worst, checked


def check_padding(x, got, fill):
    for r in range(x.rows):
        n = int(x.context_lens[r])
        tail = got[r, n:]
        if np.isnan(fill):
            assert np.all(np.isnan(tail)), f"row {r}: padding written"
        else:
            assert np.all(tail == fill), f"row {r}: padding written"


def check_hist(lens, got_logits, got_hist, hist_in=None):
    want = O.coarse_histogram(got_logits, lens, hist_in)
    if not np.array_equal(got_hist, want):
        r = int(np.nonzero((got_hist != want).any(axis=1))[0][0])
        d = np.nonzero(got_hist[r] != want[r])[0][:8]
        raise AssertionError(f"histogram row {r} differs at bins {d.tolist()}: "
                             f"got {got_hist[r, d].tolist()} want {want[r, d].tolist()}")


def check_topk(got_idx, scores, lens, k, key_dtype):
    want = O.topk_rows(scores, lens, k, key_dtype)
    for r in range(got_idx.shape[0]):
        g = got_idx[r]
        n_sel = int(np.sum(want[r] >= 0))
        sel = np.sort(g[g >= 0])
        assert np.all(g[g < 0] == -1), f"row {r}: stray values {np.unique(g[g < 0])}"
        assert sel.size == n_sel, f"row {r}: {sel.size} selected, want {n_sel}"
        assert np.array_equal(sel, want[r, :n_sel]), (
            f"row {r} (key {key_dtype}, k {k}): index sets differ in "
            f"{np.setxor1d(sel, want[r, :n_sel]).size} columns")
