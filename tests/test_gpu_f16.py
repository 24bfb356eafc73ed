"""FP16 logits output (vLLM PR #52696 "Summary": the indexer stores FP16
logits and the selector reads them): the HIP path vs the CPU oracle.

indexer_logits_f16 must write exactly the halves the float32 path's logits
round to, with the same histogram; the oracle accepts a half when some
float32 within the logit tolerance rounds to it.  topk_rows_f16 must select
the oracle's set from the GPU's own halves, with and without the producer's
histogram."""
import numpy as np
import pytest
import torch

import gen
import oracle as O
from tests.gpu_harness import (PATHS, DevInputs, announce, check_hist, check_logits, check_logits_full, check_topk,
                               on_path, topk_f16)

pytestmark = pytest.mark.gpu


def _as_f32(h):
    return h.cpu().numpy().astype(np.float32)


def _check_padding_f16(x, got, fill):
    for r in range(x.rows):
        n = int(x.context_lens[r])
        tail = got[r, n:]
        assert np.all(tail == np.float16(fill)), f"row {r}: padding written"


@pytest.mark.parametrize("next_n", [1, 2, 3, 4])
def test_f16_matches_rounded_f32_path(gpu, next_n):
    x = gen.make_indexer_inputs(f"f16/n{next_n}", B=3, next_n=next_n, base_lens=[700, 1, 2500],
                                seed=700 + next_n, weight_scale=2.0)
    d = DevInputs(x)
    announce(f"indexer_logits vs indexer_logits_f16 next_n={next_n}")
    l32, h32 = d.run(with_hist=True)
    l16, h16 = d.run_f16(with_hist=True)
    g32 = l32.cpu().numpy()
    g16 = l16.cpu().numpy()
    for r in range(x.rows):
        n = int(x.context_lens[r])
        want = O.fp16_rne(g32[r, :n]).view(np.uint16)
        got = g16[r, :n].view(np.uint16)
        assert np.array_equal(got, want), f"row {r}: halves differ from the rounded float32 logits"
    assert torch.equal(h16, h32), "histograms of the two outputs differ"
    check_logits(x, g16, sample=None, seed=1)
    _check_padding_f16(x, g16, float("inf"))


@pytest.mark.parametrize("name", ["tiny_decode", "long_decode", "spec_verify/mixed",
                                  "varlen_decode"])
def test_f16_workload_parity(gpu, name):
    announce(f"generate {name}")
    x = gen.config_inputs(name)
    d = DevInputs(x)
    announce(f"indexer_logits_f16 {name}: rows={x.rows} stride={d.f16_stride()}")
    lg, h = d.run_f16(with_hist=True)
    got = lg.cpu().numpy()
    worst, _ = check_logits_full(x, got)
    announce(f"{name}: max |err|/bound (halves) = {worst:.3g}")
    _check_padding_f16(x, got, float("inf"))
    scores = _as_f32(lg)
    check_hist(x.context_lens, scores, h.cpu().numpy())
    for use_hist in (True, False):
        announce(f"topk_rows_f16 {name} hist={'producer' if use_hist else 'NULL'}")
        idx = topk_f16(lg, h if use_hist else None, d.lens, 2048)
        check_topk(idx.cpu().numpy(), scores, x.context_lens, 2048, O.KEY_FP16)
    del d, lg, h
    torch.cuda.empty_cache()


@pytest.mark.parametrize("path", PATHS)
def test_f16_ties_and_stale_histogram(gpu, path):
    """Many equal halves (ties broken by the lower column) and a stale
    histogram (the selector must fall back and stay exact)."""
    rng = np.random.default_rng(41)
    rows, stride = 3, 20000
    vals = rng.choice(np.array([1.0, 1.5, 2.0, -0.5, np.inf, np.nan], np.float32), size=(rows, stride),
                      p=[0.4, 0.2, 0.05, 0.3, 0.03, 0.02]).astype(np.float16)
    lens = np.array([stride, 12345, 4000], np.int32)
    lg, ln = on_path(torch.from_numpy(vals).to("cuda:0"), torch.from_numpy(lens).to("cuda:0"), path)
    vals, lens = lg.cpu().numpy(), ln.cpu().numpy()
    for hist in (None, torch.full((rows, 1024), 3, dtype=torch.int32, device="cuda:0")):
        for k in (1, 100, 2048, 8192):
            announce(f"topk_rows_f16 ties k={k} hist={'stale' if hist is not None else 'NULL'} "
                     f"path={path}")
            idx = topk_f16(lg, hist, ln, k)
            check_topk(idx.cpu().numpy(), vals.astype(np.float32), lens, k, O.KEY_FP16)
