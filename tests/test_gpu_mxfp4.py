"""MXFP4 keys (block-scaled E2M1 in packed 68-byte tokens; SGLang PR #38944,
vLLM PR #52696) through indexer_logits_mxfp4, against the CPU oracle: logits
within the tolerance, histogram and top-k bit-exact from the GPU's logits,
padding untouched, at small ragged sizes and at the full MXFP4 workloads."""
import numpy as np
import pytest
import torch

import gen
import oracle as O
from tests.gpu_harness import (DevInputs, announce, check_hist, check_logits, check_logits_full, check_padding,
                               check_topk, topk)

pytestmark = pytest.mark.gpu

INF = float("inf")

SMALL = [
    (1, 51, [1000, 130, 5000, 64, 4097]),
    (2, 52, [777, 2049, 63]),
    (3, 53, [3000, 65, 1]),
    (4, 54, [4096, 1500, 129]),
]


def _check_all(x, lg, h, sample=None, keys=(O.KEY_FP32, O.KEY_FP16)):
    got = lg.cpu().numpy()
    worst = check_logits_full(x, got)[0] if sample == "all" else check_logits(x, got, sample=sample, seed=5)
    check_padding(x, got, INF)
    check_hist(x.context_lens, got, h.cpu().numpy())
    for key in keys:
        idx = topk(lg, h, torch.from_numpy(x.context_lens).to(lg.device), 2048, key)
        check_topk(idx.cpu().numpy(), got, x.context_lens, 2048, key)
    return worst


@pytest.mark.parametrize("next_n,seed,base", SMALL, ids=[f"next_n{s[0]}" for s in SMALL])
def test_mxfp4_small(gpu, next_n, seed, base):
    x = gen.make_indexer_inputs(f"mx{next_n}", len(base), next_n, base, seed, kfmt="mxfp4")
    d = DevInputs(x)
    announce(f"indexer_logits_mxfp4 small next_n={next_n} lens={base}")
    lg, h = d.run(with_hist=True, fill=INF)
    worst = _check_all(x, lg, h)
    announce(f"mxfp4 next_n={next_n}: max |err|/bound = {worst:.3g}")
    lg2, _ = d.run(with_hist=False, fill=INF)
    assert torch.equal(lg.view(torch.int32), lg2.view(torch.int32)), "histogram changes the logits"


def test_mxfp4_wide_block_scales(gpu):
    # block scales from 2^-63 to 2^73 and different in every block of a key:
    # the four partial dots of a key differ by up to 2^136, and every value
    # stays a normal float32 (no head sum can overflow, no product is
    # subnormal), the range where float32 evaluation order cannot matter
    # beyond the tolerance
    x = gen.make_indexer_inputs("mx_scales", 2, 2, [700, 333], 57, kfmt="mxfp4")
    rng = np.random.default_rng(8)
    sc = rng.integers(100, 155, size=x.kv_pages.shape[:2] + (4,)).astype(np.uint8)
    pick = rng.random(x.kv_pages.shape[:2] + (4,))
    sc[pick < 0.05] = 64
    sc[pick > 0.95] = 200
    x.kv_pages[..., 64:68] = sc
    d = DevInputs(x)
    announce("indexer_logits_mxfp4 wide block scales")
    lg, h = d.run(with_hist=True, fill=INF)
    _check_all(x, lg, h)


@pytest.mark.parametrize("name", gen.MXFP4_CONFIG_NAMES)
def test_mxfp4_workload_parity(gpu, name):
    announce(f"generate {name}")
    x = gen.config_inputs(name)
    d = DevInputs(x)
    announce(f"indexer_logits_mxfp4 {name}: B={x.B} next_n={x.next_n} stride={x.logits_stride}")
    lg, h = d.run(with_hist=True, fill=INF)
    worst = _check_all(x, lg, h, sample="all")
    announce(f"{name}: max |err|/bound = {worst:.3g}")
    del d, lg, h
    torch.cuda.empty_cache()
