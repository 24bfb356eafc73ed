"""HIP path vs the CPU oracle at the full decode workloads, in the launch
configuration the benchmark times: every live logit within tolerance, the
whole histogram and every top-k index set bit-exact from the GPU's own logits."""
import numpy as np
import pytest
import torch

import gen
import oracle as O
from tests.gpu_harness import (DEV, DevInputs, announce, check_hist, check_logits_full,
                               check_padding, check_topk, topk)

pytestmark = pytest.mark.gpu

# keys each workload selects with
KEYS = {
    "tiny_decode": (O.KEY_FP32, O.KEY_FP16),
    "long_decode": (O.KEY_FP32, O.KEY_FP16),
    "spec_verify/fine": (O.KEY_FP32, O.KEY_FP16),
    "spec_verify/unit": (O.KEY_FP32, O.KEY_FP16),
    "spec_verify/mixed": (O.KEY_FP32, O.KEY_FP16),
    "varlen_decode": (O.KEY_FP16, O.KEY_FP32),
    "very_long": (O.KEY_FP32, O.KEY_FP16),
}


@pytest.mark.parametrize("name", gen.CONFIG_NAMES)
def test_workload_parity(gpu, name):
    announce(f"generate {name}")
    x = gen.config_inputs(name)
    d = DevInputs(x)
    announce(f"indexer_logits {name}: B={x.B} next_n={x.next_n} rows={x.rows} "
             f"stride={x.logits_stride} pages={x.num_pages}")
    lg, h = d.run(with_hist=True, fill=float("inf"))
    got = lg.cpu().numpy()
    hist = h.cpu().numpy()
    worst, checked = check_logits_full(x, got)
    announce(f"{name}: {checked} logits checked, max |err|/bound = {worst:.3g}")
    check_padding(x, got, float("inf"))
    check_hist(x.context_lens, got, hist)
    for key in KEYS[name]:
        announce(f"topk_rows {name} key={key}")
        idx = topk(lg, h, d.lens, 2048, key)
        check_topk(idx.cpu().numpy(), got, x.context_lens, 2048, key)
    del d, lg, h
    torch.cuda.empty_cache()


@pytest.mark.parametrize("key", [O.KEY_FP16, O.KEY_FP32])
def test_very_long_score_rows(gpu, key):
    announce("generate very_long score rows")
    s = gen.very_long_scores()
    lens = np.full(s.shape[0], s.shape[1], dtype=np.int32)
    st = torch.from_numpy(s).to(DEV)
    ln = torch.from_numpy(lens).to(DEV)
    announce(f"topk_rows hist=NULL [4, 1048576] key={key}")
    idx = topk(st, None, ln, 2048, key)
    check_topk(idx.cpu().numpy(), s, lens, 2048, key)
    h = torch.zeros((4, 1024), dtype=torch.int32, device=DEV)
    pmqa_hist = __import__("paged_mqa_logits_indexer_amd")
    pmqa_hist.score_histogram(st, ln, h)
    torch.cuda.synchronize()
    check_hist(lens, s, h.cpu().numpy())
