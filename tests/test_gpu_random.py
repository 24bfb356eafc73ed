"""Seeded random call shapes through the decode path: batch size (including
the many-request grid), rows per request, lengths around page and share
edges, weight scale (fine, unit and saturating score ranges), a few
infinite K scales, FP8 or MXFP4 K, and k.  Each call is checked element by
element against the CPU oracle (logits within the tolerance, columns past a
row's length untouched), the histogram and the top-k bit-exact from the
GPU's own logits, the FP16-output variant against the float32 logits it
rounds, and the histogram-off call bitwise equal to the histogram-on one."""
import numpy as np
import pytest
import torch

import gen
import oracle as O
from tests.gpu_harness import (DevInputs, announce, check_hist, check_logits, check_padding,
                               check_topk, topk)

pytestmark = pytest.mark.gpu

INF = float("inf")
EDGE_LENS = [0, 1, 63, 64, 65, 127, 4095, 4096, 4097, 8192, 8193]


def _shape(seed):
    rng = np.random.default_rng(6100 + seed)
    next_n = int(rng.integers(1, 5))
    kfmt = "mxfp4" if seed % 3 == 2 else "fp8"
    # one-row requests reach the many-request grid (32 requests or more)
    B = int(rng.integers(1, 49 if next_n == 1 else 13))
    # odd seeds reach rows longer than one top-k workgroup takes (16384)
    hi = 24000 if seed % 2 else 9000
    base = np.where(rng.random(B) < 0.3, rng.choice(EDGE_LENS, B), rng.integers(0, hi, B))
    scale = float(rng.choice([1.0, 4.0, 16.0]))
    inf_frac = 0.01 if (kfmt == "fp8" and seed % 4 == 3) else 0.0
    pad = int(rng.integers(0, 3)) * 8
    stride = int(max(4, -(-(int(base.max()) + next_n) // 8) * 8 + pad))
    k = int(rng.choice([1, 100, 2048]))
    return dict(next_n=next_n, kfmt=kfmt, B=B, base=base.astype(np.int64).tolist(), scale=scale,
                inf_frac=inf_frac, stride=stride, k=k)


@pytest.mark.parametrize("seed", range(16))
def test_random_call_shapes(gpu, seed):
    s = _shape(seed)
    x = gen.make_indexer_inputs(f"rand{seed}", s["B"], s["next_n"], s["base"], 7000 + seed,
                                weight_scale=s["scale"], inf_frac=s["inf_frac"],
                                logits_stride=s["stride"], kfmt=s["kfmt"])
    d = DevInputs(x)
    announce(f"random shape seed={seed} B={s['B']} next_n={s['next_n']} kfmt={s['kfmt']} "
             f"scale={s['scale']} inf={s['inf_frac']} stride={s['stride']} k={s['k']} "
             f"lens={s['base']}")
    lg, h = d.run(with_hist=True, fill=INF)
    got = lg.cpu().numpy()
    check_logits(x, got)
    check_padding(x, got, INF)
    check_hist(x.context_lens, got, h.cpu().numpy())
    lg_off, _ = d.run(with_hist=False, fill=INF)
    assert torch.equal(lg.view(torch.int32), lg_off.view(torch.int32)), "histogram changes the logits"
    for key in (O.KEY_FP32, O.KEY_FP16):
        announce(f"random shape seed={seed} topk_rows key={key} k={s['k']}")
        idx = topk(lg, h, d.lens, s["k"], key)
        check_topk(idx.cpu().numpy(), got, x.context_lens, s["k"], key)
    if s["kfmt"] == "fp8":
        announce(f"random shape seed={seed} indexer_logits_f16")
        lg16, h16 = d.run_f16(with_hist=True, fill=INF)
        got16 = lg16.cpu().numpy()[:, :x.logits_stride]
        live = np.arange(x.logits_stride)[None, :] < x.context_lens[:, None]
        want16 = got.astype(np.float16)
        nan = np.isnan(want16)
        assert np.all(np.isnan(got16[live & nan])), "a NaN logit is not NaN in FP16"
        cmp = live & ~nan
        assert np.array_equal(np.where(cmp, got16, 0).view(np.uint16),
                              np.where(cmp, want16, 0).view(np.uint16))
        assert np.all(np.isinf(got16[~live]))
        assert np.array_equal(h16.cpu().numpy(), h.cpu().numpy())
