"""topk_rows_noalloc -- top-k with the library's fixed per-GPU scratch -- against
topk_rows with a caller's workspace, both through the C ABI (ctypes), on two
calls in a row (the second on a smaller input), with FP32 and FP16 keys, with
the producer's histogram and without one, on rows that take the chunked path
(more than 16384 scores per row) and on rows that do not; index sets must be
identical and equal to the oracle's."""
import ctypes

import numpy as np
import pytest
import torch

import oracle as O
import paged_mqa_logits_indexer_amd as pmqa
from tests.gpu_harness import DEV, announce, check_topk

pytestmark = pytest.mark.gpu


def _vp(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream(DEV).cuda_stream)


def _noalloc(lib, s, h, ln, k, key):
    idx = torch.full((s.shape[0], k), -7, dtype=torch.int32, device=DEV)
    st = lib.topk_rows_noalloc(_vp(s), s.stride(0), _vp(h), _vp(ln), s.shape[0], k, key, _vp(idx),
                               _stream())
    assert st == 0, pmqa.indexer_status_str(st)
    return idx


def _with_workspace(lib, s, h, ln, k, key):
    idx = torch.full((s.shape[0], k), -7, dtype=torch.int32, device=DEV)
    nbytes = lib.topk_workspace_bytes(s.shape[0], s.stride(0), k)
    ws = torch.zeros(max(nbytes, 256), dtype=torch.uint8, device=DEV)
    st = lib.topk_rows(_vp(s), s.stride(0), _vp(h), _vp(ln), s.shape[0], k, key, _vp(idx), _vp(ws),
                       ws.numel(), _stream())
    assert st == 0, pmqa.indexer_status_str(st)
    return idx


def _scores(rows, stride, seed):
    """Mixture rows (N(0, var 4) with 1% N(40, var 10) outliers) plus ties,
    ragged lengths and a few NaNs."""
    rng = np.random.default_rng(seed)
    x = (rng.standard_normal((rows, stride)) * 2.0).astype(np.float32)
    out = rng.random((rows, stride)) < 0.01
    x[out] = (40.0 + rng.standard_normal(int(out.sum())) * np.sqrt(10.0)).astype(np.float32)
    x[:, rng.integers(0, stride, stride // 50)] = np.float32(3.5)
    x[rng.random((rows, stride)) < 0.001] = np.nan
    lens = rng.integers(stride // 2, stride + 1, rows).astype(np.int32)
    lens[0] = stride
    return x, lens


@pytest.mark.parametrize("shapes", [((8, 131072), (3, 40000)), ((4, 16384), (2, 5000))],
                         ids=["chunked", "one_workgroup"])
def test_noalloc_matches_workspace_entry_point(gpu, shapes):
    lib = pmqa.load_library()
    for call, (rows, stride) in enumerate(shapes):
        x, lens = _scores(rows, stride, 900 + call)
        s = torch.from_numpy(x).to(DEV)
        ln = torch.from_numpy(lens).to(DEV)
        h = torch.zeros((rows, 1024), dtype=torch.int32, device=DEV)
        pmqa.score_histogram(s, ln, h)
        for key in (O.KEY_FP32, O.KEY_FP16):
            for hist in (h, None):
                for k in (2048, 37):
                    announce(f"topk_rows_noalloc call={call} rows={rows} stride={stride} key={key} "
                             f"hist={'on' if hist is not None else 'none'} k={k}")
                    got = _noalloc(lib, s, hist, ln, k, key)
                    ref = _with_workspace(lib, s, hist, ln, k, key)
                    torch.cuda.synchronize()
                    g = np.sort(got.cpu().numpy(), axis=1)
                    r = np.sort(ref.cpu().numpy(), axis=1)
                    assert np.array_equal(g, r), f"noalloc differs from topk_rows (call {call})"
                    check_topk(got.cpu().numpy(), x, lens, k, key)


def test_noalloc_refuses_rows_beyond_its_scratch(gpu):
    lib = pmqa.load_library()
    s = torch.zeros((129, 16388), dtype=torch.float32, device=DEV)
    ln = torch.full((129,), 16388, dtype=torch.int32, device=DEV)
    idx = torch.empty((129, 8), dtype=torch.int32, device=DEV)
    st = lib.topk_rows_noalloc(_vp(s), s.stride(0), None, _vp(ln), 129, 8, 0, _vp(idx), _stream())
    assert st == 6, pmqa.indexer_status_str(st)  # IDX_ESCRATCH, nothing launched
