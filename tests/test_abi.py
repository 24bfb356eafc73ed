"""The C ABI on the host: the library loads, exports every entry point the
header declares, and rejects bad arguments with the documented status before
anything is launched (no GPU is touched by these tests)."""
import ctypes
import os
import re

import pytest

import paged_mqa_logits_indexer_amd as pmqa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "paged_mqa_indexer.h")

IDX_OK, IDX_EINVAL, IDX_EUNSUPPORTED, IDX_EALIGN, IDX_ELAUNCH, IDX_EWORKSPACE, IDX_ESCRATCH = range(7)


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?[A-Za-z_][\w\s\*]*?\b([a-z_][a-z0-9_]*)\s*\(",
                       text, flags=re.M)
    return sorted(set(n for n in names if n not in ("defined",)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(pmqa.library_path()):
        pytest.fail("library not built: run python -m paged_mqa_logits_indexer_amd.build")
    return pmqa.load_library()


def test_header_declares_the_entry_points():
    assert declared_functions() == sorted(pmqa.EXPORTED_SYMBOLS)


def test_library_exports_every_declared_symbol(lib):
    for name in declared_functions():
        assert hasattr(lib, name), name
    out = os.popen(f"nm -D --defined-only {pmqa.library_path()}").read()
    exported = set(re.findall(r"\bT (\w+)$", out, flags=re.M))
    assert set(declared_functions()) <= exported


def test_status_strings(lib):
    for code in range(7):
        assert pmqa.indexer_status_str(code).startswith("IDX_")
    assert "unknown" in pmqa.indexer_status_str(99)


def per_row_bytes(stride, k):
    """The documented layout: one record per row -- two counter pairs padded
    to 256 bytes, a 256-bin sub-histogram, a histogram, 16384 candidates and
    1024 per-workgroup counts (whatever the stride and k)."""
    return 256 + 1024 + 4096 + 8 * 16384 + 4 * 1024


def test_workspace_query(lib):
    assert pmqa.topk_workspace_bytes(0, 1024, 2048) == 0
    assert pmqa.topk_workspace_bytes(4, 0, 2048) == 0
    assert pmqa.topk_workspace_bytes(4, 1024, 0) == 0
    for rows, stride, k in ((1, 131072, 2048), (8, 131072, 2048), (3, 4100, 1), (64, 262144, 8192),
                            (4, 1 << 20, 2048)):
        got = pmqa.topk_workspace_bytes(rows, stride, k)
        assert got == rows * per_row_bytes(stride, k), (rows, stride, k)


# Fake but aligned device addresses: every call below fails validation before
# any of them could be dereferenced or anything launched.
A = 0x10000


def logits_call(lib, **kw):
    args = dict(q=A, kv=A, sc=A, w=A, bt=A, lens=A, B=8, next_n=1, num_pages=16, max_pages=4,
                logits=A, stride=256, hist=None, stream=None)
    args.update(kw)
    return lib.indexer_logits(args["q"], args["kv"], args["sc"], args["w"], args["bt"],
                              args["lens"], args["B"], args["next_n"], args["num_pages"],
                              args["max_pages"], args["logits"], args["stride"], args["hist"],
                              args["stream"])


@pytest.mark.parametrize("kw,status", [
    (dict(q=None), IDX_EINVAL),
    (dict(kv=None), IDX_EINVAL),
    (dict(lens=None), IDX_EINVAL),
    (dict(logits=None), IDX_EINVAL),
    (dict(B=0), IDX_EINVAL),
    (dict(num_pages=0), IDX_EINVAL),
    (dict(max_pages=-1), IDX_EINVAL),
    (dict(stride=0), IDX_EINVAL),
    (dict(next_n=0), IDX_EUNSUPPORTED),
    (dict(next_n=5), IDX_EUNSUPPORTED),
    (dict(B=4097), IDX_EUNSUPPORTED),
    (dict(B=20000, next_n=4), IDX_EUNSUPPORTED),
    (dict(B=4096, max_pages=1 << 20), IDX_EUNSUPPORTED),
    (dict(q=A + 8), IDX_EALIGN),
    (dict(kv=A + 4), IDX_EALIGN),
    (dict(w=A + 4), IDX_EALIGN),
    (dict(sc=A + 2), IDX_EALIGN),
    (dict(logits=A + 4), IDX_EALIGN),
    (dict(stride=258), IDX_EALIGN),
    (dict(hist=A + 4), IDX_EALIGN),
])
def test_indexer_logits_rejects(lib, kw, status):
    assert logits_call(lib, **kw) == status


def test_fp16_logits_checks(lib):
    """indexer_logits_f16 runs the same checks; its rows are 16-byte
    multiples of halves (stride % 8 == 0)."""
    f16 = lib.indexer_logits_f16
    assert f16(None, A, A, A, A, A, 8, 1, 16, 4, A, 256, None, None) == IDX_EINVAL
    assert f16(A, A, A, A, A, A, 8, 5, 16, 4, A, 256, None, None) == IDX_EUNSUPPORTED
    assert f16(A, A, A, A, A, A, 8, 1, 16, 4, A, 260, None, None) == IDX_EALIGN  # 260 % 8
    assert f16(A, A, A, A, A, A, 8, 1, 16, 4, A + 8, 256, None, None) == IDX_EALIGN
    # stride 260 is fine for float32 rows (a multiple of 4) -- it fails later on
    # nothing host-checkable, so use a bad alignment elsewhere to stay off the GPU
    assert logits_call(lib, stride=260, hist=A + 4) == IDX_EALIGN


def test_fp16_topk_checks(lib):
    f16 = lib.topk_rows_f16
    assert f16(None, 256, None, A, 8, 2048, A, A, 1 << 30, None) == IDX_EINVAL
    assert f16(A, 256, None, A, 8, 0, A, A, 1 << 30, None) == IDX_EINVAL
    assert f16(A, 260, None, A, 8, 2048, A, A, 1 << 30, None) == IDX_EALIGN
    assert f16(A, 256, None, A, 8, 2048, A, A, 16, None) == IDX_EWORKSPACE


def test_time_next_call_is_consumed_by_a_failing_call(lib):
    """Arming takes no device action; the next call disarms it even when its
    checks fail (fake handles are never dereferenced on the failing path)."""
    assert lib.indexer_time_next_call(A, A) == IDX_OK
    assert logits_call(lib, q=None) == IDX_EINVAL
    assert lib.indexer_time_next_call(None, None) == IDX_OK
    assert lib.hbm_read_probe(A + 4, 64, A, None) == IDX_EALIGN



def topk_call(lib, **kw):
    args = dict(logits=A, stride=256, hist=None, lens=A, rows=8, k=2048, key=0, idx=A, ws=A,
                ws_bytes=1 << 30, stream=None)
    args.update(kw)
    return lib.topk_rows(args["logits"], args["stride"], args["hist"], args["lens"], args["rows"],
                         args["k"], args["key"], args["idx"], args["ws"], args["ws_bytes"],
                         args["stream"])


@pytest.mark.parametrize("kw,status", [
    (dict(logits=None), IDX_EINVAL),
    (dict(lens=None), IDX_EINVAL),
    (dict(idx=None), IDX_EINVAL),
    (dict(ws=None), IDX_EINVAL),
    (dict(rows=0), IDX_EINVAL),
    (dict(k=0), IDX_EINVAL),
    (dict(k=8193), IDX_EINVAL),
    (dict(stride=-4), IDX_EINVAL),
    (dict(key=2), IDX_EUNSUPPORTED),
    (dict(rows=65536), IDX_EUNSUPPORTED),
    (dict(logits=A + 4), IDX_EALIGN),
    (dict(stride=6), IDX_EALIGN),
    (dict(ws=A + 128), IDX_EALIGN),
    (dict(hist=A + 4), IDX_EALIGN),
    (dict(ws_bytes=1024), IDX_EWORKSPACE),
    (dict(stride=(1 << 23) + 4), IDX_EUNSUPPORTED),
])
def test_topk_rows_rejects(lib, kw, status):
    assert topk_call(lib, **kw) == status


def noalloc_call(lib, **kw):
    args = dict(logits=A, stride=256, hist=None, lens=A, rows=8, k=2048, key=0, idx=A, stream=None)
    args.update(kw)
    return lib.topk_rows_noalloc(args["logits"], args["stride"], args["hist"], args["lens"],
                                 args["rows"], args["k"], args["key"], args["idx"], args["stream"])


@pytest.mark.parametrize("kw,status", [
    (dict(logits=None), IDX_EINVAL),
    (dict(lens=None), IDX_EINVAL),
    (dict(idx=None), IDX_EINVAL),
    (dict(rows=0), IDX_EINVAL),
    (dict(k=8193), IDX_EINVAL),
    (dict(key=2), IDX_EUNSUPPORTED),
    (dict(stride=(1 << 23) + 4), IDX_EUNSUPPORTED),
    (dict(logits=A + 4), IDX_EALIGN),
    (dict(hist=A + 4), IDX_EALIGN),
    # the fixed scratch holds 128 rows of the chunked path (stride > 16384)
    (dict(rows=129, stride=16388), IDX_ESCRATCH),
    (dict(rows=65535, stride=1 << 20), IDX_ESCRATCH),
])
def test_topk_rows_noalloc_rejects(lib, kw, status):
    assert noalloc_call(lib, **kw) == status
    assert "IDX_ESCRATCH" in pmqa.indexer_status_str(IDX_ESCRATCH)


@pytest.mark.parametrize("kw,status", [
    (dict(src=None), IDX_EINVAL),
    (dict(nbytes=0), IDX_EINVAL),
    (dict(src=A + 8), IDX_EALIGN),
    (dict(nbytes=100), IDX_EALIGN),
])
def test_probe_rejects(lib, kw, status):
    args = dict(src=A, nbytes=1 << 20, sink=A)
    args.update(kw)
    assert lib.hbm_read_probe(args["src"], args["nbytes"], args["sink"], None) == status
    assert lib.hbm_read_probe_nt(args["src"], args["nbytes"], args["sink"], None) == status


@pytest.mark.parametrize("kw,status", [
    (dict(scores=None), IDX_EINVAL),
    (dict(hist=None), IDX_EINVAL),
    (dict(rows=0), IDX_EINVAL),
    (dict(stride=0), IDX_EINVAL),
    (dict(rows=70000), IDX_EUNSUPPORTED),
    (dict(scores=A + 4), IDX_EALIGN),
    (dict(stride=10), IDX_EALIGN),
    (dict(hist=A + 4), IDX_EALIGN),
])
def test_score_histogram_rejects(lib, kw, status):
    args = dict(scores=A, stride=1024, lens=A, rows=4, hist=A)
    args.update(kw)
    assert lib.score_histogram(args["scores"], args["stride"], args["lens"], args["rows"],
                               args["hist"], None) == status


def test_binding_refuses_cpu_tensors(lib):
    import torch
    q = torch.zeros(1, 32, 128, dtype=torch.uint8)
    with pytest.raises((ValueError, TypeError)):
        pmqa.indexer_logits(q, q, q, q, q, q, 1, q)


def mxfp4_call(lib, **kw):
    args = dict(q=A, kv=A, w=A, bt=A, lens=A, B=8, next_n=1, num_pages=16, max_pages=4,
                logits=A, stride=256, hist=None, stream=None)
    args.update(kw)
    return lib.indexer_logits_mxfp4(args["q"], args["kv"], args["w"], args["bt"], args["lens"],
                                    args["B"], args["next_n"], args["num_pages"],
                                    args["max_pages"], args["logits"], args["stride"],
                                    args["hist"], args["stream"])


@pytest.mark.parametrize("kw,status", [
    (dict(q=None), IDX_EINVAL),
    (dict(kv=None), IDX_EINVAL),
    (dict(logits=None), IDX_EINVAL),
    (dict(next_n=5), IDX_EUNSUPPORTED),
    (dict(B=0), IDX_EINVAL),
    (dict(kv=A + 4), IDX_EALIGN),
    (dict(stride=254), IDX_EALIGN),
    (dict(hist=A + 4), IDX_EALIGN),
])
def test_mxfp4_logits_rejects_before_launch(lib, kw, status):
    # no k_scales argument: the scales travel inside the 68-byte tokens
    assert mxfp4_call(lib, **kw) == status


def prefill_call(lib, mx=False, **kw):
    args = dict(q=A, kv=A, sc=A, w=A, bt=A, max_pages=4, cu=A, requests=2, tokens=40, lens=A,
                num_pages=16, logits=A, stride=256, stream=None)
    args.update(kw)
    tail = (args["w"], args["bt"], args["max_pages"], args["cu"], args["requests"], args["tokens"],
            args["lens"], args["num_pages"], args["logits"], args["stride"], args["stream"])
    if mx:
        return lib.indexer_prefill_logits_mxfp4(args["q"], args["kv"], *tail)
    return lib.indexer_prefill_logits(args["q"], args["kv"], args["sc"], *tail)


@pytest.mark.parametrize("mx", [False, True])
@pytest.mark.parametrize("kw,status", [
    (dict(q=None), IDX_EINVAL),
    (dict(kv=None), IDX_EINVAL),
    (dict(cu=None), IDX_EINVAL),
    (dict(lens=None), IDX_EINVAL),
    (dict(bt=None), IDX_EINVAL),
    (dict(logits=None), IDX_EINVAL),
    (dict(requests=0), IDX_EINVAL),
    (dict(tokens=0), IDX_EINVAL),
    (dict(max_pages=0), IDX_EINVAL),
    (dict(num_pages=-1), IDX_EINVAL),
    (dict(requests=4097), IDX_EUNSUPPORTED),
    (dict(tokens=65536), IDX_EUNSUPPORTED),
    (dict(requests=4096, max_pages=1 << 20), IDX_EUNSUPPORTED),
    (dict(q=A + 8), IDX_EALIGN),
    (dict(w=A + 4), IDX_EALIGN),
    (dict(cu=A + 2), IDX_EALIGN),
    (dict(logits=A + 4), IDX_EALIGN),
    (dict(stride=258), IDX_EALIGN),
])
def test_prefill_rejects_before_launch(lib, mx, kw, status):
    assert prefill_call(lib, mx=mx, **kw) == status


def test_prefill_needs_scales_for_fp8(lib):
    assert prefill_call(lib, sc=None) == IDX_EINVAL


@pytest.mark.parametrize("kw,status", [
    (dict(pool=None), IDX_EINVAL),
    (dict(table=None), IDX_EINVAL),
    (dict(n=0), IDX_EINVAL),
    (dict(num=0), IDX_EINVAL),
    (dict(pool=A + 8), IDX_EALIGN),
    (dict(scales=A + 2), IDX_EALIGN),
])
def test_gather_probe_rejects(lib, kw, status):
    args = dict(pool=A, scales=A, table=A, n=64, num=64, sink=A)
    args.update(kw)
    assert lib.hbm_gather_probe(args["pool"], args["scales"], args["table"], args["n"], args["num"],
                                args["sink"], None) == status


@pytest.mark.parametrize("kw", [
    dict(out=None), dict(mode=-1), dict(mode=3), dict(waves=0), dict(waves=9), dict(iters=0),
    dict(iters=(1 << 20) + 1),
])
def test_coissue_probe_rejects_before_any_device_query(lib, kw):
    args = dict(mode=2, waves=1, iters=16, out=A, out_len=1 << 20)
    args.update(kw)
    assert lib.mfma_valu_probe(args["mode"], args["waves"], args["iters"], args["out"], args["out_len"],
                               None) == IDX_EINVAL


@pytest.mark.parametrize("kw,status", [
    (dict(scores=None), IDX_EINVAL),
    (dict(table=None), IDX_EINVAL),
    (dict(out=None), IDX_EINVAL),
    (dict(k=0), IDX_EINVAL),
    (dict(k=8193), IDX_EINVAL),
    (dict(kb=0), IDX_EINVAL),
    (dict(key=7), IDX_EUNSUPPORTED),
    (dict(stride=16388), IDX_EUNSUPPORTED),
    (dict(kb=(1 << 17) + 1), IDX_EUNSUPPORTED),
    (dict(scores=A + 8), IDX_EALIGN),
    (dict(stride=4098), IDX_EALIGN),
    (dict(hist=A + 4), IDX_EALIGN),
])
def test_sparse_topk_rejects(lib, kw, status):
    args = dict(scores=A, stride=4096, hist=None, lens=A, rows=4, k=2048, key=0, table=A, kb=512, out=A)
    args.update(kw)
    assert lib.sparse_topk(args["scores"], args["stride"], args["hist"], args["lens"], args["rows"], args["k"],
                           args["key"], args["table"], args["kb"], args["out"], None) == status
