"""Ragged prefill (extend) logits (SGLang PR #38944, the SM90 FP8 prefill
commit) on the GPU: element by element against the CPU oracle on ragged
batches that span several row tiles and key chunks, with ragged tails and an
empty request; on the full extend workload bitwise against the decode kernel
(the same arithmetic) on sampled rows and within tolerance of the oracle at
sampled keys; and the ragged top-k over prefill rows, bit-exact from the
GPU's own logits."""
import numpy as np
import pytest
import torch

import gen
import oracle as O
from tests.gpu_harness import DEV, DevInputs, announce, check_topk, sample_cols, topk

pytestmark = pytest.mark.gpu

P = O.prefill
SENT = -7.0


class PrefillDev:
    def __init__(self, x):
        self.x = x
        self.d = DevInputs(x)
        self.cu = torch.from_numpy(np.ascontiguousarray(x.cu_q)).to(DEV)

    def run(self, gpu, stride=None, lens=None):
        x, d = self.x, self.d
        lg = torch.full((x.rows, stride or x.logits_stride), SENT, dtype=torch.float32, device=DEV)
        gpu.indexer_prefill_logits(d.q, d.kv, d.sc, d.w, d.bt, self.cu, d.lens if lens is None else lens, lg)
        torch.cuda.synchronize()
        return lg


def check_rows(x, got, rows, lens=None, sample=None, seed=0):
    """Rows of GPU logits against the oracle; columns past each row's length
    must still hold the sentinel."""
    lens = x.context_lens if lens is None else lens
    rng = np.random.default_rng(seed)
    for i, t in enumerate(rows):
        g_row = got[i]
        n = int(lens[t])
        assert np.all(g_row[n:] == SENT), f"row {t}: columns past its length {n} were written"
        if n == 0:
            continue
        cols = sample_cols(n, sample, rng)
        args = (x.q, x.kv_pages, x.k_scales, x.weights, x.block_table, x.cu_q, t, cols)
        want = P.prefill_logits_at(*args)
        bound = P.prefill_error_bound_at(*args)
        hsum = P.prefill_head_sum_at(*args)
        hbound = P.prefill_error_bound_at(*args, unscaled=True)
        ok = O.check_logits(g_row[cols], want, bound, hsum, hbound)
        if not ok.all():
            bad = np.nonzero(~ok)[0][:5]
            raise AssertionError(f"row {t}: {int((~ok).sum())} logits outside tolerance, e.g. cols "
                                 f"{cols[bad].tolist()} got {g_row[cols][bad].tolist()} "
                                 f"want {want[bad].tolist()}")


# Requests of 37, 64, 0, 5, 130, 16 and 1 rows over prefixes up to 4000 keys:
# partial 16-row tiles, a request without rows, 8-page chunks with a partial
# last page, a single-row request.
SMALL_Q = [37, 64, 0, 5, 130, 16, 1]
SMALL_PREFIX = [0, 100, 50, 1000, 3, 4000, 700]


@pytest.mark.parametrize("kfmt", ["fp8", "mxfp4"])
def test_prefill_small_all_keys(gpu, kfmt):
    x = gen.make_prefill_inputs("pf_small", SMALL_Q, SMALL_PREFIX, 81, kfmt=kfmt)
    pd = PrefillDev(x)
    stride = x.logits_stride + 8
    announce(f"indexer_prefill_logits small {kfmt} rows={x.rows}")
    got = pd.run(gpu, stride=stride).cpu().numpy()
    check_rows(x, got, range(x.rows))


def test_prefill_custom_row_lens(gpu):
    """Row lengths chosen freely inside each request's context: zero, one,
    exact page multiples, the full context; rows of one tile then reach very
    different key ranges."""
    x = gen.make_prefill_inputs("pf_lens", [20, 33], [600, 0], 83)
    lens = x.context_lens.copy()
    ctx = [620, 33]
    rng = np.random.default_rng(5)
    for r in range(x.B):
        for t in range(int(x.cu_q[r]), int(x.cu_q[r + 1])):
            lens[t] = rng.choice([0, 1, 64, 128, 192, ctx[r], int(rng.integers(0, ctx[r] + 1))])
    pd = PrefillDev(x)
    announce("indexer_prefill_logits custom row lengths")
    got = pd.run(gpu, lens=torch.from_numpy(lens).to(DEV)).cpu().numpy()
    check_rows(x, got, range(x.rows), lens=lens)


def test_prefill_single_row(gpu):
    x = gen.make_prefill_inputs("pf_one", [1], [0], 85)
    pd = PrefillDev(x)
    announce("indexer_prefill_logits one row, one key")
    got = pd.run(gpu, stride=4).cpu().numpy()
    check_rows(x, got, range(1))


@pytest.mark.parametrize("key_dtype", [O.KEY_FP32, O.KEY_FP16])
def test_prefill_ragged_topk(gpu, key_dtype):
    """The prefill rows feed topk_rows with context_lens = row lengths."""
    x = gen.make_prefill_inputs("pf_topk", SMALL_Q, SMALL_PREFIX, 87)
    pd = PrefillDev(x)
    announce(f"prefill -> topk_rows key={key_dtype}")
    lg = pd.run(gpu)
    idx = topk(lg, None, pd.d.lens, 256, key_dtype)
    check_topk(idx.cpu().numpy(), lg.cpu().numpy(), x.context_lens, 256, key_dtype)


def _decode_of_rows(x, d, rows):
    """The given prefill rows as a decode call: one request per row, its own
    block-table row, context length = the row's length."""
    req = P.request_of_rows(x.cu_q)[rows]
    r = torch.from_numpy(np.asarray(rows, np.int64)).to(DEV)
    q = d.q.index_select(0, r).contiguous()
    w = d.w.index_select(0, r).contiguous()
    bt = d.bt.index_select(0, torch.from_numpy(req).to(DEV)).contiguous()
    lens = d.lens.index_select(0, r).contiguous()
    return q, w, bt, lens


@pytest.mark.parametrize("name", gen.PREFILL_CONFIG_NAMES)
def test_prefill_extend_workload(gpu, name):
    """Full extend batch (8192 rows, contexts 2K..32K), in the launch shape
    the benchmark times: sampled rows bitwise equal to the decode kernel's
    logits of the same rows, and within tolerance of the oracle at sampled
    keys."""
    announce(f"generate {name}")
    x = gen.config_inputs(name)
    pd = PrefillDev(x)
    announce(f"indexer_prefill_logits {name}")
    lg = pd.run(gpu)
    rng = np.random.default_rng(89)
    edges = np.concatenate([[int(a), int(b) - 1] for a, b in zip(x.cu_q[:-1], x.cu_q[1:]) if b > a])
    rows = np.unique(np.concatenate([edges, rng.choice(x.rows, 24, replace=False)]))
    got = lg.index_select(0, torch.from_numpy(rows).to(DEV)).cpu().numpy()
    q, w, bt, lens = _decode_of_rows(x, pd.d, rows)
    dec = torch.full((rows.size, x.logits_stride), SENT, dtype=torch.float32, device=DEV)
    announce(f"indexer_logits on {rows.size} of its rows")
    if pd.d.sc is None:
        gpu.indexer_logits_mxfp4(q, pd.d.kv, w, bt, lens, 1, dec, None)
    else:
        gpu.indexer_logits(q, pd.d.kv, pd.d.sc, w, bt, lens, 1, dec, None)
    torch.cuda.synchronize()
    dec = dec.cpu().numpy()
    for i, t in enumerate(rows):
        n = int(x.context_lens[t])
        assert np.array_equal(got[i, :n].view(np.uint32), dec[i, :n].view(np.uint32)), \
            f"row {t}: prefill logits differ from the decode logits of the same row"
    check_rows(x, got, rows, sample=256, seed=3)


@pytest.mark.parametrize("kfmt", ["fp8", "mxfp4"])
def test_prefill_long_ranges_cross_page_windows(gpu, kfmt):
    """A request of 1040 rows over a 48000-key prefix next to a small one:
    each of a tile's 8 workgroups walks about 96 pages, more than one
    64-page window of page ids, with the staging flushed every 16 pages.
    Sampled rows bitwise against the decode kernel, and within tolerance of
    the oracle at sampled keys; columns past each row stay untouched."""
    x = gen.make_prefill_inputs(f"pf_long_{kfmt}", [1040, 7], [48000, 300], 91, kfmt=kfmt)
    pd = PrefillDev(x)
    announce(f"indexer_prefill_logits long ranges {kfmt} rows={x.rows}")
    lg = pd.run(gpu)
    rows = np.array([0, 1, 15, 16, 517, 1023, 1038, 1039, 1040, 1046])
    got = lg.index_select(0, torch.from_numpy(rows).to(DEV)).cpu().numpy()
    q, w, bt, lens = _decode_of_rows(x, pd.d, rows)
    dec = torch.full((rows.size, x.logits_stride), SENT, dtype=torch.float32, device=DEV)
    if pd.d.sc is None:
        gpu.indexer_logits_mxfp4(q, pd.d.kv, w, bt, lens, 1, dec, None)
    else:
        gpu.indexer_logits(q, pd.d.kv, pd.d.sc, w, bt, lens, 1, dec, None)
    torch.cuda.synchronize()
    dec = dec.cpu().numpy()
    for i, t in enumerate(rows):
        n = int(x.context_lens[t])
        assert np.array_equal(got[i, :n].view(np.uint32), dec[i, :n].view(np.uint32)), \
            f"row {t}: prefill logits differ from the decode logits of the same row"
    check_rows(x, got, rows, sample=200, seed=7)
