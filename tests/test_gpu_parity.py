"""HIP path vs the CPU oracle on small seeded inputs that still span several
pages, ragged tails and every next_n, plus the edge cases of the method."""
import numpy as np
import pytest
import torch

import gen
import paged_mqa_logits_indexer_amd as pmqa
import oracle as O
from tests import oracle_pins as P
from tests.gpu_harness import (DEV, PATHS, DevInputs, announce, check_hist, check_logits,
                               check_padding, check_topk, on_path, topk)

pytestmark = pytest.mark.gpu

INF = float("inf")


def _scores_dev(rows_list):
    """Pack rows of different lengths into one [rows, stride] buffer (+inf pad)."""
    n = max(len(r) for r in rows_list)
    stride = max(4, -(-n // 4) * 4)
    buf = np.full((len(rows_list), stride), np.inf, dtype=np.float32)
    lens = np.zeros(len(rows_list), dtype=np.int32)
    for i, r in enumerate(rows_list):
        buf[i, :len(r)] = r
        lens[i] = len(r)
    return buf, lens


def _edge_rows():
    """Rows that hit every bin regime, rounding edge and special value."""
    enc = np.arange(65536, dtype=np.uint32).astype(np.uint16).view(np.float16).astype(np.float32)
    vals = P._fp16_positive_values()
    mids = np.array([float((vals[i] + vals[i + 1]) / 2) for i in range(len(vals) - 1)],
                    dtype=np.float32)
    mids = np.concatenate([mids, np.nextafter(mids, np.float32(np.inf)),
                           np.nextafter(mids, np.float32(0))])
    mids = np.concatenate([mids, -mids[::3]])
    rng = np.random.default_rng(77)
    bits = rng.integers(0, 2 ** 32, 200_000, dtype=np.uint64).astype(np.uint32)
    rnd = bits.view(np.float32)
    golden, _ = P.load_golden_bins()
    return [enc, mids, rnd, golden, np.zeros(0, np.float32), enc[:5]]


def test_bins_of_every_fp16_encoding_and_rounding_edge(gpu):
    rows = _edge_rows()
    buf, lens = _scores_dev(rows)
    s = torch.from_numpy(buf).to(DEV)
    ln = torch.from_numpy(lens).to(DEV)
    h = torch.zeros((len(rows), 1024), dtype=torch.int32, device=DEV)
    announce(f"score_histogram edge rows {buf.shape}")
    gpu.score_histogram(s, ln, h)
    torch.cuda.synchronize()
    check_hist(lens, buf, h.cpu().numpy())
    # accumulates on a second call
    gpu.score_histogram(s, ln, h)
    torch.cuda.synchronize()
    check_hist(lens, buf, h.cpu().numpy(), hist_in=O.coarse_histogram(buf, lens))


@pytest.mark.parametrize("path", PATHS)
@pytest.mark.parametrize("key", [O.KEY_FP32, O.KEY_FP16])
@pytest.mark.parametrize("k", [1, 100, 2048, 8192])
def test_topk_edge_rows_without_histogram(gpu, key, k, path):
    rows = _edge_rows()
    buf, lens = _scores_dev(rows)
    s, ln = on_path(torch.from_numpy(buf).to(DEV), torch.from_numpy(lens).to(DEV), path)
    announce(f"topk_rows hist=NULL edge rows k={k} key={key} path={path}")
    idx = topk(s, None, ln, k, key)
    check_topk(idx.cpu().numpy(), s.cpu().numpy(), ln.cpu().numpy(), k, key)


def _small_inputs(next_n, seed, base, weight_scale=1.0, inf_frac=0.0):
    return gen.make_indexer_inputs(f"small{next_n}", len(base), next_n, base, seed,
                                   weight_scale=weight_scale, inf_frac=inf_frac)


SMALL = [
    (1, 11, [1000, 130, 5000, 64, 4097]),
    (2, 12, [777, 2049, 63]),
    (3, 13, [3000, 65, 1]),
    (4, 14, [4096, 1500, 129]),
]


@pytest.mark.parametrize("next_n,seed,base", SMALL, ids=[f"next_n{s[0]}" for s in SMALL])
def test_small_logits_hist_topk(gpu, next_n, seed, base):
    x = _small_inputs(next_n, seed, base)
    d = DevInputs(x)
    announce(f"indexer_logits small next_n={next_n} lens={x.context_lens.tolist()}")
    lg, h = d.run(with_hist=True, fill=INF)
    got = lg.cpu().numpy()
    check_logits(x, got)
    check_padding(x, got, INF)
    check_hist(x.context_lens, got, h.cpu().numpy())
    for key in (O.KEY_FP32, O.KEY_FP16):
        for k in (64, 2048):
            announce(f"topk_rows small next_n={next_n} k={k} key={key}")
            idx = topk(lg, h, d.lens, k, key)
            check_topk(idx.cpu().numpy(), got, x.context_lens, k, key)


@pytest.mark.parametrize("variant,scale,inf_frac", [("unit", 16.0, 0.0), ("mixed", 4.0, 0.01)])
def test_small_unit_and_mixed_regimes(gpu, variant, scale, inf_frac):
    x = _small_inputs(4, 31, [2500, 700], weight_scale=scale, inf_frac=inf_frac)
    d = DevInputs(x)
    announce(f"indexer_logits {variant} regime")
    lg, h = d.run(with_hist=True, fill=INF)
    got = lg.cpu().numpy()
    check_logits(x, got)
    check_hist(x.context_lens, got, h.cpu().numpy())
    for key in (O.KEY_FP32, O.KEY_FP16):
        idx = topk(lg, h, d.lens, 512, key)
        check_topk(idx.cpu().numpy(), got, x.context_lens, 512, key)


def test_zero_length_and_tiny_rows(gpu):
    x = gen.make_indexer_inputs("tiny_rows", 5, 1, [0, 1, 63, 64, 65], 41)
    d = DevInputs(x)
    announce("indexer_logits rows of length 0/1/63/64/65")
    lg, h = d.run(with_hist=True, fill=INF)
    got = lg.cpu().numpy()
    check_logits(x, got)
    check_padding(x, got, INF)
    check_hist(x.context_lens, got, h.cpu().numpy())
    assert int(h[0].sum()) == 0
    for key in (O.KEY_FP32, O.KEY_FP16):
        idx = topk(lg, h, d.lens, 2048, key).cpu().numpy()
        check_topk(idx, got, x.context_lens, 2048, key)
        assert np.all(idx[0] == -1)
    # verify rows where the first token sees no key
    y = gen.make_indexer_inputs("tiny_verify", 2, 3, [0, 5], 42)
    e = DevInputs(y)
    lg2, h2 = e.run(with_hist=True, fill=INF)
    got2 = lg2.cpu().numpy()
    check_logits(y, got2)
    check_padding(y, got2, INF)
    check_hist(y.context_lens, got2, h2.cpu().numpy())


def test_many_requests_persistent_grid(gpu):
    """B >= 32 one-row requests take the persistent grid (64-page shares
    dealt round robin from the lengths): element by element against the
    oracle with empty, tiny and multi-share rows, and bitwise against the
    same requests scored by two calls of 20 (the (chunks, B) grid)."""
    rng = np.random.default_rng(4040)
    lens = rng.integers(0, 9000, 40)
    lens[:6] = [0, 1, 63, 64, 4096, 8193]  # empty, one key, page edges, share edges
    x = gen.make_indexer_inputs("persist40", 40, 1, lens.tolist(), 43, logits_stride=9216)
    d = DevInputs(x)
    announce(f"indexer_logits persistent grid B=40 lens={x.context_lens.tolist()}")
    lg, h = d.run(with_hist=True, fill=INF)
    got = lg.cpu().numpy()
    check_logits(x, got)
    check_padding(x, got, INF)
    check_hist(x.context_lens, got, h.cpu().numpy())
    for key in (O.KEY_FP32, O.KEY_FP16):
        idx = topk(lg, h, d.lens, 2048, key)
        check_topk(idx.cpu().numpy(), got, x.context_lens, 2048, key)
    # the same requests in two halves of 20: the (chunks, B) grid
    halves = []
    for r0 in (0, 20):
        lg2 = d.new_logits(INF)
        h2 = d.new_hist()
        sl = slice(r0, r0 + 20)
        pmqa.indexer_logits(d.q[sl].contiguous(), d.kv, d.sc, d.w[sl].contiguous(), d.bt[sl].contiguous(),
                            d.lens[sl].contiguous(), 1, lg2[sl], h2[sl])
        halves.append((lg2[sl], h2[sl]))
    torch.cuda.synchronize()
    got2 = torch.cat([a for a, _ in halves]).cpu().numpy()
    h_2 = torch.cat([b for _, b in halves]).cpu().numpy()
    assert np.array_equal(got.view(np.uint32), got2.view(np.uint32)), "persistent grid differs from the static grid"
    assert np.array_equal(h.cpu().numpy(), h_2)
    # FP16 output through the persistent grid: the halves the float32 logits
    # round to (round to nearest even), the same histogram
    announce("indexer_logits_f16 persistent grid B=40")
    lg16, h16 = d.run_f16(with_hist=True, fill=INF)
    got16 = lg16.cpu().numpy()[:, :x.logits_stride]
    live = np.arange(x.logits_stride)[None, :] < x.context_lens[:, None]
    want16 = got.astype(np.float16)
    assert np.array_equal(np.where(live, got16, 0).view(np.uint16), np.where(live, want16, 0).view(np.uint16))
    assert np.all(np.isinf(got16[~live]))
    assert np.array_equal(h16.cpu().numpy(), h.cpu().numpy())


def test_histogram_off_is_bitwise_identical_and_counts_accumulate(gpu):
    x = _small_inputs(2, 51, [3333, 999])
    d = DevInputs(x)
    announce("indexer_logits hist on/off and accumulate")
    lg_on, h = d.run(with_hist=True, fill=0.0)
    lg_off, _ = d.run(with_hist=False, fill=0.0)
    assert torch.equal(lg_on.view(torch.int32), lg_off.view(torch.int32))
    first = h.clone()
    d.logits(lg_on, h)  # second call on the same histogram
    torch.cuda.synchronize()
    assert torch.equal(h, 2 * first)
    # repeated runs are deterministic
    lg3, h3 = d.run(with_hist=True, fill=0.0)
    assert torch.equal(lg3.view(torch.int32), lg_off.view(torch.int32))
    assert torch.equal(h3, first)


@pytest.mark.parametrize("path", PATHS)
def test_topk_stale_histograms_stay_exact(gpu, path):
    x = _small_inputs(1, 61, [20000, 9000, 3000, 12000])
    d = DevInputs(x)
    announce(f"topk_rows stale histograms path={path}")
    lg, h = d.run(with_hist=True, fill=INF)
    lg, ln = on_path(lg, d.lens, path)
    got = lg.cpu().numpy()
    lens = ln.cpu().numpy()
    stale = {
        "zeros": torch.zeros_like(h),
        "doubled": 2 * h,
        "rolled": torch.roll(h, 1, dims=0),
        "shifted": torch.roll(h, 37, dims=1),
        "random": torch.randint(0, 50, h.shape, dtype=torch.int32, device=DEV),
        "huge": torch.full_like(h, 3000),
    }
    for name, hs in stale.items():
        for key in (O.KEY_FP32, O.KEY_FP16):
            for k in (1, 2048, 5000):
                announce(f"topk_rows stale={name} key={key} k={k}")
                idx = topk(lg, hs, ln, k, key)
                check_topk(idx.cpu().numpy(), got, lens, k, key)


@pytest.mark.parametrize("path", PATHS)
def test_topk_threshold_bin_overflow_falls_back_exactly(gpu, path):
    rng = np.random.default_rng(71)
    n = 30000
    rows = [
        np.full(n, 1.0, np.float32),                               # one value
        (np.float32(5.0) + rng.integers(0, 64, n).astype(np.float32)
         * np.float32(2.0 ** -8)).astype(np.float32),              # one fine bin, many values
        np.concatenate([np.full(9000, 3.0, np.float32),
                        rng.standard_normal(n - 9000).astype(np.float32)]),
        np.where(rng.random(n) < 0.5, np.float32(np.nan), np.float32(2.0)).astype(np.float32),
    ]
    buf, lens = _scores_dev(rows)
    s, ln = on_path(torch.from_numpy(buf).to(DEV), torch.from_numpy(lens).to(DEV), path)
    buf, lens = s.cpu().numpy(), ln.cpu().numpy()
    h = torch.zeros((len(rows), 1024), dtype=torch.int32, device=DEV)
    gpu.score_histogram(s, ln, h)
    for key in (O.KEY_FP32, O.KEY_FP16):
        for k in (2048, 8192):
            announce(f"topk_rows overflow rows key={key} k={k} path={path}")
            idx = topk(s, h, ln, k, key)
            check_topk(idx.cpu().numpy(), buf, lens, k, key)
            idx = topk(s, None, ln, k, key)
            check_topk(idx.cpu().numpy(), buf, lens, k, key)


@pytest.mark.parametrize("path", PATHS)
def test_topk_ties_go_to_lower_columns(gpu, path):
    # equal keys spread over one or many chunks and both refine paths
    n = 50000
    rng = np.random.default_rng(81)
    a = rng.integers(0, 5, n).astype(np.float32)             # few distinct values
    b = (np.float32(100.0) + rng.integers(0, 3, n).astype(np.float32)
         * np.float32(2.0 ** -12)).astype(np.float32)        # fp16 ties, fp32 distinct
    c = np.zeros(n, np.float32)
    c[rng.integers(0, n, n // 2)] = -0.0                     # +0 / -0 mix
    buf, lens = _scores_dev([a, b, c])
    s, ln = on_path(torch.from_numpy(buf).to(DEV), torch.from_numpy(lens).to(DEV), path)
    buf, lens = s.cpu().numpy(), ln.cpu().numpy()
    h = torch.zeros((3, 1024), dtype=torch.int32, device=DEV)
    gpu.score_histogram(s, ln, h)
    for key in (O.KEY_FP32, O.KEY_FP16):
        for k in (7, 2048, 6000):
            announce(f"topk_rows ties key={key} k={k} path={path}")
            idx = topk(s, h, ln, k, key)
            check_topk(idx.cpu().numpy(), buf, lens, k, key)


def _register_bin_row(rng, n, n_above, inside, ties, below):
    """A row whose threshold bin [20, 21) holds `inside` distinct values above
    20.5, `ties` copies of 20.5 (one of them in the last column) and `below`
    distinct values under it, with n_above distinct values in [25, 200) and
    the rest far below the bin: a bin of a few hundred candidates."""
    above = rng.uniform(25.0, 200.0, n_above).astype(np.float32)
    hi = rng.uniform(20.5, 21.0, inside * 2).astype(np.float32)
    hi = np.unique(hi[hi > np.float32(20.5)])[:inside]
    lo = np.unique(rng.uniform(20.0, 20.5, below * 2).astype(np.float32))[:below]
    rest = np.clip(rng.standard_normal(n - n_above - len(hi) - ties - len(lo)) * 2.0, -15, 15)
    row = np.concatenate([above, hi, np.full(ties - 1, 20.5, np.float32), lo,
                          rest.astype(np.float32)])
    rng.shuffle(row)
    return np.concatenate([row, np.array([20.5], np.float32)])


@pytest.mark.parametrize("path", ["as_is", "wide"])
def test_topk_threshold_bin_selected_from_registers(gpu, path):
    # threshold bins of a few hundred candidates (all of them in the finish
    # pass's early loads): ties at the final key cut by column with more than
    # 64 ties, a bin whose keys are all equal, and few ties; rows of lengths
    # that are not powers of two (the column bound comes from the length)
    rng = np.random.default_rng(2024)
    # 1500 candidates all in even 4096-column chunks: more than 1024 come from
    # the front list, so they reach the finish pass through LDS first
    row = np.clip(rng.standard_normal(40000) * 2.0, -15, 15).astype(np.float32)
    even = np.concatenate([np.arange(c * 4096, min(c * 4096 + 4096, 40000)) for c in range(0, 10, 2)])
    cols = rng.choice(even, 1900 + 1500, replace=False)
    row[cols[:1900]] = rng.uniform(25.0, 200.0, 1900).astype(np.float32)
    row[cols[1900:]] = np.round(rng.uniform(20.0, 21.0, 1500) * 64) / np.float32(64)  # ties
    cases = [  # (row, k)
        (_register_bin_row(rng, 40000, 1900, 100, 300, 100), 2048),
        (_register_bin_row(rng, 39999, 1900, 0, 500, 0), 2048),
        (_register_bin_row(rng, 25001, 1900, 100, 40, 300), 2020),
        (_register_bin_row(rng, 65537, 1900, 60, 200, 60), 2000),
        (row, 2048),
    ]
    for ci, (row, k) in enumerate(cases):
        buf, lens = _scores_dev([row])
        s, ln = on_path(torch.from_numpy(buf).to(DEV), torch.from_numpy(lens).to(DEV), path)
        buf, lens = s.cpu().numpy(), ln.cpu().numpy()
        h = torch.zeros((1, 1024), dtype=torch.int32, device=DEV)
        gpu.score_histogram(s, ln, h)
        for key in (O.KEY_FP32, O.KEY_FP16):
            announce(f"topk_rows register-path bin case={ci} key={key} k={k} path={path}")
            idx = topk(s, h, ln, k, key)
            check_topk(idx.cpu().numpy(), buf, lens, k, key)


def test_topk_row_of_more_than_512_chunks(gpu):
    # the last workgroup adds up and gathers the chunk slots 512 at a time
    n = 512 * 8192 + 5000
    rng = np.random.default_rng(95)
    buf = (rng.standard_normal((1, n), dtype=np.float32) * np.float32(3.0)).astype(np.float32)
    buf[0, rng.integers(0, n, 3000)] = np.float32(7.5)          # ties across many chunks
    lens = np.array([n - 3], np.int32)
    s = torch.from_numpy(buf).to(DEV)
    ln = torch.from_numpy(lens).to(DEV)
    h = torch.zeros((1, 1024), dtype=torch.int32, device=DEV)
    gpu.score_histogram(s, ln, h)
    for key in (O.KEY_FP32, O.KEY_FP16):
        announce(f"topk_rows {n}-score row key={key}")
        idx = topk(s, h, ln, 2048, key)
        check_topk(idx.cpu().numpy(), buf, lens, 2048, key)


def _threshold(hist_row, k):
    """The selector's threshold bin of one histogram row: the least bin whose
    running count reaches k (1024 when the row holds at most k), with the
    histogram's count before it and in it."""
    c = np.cumsum(hist_row.astype(np.int64))
    if c[-1] <= k:
        return 1024, int(c[-1]), 0
    b = int(np.argmax(c >= k))
    return b, int(c[b] - hist_row[b]), int(hist_row[b])


@pytest.mark.parametrize("key", [O.KEY_FP32, O.KEY_FP16])
def test_topk_garbage_workspace_with_stale_histogram(gpu, key):
    """A workspace nobody initialised, together with a stale histogram: random
    bytes, 0xA5 everywhere, and counters crafted so that, added to this
    call's true counts, they equal the stale histogram's own counts -- the
    case a check of the counters against the histogram alone would pass
    with shifted places.  Every call exact, and the next call on the same
    workspace (now left clean) too."""
    x = _small_inputs(1, 61, [20000, 9000, 3000, 12000])
    d = DevInputs(x)
    announce(f"topk_rows garbage workspace + stale histogram key={key}")
    lg, h = d.run(with_hist=True, fill=INF)
    got = lg.cpu().numpy()
    lens = x.context_lens
    rows = x.rows
    rec = gpu.topk_workspace_bytes(1, lg.shape[1], 1)
    assert rec % 8 == 0
    stale = {
        "exact": h.clone(),
        "zeros": torch.zeros_like(h),
        "doubled": 2 * h,
        "rolled": torch.roll(h, 1, dims=0),
        "shifted": torch.roll(h, 37, dims=1),
    }
    rng = np.random.default_rng(5)
    for k in (100, 2048):
        for name, hs in stale.items():
            hs_np = hs.cpu().numpy()
            for fill in ("random", "a5", "crafted"):
                if fill == "random":
                    ws = torch.from_numpy(rng.integers(0, 256, rows * rec, dtype=np.uint8)).to(DEV)
                else:
                    ws = torch.full((rows * rec,), 0xA5, dtype=torch.uint8, device=DEV)
                if fill == "crafted":
                    counters = np.zeros((rows, 2), np.uint64)
                    for r in range(rows):
                        b, before, count = _threshold(hs_np[r], k)
                        bins = O.coarse_bin(got[r, :int(lens[r])])
                        live = bins >= 0
                        gt = int(np.sum(live & (bins < b)))
                        eq = int(np.sum(bins == b))
                        g_gt = (before - gt) % (1 << 32)
                        g_eq = (count - eq) % (1 << 32)
                        counters[r, 0] = np.uint64(g_gt | (g_eq << 32))
                    w64 = ws.view(torch.int64).view(rows, rec // 8)
                    w64[:, 0:2] = torch.from_numpy(counters.view(np.int64)).to(DEV)
                for call in range(2):
                    announce(f"topk_rows ws={fill} stale={name} k={k} key={key} call={call}")
                    idx = topk(lg, hs, d.lens, k, key, workspace=ws)
                    check_topk(idx.cpu().numpy(), got, lens, k, key)


@pytest.mark.parametrize("key", [O.KEY_FP32, O.KEY_FP16])
def test_topk_empty_rows_with_a_stale_threshold_slot(gpu, key):
    """The finish pass takes b* from the record the collect pass wrote; a row
    with no live score runs no collect workgroup, so it reads whatever the
    slot holds (all bins, bin 0, a middle bin, a negative value, 0xA5 bytes):
    it must still come out as padding only, next to normal rows."""
    rng = np.random.default_rng(515)
    stride = 40000
    rows = [np.zeros(0, np.float32), rng.standard_normal(30000).astype(np.float32),
            np.zeros(0, np.float32), np.array([2.5], np.float32), np.zeros(0, np.float32)]
    buf, lens = _scores_dev(rows)
    buf = np.concatenate([buf, np.full((buf.shape[0], stride - buf.shape[1]), np.inf, np.float32)], axis=1)
    s_, ln = torch.from_numpy(buf).to(DEV), torch.from_numpy(lens).to(DEV)
    h = torch.zeros((len(rows), 1024), dtype=torch.int32, device=DEV)
    gpu.score_histogram(s_, ln, h)
    rec = gpu.topk_workspace_bytes(1, stride, 1)
    for slot in (1024, 0, 600, -5, None):
        ws = torch.full((len(rows) * rec,), 0xA5, dtype=torch.uint8, device=DEV)
        w32 = ws.view(torch.int32).view(len(rows), rec // 4)
        w32[:, 0:4] = 0  # clean counter pairs
        if slot is not None:
            w32[:, 4] = slot  # the b* slot after the two pairs
        for k in (1, 2048):
            announce(f"topk_rows empty rows, b* slot {slot}, k={k} key={key}")
            idx = topk(s_, h, ln, k, key, workspace=ws)
            check_topk(idx.cpu().numpy(), buf, lens, k, key)


@pytest.mark.parametrize("key", [O.KEY_FP32, O.KEY_FP16])
def test_topk_without_histogram_reuses_its_workspace(gpu, key):
    """hist=NULL on rows longer than 8192: the selector builds its histograms
    in the workspace, and every call leaves them zero for the next.  A
    workspace that starts as garbage, then calls on different rows through
    the same workspace: each result exact."""
    rng = np.random.default_rng(606)
    n = 40000
    ws = torch.full((gpu.topk_workspace_bytes(3, n, 2048),), 0xA5, dtype=torch.uint8, device=DEV)
    for call in range(4):
        rows = [rng.standard_normal(n).astype(np.float32) * np.float32(2.0 ** call),
                np.round(rng.standard_normal(n - 1001) * 3).astype(np.float32),  # many ties
                np.where(rng.random(n - 7) < 0.01, np.float32(40.0), rng.standard_normal(n - 7)).astype(np.float32)]
        buf, lens = _scores_dev(rows)
        s_, ln = torch.from_numpy(buf).to(DEV), torch.from_numpy(lens).to(DEV)
        announce(f"topk_rows hist=NULL workspace reuse call={call} key={key}")
        idx = topk(s_, None, ln, 2048, key, workspace=ws)
        check_topk(idx.cpu().numpy(), buf, lens, 2048, key)


def test_calls_replay_in_a_hip_graph(gpu):
    # one row of one selector chunk, one of several (the arrival counters of
    # a replayed launch must start from zero again); the workspace starts
    # out as garbage and eager calls on it run between the replays
    x = _small_inputs(2, 91, [5000, 30000])
    d = DevInputs(x)
    k = 2048
    lg = d.new_logits(INF)
    h = d.new_hist()
    idx = torch.full((x.rows, k), -7, dtype=torch.int32, device=DEV)
    ws = torch.full((gpu.topk_workspace_bytes(x.rows, x.logits_stride, k),), 0xA5, dtype=torch.uint8,
                    device=DEV)
    announce("eager reference for graph replay")
    d.logits(lg, h)
    gpu.topk_rows(lg, h, d.lens, k, O.KEY_FP32, idx, ws)
    torch.cuda.synchronize()
    ref_lg, ref_h, ref_idx = lg.clone(), h.clone(), np.sort(idx.cpu().numpy(), axis=1)
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            h.zero_()
            d.logits(lg, h)
            gpu.topk_rows(lg, h, d.lens, k, O.KEY_FP32, idx, ws)
    torch.cuda.synchronize()
    for rep in range(4):
        announce(f"graph replay {rep}")
        lg.fill_(-1.0)
        idx.fill_(-7)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(h, ref_h)
        assert np.array_equal(np.sort(idx.cpu().numpy(), axis=1), ref_idx)
        live = torch.from_numpy(np.arange(x.logits_stride)[None, :] < x.context_lens[:, None]).to(DEV)
        assert torch.equal(torch.where(live, lg, 0.0), torch.where(live, ref_lg, 0.0))
        _ = (lg * 2).sum().item()  # unrelated eager work between replays
        idx2 = torch.full((x.rows, k), -7, dtype=torch.int32, device=DEV)
        gpu.topk_rows(lg, h, d.lens, k, O.KEY_FP32, idx2, ws)  # same workspace, eager
        torch.cuda.synchronize()
        assert np.array_equal(np.sort(idx2.cpu().numpy(), axis=1), ref_idx)


def test_topk_without_histogram_replays_in_a_hip_graph(gpu):
    """hist=NULL on long rows in a captured graph: the selector's own
    histogram lives in the workspace, which each call leaves zero, so every
    replay (with eager calls on the same workspace between them) is exact."""
    rng = np.random.default_rng(707)
    rows = [rng.standard_normal(30000).astype(np.float32),
            np.round(rng.standard_normal(20001) * 4).astype(np.float32)]
    buf, lens = _scores_dev(rows)
    s_, ln = torch.from_numpy(buf).to(DEV), torch.from_numpy(lens).to(DEV)
    k = 2048
    ws = torch.full((gpu.topk_workspace_bytes(2, buf.shape[1], k),), 0xA5, dtype=torch.uint8, device=DEV)
    idx = torch.full((2, k), -7, dtype=torch.int32, device=DEV)
    announce("topk_rows hist=NULL eager before capture")
    gpu.topk_rows(s_, None, ln, k, O.KEY_FP16, idx, ws)
    torch.cuda.synchronize()
    check_topk(idx.cpu().numpy(), buf, lens, k, O.KEY_FP16)
    ref = np.sort(idx.cpu().numpy(), axis=1)
    g = torch.cuda.CUDAGraph()
    st = torch.cuda.Stream()
    st.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(st):
        with torch.cuda.graph(g, stream=st):
            gpu.topk_rows(s_, None, ln, k, O.KEY_FP16, idx, ws)
    torch.cuda.synchronize()
    for rep in range(3):
        announce(f"hist=NULL graph replay {rep}")
        idx.fill_(-7)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(np.sort(idx.cpu().numpy(), axis=1), ref)
        idx2 = torch.full((2, k), -7, dtype=torch.int32, device=DEV)
        gpu.topk_rows(s_, None, ln, k, O.KEY_FP16, idx2, ws)  # same workspace, eager
        torch.cuda.synchronize()
        assert np.array_equal(np.sort(idx2.cpu().numpy(), axis=1), ref)


@pytest.mark.parametrize("key", [O.KEY_FP32, O.KEY_FP16])
def test_topk_fallback_overflow_shapes(gpu, key):
    """Threshold bins over the 8192-candidate capacity send rows to the
    whole-row select: scores spread over the saturating bin (the keys under
    the chosen digit prefix soon fit the LDS buffer and the row is finished
    there), 20,000 copies of one saturating value (no prefix narrows them:
    ties cut by column at the last digit), and a row of 8192 + 1 equal scores
    in a unit bin next to larger ones."""
    rng = np.random.default_rng(808)
    rows = [np.concatenate([rng.uniform(223, 4000, 16000), rng.standard_normal(24000) * 50]).astype(np.float32),
            np.concatenate([np.full(20000, 300.0), rng.standard_normal(20000)]).astype(np.float32),
            np.concatenate([np.full(8193, 100.0), rng.uniform(101, 150, 1000), rng.standard_normal(9000)]).astype(np.float32)]
    for r in rows:
        rng.shuffle(r)
    buf, lens = _scores_dev(rows)
    s_, ln = torch.from_numpy(buf).to(DEV), torch.from_numpy(lens).to(DEV)
    for k in (2048, 8192):
        announce(f"topk_rows overflow fallback shapes k={k} key={key}")
        idx = topk(s_, None, ln, k, key)
        check_topk(idx.cpu().numpy(), buf, lens, k, key)


def _sub_cut_rows(k, rng):
    """Rows of 40,000 scores whose threshold bin holds 2049 .. 16384 scores,
    so that the selector cuts the bin by its 256 sub-bins: spread over the
    saturating bin (many FP16 values per sub-bin), a fine bin with float32
    values between its FP16 ones, 8000 ties at one value beside spread
    values, only the bin's extreme keys (+inf, 65504, 223: the top and
    bottom sub-bins), one value only (no cut), and exactly 16384 in the
    bin."""
    n = 40000

    def row(parts):
        r = np.concatenate(parts + [rng.standard_normal(n - sum(len(p) for p in parts))]).astype(np.float32)
        rng.shuffle(r)
        return r

    above = np.full(k // 2, 200.0, np.float32)  # in a bin above the fine one
    return [
        row([rng.uniform(223.0, 60000.0, 12000)]),
        row([above, (np.float32(5.0) + rng.uniform(0, 0.25, 9000)).astype(np.float32)]),
        row([np.full(8000, 300.0), rng.uniform(223.0, 60000.0, 1000)]),
        row([np.full(100, np.inf), np.full(2400, 65504.0), np.full(2500, 223.0)]),
        row([above, np.full(6000, 7.0)]),
        row([rng.uniform(223.0, 60000.0, 16384)]),
    ]


@pytest.mark.parametrize("key", [O.KEY_FP32, O.KEY_FP16])
@pytest.mark.parametrize("k", [100, 2048, 8192])
def test_topk_threshold_bin_cut_by_sub_bins(gpu, key, k):
    """Threshold bins of more than 2048 scores are cut once more by the
    sub-bins the collect pass counts: exact with the producer's histogram and
    without one, and with a workspace whose sub-bin counts hold garbage (the
    cut is checked against the candidates' real counts, so only its speed
    may suffer), then again on the same workspace."""
    rng = np.random.default_rng(4242 + k)
    rows = _sub_cut_rows(k, rng)
    buf, lens = _scores_dev(rows)
    s_, ln = torch.from_numpy(buf).to(DEV), torch.from_numpy(lens).to(DEV)
    h = torch.zeros((len(rows), 1024), dtype=torch.int32, device=DEV)
    gpu.score_histogram(s_, ln, h)
    for hist in (h, None):
        announce(f"topk_rows sub-bin cut k={k} key={key} hist={'given' if hist is not None else 'NULL'}")
        idx = topk(s_, hist, ln, k, key)
        check_topk(idx.cpu().numpy(), buf, lens, k, key)
    rec = gpu.topk_workspace_bytes(1, buf.shape[1], k)
    ws = torch.zeros(len(rows) * rec, dtype=torch.uint8, device=DEV)
    w32 = ws.view(torch.int32).view(len(rows), rec // 4)
    # the documented record: counters in bytes 0..255, sub-bin counts in 256..1279
    w32[:, 64:320] = torch.from_numpy(rng.integers(0, 3000, (len(rows), 256), dtype=np.int32)).to(DEV)
    for call in range(2):
        announce(f"topk_rows sub-bin cut, garbage sub-bin counts k={k} key={key} call={call}")
        idx = topk(s_, h, ln, k, key, workspace=ws)
        check_topk(idx.cpu().numpy(), buf, lens, k, key)
    assert int(w32[:, 64:320].abs().sum().item()) == 0  # left zero for the next call


@pytest.mark.parametrize("key", [O.KEY_FP32, O.KEY_FP16])
@pytest.mark.parametrize("k", [1, 2048, 8192])
def test_topk_rows_up_to_16384_in_one_workgroup(gpu, key, k):
    """Rows of 8193 .. 16384 scores take the one-workgroup kernel with two
    8192-column parts per thread (candidates in column order across the part
    boundary): lengths 0, 1, 8191 .. 8193, 12000 and 16384, ties spanning both
    parts, with the producer's histogram (score_histogram) and without."""
    rng = np.random.default_rng(909 + k)
    rows = [np.zeros(0, np.float32), np.array([3.0], np.float32),
            rng.standard_normal(8191).astype(np.float32), rng.standard_normal(8192).astype(np.float32),
            rng.standard_normal(8193).astype(np.float32),
            np.round(rng.standard_normal(12000) * 2).astype(np.float32),   # ties in both parts
            rng.standard_normal(16384).astype(np.float32) * np.float32(30.0)]
    buf, lens = _scores_dev(rows)
    buf = np.concatenate([buf, np.full((buf.shape[0], 16384 - buf.shape[1]), np.inf, np.float32)], axis=1)
    s_, ln = torch.from_numpy(buf).to(DEV), torch.from_numpy(lens).to(DEV)
    h = torch.zeros((len(rows), 1024), dtype=torch.int32, device=DEV)
    gpu.score_histogram(s_, ln, h)
    for hist in (h, None):
        announce(f"topk_rows stride 16384 k={k} key={key} hist={'given' if hist is not None else 'NULL'}")
        idx = topk(s_, hist, ln, k, key)
        check_topk(idx.cpu().numpy(), buf, lens, k, key)


def test_read_probes_run_on_small_buffers(gpu):
    """The measurement aids launch on small inputs (partial chunks, a page
    list shorter than a workgroup's share, out-of-range ids clamped) and
    leave the sink alone for data whose checksum is not the marker."""
    announce("hbm_read_probe / hbm_read_probe_nt / hbm_gather_probe small buffers")
    sink = torch.zeros(1, dtype=torch.int32, device=DEV)
    src = torch.zeros(100_000 // 4 * 4, dtype=torch.int32, device=DEV)
    gpu.hbm_read_probe(src, sink)
    gpu.hbm_read_probe_nt(src, sink)
    pool = torch.zeros((10, 64, 128), dtype=torch.uint8, device=DEV)
    scales = torch.zeros((10, 64), dtype=torch.float32, device=DEV)
    plist = torch.tensor([3, 9, 0, 12, -1, 5, 5], dtype=torch.int32, device=DEV)
    gpu.hbm_gather_probe(pool, scales, plist, sink)
    torch.cuda.synchronize()
    assert int(sink.item()) == 0


def test_coissue_probe_runs_every_mode(gpu):
    """The MFMA / VALU co-issue probe: every mode and wave count launches and
    writes one finite value per thread; a too-short output is refused."""
    cus = torch.cuda.get_device_properties(DEV).multi_processor_count
    for wps in (1, 2):
        out = torch.full((cus * wps * 256 + 5,), float("nan"), dtype=torch.float32, device=DEV)
        for mode in (0, 1, 2):
            announce(f"mfma_valu_probe mode={mode} waves/SIMD={wps}")
            out.fill_(float("nan"))
            gpu.mfma_valu_probe(mode, wps, 64, out)
            torch.cuda.synchronize()
            got = out[:cus * wps * 256]
            assert bool(torch.isfinite(got).all()), (mode, wps)
            assert bool(torch.isnan(out[cus * wps * 256:]).all()), "written past the grid"
    with pytest.raises(pmqa.IndexerError):
        gpu.mfma_valu_probe(2, 1, 16, torch.zeros(cus * 256 - 1, dtype=torch.float32, device=DEV))
