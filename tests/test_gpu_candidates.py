"""Two-level candidate indexer (SGLang PR #38944) on the GPU against the CPU
oracle: block maxima, the sorted block table with its page transform, sparse
logits over the published blocks, and the whole consumer chain (block
top-k -> sort -> sparse logits -> top-k inside the sparse row -> logical
positions), each integer stage bit-exact from the GPU's own inputs."""
import numpy as np
import pytest
import torch

import gen
import oracle as O
from tests.gpu_harness import DEV, DevInputs, announce, check_logits, check_topk, topk

pytestmark = pytest.mark.gpu

C = O.candidates
BIG = 2 ** 31 - 1
SENT = -7.0


def test_block_amax8(gpu):
    rng = np.random.default_rng(71)
    rows, stride = 7, 4104
    sc = (rng.standard_normal((rows, stride)) * 3).astype(np.float32)
    sc[rng.random((rows, stride)) < 0.05] = np.nan
    sc[0, 64:72] = np.nan                    # a block of NaNs only
    sc[1, rng.integers(0, stride, 20)] = np.inf
    sc[2, rng.integers(0, stride, 20)] = -np.inf
    lens = np.array([4104, 4097, 8, 1, 0, 1000, 3999], np.int32)
    s = torch.from_numpy(sc).to(DEV)
    ln = torch.from_numpy(lens).to(DEV)
    width = -(-stride // 8)
    out = torch.full((rows, width + 3), SENT, dtype=torch.float32, device=DEV)
    out2 = torch.full((rows, width + 3), SENT, dtype=torch.float32, device=DEV)
    h = torch.zeros((rows, 1024), dtype=torch.int32, device=DEV)
    bl = torch.full((rows,), -5, dtype=torch.int32, device=DEV)
    announce("block_amax8")
    gpu.block_amax8(s, ln, out)
    gpu.block_amax8(s, ln, out2, h, block_lens=bl)
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    assert np.array_equal(got, out2.cpu().numpy(), equal_nan=True), "the histogram changes the maxima"
    want = C.block_amax8(sc, lens)
    blk_lens = -(-lens.astype(np.int64) // 8)
    assert np.array_equal(bl.cpu().numpy(), blk_lens), "block counts (lengths of the block rows)"
    assert np.array_equal(h.cpu().numpy(), O.coarse_histogram(got[:, :width], blk_lens)), \
        "histogram of the block maxima differs"
    for r in range(rows):
        nb = -(-int(lens[r]) // 8)
        g, w = got[r, :nb], want[r, :nb]
        assert np.array_equal(g, w, equal_nan=True), f"row {r}: block maxima differ"
        assert np.all(got[r, nb:] == SENT), f"row {r}: written past ceil(len / 8)"


def _random_blocks(rng, lens, kb, dup=False):
    rows = len(lens)
    blocks = np.full((rows, kb), -1, np.int32)
    for r in range(rows):
        nb = -(-int(lens[r]) // 8)
        if nb == 0:
            continue
        n = min(kb - r % 3, nb)
        pick = rng.choice(nb, size=n, replace=False).astype(np.int32)
        if dup and n > 4:
            pick[1] = pick[0]        # a repeat, dropped by the sort
            pick[2] = nb + 5         # out of range, dropped
        blocks[r, :n] = pick
    return blocks


@pytest.mark.parametrize("in_place", [False, True])
def test_sort_candidate_blocks(gpu, in_place):
    rng = np.random.default_rng(73)
    x = gen.make_indexer_inputs("sortblk", 4, 2, [30000, 100, 9000, 777], 17)
    kb = 96
    lens = x.context_lens
    blocks = _random_blocks(rng, lens, kb, dup=True)
    max_len = int(lens.max())
    d = DevInputs(x)
    bl = torch.from_numpy(blocks).to(DEV)
    table = bl if in_place else torch.full_like(bl, -5)
    slots = torch.full_like(bl, -5)
    slens = torch.zeros(x.rows, dtype=torch.int32, device=DEV)
    announce(f"sort_candidate_blocks in_place={in_place}")
    gpu.sort_candidate_blocks(bl, d.lens, max_len, d.bt, x.next_n, table, slots, slens)
    torch.cuda.synchronize()
    n_blocks = -(-lens.astype(np.int64) // 8)
    want_t, want_s = C.sort_candidate_blocks(blocks, n_blocks, x.block_table, x.next_n)
    assert np.array_equal(table.cpu().numpy(), want_t)
    assert np.array_equal(slots.cpu().numpy(), want_s)
    assert np.array_equal(slens.cpu().numpy(), C.sparse_row_lens(want_t, lens))


@pytest.mark.parametrize("kfmt", ["fp8", "mxfp4"])
def test_sparse_logits(gpu, kfmt):
    rng = np.random.default_rng(75)
    x = gen.make_indexer_inputs("sparse", 3, 2, [20000, 3000, 700], 19, kfmt=kfmt)
    d = DevInputs(x)
    kb = 200
    lens = x.context_lens
    blocks = _random_blocks(rng, lens, kb)
    for r in range(x.rows):  # the newest block is always published
        nb = -(-int(lens[r]) // 8)
        if nb > kb:
            blocks[r, 0] = nb - 1
    n_blocks = -(-lens.astype(np.int64) // 8)
    table, slots = C.sort_candidate_blocks(blocks, n_blocks, x.block_table, x.next_n)
    stride = kb * 8 + 12
    lg = torch.full((x.rows, stride), float("inf"), dtype=torch.float32, device=DEV)
    announce(f"indexer_sparse_logits {kfmt}")
    gpu.indexer_sparse_logits(d.q, d.kv, d.sc, d.w, torch.from_numpy(table).to(DEV),
                              torch.from_numpy(slots).to(DEV), d.lens, lg)
    torch.cuda.synchronize()
    got = lg.cpu().numpy()
    want = C.sparse_logits(x.q, x.kv_pages, x.k_scales, x.weights, x.block_table, table, lens,
                           x.next_n)
    assert np.all(np.isinf(got[:, kb * 8:])), "columns past the table were written"
    got = got[:, :kb * 8]
    for r in range(x.rows):
        live = ~np.isnan(want[r])
        assert np.all(np.isinf(got[r, ~live])), f"row {r}: a column that is not live was written"
        cols = np.nonzero(live)[0]
        keys = C.sparse_to_logical(table[r:r + 1], cols[None, :])[0]
        bound = O.logits_error_bound_at(x.q, x.kv_pages, x.k_scales, x.weights, x.block_table,
                                        x.next_n, r, keys)
        ok = O.check_logits(got[r, cols], want[r, cols], bound)
        assert ok.all(), f"row {r}: {int((~ok).sum())} sparse logits outside tolerance"


@pytest.mark.parametrize("name,kb_blocks", [("long_decode", 512), ("spec_verify/fine", 256),
                                            ("long_decode/mxfp4", 512)])
def test_candidate_chain(gpu, name, kb_blocks):
    """Dense logits -> block maxima -> block top-k -> sorted table -> sparse
    logits -> top-2048 inside the sparse row -> logical positions."""
    announce(f"generate {name}")
    x = gen.config_inputs(name)
    d = DevInputs(x)
    lens = x.context_lens
    lg, _ = d.run(with_hist=False, fill=float("inf"))
    dense = lg.cpu().numpy()
    width = -(-(-(-x.logits_stride // 8)) // 4) * 4  # ceil(stride / 8), 16-byte rows for the top-k
    am = torch.full((x.rows, width), SENT, dtype=torch.float32, device=DEV)
    ah = torch.zeros((x.rows, 1024), dtype=torch.int32, device=DEV)
    announce(f"{name}: block_amax8")
    blens = torch.full((x.rows,), -5, dtype=torch.int32, device=DEV)
    gpu.block_amax8(lg, d.lens, am, ah, block_lens=blens)
    torch.cuda.synchronize()
    assert np.array_equal(blens.cpu().numpy(), -(-lens.astype(np.int64) // 8))
    announce(f"{name}: block top-{kb_blocks}")
    bsel = topk(am, ah, blens, kb_blocks, O.KEY_FP32)
    am_h = am.cpu().numpy()
    want_am = C.block_amax8(dense, lens)
    for r in range(x.rows):
        nb = -(-int(lens[r]) // 8)
        assert np.array_equal(am_h[r, :nb], want_am[r, :nb], equal_nan=True), f"row {r}: amax8"
    check_topk(bsel.cpu().numpy(), np.where(np.isnan(am_h), np.nan, am_h), blens.cpu().numpy(),
               kb_blocks, O.KEY_FP32)
    table = torch.empty_like(bsel)
    slots = torch.empty_like(bsel)
    slens = torch.zeros(x.rows, dtype=torch.int32, device=DEV)
    announce(f"{name}: sort_candidate_blocks")
    gpu.sort_candidate_blocks(bsel, d.lens, x.logits_stride, d.bt, x.next_n, table, slots, slens)
    n_blocks = -(-lens.astype(np.int64) // 8)
    want_t, want_s = C.sort_candidate_blocks(bsel.cpu().numpy(), n_blocks, x.block_table, x.next_n)
    tab = table.cpu().numpy()
    assert np.array_equal(tab, want_t) and np.array_equal(slots.cpu().numpy(), want_s)
    stride = kb_blocks * 8
    sl = torch.full((x.rows, stride), float("inf"), dtype=torch.float32, device=DEV)
    announce(f"{name}: indexer_sparse_logits")
    gpu.indexer_sparse_logits(d.q, d.kv, d.sc, d.w, table, slots, d.lens, sl)
    torch.cuda.synchronize()
    sparse = sl.cpu().numpy()
    # the sparse logits are the dense GPU logits at the listed positions (same kernel arithmetic)
    for r in range(x.rows):
        n = int(slens[r].item())
        keys = C.sparse_to_logical(tab[r:r + 1], np.arange(n)[None, :])[0]
        assert np.array_equal(sparse[r, :n].view(np.int32), dense[r, keys].view(np.int32)), \
            f"row {r}: sparse logits differ from the dense logits at the listed keys"
    announce(f"{name}: top-2048 inside the sparse rows")
    sel = topk(sl, None, slens, 2048, O.KEY_FP32)
    check_topk(sel.cpu().numpy(), sparse, slens.cpu().numpy(), 2048, O.KEY_FP32)
    pos = torch.empty_like(sel)
    gpu.sparse_to_logical(sel, table, pos)
    torch.cuda.synchronize()
    want_pos = C.sparse_to_logical(tab, sel.cpu().numpy())
    assert np.array_equal(pos.cpu().numpy(), want_pos)
    announce(f"{name}: sparse_topk (top-k and map in one launch)")
    fused = torch.full_like(sel, -9)
    gpu.sparse_topk(sl, None, slens, 2048, O.KEY_FP32, table, fused)
    torch.cuda.synchronize()
    assert np.array_equal(np.sort(fused.cpu().numpy(), axis=1), np.sort(want_pos, axis=1))
    del d, lg, am, sl
    torch.cuda.empty_cache()


def test_candidate_chain_replays_in_a_hip_graph(gpu):
    """The consumer chain (block maxima with histogram and block counts,
    block top-k, sort, sparse logits, top-k in the sparse row, map back)
    captured in one HIP graph: every replay, with eager work and an eager
    run of the chain on the same workspaces between replays, gives the
    eager chain's logical positions."""
    x = gen.make_indexer_inputs("cand_graph", 4, 1, [20000, 9000, 40000, 3000], 77)
    d = DevInputs(x)
    kb, k = 512, 2048
    lg = d.new_logits(float("inf"))
    d.logits(lg, None)
    rows = x.rows
    width = -(-(-(-x.logits_stride // 8)) // 4) * 4
    am = torch.empty((rows, width), dtype=torch.float32, device=DEV)
    ah = torch.zeros((rows, 1024), dtype=torch.int32, device=DEV)
    blens = torch.empty(rows, dtype=torch.int32, device=DEV)
    bsel = torch.empty((rows, kb), dtype=torch.int32, device=DEV)
    table, slots = torch.empty_like(bsel), torch.empty_like(bsel)
    slens = torch.empty(rows, dtype=torch.int32, device=DEV)
    sparse = torch.empty((rows, kb * 8), dtype=torch.float32, device=DEV)
    ssel = torch.empty((rows, k), dtype=torch.int32, device=DEV)
    pos = torch.empty_like(ssel)
    ws_b = torch.full((gpu.topk_workspace_bytes(rows, width, kb),), 0xA5, dtype=torch.uint8, device=DEV)
    ws_s = torch.full((gpu.topk_workspace_bytes(rows, kb * 8, k),), 0xA5, dtype=torch.uint8, device=DEV)

    def chain():
        ah.zero_()
        gpu.block_amax8(lg, d.lens, am, ah, block_lens=blens)
        gpu.topk_rows(am, ah, blens, kb, O.KEY_FP32, bsel, ws_b)
        gpu.sort_candidate_blocks(bsel, d.lens, x.logits_stride, d.bt, x.next_n, table, slots, slens)
        gpu.indexer_sparse_logits(d.q, d.kv, d.sc, d.w, table, slots, d.lens, sparse)
        gpu.topk_rows(sparse, None, slens, k, O.KEY_FP32, ssel, ws_s)
        gpu.sparse_to_logical(ssel, table, pos)

    announce("candidate chain: eager reference")
    chain()
    torch.cuda.synchronize()
    ref = np.sort(pos.cpu().numpy(), axis=1)
    # the final positions are the oracle's top-k of the dense logits over the listed blocks
    assert np.all(ref[:, -1] < x.logits_stride)
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            chain()
    torch.cuda.synchronize()
    for rep in range(4):
        announce(f"candidate chain graph replay {rep}")
        pos.fill_(-7)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(np.sort(pos.cpu().numpy(), axis=1), ref), f"replay {rep}"
        _ = (lg * 2).sum().item()  # unrelated eager work between replays
        pos.fill_(-7)
        chain()  # the same buffers and workspaces, eager
        torch.cuda.synchronize()
        assert np.array_equal(np.sort(pos.cpu().numpy(), axis=1), ref), f"eager after replay {rep}"



@pytest.mark.parametrize("key", [O.KEY_FP32, O.KEY_FP16])
@pytest.mark.parametrize("k", [1, 100, 2048, 8192])
def test_sparse_topk_edges(gpu, key, k):
    """sparse_topk against the oracle's top-k mapped through the table
    (sparse_to_logical's definition): rows of one and two 8192-column parts,
    lengths 0, 1 and below k, live columns past the table (kb * 8 < len),
    table padding (INT32_MAX), ties, with the histogram given and without."""
    rng = np.random.default_rng(3030 + k)
    for stride in (4096, 12000):
        rows = 6
        kb = stride // 8 - 3  # the last 24 columns lie past every table
        sc = (np.round(rng.standard_normal((rows, stride)) * 3)).astype(np.float32)
        lens = np.array([stride, 0, 1, min(stride, k // 2 + 5), stride - 7, stride // 3], np.int32)
        table = np.sort(rng.choice(1 << 16, size=(rows, kb), replace=True), axis=1).astype(np.int32)
        table[4, kb // 2:] = np.iinfo(np.int32).max  # padded second half
        s_ = torch.from_numpy(sc).to(DEV)
        ln = torch.from_numpy(lens).to(DEV)
        tb = torch.from_numpy(table).to(DEV)
        h = torch.zeros((rows, 1024), dtype=torch.int32, device=DEV)
        gpu.score_histogram(s_, ln, h)
        want = C.sparse_to_logical(table, O.topk_rows(sc, lens, k, key))
        for hist in (h, None):
            announce(f"sparse_topk stride={stride} k={k} key={key} hist={'given' if hist is not None else 'NULL'}")
            out = torch.full((rows, k), -9, dtype=torch.int32, device=DEV)
            gpu.sparse_topk(s_, hist, ln, k, key, tb, out)
            torch.cuda.synchronize()
            got = out.cpu().numpy()
            for r in range(rows):
                assert np.array_equal(np.sort(got[r]), np.sort(want[r])), f"stride {stride} row {r}"
