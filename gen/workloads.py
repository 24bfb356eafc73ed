"""Seeded synthetic inputs for the paged MQA indexer.

Input synthesis only: this module holds none of the method's arithmetic (no
fp8 decode, no dot products, no binning, no selection).  FP8 E4M3FN encoding
is done with PyTorch's own CPU cast.  Both the HIP path (tests, bench, smoke)
and the CPU oracle consume what it produces.

The workloads follow the five decode configurations the indexer is measured
on (H=32, D=128, 64-token pages):

  tiny_decode    B=1,  next_n=1, L=4096
  long_decode    B=8,  next_n=1, L=131072
  spec_verify    B=16, next_n=4, L=32768 (row j of a request sees L+j keys);
                 variants fine / unit / mixed scale the head weights so the
                 scores land below 16, mostly in 16..223, or across all three
                 regimes, and "mixed" sets the K scale of 1% of the pool slots
                 to +inf
  varlen_decode  B=64, next_n=1, L log-uniform in [8192, 262144], stride 262144
  very_long      B=4,  next_n=1, L=1048576; plus score rows [4, 1048576] drawn
                 from 0.99 N(0, var 4) + 0.01 N(40, var 10)

and one ragged prefill (extend) batch, the second workload of the pages'
prefill path:

  prefill/extend 4 requests x 2048 new tokens over cached prefixes of 0, 6K,
                 14K and 30K keys (contexts 2K, 8K, 16K, 32K); row i of a
                 request sees prefix + 1 + i keys (causal); 8192 rows

Value recipe: Q ~ N(0,1) cast to e4m3; K rows ~ N(0,1), per-token scale
absmax/448, codes = e4m3(k / scale); head weights N(0,1)/sqrt(32) times the
variant's factor.  MXFP4 K (the "/mxfp4" workloads): the same K rows, each
block of 32 dimensions scaled by 2^(floor(log2(absmax)) - 2) (E8M0 byte) and
its elements rounded to the nearest E2M1 value (ties to the even code,
saturated at +-6), packed 68 bytes per token.  Physical pages are a seeded permutation of one pool that
has ~1% spare pages.  Slots of a request's last page past its longest row and
the spare pages hold K = 448 with scale 1e6, so an unmasked read shows up as a
huge score.
"""

from __future__ import annotations

import dataclasses
import math

import numpy as np
import torch

HEADS = 32
DIM = 128
PAGE = 64

SEEDS = {
    "tiny_decode": 101,
    "long_decode": 202,
    "spec_verify/fine": 301,
    "spec_verify/unit": 302,
    "spec_verify/mixed": 303,
    "varlen_decode": 404,
    "very_long": 505,
    "very_long/scores": 506,
    "long_decode/mxfp4": 212,
    "spec_verify/mxfp4": 311,
    "prefill/extend": 601,
    "prefill/extend_mxfp4": 611,
}

# Ragged prefill (extend) batch: four requests append 2048 tokens each to
# cached prefixes, so their contexts hold 2K, 8K, 16K and 32K keys.
PREFILL_Q_LENS = (2048, 2048, 2048, 2048)
PREFILL_PREFIX_LENS = (0, 6144, 14336, 30720)

# Head-weight factors for the three verify variants.
VERIFY_WEIGHT_SCALE = {"fine": 0.25, "unit": 16.0, "mixed": 4.0}


@dataclasses.dataclass
class IndexerInputs:
    """Host (numpy) arrays of one indexer call, in the library's layouts."""

    name: str
    q: np.ndarray            # uint8 [rows, 32, 128]   e4m3fn codes
    kv_pages: np.ndarray     # uint8 [num_pages, 64, 128] e4m3fn codes, or
                             #       [num_pages, 64, 68] packed MXFP4 tokens
    k_scales: np.ndarray     # f32   [num_pages, 64] (None with MXFP4 pages)
    weights: np.ndarray      # f32   [rows, 32]
    block_table: np.ndarray  # int32 [B, max_pages]
    context_lens: np.ndarray  # int32 [rows]
    next_n: int               # rows per request (0 for a ragged prefill batch)
    logits_stride: int
    cu_q: np.ndarray = None   # int32 [B + 1] row offsets of a ragged prefill batch

    @property
    def B(self) -> int:
        return self.block_table.shape[0]

    @property
    def rows(self) -> int:
        return self.q.shape[0]

    @property
    def num_pages(self) -> int:
        return self.kv_pages.shape[0]

    @property
    def max_pages(self) -> int:
        return self.block_table.shape[1]

    def request_keys(self) -> np.ndarray:
        """Longest row length of each request (the keys its K sweep reads)."""
        if self.cu_q is not None:
            return np.array([int(self.context_lens[a:b].max()) if b > a else 0
                             for a, b in zip(self.cu_q[:-1], self.cu_q[1:])], dtype=np.int64)
        return self.context_lens.reshape(self.B, self.next_n).max(axis=1)

    @property
    def mxfp4(self) -> bool:
        return self.kv_pages.shape[-1] == MXFP4_TOKEN_BYTES

    def k_bytes(self) -> int:
        """Bytes of K rows the indexer must read per request and key: 128
        (FP8 codes; the scale is counted apart) or 68 (MXFP4 token)."""
        return int(self.request_keys().astype(np.int64).sum()) * int(self.kv_pages.shape[-1])


MXFP4_TOKEN_BYTES = 68
_E2M1_POS = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0], dtype=np.float64)


def to_mxfp4_tokens(k: np.ndarray) -> np.ndarray:
    """float32 [n, 128] -> uint8 [n, 68] packed MXFP4 tokens (see module doc)."""
    k = np.asarray(k, dtype=np.float64)
    n = k.shape[0]
    blocks = k.reshape(n, 4, 32)
    amax = np.abs(blocks).max(axis=2)
    e = np.where(amax > 0, np.floor(np.log2(np.where(amax > 0, amax, 1.0))) - 2, -127)
    e = np.clip(e, -127, 127).astype(np.int64)
    v = blocks / np.ldexp(1.0, e)[:, :, None]
    a = np.minimum(np.abs(v), 6.0)
    # nearest E2M1 magnitude, ties to the even code (codes 0..7 by magnitude)
    hi = np.searchsorted(_E2M1_POS, a, side="left").clip(0, 7)
    lo = (hi - 1).clip(0, 7)
    dlo, dhi = a - _E2M1_POS[lo], _E2M1_POS[hi] - a
    mag = np.where(dlo < dhi, lo, np.where(dhi < dlo, hi, np.where(lo % 2 == 0, lo, hi)))
    codes = (mag | np.where((v < 0) & (mag > 0), 8, 0)).astype(np.uint8).reshape(n, 128)
    out = np.empty((n, MXFP4_TOKEN_BYTES), dtype=np.uint8)
    out[:, :64] = codes[:, 0::2] | (codes[:, 1::2] << 4)
    out[:, 64:] = (e + 127).astype(np.uint8)
    return out


def to_e4m3fn_codes(x: np.ndarray) -> np.ndarray:
    """uint8 E4M3FN codes of float32 values (saturated to +-448 first)."""
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    t = t.clamp_(-448.0, 448.0).to(torch.float8_e4m3fn)
    return t.view(torch.uint8).numpy()


def make_indexer_inputs(name, B, next_n, base_lens, seed, weight_scale=1.0,
                        inf_frac=0.0, logits_stride=None, max_pages=None,
                        spare_frac=0.01, pages_per_chunk=4096, kfmt="fp8"):
    """Build one indexer call.

    base_lens: int per request; row j of request b sees base_lens[b] + j keys.
    kfmt: "fp8" (E4M3 codes + per-token scales) or "mxfp4" (packed tokens).
    """
    return _make_inputs(name, np.full(B, next_n, dtype=np.int64), base_lens, seed, weight_scale,
                        inf_frac, logits_stride, max_pages, spare_frac, pages_per_chunk, kfmt)


def make_prefill_inputs(name, q_lens, prefix_lens, seed, weight_scale=1.0, logits_stride=None,
                        max_pages=None, kfmt="fp8"):
    """A ragged prefill (extend) batch: request b appends q_lens[b] tokens to a
    cached prefix of prefix_lens[b] keys, so its context holds
    prefix_lens[b] + q_lens[b] keys and its row i (causal) sees
    prefix_lens[b] + 1 + i of them.  Rows are packed request after request;
    cu_q holds the row offsets.  A request may have no rows."""
    q_lens = np.asarray(q_lens, dtype=np.int64)
    prefix_lens = np.asarray(prefix_lens, dtype=np.int64).reshape(q_lens.shape)
    x = _make_inputs(name, q_lens, prefix_lens + 1, seed, weight_scale, 0.0, logits_stride,
                     max_pages, 0.01, 4096, kfmt)
    x.cu_q = np.concatenate([[0], np.cumsum(q_lens)]).astype(np.int32)
    x.next_n = 0
    return x


def _make_inputs(name, n_rows, base_lens, seed, weight_scale, inf_frac, logits_stride,
                 max_pages, spare_frac, pages_per_chunk, kfmt):
    """Requests of n_rows[b] rows each; row j of request b sees base_lens[b] + j
    keys (the K slots of its context up to base_lens[b] + n_rows[b] - 1)."""
    mx = kfmt == "mxfp4"
    rng = np.random.Generator(np.random.PCG64(seed))
    n_rows = np.asarray(n_rows, dtype=np.int64)
    B = n_rows.shape[0]
    base_lens = np.asarray(base_lens, dtype=np.int64).reshape(B)
    rows = int(n_rows.sum())
    lens = np.concatenate([base_lens[b] + np.arange(n_rows[b]) for b in range(B)] or
                          [np.zeros(0, np.int64)]).astype(np.int64)
    next_n = int(n_rows[0]) if B else 0
    req_keys = np.maximum(base_lens + n_rows - 1, 0)
    req_pages = -(-req_keys // PAGE)
    used = int(req_pages.sum())
    num_pages = used + max(1, int(math.ceil(used * spare_frac)))
    if max_pages is None:
        max_pages = int(req_pages.max()) if B else 1
    if logits_stride is None:
        logits_stride = int(lens.max()) if rows else 1
        logits_stride = -(-logits_stride // 4) * 4

    # Q and head weights.
    q = to_e4m3fn_codes(rng.standard_normal((rows, HEADS, DIM), dtype=np.float32))
    weights = (rng.standard_normal((rows, HEADS), dtype=np.float32)
               / np.float32(math.sqrt(HEADS)) * np.float32(weight_scale))

    # K pool, generated in chunks of pages to bound host memory.
    kv_pages = np.empty((num_pages, PAGE, MXFP4_TOKEN_BYTES if mx else DIM), dtype=np.uint8)
    k_scales = None if mx else np.empty((num_pages, PAGE), dtype=np.float32)
    for p0 in range(0, num_pages, pages_per_chunk):
        p1 = min(num_pages, p0 + pages_per_chunk)
        k = rng.standard_normal(((p1 - p0) * PAGE, DIM), dtype=np.float32)
        if mx:
            kv_pages[p0:p1] = to_mxfp4_tokens(k).reshape(p1 - p0, PAGE, MXFP4_TOKEN_BYTES)
            continue
        sc = np.abs(k).max(axis=1) / np.float32(448.0)
        kv_pages[p0:p1] = to_e4m3fn_codes(k / sc[:, None]).reshape(p1 - p0, PAGE, DIM)
        k_scales[p0:p1] = sc.reshape(p1 - p0, PAGE)

    # Page table: a seeded permutation of the pool.
    perm = rng.permutation(num_pages).astype(np.int32)
    block_table = np.zeros((B, max_pages), dtype=np.int32)
    offs = np.concatenate([[0], np.cumsum(req_pages)])
    for b in range(B):
        block_table[b, :req_pages[b]] = perm[offs[b]:offs[b + 1]]
    spare = perm[used:]

    # Poison: spare pages and slots past each request's longest row (FP8:
    # K = 448 with scale 1e6; MXFP4: every element +6 with scale 2^127).
    def poison(page, tail=0):
        if mx:
            kv_pages[page, tail:, :64] = 0x77
            kv_pages[page, tail:, 64:] = 254
        else:
            kv_pages[page, tail:] = 0x7E
            k_scales[page, tail:] = 1e6

    poison(spare)
    for b in range(B):
        tail = int(req_keys[b] % PAGE)
        if tail:
            poison(block_table[b, req_pages[b] - 1], tail)

    if inf_frac > 0.0 and not mx:
        mask = rng.random((num_pages, PAGE)) < inf_frac
        k_scales[mask] = np.inf

    return IndexerInputs(name=name, q=q, kv_pages=kv_pages, k_scales=k_scales,
                         weights=weights, block_table=block_table,
                         context_lens=lens.astype(np.int32), next_n=next_n,
                         logits_stride=int(logits_stride))


def config_inputs(name: str) -> IndexerInputs:
    """The named decode workload at its full size."""
    if name == "long_decode/mxfp4":
        return make_indexer_inputs(name, 8, 1, [131072] * 8, SEEDS[name], kfmt="mxfp4")
    if name == "spec_verify/mxfp4":
        return make_indexer_inputs(name, 16, 4, [32768] * 16, SEEDS[name],
                                   weight_scale=VERIFY_WEIGHT_SCALE["fine"], kfmt="mxfp4")
    if name in ("prefill/extend", "prefill/extend_mxfp4"):
        return make_prefill_inputs(name, PREFILL_Q_LENS, PREFILL_PREFIX_LENS, SEEDS[name],
                                   kfmt="mxfp4" if name.endswith("mxfp4") else "fp8")
    if name == "tiny_decode":
        return make_indexer_inputs(name, 1, 1, [4096], SEEDS[name])
    if name == "long_decode":
        return make_indexer_inputs(name, 8, 1, [131072] * 8, SEEDS[name])
    if name.startswith("spec_verify/"):
        variant = name.split("/", 1)[1]
        return make_indexer_inputs(
            name, 16, 4, [32768] * 16, SEEDS[name],
            weight_scale=VERIFY_WEIGHT_SCALE[variant],
            inf_frac=0.01 if variant == "mixed" else 0.0)
    if name == "varlen_decode":
        rng = np.random.Generator(np.random.PCG64(SEEDS[name] + 1000))
        lens = np.floor(np.exp(rng.uniform(math.log(8192), math.log(262144), 64)))
        return make_indexer_inputs(name, 64, 1, lens.astype(np.int64), SEEDS[name],
                                   logits_stride=262144, max_pages=262144 // PAGE)
    if name == "very_long":
        return make_indexer_inputs(name, 4, 1, [1048576] * 4, SEEDS[name])

    raise KeyError(name)


CONFIG_NAMES = ("tiny_decode", "long_decode", "spec_verify/fine",
                "spec_verify/unit", "spec_verify/mixed", "varlen_decode",
                "very_long")
MXFP4_CONFIG_NAMES = ("long_decode/mxfp4", "spec_verify/mxfp4")
PREFILL_CONFIG_NAMES = ("prefill/extend", "prefill/extend_mxfp4")


def very_long_scores(rows=4, n=1048576, seed=None) -> np.ndarray:
    """float32 [rows, n]: 0.99 N(0, var 4) + 0.01 N(40, var 10), seeded."""
    if seed is None:
        seed = SEEDS["very_long/scores"]
    rng = np.random.Generator(np.random.PCG64(seed))
    base = rng.standard_normal((rows, n), dtype=np.float32) * np.float32(2.0)
    out = rng.standard_normal((rows, n), dtype=np.float32) * np.float32(math.sqrt(10.0))
    out += np.float32(40.0)
    mask = rng.random((rows, n)) < 0.01
    return np.where(mask, out, base).astype(np.float32)
