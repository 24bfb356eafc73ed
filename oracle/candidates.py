"""Plain CPU oracle of the two-level candidate indexer's consumer path.

TEST INFRASTRUCTURE ONLY, like indexer_oracle: only ``tests/``,
``__graft_entry__.smoke()`` and ``bench.py``'s cpu_baseline leg may use it.

Source: [P2] SGLang PR #38944, "[DSV4.1] Enable the two-level candidate
indexer on DeepGEMM's paged sparse MQA logits": the candidate-source layer
publishes, per query row, an ascending logical block table (blocks of 8
tokens); the layers after it score the published blocks only (paged sparse
MQA logits) and select inside that sparse row.  The commit that replaces the
source layer's torch pieces defines

* ``block_amax8``            -- amax8_varlen: the maximum of every 8 consecutive
                                fp32 scores for the first ceil(len / 8) blocks
                                of a row; the newest block is written as +inf
                                (always selected); nothing past that count;
* ``sort_candidate_blocks``  -- the selected block ids (any order, -1 padded)
                                as an ascending table padded with INT32_MAX,
                                plus the same blocks as pool slots / 8 through
                                the row's page table; rows with at most k
                                blocks get the identity table;

and the consumer side is

* ``sparse_logits``          -- the indexer logits at the published positions
                                only, block i of the table filling sparse
                                columns 8i .. 8i+7;
* ``sparse_row_lens``        -- the live columns of each sparse row;
* ``sparse_to_logical``      -- sparse column -> logical key position.

Readings taken where the page is silent: scores that are NaN are ignored by
the block maximum (NaN only when every live score of the block is NaN); the
sort drops ids outside [0, ceil(len / 8)) and repeats (a block is listed
once);
block b covers keys 8b .. 8b+7, only keys below the row length are live; the
pool slot of logical key s is page * 64 + s % 64 with page the row's block
table entry s // 64, so block b's slot / 8 is page * 8 + b % 8; the sparse
row of a table is its blocks' live keys in table order.
"""

from __future__ import annotations

import numpy as np

from .indexer_oracle import PAGE_SIZE, indexer_logits_at

BLOCK = 8
INT32_MAX = np.iinfo(np.int32).max


def block_amax8(scores, lens, fill=np.nan):
    """float32 [rows, max_blocks]: NaN-ignoring maximum of each 8-score block
    of live scores, +inf for the newest block, ``fill`` past the count."""
    scores = np.asarray(scores, dtype=np.float32)
    lens = np.asarray(lens, dtype=np.int64)
    rows = scores.shape[0]
    nb = (lens + BLOCK - 1) // BLOCK
    width = int(nb.max()) if rows else 0
    out = np.full((rows, max(width, 1)), fill, dtype=np.float32)
    for r in range(rows):
        n = int(lens[r])
        for j in range(int(nb[r])):
            blk = scores[r, BLOCK * j:min(n, BLOCK * j + BLOCK)]
            with np.errstate(invalid="ignore"):
                out[r, j] = np.fmax.reduce(blk)  # NaN only if all are NaN
        if nb[r] > 0:
            out[r, nb[r] - 1] = np.inf
    return out


def sort_candidate_blocks(blocks, n_blocks, block_table, next_n):
    """Ascending INT32_MAX-padded block table and the pool-slot / 8 table.

    blocks     int32 [rows, kb]: selected block ids, any order, -1 padded
    n_blocks   int   [rows]: blocks the row has (ceil(len / 8))
    block_table int32 [B, max_pages], rows b*next_n .. b*next_n+next_n-1 use row b
    """
    blocks = np.asarray(blocks, dtype=np.int64)
    rows, kb = blocks.shape
    table = np.full((rows, kb), INT32_MAX, dtype=np.int64)
    slots = np.full((rows, kb), INT32_MAX, dtype=np.int64)
    for r in range(rows):
        n = int(n_blocks[r])
        if n <= kb:
            ids = np.arange(n)
        else:
            b = blocks[r]
            ids = np.unique(b[(b >= 0) & (b < n)])
        table[r, :len(ids)] = ids
        pages = np.asarray(block_table[r // next_n], dtype=np.int64)[(ids * BLOCK) // PAGE_SIZE]
        slots[r, :len(ids)] = (pages * PAGE_SIZE + (ids * BLOCK) % PAGE_SIZE) // BLOCK
    return table.astype(np.int32), slots.astype(np.int32)


def sparse_row_lens(table, lens):
    """Live columns of each sparse row: the live keys of its listed blocks."""
    table = np.asarray(table, dtype=np.int64)
    out = np.zeros(table.shape[0], dtype=np.int64)
    for r in range(table.shape[0]):
        ids = table[r][table[r] != INT32_MAX]
        out[r] = int(np.clip(int(lens[r]) - ids * BLOCK, 0, BLOCK).sum())
    return out


def sparse_to_logical(table, cols):
    """Logical key position of sparse column c of each row: 8 * table[c // 8] + c % 8.

    Outside that definition (a reading): -1 stays -1, and a column past the
    row's table (c >= 8 * kb) or on a padding entry (INT32_MAX) has no key
    and gives -1 as well.
    """
    table = np.asarray(table, dtype=np.int64)
    cols = np.asarray(cols, dtype=np.int64)
    kb = table.shape[1]
    out = np.full(cols.shape, -1, dtype=np.int64)
    ok = (cols >= 0) & (cols < BLOCK * kb)
    r = np.nonzero(ok)
    blocks = table[r[0], cols[ok] // BLOCK]
    out[ok] = np.where(blocks == INT32_MAX, -1, BLOCK * blocks + cols[ok] % BLOCK)
    return out


def sparse_logits(q, kv_pages, k_scales, weights, block_table, table, lens, next_n,
                  fill=np.nan):
    """float32 [rows, kb * 8]: the logits of the listed blocks' live keys, block
    i of the table at columns 8i .. 8i+7; ``fill`` elsewhere."""
    table = np.asarray(table, dtype=np.int64)
    rows, kb = table.shape
    out = np.full((rows, kb * BLOCK), fill, dtype=np.float32)
    for r in range(rows):
        ids = table[r][table[r] != INT32_MAX]
        if ids.size == 0:
            continue
        keys = (ids[:, None] * BLOCK + np.arange(BLOCK)[None, :]).reshape(-1)
        cols = np.arange(keys.size)
        live = keys < int(lens[r])
        if live.any():
            out[r, cols[live]] = indexer_logits_at(q, kv_pages, k_scales, weights, block_table,
                                                   next_n, r, keys[live])
    return out
