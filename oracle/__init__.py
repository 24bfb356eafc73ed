"""CPU oracle of the paged MQA indexer (test infrastructure only).

Only ``tests/``, ``__graft_entry__.smoke()`` and ``bench.py``'s cpu_baseline
leg may import this package; the HIP library never does.
"""
from .indexer_oracle import *  # noqa: F401,F403
from .indexer_oracle import (  # noqa: F401
    E2M1, E4M3FN, KEY_FP16, KEY_FP32, MXFP4_BLOCK, MXFP4_TOKEN_BYTES, NUM_BINS, PAGE_SIZE,
    HEAD_DIM, NUM_HEADS, decode_e8m0, dequant_mxfp4_tokens, e2m1_decode_table, is_mxfp4_pages,
    check_logits, check_logits_f16, coarse_bin, coarse_histogram, decode_e4m3fn,
    e4m3fn_decode_table, fp16_rne, head_sum_at, indexer_logits,
    indexer_logits_at, logits_error_bound_at, score_keys, topk_row, topk_rows,
)
from . import candidates  # noqa: F401,E402
from . import prefill  # noqa: F401,E402
