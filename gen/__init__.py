"""Seeded synthetic inputs shared by tests, the benchmark and the smoke run."""
from .workloads import (  # noqa: F401
    CONFIG_NAMES, MXFP4_CONFIG_NAMES, PREFILL_CONFIG_NAMES, SEEDS, IndexerInputs, config_inputs,
    make_indexer_inputs, make_prefill_inputs,
    to_e4m3fn_codes, to_mxfp4_tokens, very_long_scores,
)
