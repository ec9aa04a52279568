"""Seeded synthetic inputs shared by the tests, the bench and the oracle checks."""
from .workloads import (Workload, ALL, BY_NAME, TINY_DECODE, SPEC_DECODE_32K,
                        PREFILL_128K, INT8_DECODE_64K, DECODE_256K, RAGGED,
                        RAGGED_DECODE_256K, RAGGED_PREFILL_64K, scaled)
from .generate import (make_inputs, torch_dtype, integer_scores, indexer_like_scores,
                       make_append_inputs, make_new_tokens, rope_tables,
                       make_rope_inputs, make_aux_inputs)

__all__ = ["Workload", "ALL", "BY_NAME", "TINY_DECODE", "SPEC_DECODE_32K",
           "PREFILL_128K", "INT8_DECODE_64K", "DECODE_256K", "RAGGED",
           "RAGGED_DECODE_256K", "RAGGED_PREFILL_64K", "scaled",
           "make_inputs", "torch_dtype", "integer_scores", "indexer_like_scores",
           "make_append_inputs", "make_new_tokens", "rope_tables", "make_rope_inputs",
           "make_aux_inputs"]
