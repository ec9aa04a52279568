"""FP64 CPU oracle of the sparse GQA attention hot path -- test infrastructure only.

Importable by the tests, by __graft_entry__.smoke() and by the bench's
CPU-baseline leg; never by the library.  See dsa_oracle.py for what each
function computes and which passage it follows.
"""
from .dsa_oracle import (query_position, indexer_scores_row, indexer_scores,
                         topk_row, topk, dequantize, attention_row,
                         sparse_attention)

__all__ = ["query_position", "indexer_scores_row", "indexer_scores",
           "topk_row", "topk", "dequantize", "attention_row",
           "sparse_attention"]
