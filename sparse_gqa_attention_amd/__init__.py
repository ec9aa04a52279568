"""Dynamic sparse GQA attention on MI355X (gfx950): indexer -> top-k -> attention.

The compute runs in libdsa.so (hand-written HIP kernels behind the C ABI of
include/dsa.h); this package is its Python binding.
"""
from .dsa import (DsaError, dsa_abi_version, dsa_last_error, dsa_indexer_score,
                  dsa_topk_workspace_bytes, dsa_topk, attention_args,
                  dsa_attention_workspace_bytes, dsa_attention_decode,
                  dsa_attention_prefill, dsa_attention_decode_noalloc, dsa_describe_plan,
                  plan_fields, DSA_PLAN_INDEXER, DSA_PLAN_TOPK, DSA_PLAN_ATTENTION_DECODE,
                  DSA_PLAN_ATTENTION_PREFILL, dsa_cache_append,
                  cache_append_args, dsa_rmsnorm_rope, dsa_rmsnorm_rope_multi, rope_args, EXPORTS,
                  LIB)

__all__ = ["DsaError", "dsa_abi_version", "dsa_last_error", "dsa_indexer_score",
           "dsa_topk_workspace_bytes", "dsa_topk", "attention_args",
           "dsa_attention_workspace_bytes", "dsa_attention_decode",
           "dsa_attention_prefill", "dsa_attention_decode_noalloc", "dsa_describe_plan",
           "plan_fields", "DSA_PLAN_INDEXER", "DSA_PLAN_TOPK", "DSA_PLAN_ATTENTION_DECODE",
           "DSA_PLAN_ATTENTION_PREFILL", "dsa_cache_append",
           "cache_append_args", "dsa_rmsnorm_rope", "dsa_rmsnorm_rope_multi", "rope_args", "EXPORTS",
           "LIB"]
