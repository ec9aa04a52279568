"""Shapes and storage dtypes of the synthetic workloads.

Each workload is one layer of dynamic sparse GQA attention: an indexer scores
every cached token against each query token, a per-query top-k picks the keys,
and softmax attention runs over the picked keys only.  The geometry follows the
pages' model: query/KV group ratio 12, speculative decode with 8 query tokens,
2048-key chunks and a 256K context (ORT PR #33997 "Support FP16 KV cache ..."
Description items 2-3; ORT PR #33802 "Optimize ... for SM12x and 256K context"
Summary items 1-2).  Nothing here holds any of the method's arithmetic.
"""
from dataclasses import dataclass, field
from typing import Optional


@dataclass(frozen=True)
class Workload:
    name: str
    seed: int
    B: int                 # batch (sequences)
    S: int                 # query tokens per sequence in this step
    L: int                 # cached tokens per sequence (= cache capacity here)
    H_q: int               # query heads
    H_kv: int              # KV heads (GQA groups)
    D: int                 # head dim
    q_dtype: str           # "f32" | "f16" | "bf16"
    kv_dtype: str          # "f32" | "f16" | "bf16" | "i8"
    out_dtype: str         # "f32" | "f16" | "bf16"
    k: int                 # keys kept per query token
    H_idx: Optional[int] = None   # indexer heads (None: no indexer, dense selection)
    D_idx: Optional[int] = None   # indexer dim
    idx_dtype: str = "bf16"
    kv_len: Optional[tuple] = None   # per-sequence live length (None: every sequence full)
    note: str = field(default="", compare=False)

    @property
    def live_lengths(self):
        return list(self.kv_len) if self.kv_len is not None else [self.L] * self.B

    @property
    def max_kv_len(self) -> int:
        """Runtime capacity bound handed to the launches (<= L, the cache capacity)."""
        return max(self.live_lengths)

    @property
    def decode_form(self) -> bool:
        """Split-K decode attention for short query runs, prefill form otherwise."""
        return self.S <= 16

    @property
    def has_indexer(self) -> bool:
        return self.H_idx is not None

    @property
    def ratio(self) -> int:
        return self.H_q // self.H_kv

    def positions(self):
        """Absolute position of query token s: the last S slots of the cache."""
        return [self.L - self.S + s for s in range(self.S)]


TINY_DECODE = Workload(
    name="tiny_decode_1k", seed=1, B=1, S=1, L=1024, H_q=4, H_kv=1, D=64,
    q_dtype="f32", kv_dtype="f32", out_dtype="f32", k=128, H_idx=4, D_idx=32,
    note="1 query token, 1K context, FP32 KV, 4x32 indexer, top-128")

SPEC_DECODE_32K = Workload(
    name="spec_decode_32k", seed=2, B=1, S=8, L=32768, H_q=24, H_kv=2, D=128,
    q_dtype="bf16", kv_dtype="f16", out_dtype="bf16", k=2048, H_idx=16, D_idx=64,
    note="8 speculative tokens at 32760..32767, FP16 KV, ratio 12, top-2048")

PREFILL_128K = Workload(
    name="prefill_128k", seed=3, B=1, S=2048, L=131072, H_q=24, H_kv=2, D=128,
    q_dtype="bf16", kv_dtype="bf16", out_dtype="bf16", k=2048, H_idx=16, D_idx=64,
    note="2048-token prefill chunk after 129024 cached tokens, BF16 KV")

INT8_DECODE_64K = Workload(
    name="int8_batched_decode_64k", seed=4, B=8, S=1, L=65536, H_q=48, H_kv=8, D=128,
    q_dtype="bf16", kv_dtype="i8", out_dtype="bf16", k=65536,
    note="batch 8, INT8 KV with per-token per-KV-head scales, dense selection (k = L)")

DECODE_256K = Workload(
    name="decode_256k", seed=5, B=1, S=8, L=262144, H_q=24, H_kv=2, D=128,
    q_dtype="bf16", kv_dtype="f16", out_dtype="bf16", k=2048, H_idx=16, D_idx=64,
    note="8 tokens at 262136..262143, FP16 KV, 128 chunks of 2048 keys")

RAGGED_DECODE_256K = Workload(
    name="ragged_decode_256k", seed=6, B=4, S=8, L=262144, H_q=24, H_kv=2, D=128,
    q_dtype="bf16", kv_dtype="f16", out_dtype="bf16", k=2048, H_idx=16, D_idx=64,
    kv_len=(200000, 70001, 9000, 131072),
    note="4 sequences of different live lengths in a 256K-capacity cache; launches sized "
         "by the runtime bound max(kv_len) = 200000")

RAGGED_PREFILL_64K = Workload(
    name="ragged_prefill_64k", seed=7, B=3, S=512, L=65536, H_q=24, H_kv=2, D=128,
    q_dtype="bf16", kv_dtype="bf16", out_dtype="bf16", k=2048, H_idx=16, D_idx=64,
    kv_len=(65536, 20000, 512),
    note="512-token prefill chunks of 3 sequences: after 65024 and 19488 cached tokens, and "
         "a fresh sequence (kv_len == S)")

ALL = (TINY_DECODE, SPEC_DECODE_32K, PREFILL_128K, INT8_DECODE_64K, DECODE_256K)
RAGGED = (RAGGED_DECODE_256K, RAGGED_PREFILL_64K)
BY_NAME = {w.name: w for w in ALL + RAGGED}


def scaled(w: Workload, **overrides) -> Workload:
    """A copy of `w` with some fields replaced (smaller parity cases)."""
    d = {f: getattr(w, f) for f in w.__dataclass_fields__}
    d.update(overrides)
    return Workload(**d)
