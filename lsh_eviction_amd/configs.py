"""Named workload shapes for the HashEvict decode path.

Each shape is one eviction workload: a batch of sequences, each with a GQA
group of query heads per KV head, a prompt that is prefilled into a cache of a
fixed budget of slots, and a number of decode steps.  The shapes follow the
Llama-3-8B / Llama-3-70B attention layer geometry (32/8 and 64/8 heads,
head_dim 128) used on the TTKV page's evaluation (Introduction, model list),
and budgets inside and just beyond the 30-70 % compression range reported on
the HashEvict page (abstract).

This module holds no arithmetic of the method; it only names sizes.
"""
from __future__ import annotations

import dataclasses
from typing import Optional, Tuple


@dataclasses.dataclass(frozen=True)
class Shape:
    name: str
    index: int                    # seed offset of the workload
    batch: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    n_bits: int
    kv_dtype: str                 # "f32" or "bf16"
    prompt: int                   # fixed prompt length (ignored when prompt_range is set)
    budget: int                   # fixed budget (ignored when budget_frac is set)
    steps: int
    key_outliers: bool            # per-(kv head, channel) lognormal key scale
    prompt_range: Optional[Tuple[int, int]] = None   # inclusive integer range per sequence
    budget_frac: Optional[float] = None              # budget = floor(frac * prompt_b)

    @property
    def group(self) -> int:
        return self.n_q_heads // self.n_kv_heads

    @property
    def words(self) -> int:
        return (self.n_bits + 31) // 32

    def scaled(self, **kw) -> "Shape":
        """A copy with some fields replaced (smaller parity-test variants)."""
        return dataclasses.replace(self, **kw)


TINY = Shape("tiny", 0, batch=1, n_q_heads=1, n_kv_heads=1, head_dim=64, n_bits=16,
             kv_dtype="f32", prompt=256, budget=128, steps=64, key_outliers=False)

LLAMA8B = Shape("llama3_8b_layer", 1, batch=1, n_q_heads=32, n_kv_heads=8, head_dim=128,
                n_bits=32, kv_dtype="bf16", prompt=8192, budget=4096, steps=256,
                key_outliers=True)

LONG128K = Shape("long_128k", 2, batch=1, n_q_heads=32, n_kv_heads=8, head_dim=128,
                 n_bits=32, kv_dtype="bf16", prompt=131072, budget=32768, steps=128,
                 key_outliers=True)

RAGGED = Shape("ragged_b32", 3, batch=32, n_q_heads=32, n_kv_heads=8, head_dim=128,
               n_bits=16, kv_dtype="bf16", prompt=16384, budget=8192, steps=64,
               key_outliers=False, prompt_range=(4096, 16384), budget_frac=0.5)

LLAMA70B = Shape("llama3_70b_layer", 4, batch=8, n_q_heads=64, n_kv_heads=8, head_dim=128,
                 n_bits=64, kv_dtype="bf16", prompt=32768, budget=16384, steps=128,
                 key_outliers=True)

ALL = (TINY, LLAMA8B, LONG128K, RAGGED, LLAMA70B)
BY_NAME = {s.name: s for s in ALL}

SEED_BASE = 20261203
