"""Seeded synthetic inputs for the HashEvict decode path.

This module is input plumbing shared by the GPU path's tests and by the CPU
oracle's tests.  It holds none of the method's arithmetic: it draws numbers
and rounds them to the storage type, nothing else.

Recipe (one independent numpy stream per quantity, from
``SeedSequence(SEED_BASE + shape.index)``):

* R ~ N(0, 1) in fp32, shape [head_dim][n_bits] (one projection matrix per
  cache, shared by queries and keys, as the Hamming distance between a query
  and a key code only estimates their angle when both use the same
  hyperplanes).
* keys: N(0, 1), times a fixed per-(KV head, channel) scale exp(N(0, 1)) when
  ``key_outliers`` is set -- keys with a much wider range than values, as the
  TTKV page reports for Llama-3.1-8B (section 3, Figure 2).
* values: N(0, 1).  queries: N(0, 1) in fp32 (not scaled).
* bf16 storage: round-to-nearest-even of the fp32 draw; arrays of raw bf16
  bits are returned as ``uint16``.
* ragged prompts: integer-uniform on the inclusive range, budget
  floor(frac * prompt).
"""
from __future__ import annotations

import dataclasses
from typing import Dict, Optional

import numpy as np

from .configs import SEED_BASE, Shape

# stream ids inside one workload's SeedSequence
_S_R, _S_SCALE, _S_PK, _S_PV, _S_LEN, _S_DQ, _S_DK, _S_DV, _S_PQ, _S_OQ = range(10)


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round fp32 to bf16 (round to nearest, ties to even); returns uint16 bits."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    r = (u + np.uint32(0x7FFF) + lsb) >> np.uint32(16)
    return r.astype(np.uint16)


def _streams(shape: Shape, seed: Optional[int]):
    s = SEED_BASE + shape.index if seed is None else seed
    return np.random.SeedSequence(s).spawn(10)   # child i does not depend on the count


def _rng(ss) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(ss))


@dataclasses.dataclass
class Prompt:
    R: np.ndarray             # float32 [d][b]
    K: np.ndarray             # [B][Hkv][n_max][d]  float32, or uint16 bf16 bits
    V: np.ndarray
    prompt_lens: np.ndarray   # int32 [B]
    budgets: np.ndarray       # int32 [B]
    key_scale: np.ndarray     # float32 [Hkv][d]  (ones without outliers)

    @property
    def n_max(self) -> int:
        return int(self.K.shape[2])


@dataclasses.dataclass
class Decode:
    q: np.ndarray             # float32 [steps][B][Hq][d]
    k: np.ndarray             # [steps][B][Hkv][d] float32 or uint16 bf16 bits
    v: np.ndarray


def _store(x: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "bf16":
        return f32_to_bf16_bits(x)
    return np.ascontiguousarray(x, dtype=np.float32)


def lengths(shape: Shape, seed: Optional[int] = None):
    """Prompt lengths and budgets per sequence (int32 arrays of size batch)."""
    ss = _streams(shape, seed)
    if shape.prompt_range is not None:
        lo, hi = shape.prompt_range
        n = _rng(ss[_S_LEN]).integers(lo, hi + 1, size=shape.batch).astype(np.int32)
    else:
        n = np.full(shape.batch, shape.prompt, dtype=np.int32)
    if shape.budget_frac is not None:
        s = np.floor(shape.budget_frac * n).astype(np.int32)
    else:
        s = np.full(shape.batch, shape.budget, dtype=np.int32)
    return n, s


def prompt(shape: Shape, seed: Optional[int] = None) -> Prompt:
    ss = _streams(shape, seed)
    d, b, B, H = shape.head_dim, shape.n_bits, shape.batch, shape.n_kv_heads
    R = _rng(ss[_S_R]).standard_normal((d, b), dtype=np.float32)
    if shape.key_outliers:
        scale = np.exp(_rng(ss[_S_SCALE]).standard_normal((H, d))).astype(np.float32)
    else:
        scale = np.ones((H, d), dtype=np.float32)
    n, s = lengths(shape, seed)
    n_max = int(n.max())
    gk = _rng(ss[_S_PK])
    K = gk.standard_normal((B, H, n_max, d), dtype=np.float32)
    K *= scale[None, :, None, :]
    V = _rng(ss[_S_PV]).standard_normal((B, H, n_max, d), dtype=np.float32)
    return Prompt(R=R, K=_store(K, shape.kv_dtype), V=_store(V, shape.kv_dtype),
                  prompt_lens=n, budgets=s, key_scale=scale)


def prompt_queries(shape: Shape, seed: Optional[int] = None) -> np.ndarray:
    """Query rows of the prompt tokens, fp32 [B][Hq][n_max][d] ~ N(0, 1) (the
    decode queries' distribution), for the query-driven prefill."""
    ss = _streams(shape, seed)
    n, _ = lengths(shape, seed)
    return _rng(ss[_S_PQ]).standard_normal((shape.batch, shape.n_q_heads, int(n.max()), shape.head_dim),
                                           dtype=np.float32)


def observation_queries(shape: Shape, seed: Optional[int] = None) -> np.ndarray:
    """Observation queries of the chunk prefill (those of the token decoding
    starts from), fp32 [B][Hq][d] ~ N(0, 1) like the decode queries."""
    ss = _streams(shape, seed)
    return _rng(ss[_S_OQ]).standard_normal((shape.batch, shape.n_q_heads, shape.head_dim), dtype=np.float32)


def decode(shape: Shape, steps: Optional[int] = None, seed: Optional[int] = None,
           key_scale: Optional[np.ndarray] = None) -> Decode:
    ss = _streams(shape, seed)
    T = shape.steps if steps is None else steps
    d, B, H, Hq = shape.head_dim, shape.batch, shape.n_kv_heads, shape.n_q_heads
    q = _rng(ss[_S_DQ]).standard_normal((T, B, Hq, d), dtype=np.float32)
    k = _rng(ss[_S_DK]).standard_normal((T, B, H, d), dtype=np.float32)
    if key_scale is not None:
        k *= key_scale[None, None, :, :]
    v = _rng(ss[_S_DV]).standard_normal((T, B, H, d), dtype=np.float32)
    return Decode(q=q, k=_store(k, shape.kv_dtype), v=_store(v, shape.kv_dtype))


def workload(shape: Shape, steps: Optional[int] = None, seed: Optional[int] = None) -> Dict:
    p = prompt(shape, seed)
    dec = decode(shape, steps, seed, p.key_scale if shape.key_outliers else None)
    return {"prompt": p, "decode": dec}
