"""ctypes front of the fp64 CPU oracle (``liboracle.so``) of the HashEvict path.

TEST INFRASTRUCTURE ONLY.  Only the test-suite, the package smoke check and the
CPU-baseline leg of the benchmark may import this package.  It shares no code
with the GPU library: it decodes bf16 storage itself, slices query heads into
GQA groups itself, and runs the eviction rule of the HashEvict summary page
("Technical framework", stages 1-5; abstract) in plain C.

Functions with no pin of their own: none -- see tests/test_oracle_*.py for the
brute-force, invariant, closed-form (Charikar) and exact-attention pins.
"""
from __future__ import annotations

import ctypes as C
import os
import subprocess
from typing import Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "liboracle.so")
SOURCES = [os.path.join(_HERE, "hkv_oracle.c")]

STREAM = 0
TRUNCATE = 1
QUERY = 2
CHUNK = 3
DEFAULT_CHUNK_TOKENS = 10


def build(verbose: bool = False) -> str:
    """Compile the oracle with the host C compiler (plain -O2, one thread)."""
    cmd = ["gcc", "-std=c11", "-O2", "-mpopcnt", "-fPIC", "-shared", "-Wall", "-Wextra",
           "-o", LIB_PATH + ".tmp"] + SOURCES + ["-lm"]
    if verbose:
        print(" ".join(cmd))
    subprocess.run(cmd, check=True)
    os.replace(LIB_PATH + ".tmp", LIB_PATH)
    return LIB_PATH


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            build()
        L = C.CDLL(LIB_PATH)
        P = C.c_void_p
        L.orc_create.restype = P
        L.orc_create.argtypes = [C.c_int, C.c_int, C.c_int, C.c_int, P]
        L.orc_destroy.argtypes = [P]
        L.orc_encode.argtypes = [P, P, P, P]
        L.orc_encode_many.argtypes = [P, C.c_int, P, P, P]
        L.orc_prefill.restype = C.c_int
        L.orc_prefill.argtypes = [P, C.c_int, C.c_int, P, P, P]
        L.orc_prefill_query.argtypes = [P, C.c_int, P, P, P, P, P]
        L.orc_set_value_bits.argtypes = [P, C.c_int]
        L.orc_set_value_bits.restype = C.c_int
        L.orc_quantize_row.argtypes = [P, C.c_int, C.c_int, P, P]
        L.orc_get_value_codes.argtypes = [P, P, P]
        L.orc_set_value_codes.argtypes = [P, P, P]
        L.orc_prefill_query.restype = C.c_int
        L.orc_prefill_chunks.restype = C.c_int
        L.orc_set_tier.restype = C.c_int
        L.orc_set_tier.argtypes = [P, C.c_int]
        L.orc_get_tier.restype = C.c_int64
        L.orc_get_tier.argtypes = [P, P, P, P]
        L.orc_attend_tiered.argtypes = [P, P, P]
        L.orc_prefill_chunks.argtypes = [P, C.c_int, C.c_int] + [P] * 7
        L.orc_decode_step.restype = C.c_int
        L.orc_decode_step.argtypes = [P] * 3 + [P] * 8 + [P]
        L.orc_scores.argtypes = [P, P, P]
        L.orc_attend.argtypes = [P, P, P]
        L.orc_get_state.argtypes = [P] * 7
        L.orc_set_state.argtypes = [P, P, P, P, P, C.c_int32, C.c_int64]
        L.orc_words.restype = C.c_int
        L.orc_words.argtypes = [P]
        _lib = L
    return _lib


def bf16_bits_to_f64(u: np.ndarray) -> np.ndarray:
    """Widen raw bf16 bits (uint16) to float64 (exact)."""
    w = np.ascontiguousarray(u, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return w.view(np.float32).astype(np.float64)


def widen(x: np.ndarray) -> np.ndarray:
    """fp32 values or raw bf16 bits -> float64."""
    if x.dtype == np.uint16:
        return bf16_bits_to_f64(x)
    return np.ascontiguousarray(x, dtype=np.float32).astype(np.float64)


def _p(a: Optional[np.ndarray]):
    return None if a is None else a.ctypes.data_as(C.c_void_p)


def _f64(a) -> np.ndarray:
    return np.ascontiguousarray(a, dtype=np.float64)


def _u32(a) -> Optional[np.ndarray]:
    return None if a is None else np.ascontiguousarray(a, dtype=np.uint32)


class OracleHead:
    """One eviction domain: the cache of one (sequence, KV head) pair."""

    def __init__(self, R: np.ndarray, budget: int, group: int, value_bits: int = 0, tier: int = -1):
        R = _f64(widen(R) if R.dtype != np.float64 else R)
        self.d, self.nbits = R.shape
        self.budget, self.group = int(budget), int(group)
        self.W = (self.nbits + 31) // 32
        self._R = R
        self._h = lib().orc_create(self.d, self.nbits, self.budget, self.group, _p(R))
        if not self._h:
            raise ValueError("orc_create rejected its arguments")
        self.value_bits = int(value_bits)
        if lib().orc_set_value_bits(self._h, self.value_bits) != 0:
            raise ValueError("value_bits must be 0, 4 or 8")
        self.tier_cap = int(tier)
        if self.tier_cap >= 0 and lib().orc_set_tier(self._h, self.tier_cap) != 0:
            raise ValueError("a host tier needs values stored as given")

    def __del__(self):
        h = getattr(self, "_h", None)
        if h and _lib is not None:
            _lib.orc_destroy(h)
            self._h = None

    def encode(self, X: np.ndarray):
        """Codes and flags, [n][W] uint32 each, for vectors X[n][d] (or one vector)."""
        X = _f64(X)
        one = X.ndim == 1
        X = X.reshape(-1, self.d)
        codes = np.zeros((X.shape[0], self.W), np.uint32)
        flags = np.zeros((X.shape[0], self.W), np.uint32)
        lib().orc_encode_many(self._h, X.shape[0], _p(X), _p(codes), _p(flags))
        return (codes[0], flags[0]) if one else (codes, flags)

    def prefill(self, K: np.ndarray, V: np.ndarray, policy: int = STREAM,
                inj_codes: Optional[np.ndarray] = None):
        K, V = _f64(K), _f64(V)
        n = K.shape[0]
        inj = _u32(inj_codes)
        if inj is not None:
            assert inj.shape == (n, self.W)
        rc = lib().orc_prefill(self._h, int(policy), n, _p(K), _p(V), _p(inj))
        if rc != 0:
            raise RuntimeError("orc_prefill failed (cache not empty?)")

    def prefill_query(self, K: np.ndarray, V: np.ndarray, Q: np.ndarray,
                      inj_codes: Optional[np.ndarray] = None, inj_qcodes: Optional[np.ndarray] = None):
        """QUERY rule: Q[n][group][d] are the query rows of each prompt token."""
        K, V, Q = _f64(K), _f64(V), _f64(Q)
        n = K.shape[0]
        assert Q.shape == (n, self.group, self.d)
        inj, injq = _u32(inj_codes), _u32(inj_qcodes)
        if inj is not None:
            assert inj.shape == (n, self.W)
        if injq is not None:
            assert injq.shape == (n, self.group, self.W)
        rc = lib().orc_prefill_query(self._h, n, _p(K), _p(V), _p(Q), _p(inj), _p(injq))
        if rc != 0:
            raise RuntimeError("orc_prefill_query failed (cache not empty?)")

    def prefill_chunks(self, K: np.ndarray, V: np.ndarray, qobs: Optional[np.ndarray], chunk: int,
                       inj_codes: Optional[np.ndarray] = None, inj_qcodes: Optional[np.ndarray] = None,
                       reuse: Optional[np.ndarray] = None) -> np.ndarray:
        """CHUNK rule: whole chunks of `chunk` prompt tokens kept or evicted, scored
        against the observation queries qobs[group][d].  Returns the kept chunk
        indices, [ceil(budget / chunk)] int32, -1 after the last."""
        K, V = _f64(K), _f64(V)
        n = K.shape[0]
        q = None if qobs is None else _f64(qobs)
        if q is not None:
            assert q.shape == (self.group, self.d)
        inj, injq = _u32(inj_codes), _u32(inj_qcodes)
        if inj is not None:
            assert inj.shape == (n, self.W)
        if injq is not None:
            assert injq.shape == (self.group, self.W)
        ru = None if reuse is None else np.ascontiguousarray(reuse, np.int32)
        kept = np.empty((self.budget + chunk - 1) // chunk, np.int32)
        rc = lib().orc_prefill_chunks(self._h, n, int(chunk), _p(K), _p(V), _p(q), _p(inj), _p(injq), _p(ru),
                                      _p(kept))
        if rc < 0:
            raise RuntimeError("orc_prefill_chunks failed (cache not empty?)")
        return kept

    def decode_step(self, q, k, v, inj_qcodes=None, inj_kcode=None):
        q, k, v = _f64(q).reshape(self.group, self.d), _f64(k), _f64(v)
        out = np.zeros((self.group, self.d), np.float64)
        ev = np.zeros(1, np.int32)
        qc = np.zeros((self.group, self.W), np.uint32)
        qf = np.zeros_like(qc)
        kc = np.zeros(self.W, np.uint32)
        kf = np.zeros_like(kc)
        iq, ik = _u32(inj_qcodes), _u32(inj_kcode)
        rc = lib().orc_decode_step(self._h, _p(q), _p(k), _p(v), _p(iq), _p(ik), _p(out),
                                   _p(ev), _p(qc), _p(qf), _p(kc), _p(kf))
        if rc != 0:
            raise RuntimeError("orc_decode_step failed (zero budget?)")
        return {"out": out, "evicted": int(ev[0]), "qcodes": qc, "qflags": qf,
                "kcode": kc, "kflag": kf}

    def scores(self, qcodes) -> np.ndarray:
        qc = _u32(qcodes).reshape(self.group, self.W)
        sc = np.zeros(self.budget, np.int32)
        lib().orc_scores(self._h, _p(qc), _p(sc))
        return sc

    def attend(self, q) -> np.ndarray:
        q = _f64(q).reshape(self.group, self.d)
        out = np.zeros((self.group, self.d), np.float64)
        lib().orc_attend(self._h, _p(q), _p(out))
        return out

    def attend_tiered(self, q) -> np.ndarray:
        """Attention over the cache and the host tier."""
        q = _f64(q).reshape(self.group, self.d)
        out = np.zeros((self.group, self.d), np.float64)
        lib().orc_attend_tiered(self._h, _p(q), _p(out))
        return out

    def tier(self) -> dict:
        """Host tier contents: K, V [kept][d], tok [kept], count (tokens sent, kept or not)."""
        m = max(self.tier_cap, 0)
        K = np.zeros((m, self.d)); V = np.zeros((m, self.d)); tok = np.zeros(m, np.int64)
        count = int(lib().orc_get_tier(self._h, _p(K), _p(V), _p(tok)))
        k = min(count, m)
        return {"K": K[:k], "V": V[:k], "tok": tok[:k], "count": count}

    def value_codes(self):
        """Codes [budget][d] (one int8 per element) and fp32 scales [budget] of a
        cache with quantized values."""
        S = max(self.budget, 0)
        q = np.zeros((S, self.d), np.int8)
        sc = np.zeros(S, np.float32)
        lib().orc_get_value_codes(self._h, _p(q), _p(sc))
        return q, sc

    def set_value_codes(self, q: np.ndarray, scale: np.ndarray):
        """Import codes [budget][d] (one int8 per element) and fp32 scales
        [budget] of a cache with quantized values; the held values become
        code * scale."""
        S = max(self.budget, 0)
        q = np.ascontiguousarray(q, np.int8).reshape(S, self.d)
        sc = np.ascontiguousarray(scale, np.float32).reshape(S)
        lib().orc_set_value_codes(self._h, _p(q), _p(sc))

    def state(self) -> dict:
        S = max(self.budget, 0)
        K = np.zeros((S, self.d)); V = np.zeros((S, self.d))
        code = np.zeros((S, self.W), np.uint32)
        tok = np.zeros(S, np.int64)
        n = np.zeros(1, np.int32); t = np.zeros(1, np.int64)
        lib().orc_get_state(self._h, _p(K), _p(V), _p(code), _p(tok), _p(n), _p(t))
        return {"K": K, "V": V, "code": code, "tok": tok, "n": int(n[0]), "t": int(t[0])}

    def set_state(self, st: dict):
        K, V = _f64(st["K"]), _f64(st["V"])
        code = _u32(st["code"])
        tok = np.ascontiguousarray(st["tok"], dtype=np.int64)
        lib().orc_set_state(self._h, _p(K), _p(V), _p(code), _p(tok), int(st["n"]), int(st["t"]))


def quantize_rows(V: np.ndarray, bits: int = 8):
    """The value-compression rule at `bits` (8 or 4) applied to rows V[..][d]:
    codes (one int8 per element), fp32 scales."""
    V = _f64(V)
    d = V.shape[-1]
    flat = V.reshape(-1, d)
    q = np.zeros(flat.shape, np.int8)
    sc = np.zeros(flat.shape[0], np.float32)
    for i in range(flat.shape[0]):
        lib().orc_quantize_row(_p(flat[i]), d, int(bits), _p(q[i]), _p(sc[i:i + 1]))
    return q.reshape(V.shape), sc.reshape(V.shape[:-1])


class OracleCache:
    """All eviction domains of a batch: heads[b][h] for b < B, h < Hkv.

    Query head hq belongs to KV head hq // G (contiguous groups)."""

    def __init__(self, R, budgets, n_q_heads: int, n_kv_heads: int, heads=None, value_bits: int = 0,
                 tier: int = -1, workers: int = 1):
        self.B = len(budgets)
        self.Hq, self.Hkv = int(n_q_heads), int(n_kv_heads)
        self.G = self.Hq // self.Hkv
        self.sel = heads if heads is not None else [(b, h) for b in range(self.B) for h in range(self.Hkv)]
        self.heads = {(b, h): OracleHead(R, int(budgets[b]), self.G, value_bits, tier) for (b, h) in self.sel}
        # Heads are independent eviction domains and the C oracle keeps no
        # global state, so with workers > 1 the calls of different heads run in
        # host threads side by side (each head's own work stays one plain,
        # single-threaded C call; ctypes releases the interpreter lock).
        self.workers = max(1, int(workers))

    def map_heads(self, fn):
        """{(b, h): fn((b, h), head)} over the selected heads, in threads when workers > 1."""
        items = list(self.heads.items())
        if self.workers == 1 or len(items) == 1:
            return {key: fn(key, o) for key, o in items}
        from concurrent.futures import ThreadPoolExecutor
        with ThreadPoolExecutor(max_workers=min(self.workers, len(items))) as ex:
            outs = list(ex.map(lambda kv: fn(kv[0], kv[1]), items))
        return {key: r for (key, _), r in zip(items, outs)}

    def prefill(self, K, V, prompt_lens, policy=STREAM, inj_codes=None, Q=None, inj_qcodes=None,
                chunk=DEFAULT_CHUNK_TOKENS, reuse=None):
        """K, V [B][Hkv][n_max][d]; with policy QUERY also Q [B][Hq][n_max][d] (fp32) and
        optionally inj_qcodes [B][Hq][n_max][W]; with policy CHUNK, Q [B][Hq][d] are the
        observation queries, inj_qcodes [B][Hq][W] and reuse [B][Hkv][k] kept lists.
        Under CHUNK returns the kept lists {(b, h): [ceil(S_b / chunk)] int32}."""
        G = self.G

        def one(key, o):
            b, h = key
            n = int(prompt_lens[b])
            inj = None if inj_codes is None else inj_codes[b, h, :n]
            if policy == CHUNK:
                q = None if Q is None else widen(Q[b, h * G:(h + 1) * G])
                iq = None if inj_qcodes is None else inj_qcodes[b, h * G:(h + 1) * G]
                ru = None if reuse is None else reuse[b, h]
                return o.prefill_chunks(widen(K[b, h, :n]), widen(V[b, h, :n]), q, chunk, inj, iq, ru)
            if policy == QUERY:
                q = widen(Q[b, h * G:(h + 1) * G, :n]).transpose(1, 0, 2)
                iq = None if inj_qcodes is None else np.ascontiguousarray(
                    inj_qcodes[b, h * G:(h + 1) * G, :n].transpose(1, 0, 2))
                o.prefill_query(widen(K[b, h, :n]), widen(V[b, h, :n]), q, inj, iq)
            else:
                o.prefill(widen(K[b, h, :n]), widen(V[b, h, :n]), policy, inj)
            return None

        kept = self.map_heads(one)
        return kept if policy == CHUNK else None

    def attend_tiered(self, q):
        """q [B][Hq][d]; attention over cache and host tier per head, keyed (b, h)."""
        G = self.G
        return self.map_heads(lambda key, o: o.attend_tiered(widen(q[key[0], key[1] * G:(key[1] + 1) * G])))

    def decode_step(self, q, k, v, inj_qcodes=None, inj_kcodes=None):
        """q [B][Hq][d] fp32; k, v [B][Hkv][d]; returns per-head dicts keyed (b, h)."""
        G = self.G

        def one(key, o):
            b, h = key
            iq = None if inj_qcodes is None else inj_qcodes[b, h * G:(h + 1) * G]
            ik = None if inj_kcodes is None else inj_kcodes[b, h]
            return o.decode_step(widen(q[b, h * G:(h + 1) * G]), widen(k[b, h]), widen(v[b, h]), iq, ik)

        return self.map_heads(one)
