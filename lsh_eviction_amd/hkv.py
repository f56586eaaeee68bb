"""Thin ctypes binding of libhkv.so (include/hkv.h).

Argument marshalling only: every step of the decode path runs in the HIP
kernels of libhkv.so.  The functions keep the C names; tensors are torch
tensors on the GPU (PyTorch provides device memory and streams, nothing else).
There is no fallback: if libhkv.so is missing, loading raises.
"""
from __future__ import annotations

import ctypes as C
import os
from typing import Optional, Sequence

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libhkv.so")

HKV_OK, HKV_ERR_INVALID_ARG, HKV_ERR_UNSUPPORTED, HKV_ERR_STATE, HKV_ERR_DEVICE = range(5)
HKV_F32, HKV_BF16 = 0, 1
HKV_PREFILL_STREAM, HKV_PREFILL_TRUNCATE, HKV_PREFILL_QUERY, HKV_PREFILL_CHUNK = 0, 1, 2, 3
DEFAULT_PREFILL_CHUNK = 10   # tokens per chunk when prefill_chunk is 0
HKV_DECODE_FUSED, HKV_DECODE_SPLIT = 0, 1

# every symbol include/hkv.h declares
EXPORTS = ("hkv_validate_config", "hkv_workspace_bytes", "hkv_create", "hkv_prefill",
           "hkv_prefill_queries", "hkv_prefill_chunks", "hkv_decode_step", "hkv_decode_step_static", "hkv_destroy",
           "hkv_status_str", "hkv_last_error", "hkv_config_chunk",
           "hkv_get_state", "hkv_set_state", "hkv_debug_last_codes", "hkv_debug_prefill_codes",
           "hkv_debug_prefill_query_codes", "hkv_debug_scores", "hkv_encode", "hkv_attach_tier",
           "hkv_tier_counts", "hkv_attend_tiered")


class hkv_config(C.Structure):
    _fields_ = [("batch", C.c_int32), ("n_q_heads", C.c_int32), ("n_kv_heads", C.c_int32),
                ("head_dim", C.c_int32), ("n_bits", C.c_int32), ("kv_dtype", C.c_int32),
                ("prefill_policy", C.c_int32), ("decode_schedule", C.c_int32),
                ("max_prompt", C.c_int32), ("chunk", C.c_int32), ("value_bits", C.c_int32),
                ("prefill_chunk", C.c_int32), ("tier_capacity", C.c_int32), ("budgets", C.POINTER(C.c_int32))]


class HkvError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"{status_str(status)}: {msg}")
        self.status = status


_lib = None


def load():
    """Load libhkv.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it with __graft_entry__.build() "
                           "(python -m lsh_eviction_amd.build)")
    L = C.CDLL(LIB_PATH)
    P, I, Z = C.c_void_p, C.c_int32, C.c_size_t
    cfgp = C.POINTER(hkv_config)
    sig = {
        "hkv_validate_config": (I, [cfgp]),
        "hkv_workspace_bytes": (I, [cfgp, C.POINTER(Z)]),
        "hkv_config_chunk": (I, [cfgp, C.POINTER(I)]),
        "hkv_create": (I, [cfgp, P, P, Z, P, C.POINTER(P)]),
        "hkv_prefill": (I, [P, P, P, P, I, P]),
        "hkv_prefill_queries": (I, [P, P, P, P, P, I, P]),
        "hkv_prefill_chunks": (I, [P, P, P, P, P, P, P, I, P]),
        "hkv_attach_tier": (I, [P, P, P, P, P]),
        "hkv_tier_counts": (I, [P, P, P]),
        "hkv_attend_tiered": (I, [P, P, P, P]),
        "hkv_decode_step": (I, [P, P, P, P, P, P, P]),
        "hkv_decode_step_static": (I, [P, P, P, P, P, P, P]),
        "hkv_destroy": (I, [P]),
        "hkv_status_str": (C.c_char_p, [I]),
        "hkv_last_error": (C.c_char_p, [P]),
        "hkv_get_state": (I, [P, P, P, P, P, P, P]),
        "hkv_set_state": (I, [P, P, P, P, P, P, P]),
        "hkv_debug_last_codes": (I, [P, P, P, P]),
        "hkv_debug_prefill_codes": (I, [P, P, P]),
        "hkv_debug_prefill_query_codes": (I, [P, P, P]),
        "hkv_debug_scores": (I, [P, P, P, P]),
        "hkv_encode": (I, [P, P, I, I, P, P]),
    }
    for name, (res, args) in sig.items():
        f = getattr(L, name)
        f.restype, f.argtypes = res, args
    _lib = L
    return L


def status_str(s: int) -> str:
    return load().hkv_status_str(int(s)).decode()


def make_config(batch, n_q_heads, n_kv_heads, head_dim, n_bits, kv_dtype, budgets,
                prefill_policy=HKV_PREFILL_STREAM, decode_schedule=HKV_DECODE_FUSED,
                max_prompt=0, chunk=0, value_bits=0, prefill_chunk=0, tier_capacity=0):
    b = np.ascontiguousarray(budgets, dtype=np.int32)
    cfg = hkv_config(int(batch), int(n_q_heads), int(n_kv_heads), int(head_dim), int(n_bits),
                     int(kv_dtype), int(prefill_policy), int(decode_schedule), int(max_prompt),
                     int(chunk), int(value_bits), int(prefill_chunk), int(tier_capacity),
                     b.ctypes.data_as(C.POINTER(C.c_int32)))
    cfg._keep = b          # keep the budgets array alive with the struct
    return cfg


def _require(t, name: str, shape, dtype, device: str = "cuda"):
    """The boundary takes plain pointers, so a tensor of the wrong shape, type,
    layout or device would be read out of bounds by a kernel: refuse it here
    with a Python error instead."""
    import torch
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name}: expected a torch.Tensor, got {type(t).__name__}")
    if tuple(t.shape) != tuple(int(x) for x in shape):
        raise ValueError(f"{name}: shape {tuple(t.shape)}, expected {tuple(int(x) for x in shape)}")
    if t.dtype != dtype:
        raise TypeError(f"{name}: dtype {t.dtype}, expected {dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name}: must be contiguous")
    if t.device.type != device:
        raise ValueError(f"{name}: on {t.device}, expected a {device} tensor")


def _ptr(t) -> Optional[int]:
    if t is None:
        return None
    return C.c_void_p(t.data_ptr())


def _stream(stream) -> C.c_void_p:
    import torch
    if stream is None:
        stream = torch.cuda.current_stream()
    return C.c_void_p(stream.cuda_stream)


def _check(status: int, handle=None):
    if status != HKV_OK:
        msg = load().hkv_last_error(handle).decode()
        raise HkvError(status, msg)


def hkv_validate_config(cfg: hkv_config) -> int:
    return load().hkv_validate_config(C.byref(cfg))


def hkv_workspace_bytes(cfg: hkv_config) -> int:
    n = C.c_size_t(0)
    _check(load().hkv_workspace_bytes(C.byref(cfg), C.byref(n)))
    return int(n.value)


def hkv_create(cfg: hkv_config, R: np.ndarray, workspace, stream=None) -> C.c_void_p:
    R = np.ascontiguousarray(R, dtype=np.float32)
    h = C.c_void_p()
    _check(load().hkv_create(C.byref(cfg), R.ctypes.data_as(C.c_void_p), _ptr(workspace),
                             workspace.numel() * workspace.element_size(), _stream(stream),
                             C.byref(h)))
    return h


def hkv_prefill(h, K, V, prompt_lens, n_max: int, stream=None):
    pl = np.ascontiguousarray(prompt_lens, dtype=np.int32)
    _check(load().hkv_prefill(h, _ptr(K), _ptr(V), pl.ctypes.data_as(C.c_void_p), int(n_max),
                              _stream(stream)), h)


def hkv_decode_step(h, q, k, v, out, evicted_slot, stream=None):
    _check(load().hkv_decode_step(h, _ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(evicted_slot),
                                  _stream(stream)), h)


def hkv_decode_step_static(h, q, k, v, out, evicted_slot, stream=None):
    _check(load().hkv_decode_step_static(h, _ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(evicted_slot),
                                         _stream(stream)), h)


def hkv_destroy(h):
    _check(load().hkv_destroy(h))


def hkv_last_error(h=None) -> str:
    return load().hkv_last_error(h).decode()


def hkv_get_state(h, K=None, V=None, codes=None, slot_token=None, head_state=None, stream=None):
    _check(load().hkv_get_state(h, _ptr(K), _ptr(V), _ptr(codes), _ptr(slot_token),
                                _ptr(head_state), _stream(stream)), h)


def hkv_set_state(h, K, V, codes, slot_token, head_state, stream=None):
    _check(load().hkv_set_state(h, _ptr(K), _ptr(V), _ptr(codes), _ptr(slot_token),
                                _ptr(head_state), _stream(stream)), h)


def hkv_debug_last_codes(h, qcodes, kcodes, stream=None):
    _check(load().hkv_debug_last_codes(h, _ptr(qcodes), _ptr(kcodes), _stream(stream)), h)


def hkv_debug_prefill_codes(h, codes, stream=None):
    _check(load().hkv_debug_prefill_codes(h, _ptr(codes), _stream(stream)), h)


def hkv_prefill_queries(h, K, V, Q, prompt_lens, n_max: int, stream=None):
    pl = np.ascontiguousarray(prompt_lens, dtype=np.int32)
    _check(load().hkv_prefill_queries(h, _ptr(K), _ptr(V), _ptr(Q), pl.ctypes.data_as(C.c_void_p), int(n_max),
                                      _stream(stream)), h)


def hkv_prefill_chunks(h, K, V, q_obs, reuse, kept, prompt_lens, n_max: int, stream=None):
    pl = np.ascontiguousarray(prompt_lens, dtype=np.int32)
    _check(load().hkv_prefill_chunks(h, _ptr(K), _ptr(V), _ptr(q_obs), _ptr(reuse), _ptr(kept),
                                     pl.ctypes.data_as(C.c_void_p), int(n_max), _stream(stream)), h)


def hkv_attach_tier(h, K, V, tok, stream=None):
    _check(load().hkv_attach_tier(h, _ptr(K), _ptr(V), _ptr(tok), _stream(stream)), h)


def hkv_tier_counts(h, counts, stream=None):
    _check(load().hkv_tier_counts(h, _ptr(counts), _stream(stream)), h)


def hkv_attend_tiered(h, q, out, stream=None):
    _check(load().hkv_attend_tiered(h, _ptr(q), _ptr(out), _stream(stream)), h)


def hkv_debug_prefill_query_codes(h, codes, stream=None):
    _check(load().hkv_debug_prefill_query_codes(h, _ptr(codes), _stream(stream)), h)


def hkv_debug_scores(h, qcodes, scores, stream=None):
    _check(load().hkv_debug_scores(h, _ptr(qcodes), _ptr(scores), _stream(stream)), h)


def hkv_encode(h, X, x_dtype: int, n: int, codes, stream=None):
    _check(load().hkv_encode(h, _ptr(X), int(x_dtype), int(n), _ptr(codes), _stream(stream)), h)


# ---------------------------------------------------------------------------
# convenience wrapper holding the workspace tensor
# ---------------------------------------------------------------------------
def kv_torch_dtype(kv_dtype: int):
    import torch
    return torch.bfloat16 if kv_dtype == HKV_BF16 else torch.float32


def to_device(x: np.ndarray, device="cuda"):
    """numpy fp32 -> fp32 tensor; numpy uint16 (raw bf16 bits) -> bf16 tensor."""
    import torch
    if x.dtype == np.uint16:
        return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).to(device).view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(device)


def to_numpy(t) -> np.ndarray:
    """Tensor -> numpy; bf16 tensors come back as raw uint16 bits."""
    import torch
    t = t.detach().cpu()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


def hkv_config_chunk(cfg) -> int:
    """Slots per attention split the library uses for this configuration."""
    out = C.c_int32(0)
    s = load().hkv_config_chunk(C.byref(cfg), C.byref(out))
    if s != HKV_OK:
        raise HkvError(s, "hkv_config_chunk: invalid configuration")
    return out.value


class Cache:
    """A HashEvict cache on the current GPU, in a torch-allocated workspace."""

    def __init__(self, batch, n_q_heads, n_kv_heads, head_dim, n_bits, kv_dtype, budgets, R,
                 prefill_policy=HKV_PREFILL_STREAM, decode_schedule=HKV_DECODE_FUSED, max_prompt=0,
                 chunk=0, stream=None, value_bits=0, prefill_chunk=0, tier_capacity=0):
        import torch
        self.cfg = make_config(batch, n_q_heads, n_kv_heads, head_dim, n_bits, kv_dtype, budgets,
                               prefill_policy, decode_schedule, max_prompt, chunk, value_bits,
                               prefill_chunk, tier_capacity)
        self.tier_capacity = int(tier_capacity)
        self.tier = None
        self.prefill_policy = int(prefill_policy)
        self.prefill_chunk = (int(prefill_chunk) or DEFAULT_PREFILL_CHUNK) if prefill_policy == HKV_PREFILL_CHUNK else 0
        self.value_bits = int(value_bits)
        self.B, self.Hq, self.Hkv, self.d, self.bits = batch, n_q_heads, n_kv_heads, head_dim, n_bits
        self.W = (n_bits + 31) // 32
        self.kv_dtype = kv_dtype
        self.budgets = np.asarray(budgets, dtype=np.int32)
        self.Smax = int(self.budgets.max())
        nbytes = hkv_workspace_bytes(self.cfg)
        self.workspace = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
        self.h = hkv_create(self.cfg, R, self.workspace, stream)
        self.n_max = 0
        self.chunk = hkv_config_chunk(self.cfg)

    def close(self):
        if getattr(self, "h", None):
            hkv_destroy(self.h)
            self.h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    @property
    def kept_len(self) -> int:
        """Entries per head of a kept-chunk list (HKV_PREFILL_CHUNK): ceil(Smax / C)."""
        return -(-self.Smax // self.prefill_chunk) if self.prefill_chunk else 0

    def prefill(self, K, V, prompt_lens, stream=None, Q=None, reuse=None):
        """K, V [B][Hkv][n_max][d].  HKV_PREFILL_QUERY: Q [B][Hq][n_max][d] fp32.
        HKV_PREFILL_CHUNK: Q [B][Hq][d] fp32 observation queries (may be None with
        reuse), reuse [B][Hkv][kept_len] int32 or None; returns the kept chunk
        lists [B][Hkv][kept_len] int32 (device)."""
        import torch
        kvt = kv_torch_dtype(self.kv_dtype)
        n_max = int(K.shape[2]) if isinstance(K, torch.Tensor) and K.dim() == 4 else -1
        _require(K, "K", (self.B, self.Hkv, n_max, self.d), kvt)
        _require(V, "V", (self.B, self.Hkv, n_max, self.d), kvt)
        self.n_max = n_max
        if self.prefill_policy == HKV_PREFILL_QUERY:
            _require(Q, "Q", (self.B, self.Hq, n_max, self.d), torch.float32)
        elif self.prefill_policy == HKV_PREFILL_CHUNK:
            if Q is not None:
                _require(Q, "Q", (self.B, self.Hq, self.d), torch.float32)
            if reuse is not None:
                _require(reuse, "reuse", (self.B, self.Hkv, max(self.kept_len, 1)), torch.int32)
        if self.prefill_policy == HKV_PREFILL_CHUNK:
            import torch
            kept = torch.empty((self.B, self.Hkv, max(self.kept_len, 1)), dtype=torch.int32, device="cuda")
            hkv_prefill_chunks(self.h, K, V, Q, reuse, kept, prompt_lens, self.n_max, stream)
            return kept
        if Q is None:
            hkv_prefill(self.h, K, V, prompt_lens, self.n_max, stream)
        else:
            hkv_prefill_queries(self.h, K, V, Q, prompt_lens, self.n_max, stream)
        return None

    def attach_tier(self, stream=None):
        """Allocate the host tier in pinned host memory ([B][Hkv][tier_capacity][d]
        K and V in the kv dtype, int32 token positions) and attach it; returns
        the dict of tensors (the handle keeps them alive)."""
        import torch
        dt = kv_torch_dtype(self.kv_dtype)
        shape = (self.B, self.Hkv, self.tier_capacity)
        self.tier = {"K": torch.zeros(shape + (self.d,), dtype=dt, pin_memory=True),
                     "V": torch.zeros(shape + (self.d,), dtype=dt, pin_memory=True),
                     "tok": torch.full(shape, -1, dtype=torch.int32, pin_memory=True)}
        hkv_attach_tier(self.h, self.tier["K"], self.tier["V"], self.tier["tok"], stream)
        return self.tier

    def tier_counts(self, stream=None):
        import torch
        cnt = torch.empty((self.B, self.Hkv), dtype=torch.int32, device="cuda")
        hkv_tier_counts(self.h, cnt, stream)
        return cnt

    def attend_tiered(self, q, out=None, stream=None, check=True):
        import torch
        if out is None:
            out = torch.empty((self.B, self.Hq, self.d), dtype=torch.float32, device="cuda")
        if check:
            _require(q, "q", (self.B, self.Hq, self.d), torch.float32)
            _require(out, "out", (self.B, self.Hq, self.d), torch.float32)
        hkv_attend_tiered(self.h, q, out, stream)
        return out

    def check_step_args(self, q, k, v, out, evicted):
        """Raise unless q, k, v, out, evicted have the shapes, types and layout
        hkv_decode_step reads and writes."""
        import torch
        kvt = kv_torch_dtype(self.kv_dtype)
        _require(q, "q", (self.B, self.Hq, self.d), torch.float32)
        _require(k, "k", (self.B, self.Hkv, self.d), kvt)
        _require(v, "v", (self.B, self.Hkv, self.d), kvt)
        _require(out, "out", (self.B, self.Hq, self.d), torch.float32)
        _require(evicted, "evicted", (self.B, self.Hkv), torch.int32)

    def decode_step(self, q, k, v, out=None, evicted=None, stream=None, check=True):
        """One decode step.  check=False skips the argument checks (several
        microseconds of host time per call): for loops over tensors already
        passed through check_step_args."""
        import torch
        if out is None:
            out = torch.empty((self.B, self.Hq, self.d), dtype=torch.float32, device="cuda")
        if evicted is None:
            evicted = torch.empty((self.B, self.Hkv), dtype=torch.int32, device="cuda")
        if check:
            self.check_step_args(q, k, v, out, evicted)
        hkv_decode_step(self.h, q, k, v, out, evicted, stream)
        return out, evicted

    def decode_step_static(self, q, k, v, out=None, evicted=None, stream=None, check=True):
        """decode_step with its per-step scratch in the library's static
        device array (hkv_decode_step_static): for callers that cannot
        allocate.  Calls that overlap on one GPU race."""
        import torch
        if out is None:
            out = torch.empty((self.B, self.Hq, self.d), dtype=torch.float32, device="cuda")
        if evicted is None:
            evicted = torch.empty((self.B, self.Hkv), dtype=torch.int32, device="cuda")
        if check:
            self.check_step_args(q, k, v, out, evicted)
        hkv_decode_step_static(self.h, q, k, v, out, evicted, stream)
        return out, evicted

    def get_state(self, stream=None):
        import torch
        dt = kv_torch_dtype(self.kv_dtype)
        K = torch.empty((self.B, self.Hkv, self.Smax, self.d), dtype=dt, device="cuda")
        rows = self.B * self.Hkv * self.Smax
        vrow = self.d * self.value_bits // 8   # bytes of a row of value codes
        if self.value_bits:
            V = torch.empty(rows * (vrow + 4), dtype=torch.uint8, device="cuda")
        else:
            V = torch.empty_like(K)
        codes = torch.empty((self.B, self.Hkv, self.Smax, self.W), dtype=torch.int32, device="cuda")
        tok = torch.empty((self.B, self.Hkv, self.Smax), dtype=torch.int32, device="cuda")
        st = torch.empty((self.B, self.Hkv, 2), dtype=torch.int32, device="cuda")
        hkv_get_state(self.h, K, V, codes, tok, st, stream)
        out = {"K": K, "V": V, "codes": codes, "tok": tok, "state": st}
        if self.value_bits:
            # codes [B][Hkv][Smax][d * bits / 8] (int8, or two 4-bit codes a
            # byte, element 2i in the low half of byte i), then fp32 scales
            # [B][Hkv][Smax]
            q = V[:rows * vrow].view(self.B, self.Hkv, self.Smax, vrow)
            out["Vq"] = q.view(torch.int8) if self.value_bits == 8 else q
            out["Vs"] = V[rows * vrow:].view(torch.float32).view(self.B, self.Hkv, self.Smax)
        return out

    def set_state(self, s, stream=None):
        import torch
        kvt = kv_torch_dtype(self.kv_dtype)
        rows = self.B * self.Hkv * self.Smax
        _require(s["K"], "K", (self.B, self.Hkv, self.Smax, self.d), kvt)
        if self.value_bits:
            _require(s["V"], "V", (rows * (self.d * self.value_bits // 8 + 4),), torch.uint8)
        else:
            _require(s["V"], "V", (self.B, self.Hkv, self.Smax, self.d), kvt)
        _require(s["codes"], "codes", (self.B, self.Hkv, self.Smax, self.W), torch.int32)
        _require(s["tok"], "tok", (self.B, self.Hkv, self.Smax), torch.int32)
        _require(s["state"], "state", (self.B, self.Hkv, 2), torch.int32)
        hkv_set_state(self.h, s["K"], s["V"], s["codes"], s["tok"], s["state"], stream)

    def last_codes(self, stream=None):
        import torch
        qc = torch.empty((self.B, self.Hq, self.W), dtype=torch.int32, device="cuda")
        kc = torch.empty((self.B, self.Hkv, self.W), dtype=torch.int32, device="cuda")
        hkv_debug_last_codes(self.h, qc, kc, stream)
        return qc, kc

    def prefill_codes(self, stream=None):
        import torch
        pc = torch.empty((self.B, self.Hkv, max(self.n_max, 1), self.W), dtype=torch.int32, device="cuda")
        hkv_debug_prefill_codes(self.h, pc, stream)
        return pc

    def prefill_query_codes(self, stream=None):
        import torch
        pc = torch.empty((self.B, self.Hq, max(self.n_max, 1), self.W), dtype=torch.int32, device="cuda")
        hkv_debug_prefill_query_codes(self.h, pc, stream)
        return pc

    def scores(self, qcodes, stream=None):
        import torch
        sc = torch.empty((self.B, self.Hkv, self.Smax), dtype=torch.int32, device="cuda")
        hkv_debug_scores(self.h, qcodes, sc, stream)
        return sc

    def encode(self, X, stream=None):
        import torch
        n = X.shape[0]
        codes = torch.empty((max(n, 1), self.W), dtype=torch.int32, device="cuda")
        hkv_encode(self.h, X, HKV_BF16 if X.dtype == torch.bfloat16 else HKV_F32, n, codes, stream)
        return codes[:n]


def u32(t) -> np.ndarray:
    """int32 tensor of code words -> numpy uint32."""
    return to_numpy(t).astype(np.int64).astype(np.uint32) if t.dtype != np.uint32 else t
