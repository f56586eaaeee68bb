"""The C-ABI library loads, exports every symbol include/hkv.h declares, and
rejects bad configurations on the host (no GPU needed: validation runs before
any HIP call)."""
import ctypes as C
import os
import re

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def hkv():
    from lsh_eviction_amd import build, hkv as H
    if not os.path.exists(H.LIB_PATH):
        build.build()
    H.load()
    return H


def declared_functions():
    text = open(os.path.join(ROOT, "include", "hkv.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(hkv_[a-z_]+)\s*\(", text)))


def test_exports_every_declared_symbol(hkv):
    decl = declared_functions()
    assert len(decl) >= 14
    assert sorted(hkv.EXPORTS) == decl
    lib = C.CDLL(hkv.LIB_PATH)
    for name in decl:
        assert hasattr(lib, name), name


def _cfg(hkv, **kw):
    base = dict(batch=1, n_q_heads=32, n_kv_heads=8, head_dim=128, n_bits=32, kv_dtype=hkv.HKV_BF16,
                budgets=[4096], max_prompt=8192)
    base.update(kw)
    return hkv.make_config(**base)


def test_named_shapes_validate(hkv):
    from lsh_eviction_amd import configs, datagen
    for s in configs.ALL:
        n, b = datagen.lengths(s)
        cfg = hkv.make_config(s.batch, s.n_q_heads, s.n_kv_heads, s.head_dim, s.n_bits,
                              hkv.HKV_BF16 if s.kv_dtype == "bf16" else hkv.HKV_F32, b,
                              max_prompt=int(n.max()))
        assert hkv.hkv_validate_config(cfg) == hkv.HKV_OK, s.name
        assert hkv.hkv_workspace_bytes(cfg) > 0


@pytest.mark.parametrize("kw,status", [
    (dict(n_bits=24), "UNSUPPORTED"),
    (dict(n_bits=128), "UNSUPPORTED"),
    (dict(head_dim=96), "UNSUPPORTED"),
    (dict(n_q_heads=30), "UNSUPPORTED"),
    (dict(n_q_heads=256, n_kv_heads=8), "UNSUPPORTED"),   # group 32 > 16
    (dict(budgets=[0]), "UNSUPPORTED"),
    (dict(budgets=[1 << 23], prefill_policy=1), "UNSUPPORTED"),
    (dict(budgets=[40000]), "UNSUPPORTED"),               # 160 KB code table > on-chip table
    (dict(kv_dtype=7), "UNSUPPORTED"),
    (dict(prefill_policy=4), "UNSUPPORTED"),
    (dict(tier_capacity=-1), "UNSUPPORTED"),
    (dict(tier_capacity=(1 << 28) + 1), "UNSUPPORTED"),
    (dict(tier_capacity=1000, value_bits=8), "UNSUPPORTED"),   # the tier keeps values as given
    (dict(prefill_chunk=5), "UNSUPPORTED"),                 # chunk size without the CHUNK policy
    (dict(prefill_policy=3, prefill_chunk=33), "UNSUPPORTED"),
    (dict(prefill_policy=3, prefill_chunk=-1), "UNSUPPORTED"),
    (dict(value_bits=2), "UNSUPPORTED"),
    (dict(value_bits=8, kv_dtype=0), "UNSUPPORTED"),        # int8 values need bf16 keys
    (dict(value_bits=8, decode_schedule=1), "UNSUPPORTED"), # and the fused schedule
    (dict(value_bits=4, kv_dtype=0), "UNSUPPORTED"),        # so do 4-bit values
    (dict(value_bits=4, decode_schedule=1), "UNSUPPORTED"),
    (dict(tier_capacity=1000, value_bits=4), "UNSUPPORTED"),
    (dict(budgets=[40000], prefill_policy=2), "UNSUPPORTED"),   # QUERY keeps its table on chip too
    (dict(chunk=100), "UNSUPPORTED"),
    (dict(chunk=32), "UNSUPPORTED"),
    (dict(max_prompt=-1), "UNSUPPORTED"),
    (dict(batch=0, budgets=[]), "UNSUPPORTED"),
    (dict(n_kv_heads=0), "INVALID_ARG"),
])
def test_bad_configs(hkv, kw, status):
    cfg = _cfg(hkv, **kw)
    assert hkv.hkv_validate_config(cfg) == getattr(hkv, "HKV_ERR_" + status)


def test_query_policy_validates_and_sizes_its_code_buffer(hkv):
    a = _cfg(hkv, prefill_policy=hkv.HKV_PREFILL_QUERY)
    assert hkv.hkv_validate_config(a) == hkv.HKV_OK
    # the prompt query codes ([B][Hq][max_prompt] of 4 bytes) come on top of the STREAM workspace
    extra = hkv.hkv_workspace_bytes(a) - hkv.hkv_workspace_bytes(_cfg(hkv))
    assert extra >= 32 * 8192 * 4


@pytest.mark.parametrize("budgets,heads", [([4096], 8), ([32768], 8), ([300], 1), ([1500, 800, 64], 2),
                                           ([16384] * 8, 8), ([1 << 22], 1),
                                           ([7854, 2092, 4800, 4801, 9600, 3000, 6100, 2500], 8)])
def test_default_chunk(hkv, budgets, heads):
    # chunk = 0: with equal budgets about one workgroup per compute unit,
    # ceil(sum_b S_b * Hkv / 256) rounded up to 64 in [256, 65536]; with
    # ragged ones a multiple of 64 from a quarter of that to the largest
    # budget.  The workspace (which grows with the number of splits) comes
    # out as with that chunk given explicitly.
    slots = sum(budgets) * heads
    plain = min(max(-(-(-(-slots // 256)) // 64) * 64, 256), 65536)
    kw = dict(batch=len(budgets), n_q_heads=4 * heads, n_kv_heads=heads, budgets=budgets,
              prefill_policy=hkv.HKV_PREFILL_TRUNCATE)
    auto = _cfg(hkv, **kw)
    ch = hkv.hkv_config_chunk(auto)
    assert ch % 64 == 0 and 256 <= ch <= 65536
    if len(set(budgets)) == 1:
        assert ch == plain
    else:
        assert max(256, -(-(plain // 4) // 64) * 64) <= ch <= max(plain, -(-max(budgets) // 64) * 64)
    fixed = _cfg(hkv, chunk=ch, **kw)
    assert hkv.hkv_config_chunk(fixed) == ch
    assert hkv.hkv_workspace_bytes(auto) == hkv.hkv_workspace_bytes(fixed)
    # and the comparison can tell split counts apart: half the chunk, more splits
    other = _cfg(hkv, chunk=ch // 2 // 64 * 64, **kw)
    assert hkv.hkv_workspace_bytes(auto) != hkv.hkv_workspace_bytes(other)


def test_chunk_policy_validates_and_sizes_its_score_buffer(hkv):
    a = _cfg(hkv, prefill_policy=hkv.HKV_PREFILL_CHUNK)
    assert hkv.hkv_validate_config(a) == hkv.HKV_OK
    # one int32 score per chunk of 10 prompt tokens and KV head
    extra = hkv.hkv_workspace_bytes(a) - hkv.hkv_workspace_bytes(_cfg(hkv))
    assert extra >= 8 * (8192 // 10) * 4
    one = _cfg(hkv, prefill_policy=hkv.HKV_PREFILL_CHUNK, prefill_chunk=1)
    assert hkv.hkv_workspace_bytes(one) - hkv.hkv_workspace_bytes(_cfg(hkv)) >= 8 * 8192 * 4
    # no on-chip code table: a large budget is fine
    big = _cfg(hkv, budgets=[40000], prefill_policy=hkv.HKV_PREFILL_CHUNK, prefill_chunk=32)
    assert hkv.hkv_validate_config(big) == hkv.HKV_OK


def test_tier_sizes_its_device_state(hkv):
    a = _cfg(hkv, tier_capacity=100000)
    assert hkv.hkv_validate_config(a) == hkv.HKV_OK
    # counts, the partials of the tiered attention and the prompt bitset; the tier itself is the caller's
    extra = hkv.hkv_workspace_bytes(a) - hkv.hkv_workspace_bytes(_cfg(hkv))
    assert 32 * (128 + 4) * 4 <= extra < 64 << 20


def test_truncate_allows_large_budget(hkv):
    cfg = _cfg(hkv, budgets=[40000], prefill_policy=hkv.HKV_PREFILL_TRUNCATE)
    assert hkv.hkv_validate_config(cfg) == hkv.HKV_OK


def test_null_pointers(hkv):
    L = hkv.load()
    assert L.hkv_validate_config(None) == hkv.HKV_ERR_INVALID_ARG
    cfg = _cfg(hkv)
    cfg.budgets = C.POINTER(C.c_int32)()
    assert L.hkv_validate_config(C.byref(cfg)) == hkv.HKV_ERR_INVALID_ARG
    assert L.hkv_workspace_bytes(C.byref(_cfg(hkv)), None) == hkv.HKV_ERR_INVALID_ARG
    for f, n in (("hkv_prefill", 6), ("hkv_prefill_queries", 7), ("hkv_prefill_chunks", 9),
                 ("hkv_attach_tier", 5), ("hkv_tier_counts", 3), ("hkv_attend_tiered", 4),
                 ("hkv_decode_step", 7), ("hkv_destroy", 1),
                 ("hkv_get_state", 7), ("hkv_set_state", 7), ("hkv_debug_last_codes", 4),
                 ("hkv_debug_prefill_codes", 3), ("hkv_debug_prefill_query_codes", 3), ("hkv_debug_scores", 4)):
        fn = getattr(L, f)
        args = [0 if t is C.c_int32 else None for t in fn.argtypes]
        assert len(args) == n
        assert fn(*args) == hkv.HKV_ERR_INVALID_ARG, f


def test_create_rejects_before_touching_the_gpu(hkv):
    L = hkv.load()
    cfg = _cfg(hkv)
    R = np.zeros((128, 32), np.float32)
    h = C.c_void_p()
    # NULL workspace, misaligned workspace, too small workspace
    assert L.hkv_create(C.byref(cfg), R.ctypes.data_as(C.c_void_p), None, 1 << 30, None,
                        C.byref(h)) == hkv.HKV_ERR_INVALID_ARG
    assert "workspace" in hkv.hkv_last_error(None)
    assert L.hkv_create(C.byref(cfg), R.ctypes.data_as(C.c_void_p), C.c_void_p(0x1008), 1 << 30, None,
                        C.byref(h)) == hkv.HKV_ERR_INVALID_ARG
    assert L.hkv_create(C.byref(cfg), R.ctypes.data_as(C.c_void_p), C.c_void_p(0x100000), 16, None,
                        C.byref(h)) == hkv.HKV_ERR_INVALID_ARG
    assert L.hkv_create(C.byref(cfg), None, C.c_void_p(0x100000), 1 << 40, None,
                        C.byref(h)) == hkv.HKV_ERR_INVALID_ARG
    bad = _cfg(hkv, n_bits=20)
    assert L.hkv_create(C.byref(bad), R.ctypes.data_as(C.c_void_p), C.c_void_p(0x100000), 1 << 40, None,
                        C.byref(h)) == hkv.HKV_ERR_UNSUPPORTED
    assert "n_bits" in hkv.hkv_last_error(None)
    assert not h.value


def test_workspace_grows_with_budget(hkv):
    a = hkv.hkv_workspace_bytes(_cfg(hkv, budgets=[1000]))
    b = hkv.hkv_workspace_bytes(_cfg(hkv, budgets=[2000]))
    c = hkv.hkv_workspace_bytes(_cfg(hkv, budgets=[2000, 100], batch=2))
    assert 0 < a < b < c
    # K + V of 2 x 8 heads x 2000 slots x 128 x bf16 dominate
    assert c >= 2 * 2 * 8 * 2000 * 128 * 2


def test_status_strings(hkv):
    assert hkv.status_str(0) == "HKV_OK"
    assert hkv.status_str(3) == "HKV_ERR_STATE"
    assert hkv.status_str(99) == "HKV_UNKNOWN_STATUS"


def test_quantized_values_shrink_the_workspace(hkv):
    full = hkv.hkv_workspace_bytes(_cfg(hkv))
    v8 = hkv.hkv_workspace_bytes(_cfg(hkv, value_bits=8))
    v4 = hkv.hkv_workspace_bytes(_cfg(hkv, value_bits=4))
    # V: 8 heads x 4096 slots x 128 values go from 2 bytes to 1 byte (+ a 4-byte scale per slot)
    assert full - v8 >= 8 * 4096 * (128 - 4) - 4096
    # ... and to half a byte
    assert v8 - v4 >= 8 * 4096 * 64 - 4096
    assert hkv.hkv_validate_config(_cfg(hkv, value_bits=4)) == hkv.HKV_OK


def test_binding_refuses_tensors_a_kernel_would_misread():
    # the C ABI sees plain pointers; the binding checks what it hands over
    import torch
    from lsh_eviction_amd.hkv import _require
    ok = torch.zeros(2, 4, 8)
    _require(ok, "q", (2, 4, 8), torch.float32, device="cpu")
    with pytest.raises(ValueError, match="shape"):
        _require(ok, "q", (2, 4, 16), torch.float32, device="cpu")
    with pytest.raises(TypeError, match="dtype"):
        _require(ok.to(torch.bfloat16), "q", (2, 4, 8), torch.float32, device="cpu")
    with pytest.raises(ValueError, match="contiguous"):
        _require(torch.zeros(2, 8, 4).transpose(1, 2), "q", (2, 4, 8), torch.float32, device="cpu")
    with pytest.raises(ValueError, match="cuda"):
        _require(ok, "q", (2, 4, 8), torch.float32)
    with pytest.raises(TypeError, match="torch.Tensor"):
        _require(ok.numpy(), "q", (2, 4, 8), torch.float32)
