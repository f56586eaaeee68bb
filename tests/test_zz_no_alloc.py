"""hkv_decode_step_static (per-step scratch in the library's static device
array) against hkv_decode_step (scratch in the workspace): the same kernels on
the same inputs, so outputs, evicted slots and the cache state must be
bit-identical -- over two calls in a row on different caches, the second with
a smaller input, so the array holds the first call's contents when the second
starts."""
import pytest

from lsh_eviction_amd import configs as C

pytestmark = pytest.mark.gpu


def _pair(shape, schedule=0, value_bits=0):
    from lsh_eviction_amd import datagen, hkv
    P = datagen.prompt(shape)
    kvd = hkv.HKV_BF16 if shape.kv_dtype == "bf16" else hkv.HKV_F32
    caches = [hkv.Cache(shape.batch, shape.n_q_heads, shape.n_kv_heads, shape.head_dim, shape.n_bits, kvd,
                        P.budgets, P.R, decode_schedule=schedule, max_prompt=P.n_max, value_bits=value_bits)
              for _ in range(2)]
    for c in caches:
        c.prefill(hkv.to_device(P.K), hkv.to_device(P.V), P.prompt_lens)
    return caches


def _step_both(caches, shape, s):
    import torch
    from lsh_eviction_amd import datagen, hkv
    D = datagen.decode(shape, steps=s + 1)
    args = (hkv.to_device(D.q[s]), hkv.to_device(D.k[s]), hkv.to_device(D.v[s]))
    o1, e1 = caches[0].decode_step(*args)
    o2, e2 = caches[1].decode_step_static(*args)
    torch.cuda.synchronize()
    assert torch.equal(e1, e2)
    assert torch.equal(o1, o2)


def _same_state(caches):
    import torch
    s1, s2 = caches[0].get_state(), caches[1].get_state()
    torch.cuda.synchronize()
    for key in s1:
        assert torch.equal(s1[key], s2[key]), key


@pytest.mark.parametrize("schedule,value_bits", [(0, 0), (1, 0), (0, 8), (0, 4)],
                         ids=["fused", "split", "fused_int8", "fused_int4"])
def test_static_scratch_matches_workspace_scratch(schedule, value_bits):
    big = C.LLAMA8B.scaled(batch=2, prompt=6000, budget=4000)
    small = C.LLAMA8B.scaled(batch=1, prompt=900, budget=500)
    cb = _pair(big, schedule, value_bits)
    cs = _pair(small, schedule, value_bits)
    for s in range(3):
        _step_both(cb, big, s)     # the large call fills the array ...
        _step_both(cs, small, s)   # ... and the smaller one starts from its contents
    _same_state(cb)
    _same_state(cs)
    for c in cb + cs:
        c.close()


def test_static_scratch_limit():
    """A step that needs more than the array refuses before enqueuing anything."""
    import torch
    from lsh_eviction_amd import datagen, hkv
    shape = C.TINY.scaled(prompt=(1 << 20) + 10, budget=1 << 20)
    P = datagen.prompt(shape)
    c = hkv.Cache(1, 1, 1, shape.head_dim, shape.n_bits, hkv.HKV_F32, P.budgets, P.R, max_prompt=P.n_max,
                  chunk=64, prefill_policy=hkv.HKV_PREFILL_TRUNCATE)
    c.prefill(hkv.to_device(P.K), hkv.to_device(P.V), P.prompt_lens)
    D = datagen.decode(shape, steps=1)
    with pytest.raises(hkv.HkvError) as e:
        c.decode_step_static(hkv.to_device(D.q[0]), hkv.to_device(D.k[0]), hkv.to_device(D.v[0]))
    assert e.value.status == hkv.HKV_ERR_UNSUPPORTED
    assert "static scratch" in str(e.value)
    out, ev = c.decode_step(hkv.to_device(D.q[0]), hkv.to_device(D.k[0]), hkv.to_device(D.v[0]))
    torch.cuda.synchronize()
    assert int(ev[0, 0]) >= 0
    c.close()
