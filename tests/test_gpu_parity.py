"""GPU parity of the HIP path (through the C ABI) against the fp64 CPU oracle.

Small shapes are checked on every head and every step.  The full workload
shapes run in the launch configuration the benchmark times, over their whole
decode sequences: on every KV head of the single-sequence workloads, and on
many (sequence, KV head) pairs of the batched ones, which the oracle replays
head by head.
"""
import numpy as np
import pytest

from lsh_eviction_amd import configs as C
from lsh_eviction_amd.configs import Shape

pytestmark = pytest.mark.gpu

FUSED, SPLIT = 0, 1
STREAM, TRUNCATE, QUERY, CHUNK = 0, 1, 2, 3

G16 = Shape("g16_b16", 13, batch=1, n_q_heads=16, n_kv_heads=1, head_dim=128, n_bits=16,
            kv_dtype="bf16", prompt=1100, budget=640, steps=8, key_outliers=True)

SMALL = {
    "tiny": (C.TINY, 64, 0),
    "tiny_chunk64": (C.TINY.scaled(steps=24), 24, 64),
    "llama8b_small": (C.LLAMA8B.scaled(prompt=3000, budget=1500), 16, 0),
    "ragged_small": (C.RAGGED.scaled(batch=4, prompt_range=(600, 1800)), 10, 0),
    "llama70b_small": (C.LLAMA70B.scaled(batch=2, prompt=2500, budget=1200), 10, 0),
    "d64_bf16_g2": (Shape("d64_bf16_g2", 11, batch=2, n_q_heads=4, n_kv_heads=2, head_dim=64, n_bits=32,
                          kv_dtype="bf16", prompt=900, budget=333, steps=12, key_outliers=True), 12, 128),
    "d128_f32_g1": (Shape("d128_f32_g1", 12, batch=1, n_q_heads=2, n_kv_heads=2, head_dim=128, n_bits=64,
                          kv_dtype="f32", prompt=700, budget=256, steps=10, key_outliers=False), 10, 64),
    "g16_b16": (G16, 8, 0),
    "not_full": (C.LLAMA8B.scaled(prompt=700, budget=1000), 20, 0),
    "fill_then_evict": (C.LLAMA8B.scaled(prompt=990, budget=1000), 20, 0),
    "empty_prompt": (C.TINY.scaled(prompt=0, budget=8), 14, 64),
    # group sizes that are not powers of two (padded MFMA columns, uneven records)
    "g3_d128": (Shape("g3_d128", 14, batch=2, n_q_heads=6, n_kv_heads=2, head_dim=128, n_bits=32,
                      kv_dtype="bf16", prompt=900, budget=500, steps=8, key_outliers=True), 8, 64),
    "g6_d64": (Shape("g6_d64", 15, batch=1, n_q_heads=12, n_kv_heads=2, head_dim=64, n_bits=16,
                     kv_dtype="bf16", prompt=700, budget=400, steps=8, key_outliers=False), 8, 0),
    "g12_f32": (Shape("g12_f32", 16, batch=1, n_q_heads=12, n_kv_heads=1, head_dim=128, n_bits=64,
                      kv_dtype="f32", prompt=600, budget=300, steps=6, key_outliers=False), 6, 64),
    # many sequences of short, uneven budgets (KV-head-fastest grid numbering)
    "many_sequences": (C.RAGGED.scaled(batch=40, prompt_range=(300, 900)), 6, 0),
    # ragged budgets cut into several equal splits each, run longest first
    "ragged_equal_splits": (C.RAGGED.scaled(batch=6, prompt_range=(700, 2600)), 6, 448),
    # 512 sequences of 32-150 slots, 1-3 splits of 64 each: a block list of ~1200 entries
    "many_sequences_512": (C.RAGGED.scaled(batch=512, prompt_range=(64, 300)), 3, 64),
    # the fused step's last block merges up to 512 (split, head) records
    # against one common maximum per head, in one or more batches of splits,
    # and more records with a running log-sum-exp
    "g4_two_batches": (C.LLAMA8B.scaled(prompt=8100, budget=8000), 6, 64),
    "g4_lse_merge": (C.LLAMA8B.scaled(prompt=8700, budget=8600), 6, 64),
    "g16_two_batches": (G16.scaled(prompt=1600, budget=1500), 6, 64),
    "g16_lse_merge": (G16.scaled(prompt=2200, budget=2100), 6, 64),
}


@pytest.mark.parametrize("schedule", [FUSED, SPLIT], ids=["fused", "split"])
@pytest.mark.parametrize("name", list(SMALL))
def test_small(name, schedule):
    from hkv_harness import run_case
    shape, steps, chunk = SMALL[name]
    run_case(shape, steps, schedule=schedule, policy=STREAM, chunk=chunk)


@pytest.mark.parametrize("schedule", [FUSED, SPLIT], ids=["fused", "split"])
def test_truncate_policy(schedule):
    from hkv_harness import run_case
    run_case(C.LLAMA8B.scaled(prompt=2100, budget=1000), 8, schedule=schedule, policy=TRUNCATE)


QUERY_SMALL = {
    "tiny": (C.TINY, 8, 0),
    "llama8b_small": (C.LLAMA8B.scaled(prompt=3000, budget=1500), 6, 0),
    "ragged_small": (C.RAGGED.scaled(batch=4, prompt_range=(600, 1800)), 4, 0),
    "llama70b_small": (C.LLAMA70B.scaled(batch=2, prompt=2500, budget=1200), 4, 0),
    "g16_b16": (SMALL["g16_b16"][0], 4, 0),
    "d128_f32_g1": (SMALL["d128_f32_g1"][0], 4, 64),
    "d64_bf16_g2": (SMALL["d64_bf16_g2"][0], 4, 128),
    "not_full": (C.LLAMA8B.scaled(prompt=700, budget=1000), 4, 0),
    "empty_prompt": (C.TINY.scaled(prompt=0, budget=8), 4, 64),
    "g3_d128": (SMALL["g3_d128"][0], 4, 64),
    "g12_f32": (SMALL["g12_f32"][0], 3, 64),
}


@pytest.mark.parametrize("name", list(QUERY_SMALL))
def test_query_prefill_small(name):
    """Query-driven prefill: codes of every prompt query row, the sequential
    selection and the cache it leaves, then decode steps."""
    from hkv_harness import run_case
    shape, steps, chunk = QUERY_SMALL[name]
    run_case(shape, steps, schedule=FUSED, policy=QUERY, chunk=chunk)


def test_query_prefill_full_llama3_8b_layer():
    """The 8B layer shape (8192-token prompt, 4096 slots, 4096 sequential
    evictions per head) under the query-driven prefill, sampled heads."""
    from hkv_harness import run_case
    run_case(C.LLAMA8B, 2, schedule=FUSED, policy=QUERY, heads=[(0, 0), (0, 3), (0, 7)], check_every=0)


# (shape, decode steps, attention split, tokens per prefill chunk)
CHUNK_SMALL = {
    "tiny": (C.TINY, 8, 0, 10),
    "llama8b_small": (C.LLAMA8B.scaled(prompt=3000, budget=1500), 6, 0, 10),
    "ragged_small": (C.RAGGED.scaled(batch=4, prompt_range=(600, 1800)), 4, 0, 10),
    "llama70b_small": (C.LLAMA70B.scaled(batch=2, prompt=2500, budget=1200), 4, 0, 16),
    "g16_b16_c32": (SMALL["g16_b16"][0], 4, 0, 32),
    "g16_b64_c32": (Shape("g16_b64", 14, batch=1, n_q_heads=16, n_kv_heads=1, head_dim=64, n_bits=64,
                          kv_dtype="bf16", prompt=2000, budget=700, steps=4, key_outliers=True), 4, 128, 32),
    "d64_bf16_g2_c3": (SMALL["d64_bf16_g2"][0], 4, 128, 3),
    "d128_f32_g1_c1": (SMALL["d128_f32_g1"][0], 4, 64, 1),
    "not_full": (C.LLAMA8B.scaled(prompt=700, budget=1000), 4, 0, 10),
    "budget_below_chunk": (C.TINY.scaled(prompt=100, budget=7), 9, 64, 10),
    "empty_prompt": (C.TINY.scaled(prompt=0, budget=8), 4, 64, 10),
    "many_chunks": (C.TINY.scaled(prompt=40000, budget=9000), 3, 1024, 3),   # > 1024 chunks per block pass
}


@pytest.mark.parametrize("name", list(CHUNK_SMALL))
def test_chunk_prefill_small(name):
    """Chunk-granular prefill: observation codes, kept chunk lists, the cache
    they leave (bit-exact given the GPU's codes), then decode steps, which
    first fill any slots the whole chunks left free."""
    from hkv_harness import run_case
    shape, steps, chunk, pchunk = CHUNK_SMALL[name]
    run_case(shape, steps, schedule=FUSED, policy=CHUNK, chunk=chunk, prefill_chunk=pchunk)


def test_chunk_prefill_reuse_across_layers():
    """The kept lists of one layer's cache, given to the next layer's cache
    (other keys and values, no observation queries), place the same tokens."""
    from hkv_harness import run_case
    shape = C.LLAMA8B.scaled(batch=2, prompt=2105, budget=1000)   # same lengths and budgets for any seed
    st, st2 = {}, {}
    run_case(shape, 2, schedule=FUSED, policy=CHUNK, prefill_chunk=10, stats=st)
    run_case(shape, 2, schedule=FUSED, policy=CHUNK, prefill_chunk=10, seed=777, reuse=st["kept"],
             observe=False, stats=st2)
    np.testing.assert_array_equal(st2["kept"], st["kept"])


@pytest.mark.parametrize("value_bits", [8, 4], ids=["int8", "int4"])
def test_chunk_prefill_quantized_values(value_bits):
    from hkv_harness import run_case
    run_case(C.LLAMA8B.scaled(prompt=2500, budget=1200), 4, schedule=FUSED, policy=CHUNK, prefill_chunk=10,
             value_bits=value_bits)


def test_chunk_prefill_full_long_128k():
    """The 128K workload (131072-token prompt, 32768 slots per head): 13108
    chunks per head scored, 3276 kept; sampled heads."""
    from hkv_harness import run_case
    run_case(C.LONG128K, 2, schedule=FUSED, policy=CHUNK, prefill_chunk=10, heads=[(0, 1), (0, 6)],
             check_every=0)


# (shape, decode steps, schedule, prefill policy, tier capacity)
TIER = {
    "tiny_stream": (C.TINY, 24, FUSED, STREAM, 4096),
    "tiny_split": (C.TINY, 24, SPLIT, STREAM, 4096),
    "llama8b_small_stream": (C.LLAMA8B.scaled(prompt=3000, budget=1500), 8, FUSED, STREAM, 8192),
    "llama8b_small_truncate": (C.LLAMA8B.scaled(prompt=2100, budget=1000), 6, FUSED, TRUNCATE, 4096),
    "ragged_small_query": (C.RAGGED.scaled(batch=4, prompt_range=(600, 1800)), 4, FUSED, QUERY, 4096),
    "d128_f32_g1_split": (SMALL["d128_f32_g1"][0], 6, SPLIT, STREAM, 2048),
    "g16_b16": (SMALL["g16_b16"][0], 4, FUSED, STREAM, 2048),
    "overflow": (C.LLAMA8B.scaled(prompt=3000, budget=1500), 6, FUSED, STREAM, 1000),   # capacity < spills
    "fill_then_evict": (C.LLAMA8B.scaled(prompt=990, budget=1000), 20, FUSED, STREAM, 64),
}


@pytest.mark.parametrize("name", list(TIER))
def test_host_tier_small(name):
    """Host tier in pinned host memory: the tokens leaving the cache (prefill
    drops in position order, then every eviction) with their rows, bit-exact,
    and attention over cache and tier within tolerance of the oracle's (equal
    to attention over every token while the tier has room)."""
    from hkv_harness import run_case
    shape, steps, schedule, policy, cap = TIER[name]
    run_case(shape, steps, schedule=schedule, policy=policy, tier=cap)


def test_host_tier_call_errors():
    """The tier calls check their order and their memory before enqueuing anything."""
    import torch
    from lsh_eviction_amd import hkv
    from lsh_eviction_amd import datagen
    shape = C.TINY.scaled(prompt=40, budget=16)
    P = datagen.prompt(shape)
    plain = hkv.Cache(1, 1, 1, shape.head_dim, shape.n_bits, hkv.HKV_F32, P.budgets, P.R, max_prompt=64)
    with pytest.raises(hkv.HkvError) as e:
        plain.attach_tier()                              # created without a tier capacity
    assert e.value.status == hkv.HKV_ERR_INVALID_ARG
    with pytest.raises(hkv.HkvError) as e:
        plain.tier_counts()
    assert e.value.status == hkv.HKV_ERR_STATE
    c = hkv.Cache(1, 1, 1, shape.head_dim, shape.n_bits, hkv.HKV_F32, P.budgets, P.R, max_prompt=64,
                  tier_capacity=64)
    q = torch.zeros((1, 1, shape.head_dim), device="cuda")
    with pytest.raises(hkv.HkvError) as e:
        c.attend_tiered(q)                               # no tier attached yet
    assert e.value.status == hkv.HKV_ERR_STATE
    pageable = torch.zeros((1, 1, 64, shape.head_dim))   # not pinned: the GPU cannot address it
    tok = torch.zeros((1, 1, 64), dtype=torch.int32)
    with pytest.raises(hkv.HkvError) as e:
        hkv.hkv_attach_tier(c.h, pageable, pageable.clone(), tok)
    assert e.value.status == hkv.HKV_ERR_INVALID_ARG
    c.attach_tier()
    with pytest.raises(hkv.HkvError) as e:
        c.attend_tiered(q)                               # before the prefill
    assert e.value.status == hkv.HKV_ERR_STATE
    c.prefill(hkv.to_device(P.K), hkv.to_device(P.V), P.prompt_lens)
    torch.cuda.synchronize()
    assert int(hkv.to_numpy(c.tier_counts())[0, 0]) == 40 - 16
    with pytest.raises(hkv.HkvError) as e:
        c.attach_tier()                                  # after the prefill
    assert e.value.status == hkv.HKV_ERR_STATE
    c.close(); plain.close()


def test_host_tier_chunk_prefill():
    from hkv_harness import run_case
    run_case(C.LLAMA8B.scaled(prompt=2500, budget=1200), 4, schedule=FUSED, policy=CHUNK, prefill_chunk=10,
             tier=4096)


def test_host_tier_full_long_128k():
    """The 128K workload with every dropped prompt token (98 304 per head) and
    every eviction kept in a pinned host tier; sampled heads."""
    from hkv_harness import run_case
    run_case(C.LONG128K, 2, schedule=FUSED, policy=STREAM, heads=[(0, 4)], check_every=0, tier=131072)


INT8_VALUES = {
    "llama8b_small": (C.LLAMA8B.scaled(prompt=3000, budget=1500), 12, 0),
    "ragged_small": (C.RAGGED.scaled(batch=4, prompt_range=(600, 1800)), 6, 0),
    "llama70b_small": (C.LLAMA70B.scaled(batch=2, prompt=2500, budget=1200), 6, 0),
    "d64_bf16_g2": (SMALL["d64_bf16_g2"][0], 8, 128),
    "g16_b16": (SMALL["g16_b16"][0], 6, 0),
    "not_full": (C.LLAMA8B.scaled(prompt=700, budget=1000), 8, 0),
    "fill_then_evict": (C.LLAMA8B.scaled(prompt=990, budget=1000), 16, 0),
    "empty_prompt": (C.TINY.scaled(prompt=0, budget=8, kv_dtype="bf16"), 10, 64),
    # both merges of the fused step's last block (common maximum; running log-sum-exp above 512 records)
    "g4_two_batches": (SMALL["g4_two_batches"][0], 4, 64),
    "g16_lse_merge": (SMALL["g16_lse_merge"][0], 4, 64),
    "g6_d64": (SMALL["g6_d64"][0], 6, 0),
}


@pytest.mark.parametrize("value_bits", [8, 4], ids=["int8", "int4"])
@pytest.mark.parametrize("name", list(INT8_VALUES))
def test_quantized_values_small(name, value_bits):
    """Values kept as int8 or 4-bit codes with per-row scales: codes and scales
    bit-exact, evictions exact, attention within tolerance of the oracle over
    code * scale."""
    from hkv_harness import run_case
    shape, steps, chunk = INT8_VALUES[name]
    run_case(shape, steps, schedule=FUSED, policy=STREAM, chunk=chunk, value_bits=value_bits)


@pytest.mark.parametrize("value_bits", [8, 4], ids=["int8", "int4"])
def test_quantized_values_query_prefill(value_bits):
    from hkv_harness import run_case
    run_case(C.LLAMA8B.scaled(prompt=2500, budget=1200), 4, schedule=FUSED, policy=QUERY, value_bits=value_bits)


@pytest.mark.parametrize("value_bits", [8, 4], ids=["int8", "int4"])
def test_quantized_values_full_long_128k(value_bits):
    from hkv_harness import run_case
    run_case(C.LONG128K, 3, schedule=FUSED, policy=STREAM, heads=[(0, 2)], check_every=0, value_bits=value_bits)


def test_scores_and_encoder():
    """hkv_debug_scores and hkv_encode against the oracle."""
    import torch
    import oracle
    from hkv_harness import check_codes, words_u32
    from lsh_eviction_amd import datagen, hkv
    shape = C.LLAMA70B.scaled(batch=1, prompt=1500, budget=700)
    P = datagen.prompt(shape)
    cache = hkv.Cache(1, shape.n_q_heads, shape.n_kv_heads, 128, 64, hkv.HKV_BF16, P.budgets, P.R,
                      max_prompt=P.n_max)
    cache.prefill(hkv.to_device(P.K), hkv.to_device(P.V), P.prompt_lens)
    pcodes = words_u32(cache.prefill_codes())
    rng = np.random.default_rng(5)
    qc = rng.integers(0, 2**32, size=(1, shape.n_q_heads, 2), dtype=np.uint64).astype(np.uint32)
    sc = hkv.to_numpy(cache.scores(torch.from_numpy(qc.view(np.int32)).cuda()))
    orc = oracle.OracleCache(P.R, P.budgets, shape.n_q_heads, shape.n_kv_heads)
    orc.prefill(P.K, P.V, P.prompt_lens, STREAM, inj_codes=pcodes)
    G = shape.group
    for h in range(shape.n_kv_heads):
        ref = orc.heads[(0, h)].scores(qc[0, h * G:(h + 1) * G])
        np.testing.assert_array_equal(sc[0, h], ref)
    # stand-alone encoder on fp32 and bf16 rows
    X = rng.standard_normal((1000, 128)).astype(np.float32)
    for arr in (X, datagen.f32_to_bf16_bits(X)):
        got = words_u32(cache.encode(hkv.to_device(arr)))
        ref, fl = orc.heads[(0, 0)].encode(oracle.widen(arr))
        check_codes(got, ref, fl, "hkv_encode")
    cache.close()


@pytest.mark.parametrize("value_bits", [0, 8, 4])
def test_snapshot_restore_continues_identically(value_bits):
    import torch
    from lsh_eviction_amd import datagen, hkv
    shape = C.LLAMA8B.scaled(prompt=2000, budget=900)
    wl = datagen.workload(shape, steps=12)
    P, D = wl["prompt"], wl["decode"]
    a = hkv.Cache(1, 32, 8, 128, 32, hkv.HKV_BF16, P.budgets, P.R, max_prompt=P.n_max, value_bits=value_bits)
    a.prefill(hkv.to_device(P.K), hkv.to_device(P.V), P.prompt_lens)
    for s in range(5):
        a.decode_step(hkv.to_device(D.q[s]), hkv.to_device(D.k[s]), hkv.to_device(D.v[s]))
    snap = a.get_state()
    snap = {k: v.clone() for k, v in snap.items()}
    b = hkv.Cache(1, 32, 8, 128, 32, hkv.HKV_BF16, P.budgets, P.R, max_prompt=P.n_max, value_bits=value_bits)
    b.set_state(snap)
    for s in range(5, 12):
        args = (hkv.to_device(D.q[s]), hkv.to_device(D.k[s]), hkv.to_device(D.v[s]))
        oa, ea = a.decode_step(*args)
        ob, eb = b.decode_step(*args)
        assert torch.equal(ea, eb)
        assert torch.equal(oa, ob)
    sa, sb = a.get_state(), b.get_state()
    for k in sa:
        assert torch.equal(sa[k], sb[k]), k


def test_fused_equals_split_bitwise_evictions():
    """Both schedules choose the same slots and agree on outputs to fp32 rounding."""
    import torch
    from lsh_eviction_amd import datagen, hkv
    shape = C.RAGGED.scaled(batch=6, prompt_range=(1000, 3000))
    wl = datagen.workload(shape, steps=10)
    P, D = wl["prompt"], wl["decode"]
    cs = [hkv.Cache(shape.batch, 32, 8, 128, 16, hkv.HKV_BF16, P.budgets, P.R, decode_schedule=s,
                    max_prompt=P.n_max) for s in (FUSED, SPLIT)]
    for c in cs:
        c.prefill(hkv.to_device(P.K), hkv.to_device(P.V), P.prompt_lens)
    for s in range(10):
        args = (hkv.to_device(D.q[s]), hkv.to_device(D.k[s]), hkv.to_device(D.v[s]))
        (o1, e1), (o2, e2) = cs[0].decode_step(*args), cs[1].decode_step(*args)
        assert torch.equal(e1, e2)
        assert torch.allclose(o1, o2, rtol=1e-4, atol=1e-5)


@pytest.mark.parametrize("value_bits,tier", [(0, 0), (8, 0), (4, 0), (0, 4096)], ids=["plain", "int8", "int4", "tier"])
def test_graph_replay_matches_eager(value_bits, tier):
    """A captured decode step replayed several times equals the same steps run
    eagerly (with a host tier: the same tokens spill with the same rows)."""
    import torch
    from lsh_eviction_amd import datagen, hkv
    shape = C.LLAMA8B.scaled(prompt=1500, budget=700)
    wl = datagen.workload(shape, steps=6)
    P, D = wl["prompt"], wl["decode"]
    q, k, v = (hkv.to_device(D.q[0]), hkv.to_device(D.k[0]), hkv.to_device(D.v[0]))
    caches = [hkv.Cache(1, 32, 8, 128, 32, hkv.HKV_BF16, P.budgets, P.R, max_prompt=P.n_max, value_bits=value_bits,
                        tier_capacity=tier)
              for _ in range(2)]
    for c in caches:
        if tier:
            c.attach_tier()
        c.prefill(hkv.to_device(P.K), hkv.to_device(P.V), P.prompt_lens)
    torch.cuda.synchronize()
    out = torch.empty((1, 32, 128), device="cuda")
    ev = torch.empty((1, 8), dtype=torch.int32, device="cuda")
    s = torch.cuda.Stream()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            caches[0].decode_step(q, k, v, out, ev)
    torch.cuda.synchronize()
    for step in range(6):
        q.copy_(hkv.to_device(D.q[step])); k.copy_(hkv.to_device(D.k[step])); v.copy_(hkv.to_device(D.v[step]))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        o2, e2 = caches[1].decode_step(q, k, v)
        torch.cuda.synchronize()
        assert torch.equal(ev, e2), step
        assert torch.equal(out, o2), step
    if tier:
        assert torch.equal(caches[0].tier_counts(), caches[1].tier_counts())
        torch.cuda.synchronize()
        for key in ("K", "V", "tok"):
            assert torch.equal(caches[0].tier[key], caches[1].tier[key]), key


def test_maximum_budget():
    """One head at the largest supported budget, 2^22 slots: every step scores
    a 4M-slot code table and one block merges 4096 splits; the 100 prompt
    tokens past the budget are dropped (TRUNCATE), so the steps evict."""
    from hkv_harness import run_case
    run_case(C.TINY.scaled(prompt=(1 << 22) + 100, budget=1 << 22, steps=3), 3, schedule=FUSED, policy=TRUNCATE,
             check_every=0)


def test_maximum_batch():
    """The largest supported batch, 4096 sequences of 8-40 slots (2 KV heads
    each): the block list's sequence field reaches 4095 and the grid has
    8192 blocks.  The oracle replays a spread of heads, the last sequence's
    included."""
    from hkv_harness import run_case
    shape = C.RAGGED.scaled(batch=4096, n_q_heads=8, n_kv_heads=2, prompt_range=(16, 80))
    heads = [(b, b % 2) for b in range(0, 4096, 97)] + [(4095, 0), (4095, 1), (0, 1)]
    run_case(shape, 3, schedule=FUSED, policy=STREAM, heads=heads, check_every=1)


def _ragged_pairs():
    """(sequence, KV head) pairs of the ragged batch: every head of the sequence
    with the smallest budget and of the one with the largest, and one head of
    every fourth other sequence."""
    from lsh_eviction_amd import datagen
    _, budgets = datagen.lengths(C.RAGGED)
    lo, hi = int(np.argmin(budgets)), int(np.argmax(budgets))
    pairs = [(lo, h) for h in range(8)] + [(hi, h) for h in range(8)]
    pairs += [(b, b % 8) for b in range(1, C.RAGGED.batch, 4) if b not in (lo, hi)]
    return pairs


# (shape, decode steps, heads (None: all), state compared every n steps, schedule)
FULL = {
    "llama3_8b_layer": (C.LLAMA8B, 256, None, 16, FUSED),
    "long_128k": (C.LONG128K, 128, None, 16, FUSED),
    "ragged_b32": (C.RAGGED, 64, "ragged", 16, FUSED),
    "llama3_70b_layer": (C.LLAMA70B, 128, [(0, h) for h in range(8)] + [(b, b) for b in range(1, 8)], 16, FUSED),
    # the five-launch schedule at full size
    "llama3_8b_layer_split": (C.LLAMA8B, 64, None, 16, SPLIT),
    "long_128k_split": (C.LONG128K, 16, [(0, 2), (0, 7)], 8, SPLIT),
}


@pytest.mark.parametrize("name", list(FULL))
def test_full_size_whole_decode(name):
    """Each workload at its full size, in the launch configuration the benchmark
    times, over its whole decode sequence: every decode step's codes, evicted
    slots and attention are compared, and the whole cache state (slot -> token
    map, code table, K/V rows, occupancy and position) every few steps."""
    from hkv_harness import run_case
    shape, steps, heads, every, schedule = FULL[name]
    if heads == "ragged":
        heads = _ragged_pairs()
    run_case(shape, steps, schedule=schedule, policy=STREAM, heads=heads, check_every=every, workers=16,
             label=name)


def test_set_state_rejects_bad_head_state():
    """A checkpoint whose occupancy or position would send the kernels outside
    the head's slots is refused before anything is enqueued, and the cache keeps
    working from its previous state."""
    import torch
    from lsh_eviction_amd import datagen, hkv
    shape = C.LLAMA8B.scaled(batch=2, prompt=900, budget=400)
    wl = datagen.workload(shape, steps=2)
    P, D = wl["prompt"], wl["decode"]
    c = hkv.Cache(2, 32, 8, 128, 32, hkv.HKV_BF16, P.budgets, P.R, max_prompt=P.n_max)
    c.prefill(hkv.to_device(P.K), hkv.to_device(P.V), P.prompt_lens)
    good = {k: v.clone() for k, v in c.get_state().items()}
    torch.cuda.synchronize()
    for (b, h, n, t) in [(0, 0, -1, 900), (1, 3, 401, 900), (1, 7, 400, 399)]:
        bad = {k: v.clone() for k, v in good.items()}
        bad["state"][b, h, 0] = n
        bad["state"][b, h, 1] = t
        with pytest.raises(hkv.HkvError) as e:
            c.set_state(bad)
        assert e.value.status == hkv.HKV_ERR_INVALID_ARG
        assert "head_state" in str(e.value)
    after = c.get_state()
    for k in good:
        assert torch.equal(after[k], good[k]), k
    out, ev = c.decode_step(hkv.to_device(D.q[0]), hkv.to_device(D.k[0]), hkv.to_device(D.v[0]))
    torch.cuda.synchronize()
    c.set_state(good)          # a valid checkpoint is still taken
    c.close()


# Cases for the NaN-poisoned run: (shape, steps, schedule, chunk, value_bits, tier)
POISON = {
    "tiny_fused": (C.TINY, 24, FUSED, 0, 0, 0),
    "tiny_split": (C.TINY, 24, SPLIT, 0, 0, 0),
    "ragged_small_fused": (SMALL["ragged_small"][0], 6, FUSED, 0, 0, 0),
    "ragged_small_split": (SMALL["ragged_small"][0], 6, SPLIT, 0, 0, 0),
    "many_sequences": (SMALL["many_sequences"][0], 4, FUSED, 0, 0, 0),
    "not_full_fused": (SMALL["not_full"][0], 8, FUSED, 0, 0, 0),
    "not_full_split": (SMALL["not_full"][0], 8, SPLIT, 0, 0, 0),
    "empty_prompt": (SMALL["empty_prompt"][0], 10, FUSED, 64, 0, 0),
    "g4_lse_merge": (SMALL["g4_lse_merge"][0], 3, FUSED, 64, 0, 0),
    "g16_two_batches": (SMALL["g16_two_batches"][0], 3, FUSED, 64, 0, 0),
    "int8_ragged_small": (SMALL["ragged_small"][0], 4, FUSED, 0, 8, 0),
    "int8_g16_lse_merge": (SMALL["g16_lse_merge"][0], 3, FUSED, 64, 8, 0),
    "int4_ragged_small": (SMALL["ragged_small"][0], 4, FUSED, 0, 4, 0),
    "tier_llama8b_small": (C.LLAMA8B.scaled(prompt=3000, budget=1500), 4, FUSED, 0, 0, 8192),
    "tier_tiny_split": (C.TINY, 8, SPLIT, 0, 0, 4096),
}


@pytest.mark.parametrize("name", list(POISON))
def test_nan_poisoned_partials(name, monkeypatch):
    """With HKV_DEBUG_NAN=1 every per-step partial result (fused records and
    candidate rows, split partials, tier partials) holds NaN before each step;
    parity still holds, so no step reads a partial it did not write."""
    from hkv_harness import run_case
    monkeypatch.setenv("HKV_DEBUG_NAN", "1")
    shape, steps, schedule, chunk, value_bits, tier = POISON[name]
    run_case(shape, steps, schedule=schedule, policy=STREAM, chunk=chunk, value_bits=value_bits, tier=tier)


def test_nan_poison_reaches_the_workspace(monkeypatch):
    """The switch above does poison: after a fused step the split partials,
    which that schedule does not write, still hold the NaN pattern."""
    import torch
    from lsh_eviction_amd import datagen, hkv
    monkeypatch.setenv("HKV_DEBUG_NAN", "1")
    shape = C.TINY
    wl = datagen.workload(shape, steps=1)
    P, D = wl["prompt"], wl["decode"]
    kvd = hkv.HKV_BF16 if shape.kv_dtype == "bf16" else hkv.HKV_F32
    c = hkv.Cache(shape.batch, shape.n_q_heads, shape.n_kv_heads, shape.head_dim, shape.n_bits, kvd,
                  P.budgets, P.R, max_prompt=P.n_max)
    c.prefill(hkv.to_device(P.K), hkv.to_device(P.V), P.prompt_lens)
    c.decode_step(hkv.to_device(D.q[0]), hkv.to_device(D.k[0]), hkv.to_device(D.v[0]))
    torch.cuda.synchronize()
    words = c.workspace[: c.workspace.numel() // 4 * 4].view(torch.int32)
    nan_words = int((words == 0x7FC00000).sum().item())
    nsplit = -(-int(np.max(P.budgets)) // c.chunk)
    assert nan_words >= shape.batch * shape.n_q_heads * nsplit * (shape.head_dim + 4)
    c.close()
