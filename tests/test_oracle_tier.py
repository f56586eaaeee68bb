"""Pin the oracle's host tier (a reading of the TTKV summary page: tokens
leaving the HBM cache go to a slow host tier instead of being dropped).

Attention over the cache and a tier that never overflows is attention over
every token seen so far, so it must equal dense softmax attention over the
whole prompt and every decoded token, computed here with numpy and scipy.
"""
import numpy as np
import pytest
from scipy.special import softmax


def _dense(q, K, V):
    return softmax(q @ K.T / np.sqrt(K.shape[1]), axis=1) @ V


def _prefill(oracle_mod, o, policy, K, V, rng, G):
    if policy == "stream":
        o.prefill(K, V, oracle_mod.STREAM)
    elif policy == "truncate":
        o.prefill(K, V, oracle_mod.TRUNCATE)
    elif policy == "query":
        o.prefill_query(K, V, rng.standard_normal((len(K), G, K.shape[1])))
    else:
        o.prefill_chunks(K, V, rng.standard_normal((G, K.shape[1])), 3)


@pytest.mark.parametrize("policy", ["stream", "truncate", "query", "chunk"])
@pytest.mark.parametrize("d,b,S,N,G,steps,seed", [
    (8, 16, 6, 20, 1, 12, 71),
    (16, 32, 10, 31, 4, 15, 72),
    (8, 64, 7, 5, 2, 12, 73),        # prompt within the budget: the tier fills at decode
])
def test_tiered_attention_is_full_attention(oracle_mod, policy, d, b, S, N, G, steps, seed):
    rng = np.random.default_rng(seed)
    R = rng.standard_normal((d, b))
    K = rng.standard_normal((N, d)); V = rng.standard_normal((N, d))
    o = oracle_mod.OracleHead(R, S, G, tier=1000)
    _prefill(oracle_mod, o, policy, K, V, rng, G)
    allK, allV = list(K), list(V)
    q = rng.standard_normal((G, d))
    np.testing.assert_allclose(o.attend_tiered(q), _dense(q, np.array(allK), np.array(allV)), rtol=1e-12,
                               atol=1e-12)
    for _ in range(steps):
        q = rng.standard_normal((G, d)); k = rng.standard_normal(d); v = rng.standard_normal(d)
        o.decode_step(q, k, v)
        allK.append(k); allV.append(v)
        np.testing.assert_allclose(o.attend_tiered(q), _dense(q, np.array(allK), np.array(allV)),
                                   rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("policy", ["stream", "query", "chunk"])
def test_tier_contents_and_order(oracle_mod, policy):
    """Cache and tier partition the tokens seen; the tier lists the prompt
    tokens not kept in position order, then each evicted token in step order,
    with the rows they had."""
    rng = np.random.default_rng(81)
    d, b, S, N, G = 16, 32, 9, 40, 2
    R = rng.standard_normal((d, b))
    K = rng.standard_normal((N, d)); V = rng.standard_normal((N, d))
    o = oracle_mod.OracleHead(R, S, G, tier=1000)
    _prefill(oracle_mod, o, policy, K, V, rng, G)
    held = set(int(t) for t in o.state()["tok"] if t >= 0)
    expect = [t for t in range(N) if t not in held]
    rowsK, rowsV = {t: K[t] for t in range(N)}, {t: V[t] for t in range(N)}
    for s in range(25):
        before = o.state()["tok"].copy()
        q = rng.standard_normal((G, d)); k = rng.standard_normal(d); v = rng.standard_normal(d)
        r = o.decode_step(q, k, v)
        rowsK[N + s], rowsV[N + s] = k, v
        if before[r["evicted"]] >= 0:
            expect.append(int(before[r["evicted"]]))
    tier = o.tier()
    assert list(tier["tok"]) == expect and tier["count"] == len(expect)
    cache = [int(t) for t in o.state()["tok"] if t >= 0]
    assert sorted(cache + expect) == list(range(N + 25))
    for j, t in enumerate(tier["tok"]):
        np.testing.assert_array_equal(tier["K"][j], rowsK[t])
        np.testing.assert_array_equal(tier["V"][j], rowsV[t])


def test_tier_capacity(oracle_mod):
    """Past its capacity the tier keeps counting but stores nothing more, and
    attention covers the cache and the kept entries only."""
    rng = np.random.default_rng(91)
    d, b, S, N, G, cap = 8, 16, 5, 30, 1, 7
    R = rng.standard_normal((d, b))
    K = rng.standard_normal((N, d)); V = rng.standard_normal((N, d))
    big = oracle_mod.OracleHead(R, S, G, tier=1000)
    small = oracle_mod.OracleHead(R, S, G, tier=cap)
    big.prefill(K, V); small.prefill(K, V)
    for _ in range(6):
        q = rng.standard_normal((G, d)); k = rng.standard_normal(d); v = rng.standard_normal(d)
        big.decode_step(q, k, v); small.decode_step(q, k, v)
    tb, ts = big.tier(), small.tier()
    assert ts["count"] == tb["count"] == N - S + 6
    assert list(ts["tok"]) == list(tb["tok"][:cap])
    st = small.state()
    q = rng.standard_normal((G, d))
    ref = _dense(q, np.concatenate([st["K"][:st["n"]], ts["K"]]), np.concatenate([st["V"][:st["n"]], ts["V"]]))
    np.testing.assert_allclose(small.attend_tiered(q), ref, rtol=1e-12, atol=1e-12)


def test_tier_needs_plain_values(oracle_mod):
    R = np.eye(8, 16)
    with pytest.raises(ValueError):
        oracle_mod.OracleHead(R, 4, 1, value_bits=8, tier=10)
