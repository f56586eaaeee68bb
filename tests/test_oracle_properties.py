"""Pin the oracle to closed forms, invariants and textbook routines.

* Charikar: for a Gaussian hyperplane r, P[sign(r.u) != sign(r.v)] = angle(u, v) / pi,
  so E[hamming / b] = theta / pi.
* exact attention: with budget >= tokens seen nothing is evicted, and the
  output must equal softmax(Q K^T / sqrt(d)) V over every token (numpy, fp64).
* bit order: with R[:, j] = e_j the code is the sign pattern of x.
* flags: a projection that is exactly zero is flagged; a large one is not.
* GQA: G identical query heads score exactly G times a single head.
* invariants of the cache after every step (occupancy, distinct tokens, the
  new token in the evicted slot, evicted tokens never return, the victim has
  the maximal score and every lower slot scores strictly less).
* snapshot / restore continues identically.
"""
import numpy as np
import pytest
from scipy.special import softmax


def test_charikar_closed_form(oracle_mod):
    d, b = 64, 16
    thetas = np.linspace(0.05, np.pi - 0.05, 12)
    n_pairs = 2500
    rng = np.random.default_rng(2024)
    for th in thetas:
        ham = 0
        for i in range(n_pairs // 50):
            # a fresh Gaussian R for every 50 pairs; the pairs themselves are
            # isotropic, so every (pair, bit) is an independent Bernoulli(th/pi)
            R = rng.standard_normal((d, b))
            o = oracle_mod.OracleHead(R, 1, 1)
            U = rng.standard_normal((50, d))
            U /= np.linalg.norm(U, axis=1, keepdims=True)
            W = rng.standard_normal((50, d))
            W -= (W * U).sum(1, keepdims=True) * U
            W /= np.linalg.norm(W, axis=1, keepdims=True)
            Vv = np.cos(th) * U + np.sin(th) * W
            cu, _ = o.encode(U)
            cv, _ = o.encode(Vv)
            x = (cu ^ cv).astype(np.uint32)
            ham += sum(bin(int(w)).count("1") for w in x.ravel())
        p = th / np.pi
        n = n_pairs * b
        mean = ham / n
        sigma = np.sqrt(p * (1 - p) / n)
        assert abs(mean - p) < 4.5 * sigma, (th, mean, p, sigma)


@pytest.mark.parametrize("d,b,G,N,steps", [(64, 16, 1, 40, 30), (128, 32, 4, 100, 20), (128, 64, 8, 33, 9)])
def test_exact_attention_no_eviction(oracle_mod, d, b, G, N, steps):
    rng = np.random.default_rng(d + b + G)
    R = rng.standard_normal((d, b))
    o = oracle_mod.OracleHead(R, N + steps, G)
    K = rng.standard_normal((N, d)) * np.exp(rng.standard_normal(d))
    V = rng.standard_normal((N, d))
    o.prefill(K, V)
    allK, allV = list(K), list(V)
    for t in range(steps):
        q = rng.standard_normal((G, d)); k = rng.standard_normal(d); v = rng.standard_normal(d)
        r = o.decode_step(q, k, v)
        allK.append(k); allV.append(v)
        assert r["evicted"] == N + t
        ref = softmax(q @ np.array(allK).T / np.sqrt(d), axis=1) @ np.array(allV)
        err = np.abs(r["out"] - ref).max() / np.abs(ref).max()
        assert err <= 1e-12
    assert list(o.state()["tok"]) == list(range(N + steps))


def test_uniform_logits_average_values(oracle_mod):
    """q = 0 gives equal logits, so the output is the plain mean of V."""
    d, b, N = 64, 16, 13
    rng = np.random.default_rng(5)
    o = oracle_mod.OracleHead(rng.standard_normal((d, b)), 32, 2)
    K = rng.standard_normal((N, d)); V = rng.standard_normal((N, d))
    o.prefill(K, V)
    out = o.attend(np.zeros((2, d)))
    np.testing.assert_allclose(out, np.tile(V.mean(0), (2, 1)), rtol=1e-13, atol=1e-15)


@pytest.mark.parametrize("b", [16, 32, 64])
def test_bit_order(oracle_mod, b):
    d = 128
    R = np.zeros((d, b)); R[np.arange(b), np.arange(b)] = 1.0
    o = oracle_mod.OracleHead(R, 1, 1)
    rng = np.random.default_rng(b)
    for _ in range(20):
        x = rng.standard_normal(d)
        c, f = o.encode(x)
        want = 0
        for j in range(b):
            want |= int(x[j] > 0) << j
        got = sum(int(c[w]) << (32 * w) for w in range(len(c)))
        assert got == want
        assert not f.any()


def test_flag_band(oracle_mod):
    d, b = 64, 32
    rng = np.random.default_rng(9)
    R = rng.standard_normal((d, b))
    o = oracle_mod.OracleHead(R, 1, 1)
    # x orthogonal to columns 3 and 17 exactly-ish: project them out in fp64
    x = rng.standard_normal(d)
    Q, _ = np.linalg.qr(R[:, [3, 17]])
    x = x - Q @ (Q.T @ x)
    y = x @ R
    c, f = o.encode(x)
    band = 1e-5 * np.linalg.norm(x) * np.linalg.norm(R, axis=0)
    for j in range(b):
        flagged = bool((int(f[j // 32]) >> (j % 32)) & 1)
        assert flagged == bool(abs(y[j]) < band[j])
    assert (int(f[0]) >> 3) & 1 and (int(f[0]) >> 17) & 1
    assert bin(int(f[0])).count("1") == 2


def test_gqa_identical_heads(oracle_mod):
    d, b, S, G = 64, 32, 40, 4
    rng = np.random.default_rng(3)
    R = rng.standard_normal((d, b))
    K = rng.standard_normal((S, d)); V = rng.standard_normal((S, d))
    og = oracle_mod.OracleHead(R, S, G)
    o1 = oracle_mod.OracleHead(R, S, 1)
    og.prefill(K, V); o1.prefill(K, V)
    for _ in range(10):
        q = rng.standard_normal(d)
        qc, _ = o1.encode(q)
        s1 = o1.scores(qc[None])
        sg = og.scores(np.tile(qc, (G, 1)))
        np.testing.assert_array_equal(sg, G * s1)
        k = rng.standard_normal(d); v = rng.standard_normal(d)
        rg = og.decode_step(np.tile(q, (G, 1)), k, v)
        r1 = o1.decode_step(q[None], k, v)
        assert rg["evicted"] == r1["evicted"]
        np.testing.assert_allclose(rg["out"], np.tile(r1["out"], (G, 1)), rtol=0, atol=0)


def test_gqa_grouping_in_cache(oracle_mod):
    """OracleCache hands query heads h*G .. h*G+G-1 to KV head h."""
    d, b, S, Hq, Hkv = 16, 16, 6, 8, 2
    G = Hq // Hkv
    rng = np.random.default_rng(12)
    R = rng.standard_normal((d, b)).astype(np.float32)
    K = rng.standard_normal((1, Hkv, 10, d)).astype(np.float32)
    V = rng.standard_normal((1, Hkv, 10, d)).astype(np.float32)
    cache = oracle_mod.OracleCache(R, [S], Hq, Hkv)
    cache.prefill(K, V, [10])
    q = rng.standard_normal((1, Hq, d)).astype(np.float32)
    k = rng.standard_normal((1, Hkv, d)).astype(np.float32)
    res = cache.decode_step(q, k, k)
    for h in range(Hkv):
        o = oracle_mod.OracleHead(R, S, G)
        o.prefill(K[0, h].astype(np.float64), V[0, h].astype(np.float64))
        r = o.decode_step(q[0, h * G:(h + 1) * G], k[0, h], k[0, h])
        assert r["evicted"] == res[(0, h)]["evicted"]
        np.testing.assert_array_equal(r["out"], res[(0, h)]["out"])


def test_invariants(oracle_mod):
    d, b, S, G, N, steps = 64, 32, 48, 4, 160, 120
    rng = np.random.default_rng(77)
    R = rng.standard_normal((d, b))
    o = oracle_mod.OracleHead(R, S, G)
    K = rng.standard_normal((N, d)); V = rng.standard_normal((N, d))
    o.prefill(K, V)
    st = o.state()
    assert st["n"] == S and st["t"] == N
    toks = st["tok"]
    assert len(set(toks.tolist())) == S and toks.min() >= 0 and toks.max() < N
    gone = set(range(N)) - set(toks.tolist())
    # prefill kept tokens 0..S-1 first, so every evicted token is a prompt token
    for t in range(steps):
        q = rng.standard_normal((G, d))
        qc, _ = o.encode(q)
        pre = o.scores(qc)
        before = o.state()["tok"].copy()
        r = o.decode_step(q, rng.standard_normal(d), rng.standard_normal(d), inj_qcodes=qc)
        e = r["evicted"]
        assert pre[e] == pre.max()
        assert (pre[:e] < pre[e]).all()
        after = o.state()
        assert after["n"] == S
        assert after["tok"][e] == N + t
        gone.add(int(before[e]))
        assert not (set(after["tok"].tolist()) & gone)
        assert len(set(after["tok"].tolist())) == S
        mask = np.ones(S, bool); mask[e] = False
        np.testing.assert_array_equal(after["tok"][mask], before[mask])


def test_snapshot_restore(oracle_mod):
    d, b, S, G = 32, 16, 20, 2
    rng = np.random.default_rng(4)
    R = rng.standard_normal((d, b))
    a = oracle_mod.OracleHead(R, S, G)
    K = rng.standard_normal((50, d)); V = rng.standard_normal((50, d))
    a.prefill(K, V)
    qs = rng.standard_normal((12, G, d)); ks = rng.standard_normal((12, d)); vs = rng.standard_normal((12, d))
    for i in range(5):
        a.decode_step(qs[i], ks[i], vs[i])
    snap = a.state()
    c = oracle_mod.OracleHead(R, S, G)
    c.set_state(snap)
    for i in range(5, 12):
        ra = a.decode_step(qs[i], ks[i], vs[i])
        rc = c.decode_step(qs[i], ks[i], vs[i])
        assert ra["evicted"] == rc["evicted"]
        np.testing.assert_array_equal(ra["out"], rc["out"])
    np.testing.assert_array_equal(a.state()["tok"], c.state()["tok"])


def test_threaded_heads_equal_sequential(oracle_mod):
    """Driving independent heads from several host threads gives exactly the
    results of driving them one after another."""
    rng = np.random.default_rng(9)
    B, Hq, Hkv, d, b, N = 2, 8, 4, 32, 32, 60
    R = rng.standard_normal((d, b)).astype(np.float32)
    budgets = np.array([20, 33], np.int32)
    K = rng.standard_normal((B, Hkv, N, d)).astype(np.float32)
    V = rng.standard_normal((B, Hkv, N, d)).astype(np.float32)
    lens = np.array([N, 45], np.int32)
    caches = [oracle_mod.OracleCache(R, budgets, Hq, Hkv, workers=w) for w in (1, 4)]
    for c in caches:
        c.prefill(K, V, lens, oracle_mod.STREAM)
    for _ in range(8):
        q = rng.standard_normal((B, Hq, d)).astype(np.float32)
        k = rng.standard_normal((B, Hkv, d)).astype(np.float32)
        v = rng.standard_normal((B, Hkv, d)).astype(np.float32)
        r1, r4 = (c.decode_step(q, k, v) for c in caches)
        assert list(r1) == list(r4)
        for key in r1:
            assert r1[key]["evicted"] == r4[key]["evicted"]
            np.testing.assert_array_equal(r1[key]["out"], r4[key]["out"])
    for key in caches[0].heads:
        s1, s4 = caches[0].heads[key].state(), caches[1].heads[key].state()
        np.testing.assert_array_equal(s1["tok"], s4["tok"])
