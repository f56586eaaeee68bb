"""Pin the oracle against an independent brute-force model on tiny caches.

The brute force keeps codes as boolean arrays (sign of a numpy matrix
product), Hamming distance as a count of unequal booleans, picks the victim by
sorting (-score, slot), models the cache as a slot -> token list, and attends
with scipy's softmax over a numpy matrix product.  It shares nothing with the
oracle's C code.
"""
import numpy as np
import pytest
from scipy.special import softmax


class Brute:
    def __init__(self, R, budget, group):
        self.R = np.asarray(R, np.float64)
        self.S, self.G = budget, group
        self.slots = []          # list of dicts {tok, k, v, bits}
        self.t = 0

    def bits(self, x):
        return (np.asarray(x, np.float64) @ self.R) > 0

    def _victim(self, qbits_list):
        scored = []
        for s, sl in enumerate(self.slots):
            sc = sum(int(np.count_nonzero(qb != sl["bits"])) for qb in qbits_list)
            scored.append((-sc, s))
        return sorted(scored)[0][1]

    def _place(self, qbits_list, k, v, bits):
        if len(self.slots) < self.S:
            self.slots.append(None)
            e = len(self.slots) - 1
        else:
            e = self._victim(qbits_list)
        self.slots[e] = {"tok": self.t, "k": np.array(k, np.float64), "v": np.array(v, np.float64),
                         "bits": bits}
        return e

    def prefill(self, K, V, truncate=False, Q=None):
        for t in range(len(K)):
            self.t = t
            b = self.bits(K[t])
            if Q is not None:
                self._place([self.bits(qg) for qg in Q[t]], K[t], V[t], b)
            elif truncate:
                if len(self.slots) < self.S:
                    self.slots.append({"tok": t, "k": K[t].copy(), "v": V[t].copy(), "bits": b})
            else:
                self._place([b], K[t], V[t], b)
        self.t = len(K)

    def step(self, q, k, v):
        qb = [self.bits(qg) for qg in q]
        e = self._place(qb, k, v, self.bits(k))
        self.t += 1
        Kc = np.stack([s["k"] for s in self.slots])
        Vc = np.stack([s["v"] for s in self.slots])
        out = softmax(np.asarray(q) @ Kc.T / np.sqrt(Kc.shape[1]), axis=1) @ Vc
        return e, out

    def toks(self):
        return [s["tok"] for s in self.slots] + [-1] * (self.S - len(self.slots))


@pytest.mark.parametrize("d,b,S,N,G,steps,seed,truncate", [
    (8, 16, 4, 12, 1, 20, 1, False),
    (8, 16, 8, 24, 2, 24, 2, False),
    (16, 32, 6, 20, 4, 30, 3, False),
    (64, 16, 8, 24, 1, 16, 4, False),
    (8, 64, 5, 24, 2, 20, 5, False),
    (8, 16, 6, 3, 2, 12, 6, False),      # prompt shorter than the budget
    (8, 16, 6, 20, 2, 12, 7, True),
])
def test_bruteforce(oracle_mod, d, b, S, N, G, steps, seed, truncate):
    rng = np.random.default_rng(seed)
    R = rng.standard_normal((d, b)).astype(np.float32).astype(np.float64)
    K = rng.standard_normal((N, d)); V = rng.standard_normal((N, d))
    o = oracle_mod.OracleHead(R, S, G)
    bf = Brute(R, S, G)
    o.prefill(K, V, oracle_mod.TRUNCATE if truncate else oracle_mod.STREAM)
    bf.prefill(K, V, truncate)
    assert list(o.state()["tok"]) == bf.toks()
    for _ in range(steps):
        q = rng.standard_normal((G, d)); k = rng.standard_normal(d); v = rng.standard_normal(d)
        r = o.decode_step(q, k, v)
        e, out = bf.step(q, k, v)
        assert r["evicted"] == e
        assert list(o.state()["tok"]) == bf.toks()
        np.testing.assert_allclose(r["out"], out, rtol=1e-12, atol=1e-12)


def test_constructed_ties(oracle_mod):
    """Identical keys give identical codes, so every score ties and the
    victim is always slot 0; then a single distinct key in slot 2 wins."""
    d, b, S = 8, 16, 4
    rng = np.random.default_rng(11)
    R = rng.standard_normal((d, b))
    key = rng.standard_normal(d)
    K = np.tile(key, (S, 1)); V = rng.standard_normal((S, d))
    o = oracle_mod.OracleHead(R, S, 1)
    bf = Brute(R, S, 1)
    o.prefill(K, V); bf.prefill(K, V)
    for _ in range(3):          # new tokens carry the same key: still all ties
        q = rng.standard_normal((1, d))
        r = o.decode_step(q, key, rng.standard_normal(d))
        e, _ = bf.step(q, key, np.zeros(d))
        assert r["evicted"] == e == 0
    # make slot 2 the unique farthest: store -key there via a state edit
    st = o.state()
    c_neg, _ = o.encode(-key)
    st["K"][2] = -key; st["code"][2] = c_neg
    o.set_state(st)
    q = key[None, :]                       # code of key: slot 2 differs in every bit
    r = o.decode_step(q, key, np.zeros(d))
    assert r["evicted"] == 2


@pytest.mark.parametrize("d,b,S,N,G,seed", [
    (8, 16, 4, 12, 1, 21),
    (8, 16, 5, 24, 2, 22),
    (16, 32, 6, 30, 4, 23),
    (8, 64, 5, 20, 3, 24),
    (8, 16, 6, 4, 2, 25),       # prompt shorter than the budget
])
def test_bruteforce_query_prefill(oracle_mod, d, b, S, N, G, seed):
    """The QUERY prefill rule against the brute-force model, then decode."""
    rng = np.random.default_rng(seed)
    R = rng.standard_normal((d, b)).astype(np.float32).astype(np.float64)
    K = rng.standard_normal((N, d)); V = rng.standard_normal((N, d))
    Q = rng.standard_normal((N, G, d))
    o = oracle_mod.OracleHead(R, S, G)
    bf = Brute(R, S, G)
    o.prefill_query(K, V, Q)
    bf.prefill(K, V, Q=Q)
    assert list(o.state()["tok"]) == bf.toks()
    for _ in range(6):
        q = rng.standard_normal((G, d)); k = rng.standard_normal(d); v = rng.standard_normal(d)
        r = o.decode_step(q, k, v)
        e, out = bf.step(q, k, v)
        assert r["evicted"] == e
        np.testing.assert_allclose(r["out"], out, rtol=1e-12, atol=1e-12)


def test_query_prefill_reduces_to_stream(oracle_mod):
    """With one query head per KV head and each token's query equal to its
    key, the QUERY rule scores exactly what STREAM scores: same cache."""
    rng = np.random.default_rng(31)
    d, b, S, N = 32, 32, 16, 80
    R = rng.standard_normal((d, b))
    K = rng.standard_normal((N, d)); V = rng.standard_normal((N, d))
    a = oracle_mod.OracleHead(R, S, 1)
    q = oracle_mod.OracleHead(R, S, 1)
    a.prefill(K, V, oracle_mod.STREAM)
    q.prefill_query(K, V, K[:, None, :])
    sa, sq = a.state(), q.state()
    assert list(sa["tok"]) == list(sq["tok"])
    np.testing.assert_array_equal(sa["code"], sq["code"])
    np.testing.assert_array_equal(sa["K"], sq["K"])
