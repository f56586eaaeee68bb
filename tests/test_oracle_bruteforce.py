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

    def prefill_chunks(self, K, V, qobs, C):
        """Chunk rule by sorting: the chunks come in order of (summed distance,
        higher index first) and the first floor(S / C) of them stay."""
        N = len(K)
        nch = -(-N // C)
        if N <= self.S:
            keep = set(range(nch))
        else:
            qb = [self.bits(qg) for qg in qobs]
            score = [sum(int(np.count_nonzero(q != self.bits(K[t]))) for t in range(i * C, min(N, (i + 1) * C))
                         for q in qb) for i in range(nch)]
            keep = set(sorted(range(nch), key=lambda i: (score[i], -i))[:self.S // C])
        for i in sorted(keep):
            for t in range(i * C, min(N, (i + 1) * C)):
                self.slots.append({"tok": t, "k": K[t].copy(), "v": V[t].copy(), "bits": self.bits(K[t])})
        self.t = N
        kmax = -(-self.S // C)
        return sorted(keep) + [-1] * (kmax - len(keep))

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


@pytest.mark.parametrize("d,b,S,N,G,C,seed", [
    (8, 16, 10, 47, 1, 3, 41),      # ragged last chunk
    (8, 16, 12, 60, 2, 4, 42),
    (16, 32, 20, 99, 4, 10, 43),
    (8, 16, 8, 30, 2, 1, 44),       # one token per chunk
    (8, 64, 9, 40, 3, 5, 45),
    (8, 16, 12, 9, 2, 4, 46),       # prompt shorter than the budget
    (8, 16, 3, 20, 1, 4, 47),       # budget below one chunk: nothing stays
    (4, 16, 16, 70, 2, 3, 48),      # d = 4 on 16 bits: many equal scores
])
def test_bruteforce_chunk_prefill(oracle_mod, d, b, S, N, G, C, seed):
    """The CHUNK prefill rule against sorting in the brute-force model, then decode."""
    rng = np.random.default_rng(seed)
    R = rng.standard_normal((d, b)).astype(np.float32).astype(np.float64)
    K = rng.standard_normal((N, d)); V = rng.standard_normal((N, d))
    qobs = rng.standard_normal((G, d))
    o = oracle_mod.OracleHead(R, S, G)
    bf = Brute(R, S, G)
    kept = o.prefill_chunks(K, V, qobs, C)
    assert list(kept) == bf.prefill_chunks(K, V, qobs, C)
    assert list(o.state()["tok"]) == bf.toks()
    for _ in range(S // 2 + 4):      # fills the free slots, then evicts
        q = rng.standard_normal((G, d)); k = rng.standard_normal(d); v = rng.standard_normal(d)
        r = o.decode_step(q, k, v)
        e, out = bf.step(q, k, v)
        assert r["evicted"] == e
        np.testing.assert_allclose(r["out"], out, rtol=1e-12, atol=1e-12)


def test_chunk_prefill_invariants(oracle_mod):
    """Whole chunks, token order, occupancy, and the eviction order by score."""
    rng = np.random.default_rng(51)
    d, b, S, N, G, C = 16, 16, 300, 1203, 4, 10
    R = rng.standard_normal((d, b))
    K = rng.standard_normal((N, d)); V = rng.standard_normal((N, d))
    qobs = rng.standard_normal((G, d))
    o = oracle_mod.OracleHead(R, S, G)
    kept = [int(i) for i in o.prefill_chunks(K, V, qobs, C) if i >= 0]
    nch = -(-N // C)
    assert len(kept) == S // C and kept == sorted(set(kept))
    st = o.state()
    toks = [int(t) for t in st["tok"] if t >= 0]
    assert toks == [t for i in kept for t in range(i * C, min(N, (i + 1) * C))]
    assert st["n"] == len(toks) <= S
    # scores recomputed from the oracle's own codes
    codes, _ = o.encode(K)
    qc, _ = o.encode(qobs)
    pc = np.array([bin(int(x)).count("1") for x in range(1 << 16)])
    dist = sum(pc[codes[:, 0] ^ qc[g, 0]] for g in range(G))
    score = np.array([dist[i * C:(i + 1) * C].sum() for i in range(nch)])
    ev = sorted(set(range(nch)) - set(kept))
    assert score[kept].max() <= score[ev].min()
    T = score[kept].max()
    if score[ev].min() == T:       # at the threshold the lower indices went first
        assert max(i for i in ev if score[i] == T) < min(i for i in kept if score[i] == T)


def test_chunk_prefill_reuse(oracle_mod):
    """The kept list of one layer, reused by another layer's cache, places the
    same tokens there; repeats and out-of-range entries are ignored."""
    rng = np.random.default_rng(61)
    d, b, S, N, G, C = 16, 32, 40, 133, 2, 10
    R = rng.standard_normal((d, b))
    K1, V1 = rng.standard_normal((N, d)), rng.standard_normal((N, d))
    K2, V2 = rng.standard_normal((N, d)), rng.standard_normal((N, d))
    a = oracle_mod.OracleHead(R, S, G)
    kept = a.prefill_chunks(K1, V1, rng.standard_normal((G, d)), C)
    bb = oracle_mod.OracleHead(R, S, G)
    kept2 = bb.prefill_chunks(K2, V2, None, C, reuse=kept)
    assert list(kept2) == list(kept)
    sa, sb = a.state(), bb.state()
    assert list(sa["tok"]) == list(sb["tok"])
    n = sb["n"]
    np.testing.assert_array_equal(sb["K"][:n], K2[sa["tok"][:n]])
    np.testing.assert_array_equal(sb["V"][:n], V2[sa["tok"][:n]])
    odd = np.array([kept[1], kept[1], 999, -5], np.int32)
    c = oracle_mod.OracleHead(R, S, G)
    kept3 = c.prefill_chunks(K2, V2, None, C, reuse=odd)
    assert list(kept3) == [kept[1]] + [-1] * (len(kept) - 1)
    # a prompt within the budget keeps every token whatever the list says
    f = oracle_mod.OracleHead(R, N, G)
    kf = f.prefill_chunks(K2, V2, None, C, reuse=np.array([3] + [-1] * 20, np.int32))
    assert list(f.state()["tok"]) == list(range(N)) and list(kf) == list(range(-(-N // C)))
