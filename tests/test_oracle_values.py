"""Pins of the oracle's value compression (8- or 4-bit codes with a per-row
fp32 scale): hand-worked rows (tests/golden/value_quant.txt), the rounding
bound, attention over the held values, eviction being independent of how
values are stored, and a checkpoint restore."""
import os

import numpy as np
import pytest
from scipy.special import softmax

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "value_quant.txt")


def _rows():
    rows = []
    for raw in open(GOLDEN):
        line = raw.split("#", 1)[0].strip()
        if not line:
            continue
        tag, rest = line.split(None, 1)
        assert tag in ("row", "row4")
        v, sc, codes = rest.split("|")
        rows.append((8 if tag == "row" else 4, [float(x) for x in v.split()], float(sc.split()[1]),
                     [int(x) for x in codes.split()[1:]]))
    return rows


@pytest.mark.parametrize("row", _rows(), ids=lambda r: f"{r[0]}b-{r[1][:2]}")
def test_handworked_rows(oracle_mod, row):
    bits, v, scale, codes = row
    q, s = oracle_mod.quantize_rows(np.array([v]), bits)
    assert float(s[0]) == scale
    assert q[0].tolist() == codes


def test_golden_covers_both_widths():
    assert {r[0] for r in _rows()} == {8, 4}


@pytest.mark.parametrize("bits", [8, 4])
def test_rounding_bound_and_range(oracle_mod, bits):
    Q = (1 << (bits - 1)) - 1
    rng = np.random.default_rng(41)
    V = (rng.standard_normal((300, 128)) * np.exp(rng.standard_normal((300, 1)) * 2)).astype(np.float32)
    q, s = oracle_mod.quantize_rows(V, bits)
    assert np.abs(q.astype(np.int32)).max() <= Q
    # the element of largest magnitude maps to +-Q
    i = np.abs(V).argmax(axis=1)
    assert (np.abs(q[np.arange(300), i].astype(np.int32)) == Q).all()
    # |v - code * scale| <= scale / 2 (up to the fp32 rounding of v / scale)
    err = np.abs(V.astype(np.float64) - q.astype(np.float64) * s[:, None].astype(np.float64))
    assert (err <= s[:, None] * (0.5 + 1e-6) + 1e-30).all()


@pytest.mark.parametrize("bits", [8, 4])
def test_attention_over_held_values(oracle_mod, bits):
    """With budget >= length nothing is evicted: the output is dense softmax
    attention over code * scale."""
    rng = np.random.default_rng(42)
    d, b, G, N, steps = 64, 32, 4, 60, 8
    R = rng.standard_normal((d, b))
    o = oracle_mod.OracleHead(R, N + steps, G, value_bits=bits)
    K = rng.standard_normal((N, d)); V = rng.standard_normal((N, d)).astype(np.float32)
    o.prefill(K, V)
    allK, allV = list(K), list(V)
    for t in range(steps):
        q = rng.standard_normal((G, d)); k = rng.standard_normal(d); v = rng.standard_normal(d).astype(np.float32)
        r = o.decode_step(q, k, v)
        allK.append(k); allV.append(v)
        codes, scales = o.value_codes()
        n = N + t + 1
        held = codes[:n].astype(np.float64) * scales[:n, None].astype(np.float64)
        ref = softmax(q @ np.array(allK).T / np.sqrt(d), axis=1) @ held
        np.testing.assert_allclose(r["out"], ref, rtol=1e-12, atol=1e-12)
        # and the held values are the rows as given, within half a scale step
        assert np.abs(held - np.array(allV, np.float64)).max() <= scales[:n].max() * 0.5 * (1 + 1e-6)


@pytest.mark.parametrize("bits", [8, 4])
def test_eviction_does_not_depend_on_value_storage(oracle_mod, bits):
    rng = np.random.default_rng(43)
    d, b, S, N, G = 32, 16, 12, 40, 2
    R = rng.standard_normal((d, b))
    K = rng.standard_normal((N, d)); V = rng.standard_normal((N, d))
    a = oracle_mod.OracleHead(R, S, G)
    c = oracle_mod.OracleHead(R, S, G, value_bits=bits)
    a.prefill(K, V); c.prefill(K, V)
    for _ in range(20):
        q = rng.standard_normal((G, d)); k = rng.standard_normal(d); v = rng.standard_normal(d)
        assert a.decode_step(q, k, v)["evicted"] == c.decode_step(q, k, v)["evicted"]
    assert list(a.state()["tok"]) == list(c.state()["tok"])


@pytest.mark.parametrize("bits", [8, 4])
def test_quantized_snapshot_restore(oracle_mod, bits):
    """A checkpoint of a cache with quantized values (state plus value codes and
    scales) restored into a fresh cache continues identically; the import
    makes the held values code * scale."""
    rng = np.random.default_rng(44)
    d, b, S, N, G = 32, 16, 14, 40, 2
    R = rng.standard_normal((d, b))
    a = oracle_mod.OracleHead(R, S, G, value_bits=bits)
    a.prefill(rng.standard_normal((N, d)), rng.standard_normal((N, d)).astype(np.float32))
    qs = rng.standard_normal((16, G, d)); ks = rng.standard_normal((16, d))
    vs = rng.standard_normal((16, d)).astype(np.float32)
    for i in range(6):
        a.decode_step(qs[i], ks[i], vs[i])
    snap = a.state()
    codes, scales = a.value_codes()
    c = oracle_mod.OracleHead(R, S, G, value_bits=bits)
    c.set_state(dict(snap, V=np.zeros_like(snap["V"])))   # values come from the codes alone
    c.set_value_codes(codes, scales)
    held = codes.astype(np.float64) * scales[:, None].astype(np.float64)
    np.testing.assert_array_equal(c.state()["V"], held)
    np.testing.assert_array_equal(c.state()["V"], snap["V"])
    for i in range(6, 16):
        ra = a.decode_step(qs[i], ks[i], vs[i])
        rc = c.decode_step(qs[i], ks[i], vs[i])
        assert ra["evicted"] == rc["evicted"]
        np.testing.assert_array_equal(ra["out"], rc["out"])
    ca, sa = a.value_codes()
    cc, sc = c.value_codes()
    np.testing.assert_array_equal(ca, cc)
    np.testing.assert_array_equal(sa.view(np.uint32), sc.view(np.uint32))
