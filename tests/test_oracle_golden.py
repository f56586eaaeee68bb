"""Pin the oracle's eviction rule on hand-worked cases (tests/golden)."""
import os

import numpy as np
import pytest

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "handworked_eviction.txt")
D = B = 16


def _vec(code: int) -> np.ndarray:
    return np.array([1.0 if (code >> j) & 1 else -1.0 for j in range(D)])


def _cases():
    cases, cur = [], None
    for raw in open(GOLDEN):
        line = raw.split("#", 1)[0].strip()
        if not line:
            continue
        tok = line.split()
        if tok[0] == "case":
            kv = dict(zip(tok[2::2], tok[3::2]))
            cur = {"name": tok[1], "budget": int(kv["budget"]), "group": int(kv["group"]),
                   "policy": kv["policy"], "chunk": int(kv.get("chunk", 0)), "decode": []}
        elif tok[0] == "prompt":
            cur["prompt"] = [int(x, 16) for x in tok[1:]]
        elif tok[0] == "pquery":
            cur["pquery"] = [[int(x, 16) for x in t.split(",")] for t in tok[1:]]
        elif tok[0] == "qobs":
            cur["qobs"] = [int(x, 16) for x in tok[1].split(",")]
        elif tok[0] == "kept":
            cur["kept"] = [int(x) for x in tok[1:]]
        elif tok[0] == "prefill_tok":
            cur["prefill_tok"] = [int(x) for x in tok[1:]]
        elif tok[0] == "decode":
            kv = dict(t.split("=") for t in tok[1:])
            cur["decode"].append(([int(x, 16) for x in kv["q"].split(",")], int(kv["k"], 16),
                                  int(kv["evicted"])))
        elif tok[0] == "final_tok":
            cur["final_tok"] = [int(x) for x in tok[1:]]
        elif tok[0] == "tier_tok":
            cur["tier_tok"] = [int(x) for x in tok[1:]]
        elif tok[0] == "end":
            cases.append(cur)
    return cases


@pytest.mark.parametrize("tier", [False, True], ids=["no_tier", "tier"])
@pytest.mark.parametrize("case", _cases(), ids=lambda c: c["name"])
def test_handworked(oracle_mod, case, tier):
    R = np.eye(D, B)
    if tier and "tier_tok" not in case:
        pytest.skip("no tier_tok line")
    o = oracle_mod.OracleHead(R, case["budget"], case["group"], tier=64 if tier else -1)
    K = np.stack([_vec(c) for c in case["prompt"]])
    V = np.arange(K.size, dtype=np.float64).reshape(K.shape)
    if case["policy"] == "query":
        Q = np.stack([np.stack([_vec(c) for c in row]) for row in case["pquery"]])
        o.prefill_query(K, V, Q)
    elif case["policy"] == "chunk":
        qobs = np.stack([_vec(c) for c in case["qobs"]])
        kept = o.prefill_chunks(K, V, qobs, case["chunk"])
        assert list(kept) == case["kept"]
        # the kept list, reused on a prompt with other keys, reproduces the placement
        o2 = oracle_mod.OracleHead(R, case["budget"], case["group"])
        kept2 = o2.prefill_chunks(-K, V, None, case["chunk"], reuse=kept)
        assert list(kept2) == case["kept"]
        assert list(o2.state()["tok"]) == case["prefill_tok"]
    else:
        pol = oracle_mod.STREAM if case["policy"] == "stream" else oracle_mod.TRUNCATE
        o.prefill(K, V, pol)
    st = o.state()
    assert list(st["tok"]) == case["prefill_tok"]
    # codes of the prompt are the sign patterns (bit order pin on the way)
    for s, t in enumerate(st["tok"]):
        if t >= 0:
            assert st["code"][s, 0] == case["prompt"][t]
    for qs, kc, ev in case["decode"]:
        q = np.stack([_vec(c) for c in qs])
        r = o.decode_step(q, _vec(kc), np.zeros(D))
        assert [int(c) for c in r["qcodes"][:, 0]] == qs
        assert int(r["kcode"][0]) == kc
        assert r["evicted"] == ev
    assert list(o.state()["tok"]) == case["final_tok"]
    if tier:
        t = o.tier()
        assert list(t["tok"]) == case["tier_tok"] and t["count"] == len(case["tier_tok"])
        # the tier holds the rows the tokens had: prompt rows for prompt tokens
        for j, tk in enumerate(t["tok"]):
            if tk < len(case["prompt"]):
                np.testing.assert_array_equal(t["K"][j], K[tk])
                np.testing.assert_array_equal(t["V"][j], V[tk])
