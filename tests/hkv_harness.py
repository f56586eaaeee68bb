"""Parity harness: run the HIP path through the C ABI and replay the CPU oracle.

Rules (the readings are the same on both sides):
* sign codes must agree bit for bit except on bits the oracle flags
  (|projection| < 1e-5 * ||x|| * ||R[:, j]||, where fp32 and fp64 may round to
  different signs);
* the oracle is then replayed with the GPU's codes injected, and Hamming
  scores, evicted slots, slot -> token maps, code tables and K/V bytes must be
  bit-identical;
* attention outputs: per (sequence, query head) row,
  max_i |gpu_i - ref_i| / max_i |ref_i| <= 2e-3 against the fp64 oracle.
"""
from __future__ import annotations

import json
import os
import sys
import time
from typing import Iterable, Optional, Sequence, Tuple

import numpy as np

import oracle
from lsh_eviction_amd import datagen
from lsh_eviction_amd.configs import Shape

ATTN_TOL = 2e-3


def log(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def words_u32(t) -> np.ndarray:
    from lsh_eviction_amd import hkv
    return hkv.to_numpy(t).view(np.uint32)


def check_codes(gpu: np.ndarray, ref: np.ndarray, flags: np.ndarray, what: str) -> int:
    """All unflagged bits equal; returns the number of (flagged) differing bits."""
    diff = (gpu ^ ref).astype(np.uint32)
    bad = diff & ~flags.astype(np.uint32)
    if bad.any():
        idx = np.argwhere(bad)[:5]
        raise AssertionError(f"{what}: {int(np.count_nonzero(bad))} unflagged code words differ, "
                             f"first at {idx.tolist()}")
    return int(np.unpackbits(np.ascontiguousarray(diff).view(np.uint8)).sum())


def rel_err_rows(out: np.ndarray, ref: np.ndarray) -> float:
    """max over rows of max_i |o - r| / max_i |r| (rows = last axis)."""
    num = np.abs(out - ref).max(axis=-1)
    den = np.maximum(np.abs(ref).max(axis=-1), 1e-30)
    return float((num / den).max())


def kv_bytes_equal(gpu_rows: np.ndarray, ref_rows_f64: np.ndarray, kv_dtype: str) -> bool:
    """Rows stored on the GPU (fp32 or raw bf16 bits) equal the oracle's fp64 copies."""
    return bool(np.array_equal(oracle.widen(gpu_rows), ref_rows_f64))


def run_case(shape: Shape, steps: int, schedule: int = 0, policy: int = 0, chunk: int = 0,
             heads: Optional[Sequence[Tuple[int, int]]] = None, seed: Optional[int] = None,
             check_every: int = 1, stats: Optional[dict] = None, value_bits: int = 0,
             prefill_chunk: int = 0, reuse: Optional[np.ndarray] = None, observe: bool = True,
             tier: int = 0, workers: int = 8, label: Optional[str] = None):
    """Prefill + `steps` decode steps on the GPU, replayed on the oracle for `heads`
    (all heads if None).  Raises AssertionError on any parity failure.

    Under the CHUNK policy the observation queries are passed when `observe`
    (their codes are checked and injected), `reuse` [B][Hkv][k] is passed as
    the kept list, and the GPU's kept lists are compared with the oracle's and
    returned in stats["kept"].

    The oracle drives up to `workers` heads at once from host threads.  When the
    environment names a file in HKV_PARITY_LOG, one JSON line per case is
    appended to it: worst attention error, flagged bits that differed, steps and
    heads compared.

    With tier > 0 a host tier of that capacity (pinned host memory) is attached
    before the prefill; its counts, token positions and rows are compared with
    the oracle's tier, and attention over cache and tier with the oracle's, after
    the prefill and after every step."""
    import torch
    from lsh_eviction_amd import hkv

    t0 = time.time()
    wl = datagen.workload(shape, steps=steps, seed=seed)
    P, Dd = wl["prompt"], wl["decode"]
    B, Hq, Hkv, d, bits = shape.batch, shape.n_q_heads, shape.n_kv_heads, shape.head_dim, shape.n_bits
    G, W = Hq // Hkv, (bits + 31) // 32
    kvd = hkv.HKV_BF16 if shape.kv_dtype == "bf16" else hkv.HKV_F32
    n_max = P.n_max
    log(f"[{shape.name}] B={B} Hq={Hq} Hkv={Hkv} d={d} b={bits} N<={n_max} S<={P.budgets.max()} "
        f"steps={steps} schedule={schedule} policy={policy} chunk={chunk} value_bits={value_bits} "
        f"prefill_chunk={prefill_chunk} reuse={reuse is not None} "
        f"(data {time.time()-t0:.1f}s)")

    cache = hkv.Cache(B, Hq, Hkv, d, bits, kvd, P.budgets, P.R, prefill_policy=policy,
                      decode_schedule=schedule, max_prompt=n_max, chunk=chunk, value_bits=value_bits,
                      prefill_chunk=prefill_chunk, tier_capacity=tier)
    if tier:
        cache.attach_tier()
    Kt, Vt = hkv.to_device(P.K), hkv.to_device(P.V)
    query = policy == oracle.QUERY
    chunked = policy == oracle.CHUNK
    if query:
        Qp = datagen.prompt_queries(shape, seed)
    elif chunked and observe:
        Qp = datagen.observation_queries(shape, seed)
    else:
        Qp = None
    Qt = hkv.to_device(Qp) if Qp is not None else None
    reuse_t = torch.from_numpy(np.ascontiguousarray(reuse, np.int32)).to("cuda") if reuse is not None else None
    kept_t = cache.prefill(Kt, Vt, P.prompt_lens, Q=Qt, reuse=reuse_t)
    pcodes = words_u32(cache.prefill_codes())
    qpcodes = words_u32(cache.prefill_query_codes()) if query else None
    if chunked and Qp is not None:
        qpcodes = words_u32(cache.last_codes()[0])      # observation query codes [B][Hq][W]
    kept = hkv.to_numpy(kept_t) if chunked else None
    torch.cuda.synchronize()
    del Kt, Vt, Qt

    sel = list(heads) if heads is not None else [(b, h) for b in range(B) for h in range(Hkv)]
    orc = oracle.OracleCache(P.R, P.budgets, Hq, Hkv, heads=sel, value_bits=value_bits, tier=tier if tier else -1,
                             workers=workers)

    def prefill_codes_ok(key, o):
        b, h = key
        n = int(P.prompt_lens[b])
        if n == 0:
            return 0
        codes_o, flags_o = o.encode(oracle.widen(P.K[b, h, :n]))
        fl = check_codes(pcodes[b, h, :n], codes_o, flags_o, f"prefill codes b={b} h={h}")
        if query:
            for g in range(G):
                qo, qf = o.encode(oracle.widen(Qp[b, h * G + g, :n]))
                fl += check_codes(qpcodes[b, h * G + g, :n], qo, qf, f"prefill query codes b={b} hq={h * G + g}")
        if chunked and Qp is not None:
            qo, qf = o.encode(oracle.widen(Qp[b, h * G:(h + 1) * G]))
            fl += check_codes(qpcodes[b, h * G:(h + 1) * G], qo, qf, f"observation codes b={b} h={h}")
        return fl

    flagged = sum(orc.map_heads(prefill_codes_ok).values())
    # replay the oracle's prefill with the GPU codes
    kept_o = orc.prefill(P.K, P.V, P.prompt_lens, policy, inj_codes=pcodes, Q=Qp, inj_qcodes=qpcodes,
                         chunk=cache.prefill_chunk or oracle.DEFAULT_CHUNK_TOKENS, reuse=reuse)
    if chunked:
        for (b, h) in sel:
            ko = kept_o[(b, h)]
            np.testing.assert_array_equal(kept[b, h, :len(ko)], ko, err_msg=f"kept chunks b={b} h={h}")
            assert (kept[b, h, len(ko):] == -1).all(), f"kept list tail b={b} h={h}"
        if stats is not None:
            stats["kept"] = kept
    log(f"  prefill codes ok ({flagged} flagged bits differ), {time.time()-t0:.1f}s")
    compare_state(cache, orc, sel, shape, "after prefill")
    log(f"  prefill state ok, {time.time()-t0:.1f}s")
    tworst = 0.0
    if tier:
        compare_tier(cache, orc, sel, shape, "after prefill")
        tworst = check_tiered(cache, orc, Dd.q[0], G, "after prefill")
        log(f"  prefill tier ok, tiered attention rel err {tworst:.2e}, {time.time()-t0:.1f}s")

    worst = 0.0
    dflagged = 0
    states_compared = 0
    for s in range(steps):
        q = hkv.to_device(Dd.q[s]); k = hkv.to_device(Dd.k[s]); v = hkv.to_device(Dd.v[s])
        out, ev = cache.decode_step(q, k, v)
        qc, kc = cache.last_codes()
        out = hkv.to_numpy(out); ev = hkv.to_numpy(ev)
        qc = words_u32(qc); kc = words_u32(kc)
        res = orc.decode_step(Dd.q[s], Dd.k[s], Dd.v[s], inj_qcodes=qc, inj_kcodes=kc)
        for (b, h), r in res.items():
            qo, qf = orc.heads[(b, h)].encode(oracle.widen(Dd.q[s, b, h * G:(h + 1) * G]))
            ko, kf = orc.heads[(b, h)].encode(oracle.widen(Dd.k[s, b, h]))
            dflagged += check_codes(qc[b, h * G:(h + 1) * G], qo, qf, f"step {s} qcodes b={b} h={h}")
            dflagged += check_codes(kc[b, h], ko, kf, f"step {s} kcode b={b} h={h}")
            assert ev[b, h] == r["evicted"], f"step {s} b={b} h={h}: evicted {ev[b, h]} != {r['evicted']}"
            err = rel_err_rows(out[b, h * G:(h + 1) * G].astype(np.float64), r["out"])
            worst = max(worst, err)
            assert err <= ATTN_TOL, f"step {s} b={b} h={h}: attention rel err {err:.3e} > {ATTN_TOL}"
        if check_every and (s + 1) % check_every == 0 or s == steps - 1:
            compare_state(cache, orc, sel, shape, f"after step {s}")
            states_compared += 1
            if tier:
                compare_tier(cache, orc, sel, shape, f"after step {s}")
        if tier:
            tworst = max(tworst, check_tiered(cache, orc, Dd.q[s], G, f"step {s}"))
    log(f"  {steps} decode steps ok, worst attention rel err {worst:.2e}"
        + (f", tiered {tworst:.2e}" if tier else "") + f", {time.time()-t0:.1f}s")
    if stats is not None:
        stats.update(worst=worst, flagged=flagged, tiered_worst=tworst)
    logp = os.environ.get("HKV_PARITY_LOG")
    if logp:
        rec = {"case": label or shape.name, "workload": shape.name, "schedule": "split" if schedule else "fused",
               "policy": policy, "value_bits": value_bits, "tier": tier, "chunk": cache.chunk,
               "heads": len(sel), "decode_steps": steps, "states_compared": states_compared + 1,
               "worst_attention_rel_err": worst, "tiered_worst": tworst,
               "prefill_flagged_bits_differing": flagged, "decode_flagged_bits_differing": dflagged,
               "seconds": round(time.time() - t0, 1)}
        with open(logp, "a") as fh:
            fh.write(json.dumps(rec) + "\n")
    cache.close()
    return worst


def check_tiered(cache, orc, q, G: int, when: str) -> float:
    """Attention over cache and host tier against the oracle's; returns the worst row error."""
    from lsh_eviction_amd import hkv
    out = hkv.to_numpy(cache.attend_tiered(hkv.to_device(q)))
    worst = 0.0
    for (b, h), ref in orc.attend_tiered(q).items():
        err = rel_err_rows(out[b, h * G:(h + 1) * G].astype(np.float64), ref)
        worst = max(worst, err)
        assert err <= ATTN_TOL, f"{when} b={b} h={h}: tiered attention rel err {err:.3e} > {ATTN_TOL}"
    return worst


def compare_tier(cache, orc, sel, shape: Shape, when: str):
    """Tier counts, token positions and rows, bit for bit."""
    import torch
    from lsh_eviction_amd import hkv
    cnt = hkv.to_numpy(cache.tier_counts())
    torch.cuda.synchronize()
    tk, tv, tt = cache.tier["K"], cache.tier["V"], cache.tier["tok"].numpy()
    for (b, h) in sel:
        o = orc.heads[(b, h)].tier()
        assert cnt[b, h] == o["count"], f"{when} b={b} h={h}: tier count {cnt[b, h]} != {o['count']}"
        m = len(o["tok"])
        np.testing.assert_array_equal(tt[b, h, :m], o["tok"].astype(np.int32),
                                      err_msg=f"{when} b={b} h={h}: tier token positions")
        assert kv_bytes_equal(hkv.to_numpy(tk[b, h, :m]), o["K"], shape.kv_dtype), f"{when} b={b} h={h}: tier K"
        assert kv_bytes_equal(hkv.to_numpy(tv[b, h, :m]), o["V"], shape.kv_dtype), f"{when} b={b} h={h}: tier V"


def unpack_int4(packed: np.ndarray) -> np.ndarray:
    """Two signed 4-bit codes a byte (element 2i in the low half of byte i) ->
    one int8 per element."""
    p = packed.astype(np.uint8)
    lo = ((p & 0x0F).astype(np.int8) << 4) >> 4
    hi = (p.astype(np.int8) >> 4)
    out = np.empty(p.shape[:-1] + (2 * p.shape[-1],), np.int8)
    out[..., 0::2] = lo
    out[..., 1::2] = hi
    return out


def compare_state(cache, orc, sel, shape: Shape, when: str):
    from lsh_eviction_amd import hkv
    st = cache.get_state()
    tok = hkv.to_numpy(st["tok"])
    codes = words_u32(st["codes"])
    hs = hkv.to_numpy(st["state"])
    K = hkv.to_numpy(st["K"])
    vbits = getattr(cache, "value_bits", 0)
    vq = vbits != 0
    if vq:
        Vq = st["Vq"].cpu().numpy(); Vs = st["Vs"].cpu().numpy()
        if vbits == 4:
            Vq = unpack_int4(Vq)
    else:
        V = hkv.to_numpy(st["V"])
    for (b, h) in sel:
        o = orc.heads[(b, h)].state()
        S = orc.heads[(b, h)].budget
        assert hs[b, h, 0] == o["n"] and hs[b, h, 1] == o["t"], \
            f"{when} b={b} h={h}: head state {hs[b, h].tolist()} != ({o['n']}, {o['t']})"
        np.testing.assert_array_equal(tok[b, h, :S], o["tok"].astype(np.int32),
                                      err_msg=f"{when} b={b} h={h}: slot->token map")
        n = o["n"]
        np.testing.assert_array_equal(codes[b, h, :n], o["code"][:n],
                                      err_msg=f"{when} b={b} h={h}: code table")
        assert kv_bytes_equal(K[b, h, :n], o["K"][:n], shape.kv_dtype), f"{when} b={b} h={h}: K rows"
        if vq:
            oq, osc = orc.heads[(b, h)].value_codes()
            np.testing.assert_array_equal(Vq[b, h, :n], oq[:n], err_msg=f"{when} b={b} h={h}: value codes")
            np.testing.assert_array_equal(Vs[b, h, :n].view(np.uint32), osc[:n].view(np.uint32),
                                          err_msg=f"{when} b={b} h={h}: value scales")
        else:
            assert kv_bytes_equal(V[b, h, :n], o["V"][:n], shape.kv_dtype), f"{when} b={b} h={h}: V rows"
