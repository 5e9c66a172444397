"""Checks that pin the decode-update oracle (``oracle.decode``) and the
horizon of ``oracle.selector.select_pages`` to facts fixed outside them.

Each ``check_*`` takes a namespace with the two oracle modules (``decode``,
``selector``) and raises AssertionError on a disagreement with the
hand-derived values in ``tests/golden/decode_worked.json``, a token-by-token
gather of the cache after a write, the untouched rest of the pool, running
maxima / minima of the keys the check itself wrote, or the counting
properties of the split rule.  ``test_decode_oracle.py`` runs them against
the real oracle and against planted mistakes.
"""

from __future__ import annotations

import json
import os

import numpy as np

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "decode_worked.json")


def _golden():
    with open(GOLDEN) as f:
        return json.load(f)


def _random_cache(rng, S=3, Hkv=2, P=8, D=5, lens=(13, 24, 1), max_pages=4, extra=3):
    NP = S * max_pages + extra
    k = (rng.integers(-8, 9, size=(NP, Hkv, P, D)) / 2.0).astype(np.float32)
    v = (rng.integers(-8, 9, size=(NP, Hkv, P, D)) / 2.0).astype(np.float32)
    table = rng.permutation(NP)[: S * max_pages].reshape(S, max_pages).astype(np.int32)
    return k, v, table, np.asarray(lens, dtype=np.int32)


def _row(pool, table, t, P, kvh):
    return pool[table[t // P], kvh, t % P]


def check_golden_append(ns):
    g = _golden()["append"]
    P, Hkv, D, lg = g["P"], g["Hkv"], g["D"], g["logical"]
    table = np.asarray(g["block_table"], dtype=np.int32)
    k = np.zeros((g["NP"], Hkv, P, D), dtype=np.float32)
    for t, key in enumerate(g["keys_by_token"]):
        k[table[0, t // P], 0, t % P] = key
    v = np.zeros_like(k)
    kn = np.asarray(g["k_new"], dtype=np.float32)[None, None]
    vn = np.asarray(g["v_new"], dtype=np.float32)[None, None]
    lens = np.array([g["L"]], dtype=np.int32)
    k2, v2 = ns.decode.append_kv(k, v, table, lens, kn, vn)
    assert k2[g["written_phys"], 0, g["written_slot"]].tolist() == g["k_new"]
    assert v2[g["written_phys"], 0, g["written_slot"]].tolist() == g["v_new"]
    changed = np.argwhere(np.any(k2 != k, axis=-1))
    assert changed.tolist() == [[g["written_phys"], 0, g["written_slot"]]], changed.tolist()
    for which, pool, L in (("stats_before", k, g["L"]), ("stats_after", k2, g["L"] + 1)):
        want = g[which]
        st = ns.selector.page_stats(pool, table, np.array([L], dtype=np.int32), logical=lg)
        assert st[want["phys"], 0, want["sub"], 0].tolist() == want["kmax"], which
        assert st[want["phys"], 0, want["sub"], 1].tolist() == want["kmin"], which
    full = np.array([g["full_L"]], dtype=np.int32)
    k3, v3 = ns.decode.append_kv(k, v, table, full, kn, vn)
    assert np.array_equal(k3, k) and np.array_equal(v3, v), "a full cache must not change"


def check_append_gather(ns):
    """After the write, token L of every request reads back the new rows
    through the (shuffled) table, tokens below L read back what they held,
    and no other slot of the pool changed."""
    rng = np.random.default_rng(21)
    k, v, table, lens = _random_cache(rng, lens=(13, 32, 0))  # request 1 is full (4 pages x 8)
    S, Hkv, D = 3, k.shape[1], k.shape[3]
    P = k.shape[2]
    kn = (rng.integers(-8, 9, size=(S, Hkv, D)) / 2.0 + 100).astype(np.float32)
    vn = (rng.integers(-8, 9, size=(S, Hkv, D)) / 2.0 - 100).astype(np.float32)
    k2, v2 = ns.decode.append_kv(k, v, table, lens, kn, vn)
    touched = np.zeros(k.shape[:3], dtype=bool)
    for s in range(S):
        L = int(lens[s])
        for kvh in range(Hkv):
            for t in range(min(L, table.shape[1] * P)):
                assert np.array_equal(_row(k2, table[s], t, P, kvh), _row(k, table[s], t, P, kvh))
            if L < table.shape[1] * P:
                assert np.array_equal(_row(k2, table[s], L, P, kvh), kn[s, kvh]), (s, kvh)
                assert np.array_equal(_row(v2, table[s], L, P, kvh), vn[s, kvh]), (s, kvh)
                touched[table[s, L // P], kvh, L % P] = True
    assert np.array_equal(k2[~touched], k[~touched]) and np.array_equal(v2[~touched], v[~touched])
    assert touched.sum() == 2 * Hkv  # requests 0 and 2 wrote, request 1 was full


def check_append_running_stats(ns):
    """Ten appends across logical- and physical-page boundaries: after each,
    the statistics of the logical page holding the newest token equal the
    running max / min of the keys written into it so far."""
    rng = np.random.default_rng(22)
    P, lg, D, Hkv = 8, 4, 3, 2
    k, v, table, lens = _random_cache(rng, S=1, Hkv=Hkv, P=P, D=D, lens=(13,), max_pages=4)
    written = {}
    for step in range(10):
        kn = (rng.integers(-8, 9, size=(1, Hkv, D)) / 2.0).astype(np.float32)
        t = int(lens[0])
        k, v = ns.decode.append_kv(k, v, table, lens, kn, kn)
        lens = lens + 1
        start = (t // lg) * lg
        for u in range(start, t + 1):
            written.setdefault(u, _row(k, table[0], u, P, 0).copy())
        st = ns.selector.page_stats(k, table, lens, logical=lg)
        rows = np.stack([written[u] for u in range(start, t + 1)])
        phys, sub = table[0, t // P], (t % P) // lg
        assert np.array_equal(st[phys, 0, sub, 0], rows.max(0)), step
        assert np.array_equal(st[phys, 0, sub, 1], rows.min(0)), step
        assert np.array_equal(written[t], kn[0, 0]), step


def check_golden_bounds(ns):
    for case in _golden()["bounds"]:
        mask = np.asarray(case["mask"], dtype=np.uint8)[None, None]
        got = ns.decode.kept_page_bounds(mask, np.array([case["L"]]), case["P"], case["b"],
                                         horizon=case["horizon"])
        assert got[0, 0].tolist() == case["bounds"], (case, got[0, 0].tolist())


def check_bounds_properties(ns):
    """Monotone, from 0 to E = min(L + horizon, capacity); split j holds
    floor((j+1)K/b) - floor(jK/b) kept pages; no mask = all pages kept."""
    rng = np.random.default_rng(23)
    P, max_pages = 16, 37
    for trial in range(30):
        S, Hkv = 2, 3
        lens = rng.integers(0, max_pages * P + 1, size=S)
        mask = (rng.random((S, Hkv, max_pages)) < rng.uniform(0, 1)).astype(np.uint8)
        b = int(rng.choice([1, 2, 3, 5, 16, 40]))
        hz = int(rng.choice([0, 1, 15, 16, 100]))
        got = ns.decode.kept_page_bounds(mask, lens, P, b, horizon=hz)
        for s in range(S):
            E = min(int(lens[s]) + hz, max_pages * P)
            n = -(-E // P)
            for h in range(Hkv):
                bd = got[s, h]
                assert bd[0] == 0 and bd[b] == E and np.all(np.diff(bd) >= 0), (trial, bd)
                kept = [lp for lp in range(n) if mask[s, h, lp]]
                K = len(kept)
                for j in range(b):
                    cnt = sum(1 for lp in kept if bd[j] <= lp * P < bd[j + 1])
                    assert cnt == (j + 1) * K // b - j * K // b, (trial, s, h, j, cnt)
        ones = np.ones_like(mask)
        assert np.array_equal(ns.decode.kept_page_bounds(None, lens, P, b, horizon=hz, Hkv=Hkv,
                                                         max_pages=max_pages),
                              ns.decode.kept_page_bounds(ones, lens, P, b, horizon=hz))


def check_golden_horizon(ns):
    g = _golden()["horizon"]
    sc = np.asarray([float(x) for x in g["scores"]])[None, None]
    lens = np.array([g["L"]], dtype=np.int32)
    for case in g["cases"]:
        m = ns.selector.select_pages(sc, lens, g["P"], g["budget"], select_heads=[case["select"]],
                                     horizon=case["horizon"])
        assert m[0, 0].tolist() == case["mask"], (case, m[0, 0].tolist())


def check_horizon_properties(ns):
    """A horizon changes only the pages from ceil(L/P) to ceil((L+h)/P),
    which become 1 for every head."""
    rng = np.random.default_rng(24)
    P, max_pages = 8, 20
    sc = rng.standard_normal((3, 2, max_pages))
    lens = np.array([0, 61, 160], dtype=np.int32)
    for hz in (0, 1, 3, 4, 16, 1000):
        for flags in (None, [1, 0]):
            base = ns.selector.select_pages(sc, lens, P, 4, 1, 1, select_heads=flags)
            got = ns.selector.select_pages(sc, lens, P, 4, 1, 1, select_heads=flags, horizon=hz)
            for s in range(3):
                lo = -(-int(lens[s]) // P)
                hi = min(-(-(int(lens[s]) + hz) // P), max_pages)
                assert np.all(got[s, :, lo:hi] == 1), (hz, s)
                keep = np.ones(max_pages, dtype=bool)
                keep[lo:hi] = False
                assert np.array_equal(got[s][:, keep], base[s][:, keep]), (hz, s)


ALL_CHECKS = [
    check_golden_append,
    check_append_gather,
    check_append_running_stats,
    check_golden_bounds,
    check_bounds_properties,
    check_golden_horizon,
    check_horizon_properties,
]
