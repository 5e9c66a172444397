"""Checks that pin the page-selection oracle (``oracle.selector``) to facts
fixed outside it.

Each ``check_*`` function takes the oracle module and raises AssertionError
when it disagrees with a brute force over tokens, the upper-bound property
of the statistics, a case that reduces to plain dot products or to a library
sort, or the hand-derived worked example under ``tests/golden``.
``test_selector_oracle.py`` runs them against the real oracle and against
planted mistakes, each of which must be caught by at least one check.

Definitions referred to (LServe blog page, sections 2.2.2 and 3.1.2): per
logical page the per-dimension maximum and minimum of its keys; a physical
page's score is the maximum over its logical pages; the top-K physical pages
are kept.
"""

from __future__ import annotations

import json
import os

import numpy as np

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


# ---------------------------------------------------------------------------
# inputs built without the oracle
# ---------------------------------------------------------------------------

def _golden():
    with open(os.path.join(GOLDEN, "selector_worked.json")) as f:
        return json.load(f)


def _golden_pool(g):
    sh = g["shape"]
    pool = np.zeros((sh["NP"], sh["Hkv"], sh["P"], sh["D"]), dtype=np.float32)
    table = np.asarray(g["block_table"], dtype=np.int32)
    for t, k in enumerate(g["keys_by_token"]):
        pool[table[0, t // sh["P"]], 0, t % sh["P"]] = k
    pool[table[0, 1], 0, 3] = g["poison_slot_7"]
    pool[1, 0] = np.asarray(g["unreferenced_page_1_rows"])
    q = np.asarray(g["q"], dtype=np.float32)[None]  # [1, Hq, D]
    lens = np.array([sh["L"]], dtype=np.int32)
    return pool, table, lens, q


def _random_case(rng, S=2, Hq=4, Hkv=2, D=6, P=8, logical=4, lens=(29, 17), extra=3):
    """Random paged pool with a random table; values are small integers and
    halves, so every product and sum below is exact in float64."""
    max_pages = max(-(-L // P) for L in lens) + 1
    NP = S * max_pages + extra
    pool = (rng.integers(-8, 9, size=(NP, Hkv, P, D)) / 2.0).astype(np.float32)
    table = rng.permutation(NP)[: S * max_pages].reshape(S, max_pages).astype(np.int32)
    q = (rng.integers(-6, 7, size=(S, Hq, D)) / 2.0).astype(np.float32)
    return pool, table, np.asarray(lens, dtype=np.int32), q, P, logical


def _token_keys(pool, table, L, P, kvh, lp, sub, logical):
    """Keys of the tokens below L of logical page `sub` of page `lp`, read
    one by one."""
    rows = []
    for t in range(lp * P + sub * logical, lp * P + (sub + 1) * logical):
        if t < L:
            rows.append(pool[table[t // P], kvh, t % P].astype(np.float64))
    return rows


# ---------------------------------------------------------------------------
# checks
# ---------------------------------------------------------------------------

def check_golden_worked_example(o):
    g = _golden()
    sh = g["shape"]
    pool, table, lens, q = _golden_pool(g)
    st = o.page_stats(pool, table, lens, logical=sh["logical"])
    for name, want in g["stats"].items():
        if name == "phys1":
            assert np.all(st[1] == 0), "unreferenced page must have zero statistics"
            continue
        phys, sub = int(name[4]), int(name[-1])
        assert np.array_equal(st[phys, 0, sub, 0], want["kmax"]), (name, st[phys, 0, sub, 0])
        assert np.array_equal(st[phys, 0, sub, 1], want["kmin"]), (name, st[phys, 0, sub, 1])
    for qi, per in g["bounds"].items():
        qv = q[0, int(qi[1])].astype(np.float64)
        for name, want in per.items():
            phys, sub = int(name[4]), int(name[-1])
            got = o.logical_bound(qv, st[phys, 0, sub, 0], st[phys, 0, sub, 1])
            assert got == want, (qi, name, got, want)
    sc = o.page_scores(q, st, table, lens, sh["P"], logical=sh["logical"])
    want = [float(x) for x in g["page_scores"]]
    assert np.array_equal(sc[0, 0], want), (sc[0, 0], want)
    for case in g["selections"]:
        m = o.select_pages(sc, lens, sh["P"], case["budget"], case["keep_first"], case["keep_last"])
        assert m[0, 0].tolist() == case["mask"], (case, m[0, 0])
    ties = g["ties"]
    tsc = np.asarray(ties["scores"], dtype=np.float64)[None, None]
    tl = np.array([ties["L_pages"] * 16], dtype=np.int32)
    for case in ties["cases"]:
        m = o.select_pages(tsc, tl, 16, case["budget"])
        assert m[0, 0].tolist() == case["mask"], (case, m[0, 0])


def check_stats_brute_force(o):
    """Running max / min over the tokens, one token at a time."""
    rng = np.random.default_rng(11)
    pool, table, lens, q, P, lg = _random_case(rng)
    st = o.page_stats(pool, table, lens, logical=lg)
    Hkv, D = pool.shape[1], pool.shape[3]
    seen = np.zeros(pool.shape[0], dtype=bool)
    for s in range(len(lens)):
        L = int(lens[s])
        for lp in range(-(-L // P)):
            phys = table[s, lp]
            seen[phys] = True
            for sub in range(P // lg):
                for kvh in range(Hkv):
                    keys = _token_keys(pool, table[s], L, P, kvh, lp, sub, lg)
                    hi = [None] * D
                    lo = [None] * D
                    for k in keys:
                        for d in range(D):
                            hi[d] = k[d] if hi[d] is None or k[d] > hi[d] else hi[d]
                            lo[d] = k[d] if lo[d] is None or k[d] < lo[d] else lo[d]
                    if not keys:
                        hi = lo = [0.0] * D
                    assert st[phys, kvh, sub, 0].tolist() == hi, (s, lp, sub, kvh)
                    assert st[phys, kvh, sub, 1].tolist() == lo, (s, lp, sub, kvh)
    assert np.all(st[~seen] == 0), "pages no table references must stay zero"


def check_upper_bound(o):
    """The score bounds q . k for every key of the page and every head of the
    group, and is attained by some combination of the extreme values."""
    rng = np.random.default_rng(12)
    pool, table, lens, q, P, lg = _random_case(rng)
    st = o.page_stats(pool, table, lens, logical=lg)
    sc = o.page_scores(q, st, table, lens, P, logical=lg)
    S, Hq, D = q.shape
    Hkv = pool.shape[1]
    G = Hq // Hkv
    for s in range(S):
        L = int(lens[s])
        npg = -(-L // P)
        assert np.all(np.isneginf(sc[s, :, npg:])), "pages beyond L_s must score -inf"
        for kvh in range(Hkv):
            for lp in range(npg):
                best_dot = -np.inf
                for sub in range(P // lg):
                    for k in _token_keys(pool, table[s], L, P, kvh, lp, sub, lg):
                        for h in range(kvh * G, (kvh + 1) * G):
                            best_dot = max(best_dot, float(np.dot(q[s, h].astype(np.float64), k)))
                assert sc[s, kvh, lp] >= best_dot, (s, kvh, lp, sc[s, kvh, lp], best_dot)


def check_one_token_pages(o):
    """With one token per logical page the bound is the dot product itself,
    so a page's score is the largest q_h . k_t over its tokens and heads."""
    rng = np.random.default_rng(13)
    pool, table, lens, q, P, _ = _random_case(rng, P=4, lens=(11, 6))
    st = o.page_stats(pool, table, lens, logical=1)
    sc = o.page_scores(q, st, table, lens, P, logical=1)
    S, Hq, D = q.shape
    Hkv = pool.shape[1]
    G = Hq // Hkv
    for s in range(S):
        L = int(lens[s])
        for kvh in range(Hkv):
            for lp in range(-(-L // P)):
                dots = [float(np.dot(q[s, h].astype(np.float64), pool[table[s, t // P], kvh, t % P]))
                        for t in range(lp * P, min(L, (lp + 1) * P)) for h in range(kvh * G, (kvh + 1) * G)]
                assert sc[s, kvh, lp] == max(dots), (s, kvh, lp)


def check_sign_cases(o):
    """Non-negative q: the bound is q . kmax; non-positive q: q . kmin, with
    kmax / kmin taken by numpy over the page's keys."""
    rng = np.random.default_rng(14)
    keys = rng.integers(-8, 9, size=(5, 7)) / 2.0
    kmax, kmin = keys.max(0), keys.min(0)
    qp = np.abs(rng.integers(-6, 7, size=7)) / 2.0
    assert o.logical_bound(qp, kmax, kmin) == float(qp @ kmax)
    assert o.logical_bound(-qp, kmax, kmin) == float(-qp @ kmin)
    assert o.logical_bound(np.zeros(7), kmax, kmin) == 0.0


def check_table_permutation(o):
    """Renaming physical pages (pool and table together) permutes the
    statistics and leaves scores and masks unchanged."""
    rng = np.random.default_rng(15)
    pool, table, lens, q, P, lg = _random_case(rng)
    perm = rng.permutation(pool.shape[0])  # old page i -> new page perm[i]
    pool2 = np.empty_like(pool)
    pool2[perm] = pool
    table2 = perm[table].astype(np.int32)
    st = o.page_stats(pool, table, lens, logical=lg)
    st2 = o.page_stats(pool2, table2, lens, logical=lg)
    assert np.array_equal(st2[perm], st)
    sc = o.page_scores(q, st, table, lens, P, logical=lg)
    sc2 = o.page_scores(q, st2, table2, lens, P, logical=lg)
    assert np.array_equal(sc, sc2)
    m = o.select_pages(sc, lens, P, 2, 1, 1)
    m2 = o.select_pages(sc2, lens, P, 2, 1, 1)
    assert np.array_equal(m, m2)


def check_select_library_sort(o):
    """Distinct scores: the kept candidates are the top of numpy's sort."""
    rng = np.random.default_rng(16)
    S, Hkv, npg = 3, 2, 40
    sc = rng.permutation(S * Hkv * npg).reshape(S, Hkv, npg).astype(np.float64) - 50.0
    lens = np.full(S, npg * 16, dtype=np.int32)
    for budget, kf, kl in ((7, 0, 0), (5, 2, 3), (0, 1, 1), (40, 0, 0), (100, 3, 3)):
        m = o.select_pages(sc, lens, 16, budget, kf, kl)
        for s in range(S):
            for h in range(Hkv):
                cand = np.arange(kf, npg - kl)
                top = cand[np.argsort(-sc[s, h, cand], kind="stable")][:budget]
                want = np.zeros(npg, dtype=np.uint8)
                want[:kf] = 1
                want[npg - kl:] = 1 if kl else 0
                want[top] = 1
                assert np.array_equal(m[s, h], want), (budget, kf, kl, s, h)


def check_select_edges(o):
    """Short requests, forced pages covering everything, unselected heads,
    pages past L_s."""
    sc = np.arange(24, dtype=np.float64).reshape(1, 2, 12)[:, :, ::-1].copy()  # descending
    lens = np.array([5 * 16 + 3], dtype=np.int32)  # 6 pages
    m = o.select_pages(sc, lens, 16, 2, select_heads=[1, 0])
    assert m[0, 0].tolist() == [1, 1, 0, 0, 0, 0] + [0] * 6
    assert m[0, 1].tolist() == [1] * 6 + [0] * 6
    m = o.select_pages(sc, lens, 16, 0, keep_first=4, keep_last=4)
    assert m[0, 0].tolist() == [1] * 6 + [0] * 6
    m = o.select_pages(sc, np.array([0], dtype=np.int32), 16, 3, 1, 1)
    assert not m.any()


ALL_CHECKS = [
    check_golden_worked_example,
    check_stats_brute_force,
    check_upper_bound,
    check_one_token_pages,
    check_sign_cases,
    check_table_permutation,
    check_select_library_sort,
    check_select_edges,
]
