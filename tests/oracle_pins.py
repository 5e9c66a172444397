"""Checks that pin the fp64 oracle to facts fixed outside it.

Each ``check_*`` function raises AssertionError when the oracle disagrees with
a closed form, a 50-digit decimal brute force, an identity of the
MicroAttention equations, or the hand-derived worked example under
``tests/golden``.  ``test_oracle.py`` runs them against the real oracle and
``test_oracle_mutants.py`` runs them against planted mistakes, which each must
be caught by at least one check.

Equations referred to (Infinite-LLM page, section 方法细节):
  standard attention  m_g = max_i s_i,  out = sum_i exp(s_i - m_g) V_i / sum_j exp(s_j - m_g)
  MicroAttention      m_j = max s_i,  e_j = sum exp(s_i - m_j),  MA_j = sum exp(s_i - m_j) V_i
  aggregation         m_g = max m_j,  e_g = sum e_j exp(m_j - m_g),  out = sum MA_j exp(m_j - m_g) / e_g
"""

from __future__ import annotations

import json
import math
import os
from decimal import Decimal, getcontext
from fractions import Fraction

import numpy as np

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


# ---------------------------------------------------------------------------
# helpers that build inputs without using the oracle
# ---------------------------------------------------------------------------

def paged_from_contiguous(K, V, page_size, rng, extra_pages=2, poison=np.nan):
    """Scatter contiguous per-head rows K, V [Hkv, L, D] into a paged pool
    [NP, Hkv, P, D] under a random block table, with every unused slot and
    every unreferenced page poisoned.  Plain loops, no oracle code."""
    Hkv, L, D = K.shape
    n_log = -(-L // page_size)
    NP = n_log + extra_pages
    perm = rng.permutation(NP)[:n_log]
    kp = np.full((NP, Hkv, page_size, D), poison, dtype=np.float64)
    vp = np.full((NP, Hkv, page_size, D), poison, dtype=np.float64)
    for t in range(L):
        for h in range(Hkv):
            kp[perm[t // page_size], h, t % page_size, :] = K[h, t]
            vp[perm[t // page_size], h, t % page_size, :] = V[h, t]
    return kp, vp, perm.astype(np.int32)


def decimal_attention(q, K, V, scale):
    """exp(s_i) / sum_j exp(s_j) weighted sum, at 50 digits, with no max
    subtraction: the textbook softmax evaluated exactly enough that its only
    error is the final conversion to float."""
    getcontext().prec = 50
    sc = Decimal(scale) if not isinstance(scale, Decimal) else scale
    s = []
    for k in K:
        acc = Decimal(0)
        for qd, kd in zip(q, k):
            acc += Decimal(float(qd)) * Decimal(float(kd))
        s.append(acc * sc)
    ex = [x.exp() for x in s]
    z = sum(ex, Decimal(0))
    D = len(V[0])
    return np.array([float(sum((ex[i] * Decimal(float(V[i][d])) for i in range(len(V))), Decimal(0)) / z)
                     for d in range(D)])


def _frac_or_log(text):
    text = text.strip()
    if text == "-inf":
        return -math.inf
    if text.startswith("ln"):
        return math.log(float(Fraction(text[2:])))
    return float(Fraction(text))


# ---------------------------------------------------------------------------
# checks
# ---------------------------------------------------------------------------

def check_bf16_widen(o):
    """Known bf16 bit patterns (IEEE binary32 upper halves)."""
    bits = np.array([0x3F80, 0xC000, 0x3F81, 0x0000, 0x8000, 0x4049, 0x7F7F], dtype=np.uint16)
    want = np.array([1.0, -2.0, 1.0 + 2.0 ** -7, 0.0, -0.0, 3.140625, 3.3895313892515355e38])
    got = o.to_f64(bits)
    assert np.array_equal(got, want), (got, want)
    assert np.signbit(got[4])


def check_closed_form_scores(o):
    """D = 64 so the default scale is exactly 1/8.  q = 8 e_0 and k = e_0 give
    the score 1 (reported as m_j of a one-token split).  With k_0 = ln(3) e_0
    and k_1 = 0 the scores are ln 3 and 0, so the weights are 3/4 and 1/4."""
    D = 64
    q = np.zeros(D)
    q[0] = 8.0
    k = np.zeros((1, D))
    k[0, 0] = 1.0
    v = np.arange(D, dtype=np.float64)[None, :]
    _, m, e = o.micro_tokens(q, k, v, o.default_scale(D))
    assert m == 1.0 and e == 1.0, (m, e)
    K = np.zeros((2, D))
    K[0, 0] = math.log(3.0)
    rng = np.random.default_rng(11)
    V = rng.standard_normal((2, D))
    out = o.attention_tokens(q, K, V, o.default_scale(D))
    want = 0.75 * V[0] + 0.25 * V[1]
    assert np.max(np.abs(out - want)) < 1e-14, np.max(np.abs(out - want))


def check_single_and_equal(o):
    """One token returns its value row exactly; all-equal scores (q = 0) give
    the mean of V, e_j = number of tokens and m_j = 0."""
    rng = np.random.default_rng(5)
    D = 16
    q = rng.standard_normal(D)
    K = rng.standard_normal((1, D))
    V = rng.standard_normal((1, D))
    assert np.array_equal(o.attention_tokens(q, K, V, 0.25), V[0])
    n = 37
    K = rng.standard_normal((n, D))
    V = rng.standard_normal((n, D))
    out = o.attention_tokens(np.zeros(D), K, V, 0.25)
    assert np.max(np.abs(out - V.mean(axis=0))) < 1e-14
    MA, m, e = o.micro_tokens(np.zeros(D), K, V, 0.25)
    assert m == 0.0 and e == float(n), (m, e)
    assert np.max(np.abs(MA - V.sum(axis=0))) < 1e-12


def check_shift_invariance(o):
    """Adding the same constant c to every score leaves the output unchanged:
    k_i + c q / (scale |q|^2) raises each score by exactly c in real
    arithmetic."""
    rng = np.random.default_rng(7)
    D, n, scale = 8, 23, 0.35
    q = rng.standard_normal(D)
    K = rng.standard_normal((n, D))
    V = rng.standard_normal((n, D))
    base = o.attention_tokens(q, K, V, scale)
    for c in (-30.0, 3.0, 55.0):
        K2 = K + (c / (scale * float(q @ q))) * q[None, :]
        assert np.max(np.abs(o.attention_tokens(q, K2, V, scale) - base)) < 1e-12


def check_brute_force(o):
    """Paged oracle output against a 50-digit decimal softmax over the
    contiguous rows, on tiny problems with random block tables, a ragged last
    page, GQA grouping and NaN poison in every slot that must not be read."""
    rng = np.random.default_rng(2024)
    for trial in range(6):
        Hkv = 1 + trial % 2
        G = (1, 2, 3)[trial % 3]
        Hq = Hkv * G
        D = (2, 4, 8)[trial % 3]
        P = (2, 3, 4)[trial % 3]
        S = 2
        lens = [int(x) for x in rng.integers(1, 10, size=S)]
        scale = 1.0 / math.sqrt(D)
        q = rng.standard_normal((S, Hq, D))
        max_pages = max(-(-L // P) for L in lens)
        NPs, kps, vps, tabs, conts = [], [], [], [], []
        for s in range(S):
            K = rng.standard_normal((Hkv, lens[s], D)) * 1.5
            V = rng.standard_normal((Hkv, lens[s], D))
            kp, vp, perm = paged_from_contiguous(K, V, P, rng)
            NPs.append(kp.shape[0])
            kps.append(kp)
            vps.append(vp)
            tabs.append(perm)
            conts.append((K, V))
        # concatenate per-request pools into one pool; offset each table
        offs = np.cumsum([0] + NPs[:-1])
        k_pool = np.concatenate(kps)
        v_pool = np.concatenate(vps)
        table = np.zeros((S, max_pages), dtype=np.int32)
        for s in range(S):
            table[s, :len(tabs[s])] = tabs[s] + offs[s]
        out = o.attention(q, k_pool, v_pool, table, np.array(lens), scale=scale)
        for s in range(S):
            K, V = conts[s]
            for h in range(Hq):
                kvh = h // G
                want = decimal_attention(q[s, h], K[kvh], V[kvh], Decimal(1) / Decimal(D).sqrt())
                err = np.max(np.abs(out[s, h] - want))
                assert err < 1e-13, (trial, s, h, err)


def check_gqa_probe(o):
    """Hq = 8 query heads over Hkv = 2 KV heads with V constant per KV head
    (value = KV head id): query heads 0..3 read KV head 0 and 4..7 read KV
    head 1 (consecutive grouping), so the outputs are exactly those ids."""
    rng = np.random.default_rng(3)
    S, Hq, Hkv, D, P, L = 1, 8, 2, 4, 4, 10
    q = rng.standard_normal((S, Hq, D))
    NP = 3
    k_pool = rng.standard_normal((NP, Hkv, P, D))
    v_pool = np.zeros((NP, Hkv, P, D))
    v_pool[:, 1] = 1.0
    table = np.array([[2, 0, 1]], dtype=np.int32)
    out = o.attention(q, k_pool, v_pool, table, np.array([L]))
    want = np.array([0, 0, 0, 0, 1, 1, 1, 1], dtype=np.float64)
    assert np.max(np.abs(out[0, :, :] - want[:, None])) < 1e-14, out[0, :, 0]


def _random_problem(rng, S=2, Hq=4, Hkv=2, D=8, P=4, lens=(13, 21), extra=3):
    max_pages = max(-(-L // P) for L in lens)
    NP = S * max_pages + extra
    q = rng.standard_normal((S, Hq, D))
    k_pool = rng.standard_normal((NP, Hkv, P, D)) * 1.3
    v_pool = rng.standard_normal((NP, Hkv, P, D))
    perm = rng.permutation(NP)
    table = perm[:S * max_pages].reshape(S, max_pages).astype(np.int32)
    return q, k_pool, v_pool, table, np.array(lens)


def _random_bounds(rng, L, b):
    cuts = np.sort(rng.integers(0, L + 1, size=b - 1))
    return np.concatenate([[0], cuts, [L]]).astype(np.int32)


def check_split_identity(o):
    """merge(MicroAttention over any splits) equals unsplit attention; b = 1
    gives MA_1 / e_1 = out and m_1 = the largest score; empty and mid-page
    splits included."""
    rng = np.random.default_rng(99)
    q, kp, vp, table, lens = _random_problem(rng)
    S, Hq = q.shape[:2]
    ref = o.attention(q, kp, vp, table, lens)
    for b in (1, 2, 5, 9):
        sb = np.stack([_random_bounds(rng, int(L), b) for L in lens])[:, None, :]
        MA, m, e = o.micro_attention(q, kp, vp, table, lens, sb)
        out = o.merge(MA, m, e)
        assert np.max(np.abs(out - ref)) < 1e-12, b
        if b == 1:
            assert np.max(np.abs(MA[:, :, 0] / e[:, :, 0, None] - ref)) < 1e-12
            for s in range(S):
                for h in range(Hq):
                    kvh = h // (Hq // kp.shape[1])
                    P = kp.shape[2]
                    rows = [kp[table[s, t // P], kvh, t % P] for t in range(int(lens[s]))]
                    best = max(float(np.dot(q[s, h], r)) for r in rows) / math.sqrt(q.shape[2])
                    assert abs(m[s, h, 0] - best) < 1e-12


def check_split_order(o):
    """Permuting the partials before merging changes nothing."""
    rng = np.random.default_rng(1234)
    q, kp, vp, table, lens = _random_problem(rng)
    sb = np.stack([_random_bounds(rng, int(L), 6) for L in lens])[:, None, :]
    MA, m, e = o.micro_attention(q, kp, vp, table, lens, sb)
    ref = o.merge(MA, m, e)
    for _ in range(3):
        p = rng.permutation(6)
        assert np.max(np.abs(o.merge(MA[:, :, p], m[:, :, p], e[:, :, p]) - ref)) < 1e-12


def check_per_head_bounds(o):
    """Per-KV-head split bounds: each KV head's own splits still merge to
    unsplit attention."""
    rng = np.random.default_rng(77)
    q, kp, vp, table, lens = _random_problem(rng, Hq=6, Hkv=3)
    ref = o.attention(q, kp, vp, table, lens)
    sb = np.stack([np.stack([_random_bounds(rng, int(L), 4) for _ in range(3)]) for L in lens])
    MA, m, e = o.micro_attention(q, kp, vp, table, lens, sb)
    assert np.max(np.abs(o.merge(MA, m, e) - ref)) < 1e-12


def check_associativity(o):
    """A merge of merged groups of partials (hierarchical aggregation) equals
    the flat merge; separate token ranges computed independently and
    concatenated merge to the unsplit result."""
    rng = np.random.default_rng(31)
    q, kp, vp, table, lens = _random_problem(rng)
    sb = np.stack([_random_bounds(rng, int(L), 8) for L in lens])[:, None, :]
    MA, m, e = o.micro_attention(q, kp, vp, table, lens, sb)
    flat = o.merge(MA, m, e)
    a = o.merge_partials(MA[:, :, :3], m[:, :, :3], e[:, :, :3])
    b = o.merge_partials(MA[:, :, 3:], m[:, :, 3:], e[:, :, 3:])
    MA2 = np.stack([a[0], b[0]], axis=2)
    m2 = np.stack([a[1], b[1]], axis=2)
    e2 = np.stack([a[2], b[2]], axis=2)
    assert np.max(np.abs(o.merge(MA2, m2, e2) - flat)) < 1e-12
    # two "remote" calls over disjoint token ranges, partials concatenated
    cut = [int(L) // 3 for L in lens]
    sb1 = np.array([[[0, c, c]] for c in cut], dtype=np.int32)
    sb2 = np.array([[[c, (c + int(L)) // 2, int(L)]] for c, L in zip(cut, lens)], dtype=np.int32)
    p1 = o.micro_attention(q, kp, vp, table, lens, sb1)
    p2 = o.micro_attention(q, kp, vp, table, lens, sb2)
    cat = [np.concatenate([x, y], axis=2) for x, y in zip(p1, p2)]
    ref = o.attention(q, kp, vp, table, lens)
    assert np.max(np.abs(o.merge(*cat) - ref)) < 1e-12


def check_fold_is_union_partial(o):
    """Folding the partials of any splits (empty ones included) gives the
    MicroAttention triple of the whole token range computed in one piece:
    the same maximum, exp-sum and unnormalised sum, not only the same
    attention after division."""
    rng = np.random.default_rng(57)
    q, kp, vp, table, lens = _random_problem(rng)
    whole = np.array([[[0, int(L)]] for L in lens], dtype=np.int32)
    wMA, wm, we = o.micro_attention(q, kp, vp, table, lens, whole)
    for b in (1, 3, 8):
        sb = np.stack([_random_bounds(rng, int(L), b) for L in lens])[:, None, :]
        if b > 1:
            sb[:, :, 1] = 0  # the first split is empty
        MA, m, e = o.micro_attention(q, kp, vp, table, lens, sb)
        fMA, fm, fe = o.merge_partials(MA, m, e)
        assert np.max(np.abs(fm - wm[:, :, 0])) < 1e-12, b  # scores of subsets: fp64 rounding
        assert np.max(np.abs(fe / we[:, :, 0] - 1)) < 1e-12, b
        assert np.max(np.abs(fMA - wMA[:, :, 0]) / we[:, :, 0, None]) < 1e-12, b
    # all partials empty: the empty triple
    z = o.merge_partials(np.zeros((1, 1, 3, 2)), np.full((1, 1, 3), -np.inf), np.zeros((1, 1, 3)))
    assert np.all(z[0] == 0) and np.isneginf(z[1]).all() and np.all(z[2] == 0)


def check_mask_compaction(o):
    """Masked attention equals dense attention over a new contiguous cache that
    holds only the kept pages' tokens, copied out by plain loops."""
    rng = np.random.default_rng(8)
    S, Hq, Hkv, D, P = 2, 4, 2, 8, 4
    lens = [19, 26]
    q, kp, vp, table, lens_a = _random_problem(rng, S, Hq, Hkv, D, P, lens)
    max_pages = table.shape[1]
    mask = (rng.random((S, Hkv, max_pages)) < 0.5).astype(np.uint8)
    mask[:, :, 0] = 1
    got = o.attention(q, kp, vp, table, lens_a, block_mask=mask)
    for s in range(S):
        for kvh in range(Hkv):
            Kc, Vc = [], []
            for t in range(lens[s]):
                if mask[s, kvh, t // P]:
                    Kc.append(kp[table[s, t // P], kvh, t % P])
                    Vc.append(vp[table[s, t // P], kvh, t % P])
            for g in range(Hq // Hkv):
                h = kvh * (Hq // Hkv) + g
                want = decimal_attention(q[s, h], Kc, Vc, Decimal(1) / Decimal(D).sqrt())
                assert np.max(np.abs(got[s, h] - want)) < 1e-13, (s, h)
    # fully masked request: output 0, every split empty
    mask0 = np.zeros_like(mask)
    out0 = o.attention(q, kp, vp, table, lens_a, block_mask=mask0)
    assert np.array_equal(out0, np.zeros_like(out0))
    sb = np.array([[[0, 5, int(L)]] for L in lens], dtype=np.int32)
    MA, m, e = o.micro_attention(q, kp, vp, table, lens_a, sb, block_mask=mask0)
    assert np.all(np.isneginf(m)) and np.all(e == 0) and np.all(MA == 0)
    assert np.array_equal(o.merge(MA, m, e), np.zeros((S, Hq, D)))


def check_bounds_clamp(o):
    """A split that starts at or past L_s is empty: (0, -inf, 0)."""
    rng = np.random.default_rng(4)
    q, kp, vp, table, lens = _random_problem(rng, lens=(9, 12))
    sb = np.array([[[0, int(L), int(L) + 4]] for L in lens], dtype=np.int32)
    MA, m, e = o.micro_attention(q, kp, vp, table, lens, sb)
    assert np.all(np.isneginf(m[:, :, 1])) and np.all(e[:, :, 1] == 0) and np.all(MA[:, :, 1] == 0)
    assert np.max(np.abs(o.merge(MA, m, e) - o.attention(q, kp, vp, table, lens))) < 1e-12


def check_golden_worked_example(o):
    """The hand-derived two-split example in tests/golden (dense and masked)."""
    with open(os.path.join(GOLDEN, "worked_two_split.json")) as f:
        g = json.load(f)
    P = g["page_size"]
    L = g["seq_len"]
    D = 2
    NP = len(g["block_table"])
    kp = np.full((NP, 1, P, D), np.nan)
    vp = np.full((NP, 1, P, D), np.nan)
    for t in range(L):
        page = g["block_table"][t // P]
        kp[page, 0, t % P] = [math.log(g["key_exp_scores"][t]), 0.0]
        vp[page, 0, t % P] = g["values"][t]
    q = np.array(g["q"], dtype=np.float64)[None, None, :]
    table = np.array([g["block_table"]], dtype=np.int32)
    lens = np.array([L])
    sb = np.array([[g["split_bounds"]]], dtype=np.int32)
    for key, mask in (("expected", None), ("masked", np.array([[g["masked"]["block_mask"]]], dtype=np.uint8))):
        exp = g[key]
        MA, m, e = o.micro_attention(q, kp, vp, table, lens, sb, block_mask=mask, scale=g["scale"])
        for j in range(2):
            want_m = _frac_or_log(exp["m"][j])
            if math.isinf(want_m):
                assert np.isneginf(m[0, 0, j])
            else:
                assert abs(m[0, 0, j] - want_m) < 1e-14
            assert abs(e[0, 0, j] - _frac_or_log(exp["e"][j])) < 1e-14
            assert np.max(np.abs(MA[0, 0, j] - [_frac_or_log(x) for x in exp["MA"][j]])) < 1e-14
        out = o.merge(MA, m, e)[0, 0]
        assert np.max(np.abs(out - [_frac_or_log(x) for x in exp["out"]])) < 1e-14
        out2 = o.attention(q, kp, vp, table, lens, block_mask=mask, scale=g["scale"])[0, 0]
        assert np.max(np.abs(out2 - [_frac_or_log(x) for x in exp["out"]])) < 1e-14


ALL_CHECKS = [
    check_bf16_widen,
    check_closed_form_scores,
    check_single_and_equal,
    check_shift_invariance,
    check_brute_force,
    check_gqa_probe,
    check_split_identity,
    check_split_order,
    check_per_head_bounds,
    check_associativity,
    check_fold_is_union_partial,
    check_mask_compaction,
    check_bounds_clamp,
    check_golden_worked_example,
]
