"""Plain fp64 CPU oracle for hierarchical page selection (LServe).

TEST INFRASTRUCTURE ONLY.  Only the test suite, ``__graft_entry__.smoke()`` and
the ``cpu_baseline`` leg of ``bench.py`` may import this module.  The product
path never imports, calls or links anything here, and this module imports
nothing from the product package.

Source: the LServe blog page ("LLM长序列服务优化：LServe的块稀疏注意力技术"),
section 2.2.2 (decode phase: a physical page holds several logical pages,
each logical page keeps per-dimension key statistics k_max / k_min, and the
important physical pages are chosen from the query's similarity) and section
3.1.2 (hierarchical selection: statistics per logical page, a score per
physical page as the maximum over its logical pages, then the top-K physical
pages are the only ones loaded for attention).

Readings where the page is silent or garbled (each is also listed with its
reason in the design notes):

* the score listing of section 3.1.2 contracts a D-vector query with 2D-wide
  statistics; it is read as the per-logical-page upper bound on q . k that
  the statistics give: sum_d max(q_d * kmax_d, q_d * kmin_d), which is >= q . k
  for every key k of the logical page (and equal to it for a one-token page);
* statistics cover only the tokens below L_s; a logical page with no such
  token has zero statistics and takes no part in its physical page's score;
* with grouped query heads the mask is shared by the group, so a physical
  page's score is the maximum over the group's query heads;
* the kept set is the forced pages (the first ``keep_first`` and the last
  ``keep_last`` pages below L_s) plus the ``budget`` best-scoring other pages;
  equal scores are ordered by lower logical page index;
* KV heads whose selection flag is 0 keep every page below L_s;
* scores are raw dot-product bounds (a positive attention scale does not
  change the order, so none is applied);
* a selection reused over a chunk of decode steps (section 2.2.2) also keeps
  the pages that the chunk's appended tokens open (``horizon`` tokens past
  L_s): they hold the newest tokens, which the forced last pages keep
  anyway once they exist.

Parity status: every function here is pinned by ``tests/test_selector_oracle.py``
(brute-force statistics on tiny inputs, the upper-bound property against every
key, its equality cases, the sign special cases that reduce to plain dot
products, table-permutation invariance, a library sort on distinct scores,
the tie and budget edge cases) and by the hand-derived worked example in
``tests/golden/selector_worked.json``.
"""

from __future__ import annotations

import numpy as np

from .core import to_f64

NEG_INF = -np.inf


def n_pages(L: int, P: int) -> int:
    """Pages holding tokens [0, L)."""
    return -(-int(L) // int(P))


def page_stats(k_pool, block_table, seq_lens, logical: int = 16) -> np.ndarray:
    """Per-logical-page key statistics (LServe page, sections 2.2.2 / 3.1.2).

    k_pool: [NP, Hkv, P, D] (uint16 bf16 bit patterns or float32).
    Returns float64 [NP, Hkv, P // logical, 2, D]: index 0 = per-dimension
    maximum, index 1 = per-dimension minimum over the keys of the logical
    page's tokens below L_s of the request whose table references the page.
    Logical pages with no such token, and pages no table row references
    below L_s, stay zero.
    """
    k = to_f64(k_pool)
    NP, Hkv, P, D = k.shape
    assert P % logical == 0
    table = np.asarray(block_table)
    lens = np.asarray(seq_lens)
    out = np.zeros((NP, Hkv, P // logical, 2, D))
    for s in range(lens.shape[0]):
        L = int(lens[s])
        for lp in range(n_pages(L, P)):
            phys = int(table[s, lp])
            for sub in range(P // logical):
                t0 = lp * P + sub * logical
                n = min(logical, L - t0)
                if n <= 0:
                    continue
                rows = k[phys, :, sub * logical: sub * logical + n, :]  # [Hkv, n, D]
                out[phys, :, sub, 0, :] = rows.max(axis=1)
                out[phys, :, sub, 1, :] = rows.min(axis=1)
    return out


def logical_bound(q, kmax, kmin) -> float:
    """Upper bound on q . k over keys k with kmin <= k <= kmax (per dim)."""
    q = np.asarray(q, dtype=np.float64)
    return float(np.maximum(q * kmax, q * kmin).sum())


def page_scores(q, stats, block_table, seq_lens, P: int, logical: int = 16,
                select_heads=None) -> np.ndarray:
    """Physical-page scores [S, Hkv, max_pages] float64.

    q: [S, Hq, D]; stats as returned by ``page_stats``.  Score of logical
    page lp of request s for KV head kvh = max over the group's query heads
    h (h // G == kvh) and over the valid logical pages of the physical page
    of ``logical_bound``.  Pages at or beyond ceil(L_s / P), and every page of
    a KV head whose flag in ``select_heads`` is 0, score -inf.
    """
    q64 = to_f64(q)
    S, Hq, D = q64.shape
    Hkv = stats.shape[1]
    G = Hq // Hkv
    table = np.asarray(block_table)
    lens = np.asarray(seq_lens)
    max_pages = table.shape[1]
    out = np.full((S, Hkv, max_pages), NEG_INF)
    for s in range(S):
        L = int(lens[s])
        for kvh in range(Hkv):
            if select_heads is not None and not select_heads[kvh]:
                continue
            for lp in range(n_pages(L, P)):
                phys = int(table[s, lp])
                best = NEG_INF
                for sub in range(P // logical):
                    if lp * P + sub * logical >= L:
                        continue
                    kmax = stats[phys, kvh, sub, 0]
                    kmin = stats[phys, kvh, sub, 1]
                    for h in range(kvh * G, (kvh + 1) * G):
                        best = max(best, logical_bound(q64[s, h], kmax, kmin))
                out[s, kvh, lp] = best
    return out


def select_pages(scores, seq_lens, P: int, budget: int, keep_first: int = 0,
                 keep_last: int = 0, select_heads=None, horizon: int = 0) -> np.ndarray:
    """Block mask [S, Hkv, max_pages] uint8 from page scores.

    For each (request, KV head): pages [0, ceil(L_s / P)) are candidates;
    the first ``keep_first`` and the last ``keep_last`` of them are kept
    unconditionally; of the others the ``budget`` with the highest score are
    kept, equal scores going to the lower page index.  A KV head whose flag
    in ``select_heads`` is 0 keeps every page below L_s.  Pages from
    ceil(L_s / P) up to ceil((L_s + horizon) / P) (at most max_pages) are
    kept for every head: they receive the tokens appended while the
    selection is reused (section 2.2.2, reusable page selector).  Pages
    beyond are 0.
    """
    sc = np.asarray(scores, dtype=np.float64)
    S, Hkv, max_pages = sc.shape
    lens = np.asarray(seq_lens)
    mask = np.zeros((S, Hkv, max_pages), dtype=np.uint8)
    for s in range(S):
        npg = min(n_pages(int(lens[s]), P), max_pages)
        npg_h = min(n_pages(int(lens[s]) + int(horizon), P), max_pages)
        mask[s, :, npg:npg_h] = 1
        for kvh in range(Hkv):
            if select_heads is not None and not select_heads[kvh]:
                mask[s, kvh, :npg] = 1
                continue
            lo = min(keep_first, npg)
            hi = max(npg - keep_last, lo)
            mask[s, kvh, :lo] = 1
            mask[s, kvh, hi:npg] = 1
            cand = np.arange(lo, hi)
            if cand.size == 0 or budget <= 0:
                continue
            # order by (score descending, index ascending)
            order = cand[np.lexsort((cand, -sc[s, kvh, cand]))]
            mask[s, kvh, order[:budget]] = 1
    return mask
