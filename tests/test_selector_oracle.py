"""The page-selection oracle against its pins, and planted mistakes in it
(on the CPU) that the pins must each catch."""

import numpy as np
import pytest

import oracle.selector as sel
from selector_pins import ALL_CHECKS


@pytest.mark.parametrize("check", ALL_CHECKS, ids=lambda c: c.__name__)
def test_pin(check):
    check(sel)


_STATS = sel.page_stats
_SCORES = sel.page_scores
_SELECT = sel.select_pages
_BOUND = sel.logical_bound


def _bound_kmax_only(q, kmax, kmin):
    return float(np.dot(np.asarray(q, dtype=np.float64), kmax))


def _bound_mean(q, kmax, kmin):
    return float(np.dot(np.asarray(q, dtype=np.float64), (kmax + kmin) / 2))


def _bound_swapped(q, kmax, kmin):
    q = np.asarray(q, dtype=np.float64)
    return float(np.minimum(q * kmax, q * kmin).sum())


def _stats_all_slots(k_pool, block_table, seq_lens, logical=16):
    # statistics over every slot of a referenced page, including those past L_s
    lens = np.asarray(seq_lens)
    P = np.asarray(k_pool).shape[2]
    padded = ((lens + P - 1) // P) * P
    return _STATS(k_pool, block_table, padded, logical)


def _stats_off_by_one(k_pool, block_table, seq_lens, logical=16):
    return _STATS(k_pool, block_table, np.maximum(np.asarray(seq_lens) - 1, 0), logical)


def _scores_first_logical(q, stats, block_table, seq_lens, P, logical=16, select_heads=None):
    # only the first logical page of each physical page counts
    st = stats.copy()
    for sub in range(1, st.shape[2]):
        st[:, :, sub] = st[:, :, 0]
    return _SCORES(q, st, block_table, seq_lens, P, logical, select_heads)


def _scores_first_head(q, stats, block_table, seq_lens, P, logical=16, select_heads=None):
    # the group's first query head only
    q = np.asarray(q)
    Hkv = stats.shape[1]
    G = q.shape[1] // Hkv
    q2 = np.repeat(q[:, ::G], G, axis=1)
    return _SCORES(q2, stats, block_table, seq_lens, P, logical, select_heads)


def _scores_gqa_modulo(q, stats, block_table, seq_lens, P, logical=16, select_heads=None):
    # heads h with h % Hkv == kvh instead of h // G == kvh
    q = np.asarray(q)
    S, Hq, D = q.shape
    Hkv = stats.shape[1]
    G = Hq // Hkv
    order = [h for kvh in range(Hkv) for h in range(Hq) if h % Hkv == kvh]
    return _SCORES(q[:, order], stats, block_table, seq_lens, P, logical, select_heads)


def _select_ties_high(scores, seq_lens, P, budget, keep_first=0, keep_last=0, select_heads=None):
    # equal scores go to the higher page index: nudge each score up by a
    # tiny amount growing with the index (only ties change order)
    sc = np.asarray(scores, dtype=np.float64)
    idx = np.arange(sc.shape[2], dtype=np.float64)
    return _SELECT(sc + idx * 1e-9, seq_lens, P, budget, keep_first, keep_last, select_heads)


def _select_lowest(scores, seq_lens, P, budget, keep_first=0, keep_last=0, select_heads=None):
    return _SELECT(-np.asarray(scores, dtype=np.float64), seq_lens, P, budget, keep_first,
                   keep_last, select_heads)


def _select_budget_counts_forced(scores, seq_lens, P, budget, keep_first=0, keep_last=0,
                                 select_heads=None):
    return _SELECT(scores, seq_lens, P, max(budget - keep_first - keep_last, 0), keep_first,
                   keep_last, select_heads)


def _select_no_forced(scores, seq_lens, P, budget, keep_first=0, keep_last=0, select_heads=None):
    return _SELECT(scores, seq_lens, P, budget, 0, 0, select_heads)


MUTANTS = {
    "bound_kmax_only": ("logical_bound", _bound_kmax_only),
    "bound_mean": ("logical_bound", _bound_mean),
    "bound_min_instead_of_max": ("logical_bound", _bound_swapped),
    "stats_all_slots": ("page_stats", _stats_all_slots),
    "stats_off_by_one": ("page_stats", _stats_off_by_one),
    "scores_first_logical": ("page_scores", _scores_first_logical),
    "scores_first_head": ("page_scores", _scores_first_head),
    "scores_gqa_modulo": ("page_scores", _scores_gqa_modulo),
    "select_ties_high": ("select_pages", _select_ties_high),
    "select_lowest": ("select_pages", _select_lowest),
    "select_budget_counts_forced": ("select_pages", _select_budget_counts_forced),
    "select_no_forced": ("select_pages", _select_no_forced),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, monkeypatch):
    attr, fn = MUTANTS[name]
    monkeypatch.setattr(sel, attr, fn)
    caught = []
    for check in ALL_CHECKS:
        try:
            check(sel)
        except AssertionError:
            caught.append(check.__name__)
    assert caught, f"mutant {name} passed every pin"
