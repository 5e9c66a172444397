"""The decode-update oracle against its pins, and planted mistakes in it (on
the CPU) that the pins must each catch."""

import types

import numpy as np
import pytest

import oracle.decode as dec
import oracle.selector as sel
from decode_pins import ALL_CHECKS

NS = types.SimpleNamespace(decode=dec, selector=sel)


@pytest.mark.parametrize("check", ALL_CHECKS, ids=lambda c: c.__name__)
def test_pin(check):
    check(NS)


_APPEND = dec.append_kv
_BOUNDS = dec.kept_page_bounds
_SELECT = sel.select_pages


def _append_off_by_one(k_pool, v_pool, block_table, seq_lens, k_new, v_new):
    return _APPEND(k_pool, v_pool, block_table, np.asarray(seq_lens) - 1, k_new, v_new)


def _append_k_only(k_pool, v_pool, block_table, seq_lens, k_new, v_new):
    k, _ = _APPEND(k_pool, v_pool, block_table, seq_lens, k_new, v_new)
    return k, np.array(v_pool, copy=True)


def _append_identity_table(k_pool, v_pool, block_table, seq_lens, k_new, v_new):
    table = np.asarray(block_table)
    ident = (np.arange(table.shape[0])[:, None] * table.shape[1] + np.arange(table.shape[1])[None])
    return _APPEND(k_pool, v_pool, ident.astype(np.int32), seq_lens, k_new, v_new)


def _append_wraps_when_full(k_pool, v_pool, block_table, seq_lens, k_new, v_new):
    cap = np.asarray(block_table).shape[1] * np.asarray(k_pool).shape[2]
    return _APPEND(k_pool, v_pool, block_table, np.asarray(seq_lens) % cap, k_new, v_new)


def _bounds_ceil(block_mask, seq_lens, P, b, horizon=0, Hkv=None, max_pages=None):
    out = _BOUNDS(block_mask, seq_lens, P, b, horizon, Hkv, max_pages)
    # shift every interior bound to the next kept page (ceil of the ordinal)
    mask = None if block_mask is None else np.asarray(block_mask)
    S = out.shape[0]
    for s in range(S):
        for h in range(out.shape[1]):
            E = out[s, h, b]
            n = -(-int(E) // P)
            kept = list(range(n)) if mask is None else [lp for lp in range(n) if mask[s, h, lp]]
            K = len(kept)
            for j in range(1, b):
                o = -(-(j * K) // b)
                out[s, h, j] = P * kept[o] if o < K else E
    return out


def _bounds_ignore_mask(block_mask, seq_lens, P, b, horizon=0, Hkv=None, max_pages=None):
    if block_mask is not None:
        _, Hkv, max_pages = np.asarray(block_mask).shape
    return _BOUNDS(None, seq_lens, P, b, horizon, Hkv, max_pages)


def _bounds_ignore_horizon(block_mask, seq_lens, P, b, horizon=0, Hkv=None, max_pages=None):
    return _BOUNDS(block_mask, seq_lens, P, b, 0, Hkv, max_pages)


def _select_horizon_short(scores, seq_lens, P, budget, keep_first=0, keep_last=0,
                          select_heads=None, horizon=0):
    return _SELECT(scores, seq_lens, P, budget, keep_first, keep_last, select_heads,
                   max(horizon - 1, 0))


def _select_horizon_ignored(scores, seq_lens, P, budget, keep_first=0, keep_last=0,
                            select_heads=None, horizon=0):
    return _SELECT(scores, seq_lens, P, budget, keep_first, keep_last, select_heads, 0)


MUTANTS = {
    "append_off_by_one": (dec, "append_kv", _append_off_by_one),
    "append_k_only": (dec, "append_kv", _append_k_only),
    "append_identity_table": (dec, "append_kv", _append_identity_table),
    "append_wraps_when_full": (dec, "append_kv", _append_wraps_when_full),
    "bounds_ceil": (dec, "kept_page_bounds", _bounds_ceil),
    "bounds_ignore_mask": (dec, "kept_page_bounds", _bounds_ignore_mask),
    "bounds_ignore_horizon": (dec, "kept_page_bounds", _bounds_ignore_horizon),
    "select_horizon_short": (sel, "select_pages", _select_horizon_short),
    "select_horizon_ignored": (sel, "select_pages", _select_horizon_ignored),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, monkeypatch):
    mod, attr, fn = MUTANTS[name]
    monkeypatch.setattr(mod, attr, fn)
    caught = []
    for check in ALL_CHECKS:
        try:
            check(NS)
        except AssertionError:
            caught.append(check.__name__)
    assert caught, f"mutant {name} passed every pin"
