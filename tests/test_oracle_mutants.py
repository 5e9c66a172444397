"""Planted mistakes in the oracle (on the CPU) must each be caught by at
least one pin.  A mutant replaces one function of ``oracle.core`` for the
duration of a test; the pins then run against the mutated module."""

import math

import numpy as np
import pytest

import oracle.core as oa
from oracle_pins import ALL_CHECKS

_MICRO = oa.micro_tokens
_KEPT = oa.kept_tokens
_FOLD = oa.merge_partials


def _no_scale(q, K, scale):
    return oa.to_f64(K) @ oa.to_f64(q)


def _sqrt_scale(q, K, scale):
    return (oa.to_f64(K) @ oa.to_f64(q)) * math.sqrt(float(scale))


def _gqa_modulo(h, Hq, Hkv):
    return h % Hkv


def _gather_swapped(pool, row, kv_head, tokens, P):
    tokens = np.asarray(tokens, dtype=np.int64)
    phys = np.asarray(row, dtype=np.int64)[tokens % P]
    return np.asarray(pool)[phys % np.asarray(pool).shape[0], kv_head, tokens // P % P, :]


def _attn_sign(q, K, V, scale):
    V64 = oa.to_f64(V)
    if V64.shape[0] == 0:
        return np.zeros(V64.shape[1])
    s = oa.scores(q, K, scale)
    w = np.exp(s.max() - s)
    return (w[:, None] * V64).sum(0) / w.sum()


def _attn_transposed(q, K, V, scale):
    # contraction over the wrong axis of V when shapes allow it
    V64 = oa.to_f64(V)
    if V64.shape[0] == 0:
        return np.zeros(V64.shape[1])
    s = oa.scores(q, K, scale)
    w = np.exp(s - s.max())
    return (w[:, None] * V64).sum(0) / len(w)


def _micro_count(q, K, V, scale):
    MA, m, e = _MICRO(q, K, V, scale)
    return MA, m, float(np.asarray(V).shape[0])


def _micro_no_shift(q, K, V, scale):
    V64 = oa.to_f64(V)
    if V64.shape[0] == 0:
        return np.zeros(V64.shape[1]), -np.inf, 0.0
    s = oa.scores(q, K, scale)
    w = np.exp(s)
    return (w[:, None] * V64).sum(0), float(s.max()), float(w.sum())


def _kept_ignore_mask(seq_len, P, t0, t1, mask_row=None):
    return _KEPT(seq_len, P, t0, t1, None)


def _kept_no_clamp(seq_len, P, t0, t1, mask_row=None):
    return _KEPT(10 ** 9, P, t0, t1, mask_row)


def _weights_unshifted(m, axis):
    m = np.asarray(m, dtype=np.float64)
    m_g = np.max(m, axis=axis, keepdims=True)
    return m_g, np.where(np.isneginf(m), 0.0, 1.0)


def _widen_wrong(x):
    a = np.asarray(x)
    if a.dtype == np.uint16:
        return (a.astype(np.uint32) << np.uint32(8)).view(np.float32).astype(np.float64)
    return a.astype(np.float64)


def _fold_unweighted_sum(MA, m, e):
    MAf, mf, ef = _FOLD(MA, m, e)
    return np.asarray(MA, dtype=np.float64).sum(axis=-2), mf, ef


def _fold_normalised(MA, m, e):
    MAf, mf, ef = _FOLD(MA, m, e)
    return MAf / np.where(ef > 0, ef, 1.0)[..., None], mf, ef


MUTANTS = {
    "scores: scale dropped": ("scores", _no_scale),
    "scores: sqrt of scale": ("scores", _sqrt_scale),
    "GQA: h % Hkv": ("kv_head_of", _gqa_modulo),
    "gather: page/slot swapped": ("gather", _gather_swapped),
    "attention: exp sign flipped": ("attention_tokens", _attn_sign),
    "attention: divide by count": ("attention_tokens", _attn_transposed),
    "micro: e_j = count": ("micro_tokens", _micro_count),
    "micro: m_j not subtracted": ("micro_tokens", _micro_no_shift),
    "mask ignored": ("kept_tokens", _kept_ignore_mask),
    "seq_len clamp dropped": ("kept_tokens", _kept_no_clamp),
    "merge: weights not rescaled": ("_weights", _weights_unshifted),
    "fold: MA' not rescaled": ("merge_partials", _fold_unweighted_sum),
    "fold: MA' divided by e'": ("merge_partials", _fold_normalised),
    "bf16 widen: wrong shift": ("to_f64", _widen_wrong),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, monkeypatch):
    attr, fn = MUTANTS[name]
    original = getattr(oa, attr)
    monkeypatch.setattr(oa, attr, fn)
    caught = []
    for check in ALL_CHECKS:
        try:
            with np.errstate(all="ignore"):
                check(oa)
        except (AssertionError, IndexError, ValueError, FloatingPointError, OverflowError):
            caught.append(check.__name__)
    monkeypatch.setattr(oa, attr, original)
    assert caught, f"mutant '{name}' passed every pin"
