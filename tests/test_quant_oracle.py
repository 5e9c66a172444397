"""The 8-bit KV quantization oracle against its pins, and planted mistakes in
it (on the CPU) that the pins must each catch."""

import numpy as np
import pytest

import oracle.quant as qo
from quant_pins import ALL_CHECKS


@pytest.mark.parametrize("check", ALL_CHECKS, ids=lambda c: c.__name__)
def test_pin(check):
    check(qo)


_VALUE = qo.e4m3_value
_ENCODE = qo.e4m3_encode
_QUANT = qo.quantize_rows


def _encode_truncate(y):
    # magnitude rounded toward zero onto the grid
    y = np.asarray(y, dtype=np.float64)
    c = _ENCODE(y)
    v = np.abs(_VALUE(c))
    over = v > np.minimum(np.abs(y), 448.0)
    step_down = np.where(over & ((c & 0x7F) > 0), c - 1, c)
    return step_down.astype(np.uint8)


def _encode_ties_away(y):
    y = np.asarray(y, dtype=np.float64)
    c = _ENCODE(y)
    # at an exact midpoint move to the larger magnitude
    v = np.abs(_VALUE(c))
    up = np.abs(_VALUE(np.minimum(c & 0x7F, 0x7D) + 1))
    a = np.minimum(np.abs(y), 448.0)
    tie = (a - v) == (up - a)
    return np.where(tie & ((c & 0x7F) < 0x7E), c + 1, c).astype(np.uint8)


def _encode_no_clamp(y):
    y = np.asarray(y, dtype=np.float64)
    c = _ENCODE(y)
    return np.where(np.abs(y) > 464.0, c | 0x7F, c).astype(np.uint8)


def _encode_unsigned_zero(y):
    c = _ENCODE(y)
    return np.where((c & 0x7F) == 0, 0, c).astype(np.uint8)


def _value_bias8(codes):
    v = _VALUE(codes)
    e = (np.asarray(codes).astype(np.int64) >> 3) & 0xF
    return np.where(e > 0, v / 2.0, v)


def _value_subnormal_as_normal(codes):
    c = np.asarray(codes).astype(np.int64)
    v = _VALUE(codes)
    e = (c >> 3) & 0xF
    m = (c & 7).astype(np.float64)
    sub = (e == 0) & (m > 0)
    return np.where(sub, np.where(c & 0x80, -1.0, 1.0) * (1 + m / 8) * 2.0 ** -7, v)


def _quant_scale_127(x):
    a = np.asarray(x)
    xf = (a.astype(np.uint32) << np.uint32(16)).view(np.float32) if a.dtype == np.uint16 else a.astype(np.float32)
    s = (np.max(np.abs(xf), axis=-1) / np.float32(127)).astype(np.float32)
    safe = np.where(s > 0, s, np.float32(1)).astype(np.float32)
    return _ENCODE((xf / safe[..., None]).astype(np.float32)), s


MUTANTS = {
    "encode_truncate": ("e4m3_encode", _encode_truncate),
    "encode_ties_away": ("e4m3_encode", _encode_ties_away),
    "encode_no_clamp": ("e4m3_encode", _encode_no_clamp),
    "encode_unsigned_zero": ("e4m3_encode", _encode_unsigned_zero),
    "value_bias8": ("e4m3_value", _value_bias8),
    "value_subnormal_as_normal": ("e4m3_value", _value_subnormal_as_normal),
    "quant_scale_127": ("quantize_rows", _quant_scale_127),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, monkeypatch):
    attr, fn = MUTANTS[name]
    monkeypatch.setattr(qo, attr, fn)
    caught = []
    for check in ALL_CHECKS:
        try:
            check(qo)
        except AssertionError:
            caught.append(check.__name__)
    assert caught, f"mutant {name} passed every pin"
