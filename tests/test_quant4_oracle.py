"""The 4-bit KV quantization oracle against its pins, and planted mistakes in
it (on the CPU) that the pins must each catch."""

import numpy as np
import pytest

import oracle.quant4 as qo
from quant4_pins import ALL_CHECKS


@pytest.mark.parametrize("check", ALL_CHECKS, ids=lambda c: c.__name__)
def test_pin(check):
    check(qo)


_VALUE = qo.e2m1_value
_ENCODE = qo.e2m1_encode
_PACK = qo.pack
_QUANT = qo.quantize_rows


def _encode_truncate(y):
    # magnitude rounded toward zero onto the grid
    y = np.asarray(y, dtype=np.float64)
    c = _ENCODE(y)
    over = np.abs(_VALUE(c)) > np.minimum(np.abs(y), 6.0)
    return np.where(over & ((c & 0x7) > 0), c - 1, c).astype(np.uint8)


def _encode_ties_away(y):
    y = np.asarray(y, dtype=np.float64)
    c = _ENCODE(y)
    v = np.abs(_VALUE(c))
    up = np.abs(_VALUE(np.minimum(c & 0x7, 6) + 1))
    a = np.minimum(np.abs(y), 6.0)
    tie = (a - v) == (up - a)
    return np.where(tie & ((c & 0x7) < 0x7), c + 1, c).astype(np.uint8)


def _encode_no_clamp(y):
    # magnitudes past 6 wrap to the smallest code
    y = np.asarray(y, dtype=np.float64)
    c = _ENCODE(y)
    return np.where(np.abs(y) > 6.0, c & 0x8, c).astype(np.uint8)


def _encode_unsigned_zero(y):
    c = _ENCODE(y)
    return np.where((c & 0x7) == 0, 0, c).astype(np.uint8)


def _value_bias2(codes):
    v = _VALUE(codes)
    e = (np.asarray(codes).astype(np.int64) >> 1) & 0x3
    return np.where(e > 0, v / 2.0, v)


def _value_subnormal_as_normal(codes):
    c = np.asarray(codes).astype(np.int64)
    v = _VALUE(codes)
    sub = (((c >> 1) & 0x3) == 0) & ((c & 1) == 1)
    return np.where(sub, np.where(c & 0x8, -1.0, 1.0) * 0.75, v)


def _pack_swapped(codes):
    c = np.asarray(codes).astype(np.uint8) & np.uint8(0xF)
    return (c[..., 1::2] | (c[..., 0::2] << np.uint8(4))).astype(np.uint8)


def _quant_scale_4(x):
    a = np.asarray(x)
    xf = (a.astype(np.uint32) << np.uint32(16)).view(np.float32) if a.dtype == np.uint16 else a.astype(np.float32)
    s = (np.max(np.abs(xf), axis=-1) / np.float32(4)).astype(np.float32)
    safe = np.where(s > 0, s, np.float32(1)).astype(np.float32)
    return _PACK(_ENCODE((xf / safe[..., None]).astype(np.float32))), s


MUTANTS = {
    "encode_truncate": ("e2m1_encode", _encode_truncate),
    "encode_ties_away": ("e2m1_encode", _encode_ties_away),
    "encode_no_clamp": ("e2m1_encode", _encode_no_clamp),
    "encode_unsigned_zero": ("e2m1_encode", _encode_unsigned_zero),
    "value_bias2": ("e2m1_value", _value_bias2),
    "value_subnormal_as_normal": ("e2m1_value", _value_subnormal_as_normal),
    "pack_swapped": ("pack", _pack_swapped),
    "quant_scale_4": ("quantize_rows", _quant_scale_4),
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
