"""Checks that pin the 4-bit KV quantization oracle (``oracle.quant4``) to
facts fixed outside it: the 16 values the E2M1 format definition fixes, a
brute-force nearest-value search over every code (ties to mantissa bit 0),
the nibble order of the packing, hand-derived rows and encodings in
``tests/golden/quant4_worked.json`` and the error bound of round-to-nearest.
``test_quant4_oracle.py`` runs them against the real oracle and against
planted mistakes."""

from __future__ import annotations

import json
import math
import os

import numpy as np

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "quant4_worked.json")


def _golden():
    with open(GOLDEN) as f:
        return json.load(f)


def _brute_encode(y):
    """Nearest of the eight magnitudes the golden table lists, ties to the
    code with mantissa bit 0 (even code); |y| clamped to 6; sign bit of y."""
    table = {int(k, 16): v for k, v in _golden()["format"].items() if int(k, 16) < 8}
    codes = np.array(sorted(table))
    mags = np.array([table[c] for c in codes], dtype=np.float64)
    out = []
    for x in y:
        a = min(abs(float(x)), 6.0)
        d = np.abs(mags - a)
        pick = [int(codes[i]) for i in np.flatnonzero(d == d.min())]
        even = [p for p in pick if p % 2 == 0]
        code = (even or pick)[0]
        if math.copysign(1.0, float(x)) < 0:
            code |= 0x8
        out.append(code)
    return np.array(out, dtype=np.uint8)


def check_format_values(o):
    for code, want in _golden()["format"].items():
        got = float(o.e2m1_value(np.array([int(code, 16)]))[0])
        if want == "-0":
            assert got == 0.0 and math.copysign(1.0, got) < 0, code
        else:
            assert got == want, (code, got, want)


def check_encode_brute_force(o):
    mags = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])
    mids = (mags[:-1] + mags[1:]) / 2
    ys = [mags, -mags, mids, -mids,
          np.nextafter(mids.astype(np.float32), np.float32(0)).astype(np.float64),
          np.nextafter(mids.astype(np.float32), np.float32(1e9)).astype(np.float64),
          np.array([6.5, 100.0, -1e30, 1e-30, -1e-30])]
    rng = np.random.default_rng(41)
    ys.append(rng.standard_normal(800) * rng.choice([0.01, 0.5, 2.0, 5.0], 800))
    y = np.concatenate(ys)
    got = o.e2m1_encode(y)
    want = _brute_encode(y)
    bad = np.flatnonzero(got != want)
    assert bad.size == 0, [(float(y[i]), int(got[i]), int(want[i])) for i in bad[:5]]


def check_golden_encodings(o):
    for case in _golden()["encode"]:
        got = int(o.e2m1_encode(np.array([case["y"]]))[0])
        assert got == int(case["code"], 16), (case, hex(got))


def check_packing(o):
    """Element 2i in the low nibble of byte i, 2i + 1 in the high nibble; the
    inverse restores every code."""
    codes = np.array([[0x1, 0x2, 0x3, 0x4, 0xf, 0x0]], dtype=np.uint8)
    assert o.pack(codes).tolist() == [[0x21, 0x43, 0x0f]]
    rng = np.random.default_rng(42)
    c = rng.integers(0, 16, size=(7, 64)).astype(np.uint8)
    assert np.array_equal(o.unpack(o.pack(c)), c)


def check_golden_rows(o):
    for case in _golden()["rows"]:
        packed, s = o.quantize_rows(np.array([case["x"]], dtype=np.float32))
        assert float(s[0]) == case["scale"], (case, float(s[0]))
        assert [int(c) for c in packed[0]] == [int(c, 16) for c in case["packed"]], (case, packed)
        assert o.dequantize(packed, s)[0].tolist() == case["dequantized"], case


def check_quantize_bounds(o):
    """Random bf16 rows: the largest |x| maps to magnitude code 7 (6 s); every
    value is reconstructed within half a grid step of y = |x| / s (0.25 below
    2, 0.5 in [2, 4), 1 in [4, 6]) times s; s = amax / 6 in fp32."""
    rng = np.random.default_rng(43)
    x = (rng.standard_normal((64, 128)) * rng.choice([1e-3, 1.0, 50.0], (64, 1))).astype(np.float32)
    bits = (x.view(np.uint32) >> 16).astype(np.uint16)
    xf = (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    packed, s = o.quantize_rows(bits)
    amax = np.abs(xf).max(axis=1)
    assert np.array_equal(s, (amax.astype(np.float32) / np.float32(6)).astype(np.float32))
    codes = o.unpack(packed)
    arg = np.abs(xf).argmax(axis=1)
    assert np.all((codes[np.arange(64), arg] & 0x7) == 0x7)
    deq = o.dequantize(packed, s)
    y = np.abs(xf) / s[:, None].astype(np.float64)
    half = np.where(y < 2, 0.25, np.where(y < 4, 0.5, 1.0))
    err = np.abs(deq - xf)
    assert np.all(err <= half * s[:, None] * (1 + 1e-6) + 1e-30), float((err / (half * s[:, None])).max())


ALL_CHECKS = [
    check_format_values,
    check_encode_brute_force,
    check_golden_encodings,
    check_packing,
    check_golden_rows,
    check_quantize_bounds,
]
