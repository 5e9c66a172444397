"""Checks that pin the 8-bit KV quantization oracle (``oracle.quant``) to
facts fixed outside it: values the E4M3 format definition fixes, the
monotone structure of its grid, a brute-force nearest-value search over all
finite codes (ties to the even code), hand-derived rows and encodings in
``tests/golden/quant_worked.json`` and the reconstruction-error bound of
round-to-nearest.  ``test_quant_oracle.py`` runs them against the real oracle
and against planted mistakes."""

from __future__ import annotations

import json
import math
import os

import numpy as np

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "quant_worked.json")


def _golden():
    with open(GOLDEN) as f:
        return json.load(f)


def _finite_table(o):
    """(codes, values) of every finite code, taken from the oracle's decoder."""
    c = np.arange(256, dtype=np.uint8)
    v = o.e4m3_value(c)
    keep = ~np.isnan(v)
    return c[keep], v[keep]


def _brute_encode(y, codes, values):
    """Nearest finite value to y, ties to the even code; |y| clamped to 448;
    sign bit of y kept."""
    out = []
    pos = values >= 0
    pc, pv = codes[pos & (codes < 0x80)], values[pos & (codes < 0x80)]
    for x in y:
        a = min(abs(float(x)), 448.0)
        d = np.abs(pv - a)
        best = np.flatnonzero(d == d.min())
        pick = [int(pc[i]) for i in best]
        even = [p for p in pick if p % 2 == 0]
        code = (even or pick)[0]
        if math.copysign(1.0, float(x)) < 0:
            code |= 0x80
        out.append(code)
    return np.array(out, dtype=np.uint8)


def check_format_values(o):
    for code, want in _golden()["format"].items():
        got = float(o.e4m3_value(np.array([int(code, 16)], dtype=np.uint8))[0])
        if want == "nan":
            assert math.isnan(got), code
        elif want == "-0":
            assert got == 0.0 and math.copysign(1.0, got) < 0, code
        else:
            assert got == want, (code, got, want)


def check_grid_structure(o):
    """Positive codes 0x00..0x7e increase strictly; the step is 2^-9 over the
    subnormals and the first binade and doubles with every binade; negative
    codes mirror the positive ones; exactly two NaN codes."""
    v = o.e4m3_value(np.arange(256, dtype=np.uint8))
    assert int(np.isnan(v).sum()) == 2 and np.isnan(v[0x7F]) and np.isnan(v[0xFF])
    pos = v[:0x7F]
    steps = np.diff(pos)
    assert np.all(steps > 0)
    for e in range(16):
        lo, hi = 8 * e, min(8 * e + 8, 0x7F)
        want = 2.0 ** (max(e, 1) - 10)
        assert np.all(steps[lo:hi - 1] == want), (e, steps[lo:hi - 1])
    assert np.array_equal(v[0x80:0xFF], -pos)


def check_encode_brute_force(o):
    codes, values = _finite_table(o)
    pv = np.unique(np.abs(values))
    mids = (pv[:-1] + pv[1:]) / 2
    ys = [values, mids, -mids,
          np.nextafter(mids.astype(np.float32), np.float32(0)).astype(np.float64),
          np.nextafter(mids.astype(np.float32), np.float32(1e9)).astype(np.float64)]
    rng = np.random.default_rng(31)
    ys.append(rng.standard_normal(500) * rng.choice([0.001, 0.1, 1.0, 30.0, 300.0], 500))
    y = np.concatenate(ys)
    got = o.e4m3_encode(y)
    want = _brute_encode(y, codes, values)
    bad = np.flatnonzero(got != want)
    assert bad.size == 0, [(float(y[i]), int(got[i]), int(want[i])) for i in bad[:5]]


def check_golden_encodings(o):
    for case in _golden()["encode"]:
        got = int(o.e4m3_encode(np.array([case["y"]]))[0])
        assert got == int(case["code"], 16), (case, hex(got))


def check_golden_rows(o):
    for case in _golden()["rows"]:
        codes, s = o.quantize_rows(np.array([case["x"]], dtype=np.float32))
        assert float(s[0]) == case["scale"], (case, float(s[0]))
        assert [int(c) for c in codes[0]] == [int(c, 16) for c in case["codes"]], (case, codes)
        if "dequantized" in case:
            assert o.dequantize(codes, s)[0].tolist() == case["dequantized"]


def check_quantize_bounds(o):
    """Random bf16 rows: the largest |x| maps to code +-448; every value is
    reconstructed within half a grid step (of the E4M3 grid at |x| / s)
    times s; s = amax / 448 in fp32."""
    rng = np.random.default_rng(32)
    x = (rng.standard_normal((64, 128)) * rng.choice([1e-3, 1.0, 50.0], (64, 1))).astype(np.float32)
    bits = (x.view(np.uint32) >> 16).astype(np.uint16)  # bf16 (truncated) bit patterns
    xf = (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    codes, s = o.quantize_rows(bits)
    amax = np.abs(xf).max(axis=1)
    assert np.array_equal(s, (amax.astype(np.float32) / np.float32(448)).astype(np.float32))
    arg = np.abs(xf).argmax(axis=1)
    assert np.all((codes[np.arange(64), arg] & 0x7F) == 0x7E)
    deq = o.dequantize(codes, s)
    y = np.abs(xf) / s[:, None].astype(np.float64)
    _, ex = np.frexp(np.where(y > 0, y, 1.0))
    step = np.exp2(np.maximum(ex - 1, -6) - 3.0)
    err = np.abs(deq - xf)
    assert np.all(err <= 0.5 * step * s[:, None] * (1 + 1e-6) + 1e-30), float((err / (step * s[:, None])).max())


ALL_CHECKS = [
    check_format_values,
    check_grid_structure,
    check_encode_brute_force,
    check_golden_encodings,
    check_golden_rows,
    check_quantize_bounds,
]
