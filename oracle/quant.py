"""Plain CPU oracle for 8-bit floating-point KV pages.

TEST INFRASTRUCTURE ONLY.  Only the test suite, ``__graft_entry__.smoke()`` and
the ``cpu_baseline`` leg of ``bench.py`` may import this module.  The product
path never imports, calls or links anything here, and this module imports
nothing from the product package.

Source: LServe blog page ("LLM长序列服务优化：LServe的块稀疏注意力技术"),
section 3.2.1 (the retrieval-head cache is a growing paged store with
logical-page statistics and configurable 2-8 bit quantization) and section
3.2.2 (quantization together with sparsity).  The page fixes neither the
number format nor the scale granularity; the readings taken (also listed in
the design notes):

* 8 bits in the OCP FP8 E4M3 format: 1 sign bit, 4 exponent bits with bias 7,
  3 mantissa bits, subnormals (exponent field 0: m * 2^-9), no infinities,
  S.1111.111 is NaN, largest finite value 448 -- the 8-bit float format the
  target GPU converts in hardware;
* one fp32 scale per (token, KV head) row of K and of V: s = amax / 448 in
  fp32 (amax = the largest |x| of the row), and the code of x is the E4M3
  value nearest to y = x / s (fp32 division) after clamping y to [-448, 448],
  ties going to the even code; the sign of y is kept even when the magnitude
  rounds to zero; an all-zero row has s = 0 and codes 0;
* a quantized row stands for value(code) * s, and attention over quantized
  pages is the plain attention of ``oracle.core`` over those values.

Parity status: pinned by ``tests/test_quant_oracle.py`` (values the format
definition fixes, a brute-force nearest-value search over all 254 finite
codes with ties to even, hand-derived rows in ``tests/golden/quant_worked.json``,
reconstruction-error bounds, planted mistakes).
"""

from __future__ import annotations

import numpy as np

E4M3_MAX = 448.0


def e4m3_value(codes) -> np.ndarray:
    """float64 values of E4M3 codes (uint8 array); NaN for the NaN codes."""
    c = np.asarray(codes).astype(np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = (c & 7).astype(np.float64)
    mag = np.where(e == 0, m * 2.0 ** -9, (1.0 + m / 8.0) * np.exp2(e - 7.0))
    mag = np.where((e == 0xF) & ((c & 7) == 7), np.nan, mag)
    return sign * mag


def e4m3_encode(y) -> np.ndarray:
    """Codes (uint8) of the E4M3 values nearest to y (ties to the even code),
    after clamping |y| to 448; the sign bit is the sign bit of y."""
    y = np.asarray(y, dtype=np.float64)
    neg = np.signbit(y)
    a = np.minimum(np.abs(y), E4M3_MAX)
    # spacing of the E4M3 grid around a: 2^-9 below 2^-6, else 2^(E-3) in binade [2^E, 2^(E+1))
    _, ex = np.frexp(np.where(a > 0, a, 1.0))
    E = np.maximum(ex - 1, -6)
    spacing = np.exp2(E - 3.0)
    n = np.rint(a / spacing)  # round half to even
    v = n * spacing
    # value -> code fields
    _, vex = np.frexp(np.where(v > 0, v, 1.0))
    VE = vex - 1
    normal = v >= 2.0 ** -6
    e_field = np.where(normal, VE + 7, 0)
    m_field = np.where(normal, v / np.exp2(VE.astype(np.float64)) * 8 - 8, v / 2.0 ** -9)
    code = (e_field << 3) | m_field.astype(np.int64)
    code = np.where(v == 0, 0, code)
    return (code | np.where(neg, 0x80, 0)).astype(np.uint8)


def quantize_rows(x):
    """(codes uint8 [..., D], scales float32 [...]) of rows x [..., D]
    (bf16 bit patterns as uint16, or float32)."""
    a = np.asarray(x)
    if a.dtype == np.uint16:
        xf = (a.astype(np.uint32) << np.uint32(16)).view(np.float32)
    else:
        xf = a.astype(np.float32)
    amax = np.max(np.abs(xf), axis=-1)
    s = (amax / np.float32(E4M3_MAX)).astype(np.float32)
    safe = np.where(s > 0, s, np.float32(1.0)).astype(np.float32)
    y = (xf / safe[..., None]).astype(np.float32)
    codes = e4m3_encode(y)
    codes = np.where((s > 0)[..., None], codes, np.uint8(0)).astype(np.uint8)
    return codes, s


def dequantize(codes, scales) -> np.ndarray:
    """float64 values value(code) * scale of quantized rows."""
    return e4m3_value(codes) * np.asarray(scales, dtype=np.float64)[..., None]
