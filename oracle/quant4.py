"""Plain CPU oracle for 4-bit floating-point KV pages.

TEST INFRASTRUCTURE ONLY.  Only the test suite, ``__graft_entry__.smoke()`` and
the ``cpu_baseline`` leg of ``bench.py`` may import this module.  The product
path never imports, calls or links anything here, and this module imports
nothing from the product package.

Source: LServe blog page ("LLM长序列服务优化：LServe的块稀疏注意力技术"),
section 3.2.1 (the KV cache of retrieval heads is quantized with a
configurable 2-8 bits; the cache of streaming heads is 4-bit) and section
3.2.2 (quantization together with sparsity).  The page fixes neither the
4-bit number format nor the scale granularity; the readings taken (also
listed in the design notes):

* 4 bits in the OCP FP4 E2M1 format: 1 sign bit, 2 exponent bits with bias 1,
  1 mantissa bit; exponent field 0 is subnormal (m * 0.5), otherwise the value
  is 2^(e - 1) * (1 + m / 2); no infinities and no NaN, so the magnitudes are
  0, 0.5, 1, 1.5, 2, 3, 4, 6 -- the 4-bit float format the target GPU
  converts in hardware;
* two codes per byte: element 2i of a row in the low nibble (bits 3-0) of
  byte i, element 2i + 1 in the high nibble (bits 7-4);
* one fp32 scale per (token, KV head) row of K and of V, as for 8-bit pages:
  s = amax / 6 in fp32 (amax = the largest |x| of the row); the code of x is
  the E2M1 value nearest to y = x / s (fp32 division) after clamping |y| to 6,
  ties going to the code with mantissa bit 0; the sign of y is kept even when
  the magnitude rounds to zero; an all-zero row has s = 0 and codes 0;
* a quantized row stands for value(code) * s, and attention over quantized
  pages is the plain attention of ``oracle.core`` over those values.

Parity status: pinned by ``tests/test_quant4_oracle.py`` (the 16 values the
format definition fixes, a brute-force nearest-value search over every code
with ties to the even code, the nibble order, hand-derived rows in
``tests/golden/quant4_worked.json``, the round-to-nearest error bound,
planted mistakes).
"""

from __future__ import annotations

import numpy as np

E2M1_MAX = 6.0


def e2m1_value(codes) -> np.ndarray:
    """float64 values of 4-bit E2M1 codes (integers 0..15)."""
    c = np.asarray(codes).astype(np.int64) & 0xF
    sign = np.where(c & 0x8, -1.0, 1.0)
    e = (c >> 1) & 0x3
    m = (c & 1).astype(np.float64)
    mag = np.where(e == 0, m * 0.5, np.exp2(e - 1.0) * (1.0 + m / 2.0))
    return sign * mag


def e2m1_encode(y) -> np.ndarray:
    """4-bit codes (uint8 values 0..15) of the E2M1 values nearest to y (ties
    to the code with mantissa bit 0), after clamping |y| to 6; the sign bit is
    the sign bit of y."""
    y = np.asarray(y, dtype=np.float64)
    neg = np.signbit(y)
    a = np.minimum(np.abs(y), E2M1_MAX)
    # the grid has spacing 0.5 below 2 (0, 0.5, 1, 1.5), 1 in [2, 4) and 2 in [4, 6]
    spacing = np.where(a < 2.0, 0.5, np.where(a < 4.0, 1.0, 2.0))
    base = np.where(a < 2.0, 0.0, np.where(a < 4.0, 2.0, 4.0))
    n = np.rint((a - base) / spacing)  # round half to even: an even step count is mantissa 0
    v = base + n * spacing
    # value -> code fields (v is on the grid: 0, 0.5, 1, 1.5, 2, 3, 4, 6)
    code = np.select(
        [v == 0.0, v == 0.5, v == 1.0, v == 1.5, v == 2.0, v == 3.0, v == 4.0, v == 6.0],
        [0, 1, 2, 3, 4, 5, 6, 7])
    return (code | np.where(neg, 0x8, 0)).astype(np.uint8)


def pack(codes) -> np.ndarray:
    """Packs 4-bit codes [..., D] (D even) two per byte: element 2i in the low
    nibble of byte i, element 2i + 1 in the high nibble -> uint8 [..., D/2]."""
    c = np.asarray(codes).astype(np.uint8) & np.uint8(0xF)
    return (c[..., 0::2] | (c[..., 1::2] << np.uint8(4))).astype(np.uint8)


def unpack(packed) -> np.ndarray:
    """Inverse of pack: uint8 [..., D/2] -> 4-bit codes uint8 [..., D]."""
    b = np.asarray(packed).astype(np.uint8)
    out = np.empty(b.shape[:-1] + (2 * b.shape[-1],), dtype=np.uint8)
    out[..., 0::2] = b & np.uint8(0xF)
    out[..., 1::2] = b >> np.uint8(4)
    return out


def quantize_rows(x):
    """(packed codes uint8 [..., D/2], scales float32 [...]) of rows x
    [..., D] (bf16 bit patterns as uint16, or float32)."""
    a = np.asarray(x)
    if a.dtype == np.uint16:
        xf = (a.astype(np.uint32) << np.uint32(16)).view(np.float32)
    else:
        xf = a.astype(np.float32)
    amax = np.max(np.abs(xf), axis=-1)
    s = (amax / np.float32(E2M1_MAX)).astype(np.float32)
    safe = np.where(s > 0, s, np.float32(1.0)).astype(np.float32)
    y = (xf / safe[..., None]).astype(np.float32)
    codes = e2m1_encode(y)
    codes = np.where((s > 0)[..., None], codes, np.uint8(0)).astype(np.uint8)
    return pack(codes), s


def dequantize(packed, scales) -> np.ndarray:
    """float64 values value(code) * scale of quantized rows (packed codes)."""
    return e2m1_value(unpack(packed)) * np.asarray(scales, dtype=np.float64)[..., None]
