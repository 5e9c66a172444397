"""Seeded random shapes through the C ABI against the fp64 oracle: each case
draws the request count, head counts (G in {1, 2, 4, 8}), head dim, page
size, dtype, length mix, block table, mask, split rule, chunk count,
schedule and pool layout, then checks the two-call step (partials and
output), the one-launch step and, for bf16 cases, the same pools quantized
to 8 and to 4 bits.  The draws come from a fixed seed, so every run checks the same
cases; sizes keep the oracle at a fraction of a second per case.  Needs an
MI355X and the built libda.so.
"""

from __future__ import annotations

import sys

import numpy as np
import pytest
import torch

import oracle
import oracle.quant as oq
import oracle.quant4 as oq4
from harness import TOL_OUT, compare_out, compare_partials, host_inputs, oracle_micro, oracle_out
from long_context_decode_microattention_amd import _lib
from long_context_decode_microattention_amd import workloads as wl

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
N_CASES = 64


def draw(i: int):
    """Case i: a workload spec, a seed and the launch options."""
    rng = np.random.default_rng(1000 + i)
    G = int(rng.choice([1, 2, 4, 8]))
    Hkv = int(rng.choice([1, 2, 3, 4]))
    D = int(rng.choice([64, 128]))
    P = int(rng.choice([16, 32, 64, 128, 256]))
    dtype = wl.F32 if rng.random() < 0.25 else wl.BF16
    S = int(rng.integers(1, 5))
    if rng.random() < 0.5:
        lens = ("fixed", int(rng.integers(1, 6000)))
    else:
        lens = ("loguniform", int(rng.integers(64, 8000)))
    b = int(rng.integers(1, 9))
    splits = ("equal", b) if rng.random() < 0.6 else ("chunk", int(rng.integers(P, 4 * P + 1)))
    mask = ("lserve", 1, 1, float(rng.choice([0.1, 0.25, 0.5]))) if Hkv >= 2 and rng.random() < 0.5 else None
    if mask is not None and rng.random() < 0.5:
        splits = ("kept_pages", b)
    spec = wl.Spec(f"random case {i}", S=S, Hq=Hkv * G, Hkv=Hkv, D=D, P=P, dtype=dtype, lens=lens,
                   table="shuffled" if rng.random() < 0.7 else "identity", splits=splits, mask=mask,
                   extra_pages=int(rng.integers(0, 4)),
                   layout="head" if rng.random() < 0.3 else "page")
    chunks = int(rng.choice([0, 0, 1, 2, 5]))
    schedule = int(rng.choice([0, 0, 1, 2]))
    return spec, int(rng.integers(0, 1 << 16)), chunks, schedule


def announce(*parts):
    print("[gpu-case]", *parts, flush=True)
    sys.stdout.flush()


@pytest.fixture(autouse=True)
def _free_memory():
    yield
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


@pytest.mark.parametrize("i", range(N_CASES))
def test_random_shape(i):
    spec, seed, chunks, schedule = draw(i)
    announce("random", i, spec, "seed", seed, "chunks", chunks, "schedule", schedule)
    b = wl.build(spec, seed, DEV)
    args = (b.q, b.k_pages, b.v_pages, b.block_table, b.seq_lens, b.split_bounds, b.block_mask)
    ws = torch.empty(1 << 24, dtype=torch.uint8, device=DEV)
    MA, m, e = _lib.micro_attention(*args, scale=b.scale, chunks=chunks, schedule=schedule,
                                    workspace=ws, pool_layout=b.layout)
    out = _lib.merge(MA, m, e)
    out1 = _lib.attention(*args, scale=b.scale, chunks=chunks, schedule=schedule,
                          pool_layout=b.layout)
    torch.cuda.synchronize()
    inp = host_inputs(b)
    tol = TOL_OUT[spec.dtype]
    want = oracle_out(inp, b.scale)
    compare_out(out.cpu().numpy(), want, tol, f"case {i} out")
    compare_out(out1.cpu().numpy(), want, tol, f"case {i} one-launch out")
    oMA, om, oe = oracle_micro(inp, b.scale)
    compare_partials(MA.cpu().numpy(), m.cpu().numpy(), e.cpu().numpy(), oMA, om, oe, tol,
                     f"case {i} partials")
    if spec.dtype != wl.BF16:
        return
    # the same pools in 8 bits: attention over the dequantized values
    kc, ks = _lib.quantize_rows(b.k_pages)
    vc, vs = _lib.quantize_rows(b.v_pages)
    args8 = (b.q, kc, ks, vc, vs, b.block_table, b.seq_lens, b.split_bounds, b.block_mask)
    MA8, m8, e8 = _lib.micro_attention_fp8(*args8, scale=b.scale, chunks=chunks,
                                           schedule=schedule, workspace=ws, pool_layout=b.layout)
    out8 = _lib.merge(MA8, m8, e8)
    torch.cuda.synchronize()
    h = wl.host
    if b.layout == "head":  # the oracle takes page-major pools
        kc, ks, vc, vs = (t.transpose(0, 1).contiguous() for t in (kc, ks, vc, vs))
    kd = oq.dequantize(h(kc), h(ks))
    vd = oq.dequantize(h(vc), h(vs))
    want8 = oracle.attention(inp["q"], kd, vd, inp["block_table"], inp["seq_lens"],
                             block_mask=inp["block_mask"], scale=b.scale)
    compare_out(out8.cpu().numpy(), want8, tol, f"case {i} 8-bit out")
    # and in 4 bits (D = 64 with one query head per KV head needs pages of 32
    # tokens or more)
    if spec.D == 64 and spec.G == 1 and spec.P < 32:
        return
    kc4, ks4 = _lib.quantize_rows_fp4(b.k_pages)
    vc4, vs4 = _lib.quantize_rows_fp4(b.v_pages)
    args4 = (b.q, kc4, ks4, vc4, vs4, b.block_table, b.seq_lens, b.split_bounds, b.block_mask)
    MA4, m4, e4 = _lib.micro_attention_fp4(*args4, scale=b.scale, chunks=chunks,
                                           schedule=schedule, workspace=ws, pool_layout=b.layout)
    out4 = _lib.merge(MA4, m4, e4)
    torch.cuda.synchronize()
    if b.layout == "head":
        kc4, ks4, vc4, vs4 = (t.transpose(0, 1).contiguous() for t in (kc4, ks4, vc4, vs4))
    want4 = oracle.attention(inp["q"], oq4.dequantize(h(kc4), h(ks4)),
                             oq4.dequantize(h(vc4), h(vs4)), inp["block_table"], inp["seq_lens"],
                             block_mask=inp["block_mask"], scale=b.scale)
    compare_out(out4.cpu().numpy(), want4, tol, f"case {i} 4-bit out")
