"""Head-major pools ([Hkv, NP, P, D]) against page-major pools ([NP, Hkv, P, D])
holding the same values, through every entry point that takes pools.  Only
addresses differ between the two, so every result must be bitwise identical;
one attention case is also compared with the fp64 oracle.  Needs an MI355X
and the built libda.so."""

from __future__ import annotations

import sys

import numpy as np
import pytest
import torch

from harness import TOL_OUT, compare_out, host_inputs, oracle_out, run_gpu
from long_context_decode_microattention_amd import _lib
from long_context_decode_microattention_amd import workloads as wl

pytestmark = pytest.mark.gpu

DEV = "cuda:0"

CASES = {
    "C1": wl.CONFIGS["C1"],
    "C3": wl.CONFIGS["C3"].replace(S=6, Hq=8, Hkv=8),
    "C4": wl.CONFIGS["C4"].replace(Hq=8, Hkv=8, lens=("fixed", 16384 + 21)),
    "C5": wl.CONFIGS["C5"].replace(S=2, lens=("fixed", 16384 + 5)),
    "C5_G8_D64": wl.CONFIGS["C5"].replace(S=1, Hq=64, D=64, lens=("fixed", 8192 + 50)),
    # 16-token pages under a shuffled table (one slab per page), and 32-token
    # pages under the grouped-query kernel (one 32-row 8-bit slab per page)
    "C2": wl.CONFIGS["C2"].replace(S=2),
    "C5_P32": wl.CONFIGS["C5"].replace(S=2, P=32, lens=("fixed", 8192 + 13)),
    # the largest page size built, mid-slab splits
    "C4_P256": wl.CONFIGS["C4"].replace(Hq=4, Hkv=4, P=256, lens=("fixed", 256 * 20 + 77),
                                        splits=("equal", 5)),
}


def announce(*parts):
    print("[gpu-case]", *parts, flush=True)
    sys.stdout.flush()


@pytest.fixture(autouse=True)
def _free_memory():
    yield
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def _pair(cfg, seed=0, **kw):
    spec = CASES[cfg].replace(**kw)
    return wl.build(spec, seed, DEV), wl.build(spec.replace(layout="head"), seed, DEV)


def _same(a, b, what):
    assert torch.equal(a, b), f"{what}: head-major result differs from page-major"


@pytest.mark.parametrize("cfg", sorted(CASES))
def test_attention_layouts_identical(cfg):
    announce("layout attention", cfg)
    bp, bh = _pair(cfg)
    for chunks in (0, 3):
        rp = run_gpu(bp, chunks=chunks)
        rh = run_gpu(bh, chunks=chunks)
        for x, y, name in zip(rp, rh, ("out", "MA", "m", "e")):
            _same(x, y, f"{cfg} chunks={chunks} {name}")
    want = oracle_out(host_inputs(bh), bh.scale)
    compare_out(rh[0].cpu().numpy(), want, TOL_OUT[bh.spec.dtype], f"{cfg} head-major vs oracle")


@pytest.mark.parametrize("cfg", ["C2", "C4", "C5", "C5_G8_D64", "C5_P32"])
def test_fp8_layouts_identical(cfg):
    announce("layout fp8", cfg)
    bp, bh = _pair(cfg)
    outs = []
    for b in (bp, bh):
        kc, ks = _lib.quantize_rows(b.k_pages)
        vc, vs = _lib.quantize_rows(b.v_pages)
        MA, m, e = _lib.micro_attention_fp8(b.q, kc, ks, vc, vs, b.block_table, b.seq_lens,
                                            b.split_bounds, b.block_mask, scale=b.scale,
                                            pool_layout=b.layout)
        outs.append((_lib.merge(MA, m, e), kc, ks))
    _same(outs[0][0], outs[1][0], f"{cfg} fp8 out")
    _same(outs[0][1], outs[1][1].transpose(0, 1), f"{cfg} codes")
    _same(outs[0][2], outs[1][2].transpose(0, 1), f"{cfg} scales")


@pytest.mark.parametrize("cfg", ["C3", "C5"])
def test_selection_layouts_identical(cfg):
    announce("layout selection", cfg)
    bp, bh = _pair(cfg, table="shuffled", extra_pages=3)
    P = bp.spec.P
    flags = torch.tensor([1 if h >= bp.spec.Hkv // 2 else 0 for h in range(bp.spec.Hkv)],
                         dtype=torch.uint8, device=DEV)
    res = []
    for b in (bp, bh):
        st = _lib.page_stats(b.k_pages, b.block_table, b.seq_lens, logical=16, select_heads=flags,
                             pool_layout=b.layout)
        sc = _lib.page_scores(b.q, st, b.block_table, b.seq_lens, P=P, select_heads=flags)
        res.append((st, sc))
    _same(res[0][0], res[1][0], f"{cfg} statistics")
    _same(res[0][1], res[1][1], f"{cfg} scores")


@pytest.mark.parametrize("cfg", ["C4", "C5"])
def test_append_layouts_identical(cfg):
    """bf16 and 8-bit appends with statistics over 20 steps."""
    announce("layout append", cfg)
    bp, bh = _pair(cfg, reserve=24, table="shuffled", extra_pages=2)
    spec = bp.spec
    flags = torch.tensor([1 if h >= spec.Hkv // 2 else 0 for h in range(spec.Hkv)],
                         dtype=torch.uint8, device=DEV)
    state = []
    for b in (bp, bh):
        st = _lib.page_stats(b.k_pages, b.block_table, b.seq_lens, logical=16, select_heads=flags,
                             pool_layout=b.layout)
        st8 = st.clone()
        kc, ks = _lib.quantize_rows(b.k_pages)
        vc, vs = _lib.quantize_rows(b.v_pages)
        state.append(dict(b=b, st=st, st8=st8, kc=kc, ks=ks, vc=vc, vs=vs,
                          lens=b.seq_lens.clone()))
    for step in range(20):
        kn, vn = wl.new_tokens(spec, 6, step, DEV)
        for x in state:
            b = x["b"]
            _lib.append_kv(kn, vn, b.block_table, x["lens"], b.k_pages, b.v_pages, stats=x["st"],
                           select_heads=flags, pool_layout=b.layout)
            _lib.append_kv_fp8(kn, vn, b.block_table, x["lens"], x["kc"], x["ks"], x["vc"], x["vs"],
                               stats=x["st8"], select_heads=flags, pool_layout=b.layout)
            x["lens"] += 1
    p, h = state
    _same(p["b"].k_pages, h["b"].k_pm, f"{cfg} K pool")
    _same(p["b"].v_pages, h["b"].v_pm, f"{cfg} V pool")
    _same(p["st"], h["st"], f"{cfg} statistics (bf16 append)")
    _same(p["st8"], h["st8"], f"{cfg} statistics (8-bit append)")
    for name in ("kc", "ks", "vc", "vs"):
        _same(p[name], h[name].transpose(0, 1), f"{cfg} 8-bit {name}")
