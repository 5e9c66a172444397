"""The instance-side fold of distributed decoding (da_merge_partials) through
the C ABI: each instance folds its own splits into one triple per (request,
head) and writes it into its slot of a gather buffer; the master merges the
gathered triples with da_merge.  Checked against the fp64 oracle's attention
and its partial fold on the same inputs."""

from __future__ import annotations

import sys

import numpy as np
import pytest
import torch

import oracle
from harness import compare_out, compare_partials, host_inputs, oracle_out, run_gpu
from long_context_decode_microattention_amd import _lib
from long_context_decode_microattention_amd import workloads as wl

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def announce(*parts):
    print("[gpu-case]", *parts, flush=True)
    sys.stdout.flush()


@pytest.fixture(autouse=True)
def _free_memory():
    yield
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def _instance_inputs(b: wl.Batch, pg_lo: int, pg_hi: int):
    """The pages one instance holds: logical pages [pg_lo, pg_hi) of every
    request, copied into a compact pool of its own, and a block table that
    maps those logical pages to it (entries outside the range are 0 and are
    never read, since the instance's splits stay inside the range)."""
    S = b.spec.S
    span = pg_hi - pg_lo
    idx = torch.cat([b.block_table[s, pg_lo:pg_hi] for s in range(S)]).long()
    k = b.k_pm.index_select(0, idx).contiguous()
    v = b.v_pm.index_select(0, idx).contiguous()
    tab = torch.zeros_like(b.block_table)
    for s in range(S):
        tab[s, pg_lo:pg_hi] = torch.arange(s * span, (s + 1) * span, dtype=torch.int32,
                                           device=b.block_table.device)
    return k, v, tab


@pytest.mark.parametrize("Hq,Hkv,dtype,masked", [
    (8, 2, wl.BF16, True),    # grouped-query heads (matrix-core kernel), block-sparse upper half
    (8, 2, wl.BF16, False),
    (4, 4, wl.F32, False),    # one query head per KV head (vector kernel), fp32 pages
])
def test_instances_fold_gather_merge(Hq, Hkv, dtype, masked):
    """Four instances over uneven page ranges, three splits each (cut mid
    page): fold, gather, merge equals the oracle's attention, and each
    gathered triple equals the oracle's MicroAttention over the instance's
    whole token range."""
    P = 64
    L = P * 47 + 29  # ragged last page
    spec = wl.Spec("instances", S=2, Hq=Hq, Hkv=Hkv, D=128, P=P, dtype=dtype,
                   lens=("fixed", L), table="shuffled", splits=("equal", 1),
                   mask=("lserve", 1, 2, 0.25) if masked else None)
    announce("instances", Hq, Hkv, dtype, masked)
    b = wl.build(spec, 31, DEV)
    n = -(-L // P)
    page_cuts = [0, 5, 19, 30, n]
    n_inst = len(page_cuts) - 1
    S, D = spec.S, spec.D
    gather = (torch.full((S, Hq, n_inst, D), float("nan"), device=DEV),
              torch.full((S, Hq, n_inst), float("nan"), device=DEV),
              torch.full((S, Hq, n_inst), float("nan"), device=DEV))
    ranges = []
    for i in range(n_inst):
        lo, hi = page_cuts[i] * P, min(page_cuts[i + 1] * P, L)
        ranges.append((lo, hi))
        k, v, tab = _instance_inputs(b, page_cuts[i], page_cuts[i + 1])
        cuts = [lo, lo + (hi - lo) // 3 + 7, lo + 2 * (hi - lo) // 3 + 13, hi]
        sb = torch.tensor([[cuts]] * S, dtype=torch.int32, device=DEV)
        MA, m, e = _lib.micro_attention(b.q, k, v, tab, b.seq_lens, sb, b.block_mask,
                                        scale=b.scale)
        _lib.merge_partials(MA, m, e, out=gather, slot=i)
    out = _lib.merge(*gather)
    torch.cuda.synchronize()
    inp = host_inputs(b)
    tol = 2e-3 if dtype == wl.BF16 else 1e-5
    compare_out(out.cpu().numpy(), oracle_out(inp, b.scale), tol, "gathered")
    single, *_ = run_gpu(b)
    compare_out(single.cpu().numpy(), oracle_out(inp, b.scale), tol, "single call")

    oMA = np.zeros((S, Hq, n_inst, D))
    om = np.zeros((S, Hq, n_inst))
    oe = np.zeros((S, Hq, n_inst))
    for i, (lo, hi) in enumerate(ranges):
        sb = np.repeat(np.array([[[lo, hi]]], dtype=np.int32), S, axis=0)
        a, bm, c = oracle.micro_attention(inp["q"], inp["k_pool"], inp["v_pool"],
                                          inp["block_table"], inp["seq_lens"], sb,
                                          block_mask=inp["block_mask"], scale=b.scale)
        oMA[:, :, i], om[:, :, i], oe[:, :, i] = a[:, :, 0], bm[:, :, 0], c[:, :, 0]
    compare_partials(gather[0].cpu().numpy(), gather[1].cpu().numpy(), gather[2].cpu().numpy(),
                     oMA, om, oe, tol, "gathered triples")


def _synthetic_partials(rng, S, Hq, B, D, empty_rows=True):
    """Partials that follow the library's convention: m in [-30, 30], e > 0,
    MA of the size e times a unit vector; ~20% empty (0, -inf, 0) entries and
    one (request, head) whose entries are all empty."""
    m = rng.uniform(-30, 30, size=(S, Hq, B)).astype(np.float32)
    e = rng.uniform(1, 1000, size=(S, Hq, B)).astype(np.float32)
    MA = (rng.standard_normal((S, Hq, B, D)) * e[..., None] / 4).astype(np.float32)
    empty = rng.random((S, Hq, B)) < 0.2
    if empty_rows:
        empty[0, 0, :] = True
    m[empty] = -np.inf
    e[empty] = 0
    MA[empty] = 0
    return MA, m, e


def _to_dev(*xs):
    return [torch.from_numpy(np.ascontiguousarray(x)).to(DEV) for x in xs]


@pytest.mark.parametrize("B,D", [(1, 128), (37, 128), (300, 64), (5, 320)])
def test_fold_matches_oracle(B, D):
    """The fold of the same fp32 partials against the oracle's fold in fp64:
    m' exact (a maximum), e' and MA' within fp32 rounding of the weighted
    sums; all-empty rows give (0, -inf, 0).  D = 320 takes the kernel's
    wide-row path, B = 300 its chunked split loop."""
    rng = np.random.default_rng(B * 1000 + D)
    S, Hq = 3, 5
    MA, m, e = _synthetic_partials(rng, S, Hq, B, D)
    announce("fold", B, D)
    gMA, gm, ge = _lib.merge_partials(*_to_dev(MA, m, e))
    torch.cuda.synchronize()
    gMA, gm, ge = gMA.cpu().numpy()[:, :, 0], gm.cpu().numpy()[:, :, 0], ge.cpu().numpy()[:, :, 0]
    oMA, om, oe = oracle.merge_partials(MA, m, e)
    assert np.array_equal(gm, om.astype(np.float32)), "m' differs from the maximum"
    empty = np.isneginf(om)
    assert empty[0, 0] and np.all(ge[empty] == 0) and np.all(gMA[empty] == 0)
    full = ~empty
    assert np.max(np.abs(ge[full] - oe[full]) / oe[full]) <= 1e-5
    m64 = m.astype(np.float64)
    top = np.max(m64, axis=-1, keepdims=True)
    w = np.where(np.isneginf(m64), 0.0, np.exp(m64 - np.where(np.isneginf(top), 0.0, top)))
    scale = np.einsum("shb,shbd->shd", w, np.abs(MA.astype(np.float64)))
    assert np.max(np.abs(gMA - oMA) / np.maximum(scale, 1e-30)) <= 1e-5


def test_fold_writes_only_its_slot():
    """Every other slot of the gather buffer keeps its bytes (NaN here)."""
    rng = np.random.default_rng(7)
    MA, m, e = _synthetic_partials(rng, 2, 3, 9, 128, empty_rows=False)
    announce("fold-slot")
    n_out, slot = 3, 1
    out = (torch.full((2, 3, n_out, 128), float("nan"), device=DEV),
           torch.full((2, 3, n_out), float("nan"), device=DEV),
           torch.full((2, 3, n_out), float("nan"), device=DEV))
    _lib.merge_partials(*_to_dev(MA, m, e), out=out, slot=slot)
    torch.cuda.synchronize()
    for t in out:
        others = torch.cat([t[:, :, :slot], t[:, :, slot + 1:]], dim=2)
        assert torch.isnan(others).all()
        assert not torch.isnan(t[:, :, slot]).any()


def test_hierarchical_fold_equals_direct_merge():
    """Folding groups of partials, then folding the folds, then merging gives
    the attention of merging everything at once (the fold is associative),
    and the oracle's merge of the original partials."""
    rng = np.random.default_rng(11)
    S, Hq, B, D = 2, 4, 48, 128
    MA, m, e = _synthetic_partials(rng, S, Hq, B, D)
    dMA, dm, de = _to_dev(MA, m, e)
    announce("fold-tree")
    groups = [(0, 5), (5, 6), (6, 30), (30, 48)]
    level1 = (torch.empty((S, Hq, len(groups), D), device=DEV),
              torch.empty((S, Hq, len(groups)), device=DEV),
              torch.empty((S, Hq, len(groups)), device=DEV))
    for i, (lo, hi) in enumerate(groups):
        _lib.merge_partials(dMA[:, :, lo:hi].contiguous(), dm[:, :, lo:hi].contiguous(),
                            de[:, :, lo:hi].contiguous(), out=level1, slot=i)
    level2 = (torch.empty((S, Hq, 2, D), device=DEV), torch.empty((S, Hq, 2), device=DEV),
              torch.empty((S, Hq, 2), device=DEV))
    for i, (lo, hi) in enumerate([(0, 3), (3, 4)]):
        _lib.merge_partials(*(x[:, :, lo:hi].contiguous() for x in level1), out=level2, slot=i)
    tree = _lib.merge(*level2)
    direct = _lib.merge(dMA, dm, de)
    torch.cuda.synchronize()
    want = oracle.merge(MA, m, e)
    compare_out(tree.cpu().numpy(), want, 1e-5, "tree")
    compare_out(direct.cpu().numpy(), want, 1e-5, "direct")
    assert np.all(tree.cpu().numpy()[0, 0] == 0)  # all-empty row stays 0
