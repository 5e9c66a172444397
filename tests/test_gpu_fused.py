"""The fused decode step (da_attention / da_attention_fp8: MicroAttention
partials and their merge in one launch, the merge done by the item that
completes each (request, KV head)) through the C ABI, against the fp64
oracle on the same seeded inputs, and against the two-call path
(da_micro_attention + da_merge) on the same inputs.  Needs an MI355X and the
built libda.so.

Bars: the workload tolerance on the output against the oracle (2e-3 bf16
and 8-bit K/V, 1e-5 fp32); against the two-call path 1e-5 (bf16) / 1e-6
(fp32) max-abs, the two folding the same fp32 partials in different orders.
The group counters must be zero after every call (the next call relies on
it), checked directly on the workspace.
"""

from __future__ import annotations

import sys

import numpy as np
import pytest
import torch

import oracle
import oracle.quant as oq
from harness import TOL_OUT, compare_out, host_inputs, oracle_out
from long_context_decode_microattention_amd import _lib
from long_context_decode_microattention_amd import workloads as wl

pytestmark = pytest.mark.gpu

DEV = "cuda:0"

REDUCED = {
    "C1": wl.CONFIGS["C1"],
    "C2": wl.CONFIGS["C2"].replace(S=2),
    "C3": wl.CONFIGS["C3"].replace(S=6, Hq=8, Hkv=8),
    "C4": wl.CONFIGS["C4"].replace(Hq=8, Hkv=8, lens=("fixed", 32768)),
    "C5": wl.CONFIGS["C5"].replace(S=2, lens=("fixed", 32768)),
    # eight query heads per KV head (the dense value product over bf16 pages)
    "C5_G8": wl.CONFIGS["C5"].replace(S=1, Hq=64, lens=("fixed", 16384 + 50)),
}
TOL_SAME = {wl.F32: 1e-6, wl.BF16: 1e-5}


def announce(*parts):
    print("[gpu-case]", *parts, flush=True)
    sys.stdout.flush()


@pytest.fixture(autouse=True)
def _free_memory():
    yield
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def fused_workspace(b: wl.Batch, chunks: int = 0, schedule: int = 0):
    """A caller-owned workspace for the batch's shape, zero-filled once, and
    the size of its counter prefix."""
    sh = _lib.shape_of(b.q, b.k_pages, b.block_table, b.split_bounds, b.scale, chunks, schedule,
                       b.layout)
    nbytes, counters = _lib.attention_workspace_size(sh)
    return torch.zeros(nbytes, dtype=torch.uint8, device=DEV), counters


def fused(b: wl.Batch, ws=None, chunks: int = 0, schedule: int = 0, fuse: int = 0):
    out = _lib.attention(b.q, b.k_pages, b.v_pages, b.block_table, b.seq_lens, b.split_bounds,
                         b.block_mask, scale=b.scale, chunks=chunks, schedule=schedule,
                         workspace=ws, pool_layout=b.layout, fuse=fuse)
    torch.cuda.synchronize()
    return out


def two_call(b: wl.Batch, chunks: int = 0, schedule: int = 0):
    MA, m, e = _lib.micro_attention(b.q, b.k_pages, b.v_pages, b.block_table, b.seq_lens,
                                    b.split_bounds, b.block_mask, scale=b.scale, chunks=chunks,
                                    schedule=schedule, pool_layout=b.layout)
    out = _lib.merge(MA, m, e)
    torch.cuda.synchronize()
    return out


def max_abs(a: torch.Tensor, b: torch.Tensor) -> float:
    return float((a.double() - b.double()).abs().max())


@pytest.mark.parametrize("fuse", [0, 1, 2])
@pytest.mark.parametrize("seed", [0, 1])
@pytest.mark.parametrize("cfg", sorted(REDUCED))
def test_fused_matches_oracle_and_two_call_path(cfg, seed, fuse):
    """fuse 1: the merge in the same launch; 2: partials then the merge
    kernel; 0: the library's choice between them."""
    spec = REDUCED[cfg].replace(layout=wl.PREFERRED_LAYOUT.get(cfg, "page"))
    announce("fused", cfg, "seed", seed, "fuse", fuse)
    b = wl.build(spec, seed, DEV)
    ws, counters = fused_workspace(b)
    out = fused(b, ws, fuse=fuse)
    compare_out(out.cpu().numpy(), oracle_out(host_inputs(b), b.scale), TOL_OUT[spec.dtype],
                f"fused {cfg}/{seed}")
    ref = two_call(b)
    assert max_abs(out, ref) <= TOL_SAME[spec.dtype], f"fused vs two-call {cfg}/{seed}"
    assert int(ws[:counters].count_nonzero()) == 0, "group counters not cleared"


@pytest.mark.parametrize("fuse", [1, 2])
@pytest.mark.parametrize("schedule,chunks", [(1, 0), (2, 0), (1, 1), (1, 3), (2, 3), (1, 7),
                                             (2, 16), (1, 40)])
@pytest.mark.parametrize("cfg", ["C1", "C3", "C5"])
def test_fused_schedules_and_chunks(cfg, schedule, chunks, fuse):
    """One workgroup per item and persistent workgroups on the work queue,
    with forced chunk counts, in one launch (the merge runs over every piece
    partial; 40 pieces: more than 2 D partials per head, the merge's
    head-by-head branch) and in two (the merge kernel over them)."""
    spec = REDUCED[cfg]
    announce("fused schedule", cfg, schedule, chunks, fuse)
    b = wl.build(spec, 5, DEV)
    ws, counters = fused_workspace(b, chunks, schedule)
    out = fused(b, ws, chunks, schedule, fuse)
    compare_out(out.cpu().numpy(), oracle_out(host_inputs(b), b.scale), TOL_OUT[spec.dtype],
                f"fused {cfg} schedule={schedule} chunks={chunks} fuse={fuse}")
    assert int(ws[:counters].count_nonzero()) == 0


def test_fused_repeated_calls_and_growing_shapes():
    """The counters each call leaves at zero serve the next: ten calls on one
    workspace give identical bits; then the binding's cached workspace
    serves a small shape, a larger one (more counters, reaching over the
    small call's partials) and the small one again, each matching the
    two-call path."""
    spec = REDUCED["C5"]
    announce("fused repeat")
    b = wl.build(spec, 2, DEV)
    ws, counters = fused_workspace(b)
    first = fused(b, ws)
    for i in range(9):
        again = fused(b, ws)
        assert torch.equal(first, again), f"call {i + 2} differs"
    assert int(ws[:counters].count_nonzero()) == 0
    small = wl.build(REDUCED["C1"], 3, DEV)
    big = wl.build(REDUCED["C3"], 3, DEV)
    for bb in (small, big, small, b, small):
        got = fused(bb)  # cached workspace of the binding
        assert max_abs(got, two_call(bb)) <= TOL_SAME[bb.spec.dtype], bb.spec.name


@pytest.mark.parametrize("schedule", [1, 2])
def test_fused_many_groups_same_bits_every_call(schedule):
    """Many groups of short, chunked items (every group's last arrival
    merges partials other workgroups wrote moments before): 20 calls give
    the same bits, equal to the two calls within fp32 rounding."""
    spec = REDUCED["C3"]
    announce("fused many groups", schedule)
    b = wl.build(spec, 11, DEV)
    ws, counters = fused_workspace(b, 3, schedule)
    first = fused(b, ws, 3, schedule)
    assert max_abs(first, two_call(b, 3, schedule)) <= TOL_SAME[spec.dtype]
    for i in range(19):
        assert torch.equal(fused(b, ws, 3, schedule), first), f"call {i + 2} differs"
    assert int(ws[:counters].count_nonzero()) == 0


def test_fused_masks_empty_requests_and_poison():
    """All-masked-but-one page, only the partial last page kept, an empty
    request (output 0) and NaN in every page slot no split may read."""
    spec = wl.Spec("fused mask edge", S=3, Hq=8, Hkv=2, D=128, P=64, dtype=wl.BF16,
                   lens=("fixed", 64 * 9 + 5), splits=("equal", 4), extra_pages=3)
    announce("fused mask edge")
    b = wl.build(spec, 23, DEV)
    mask = torch.zeros((3, 2, b.block_table.shape[1]), dtype=torch.uint8, device=DEV)
    mask[0, 0, 4] = 1
    mask[1, 1, 9] = 1
    mask[2, :, :] = 1
    b.block_mask = mask
    b.seq_lens[2] = 0
    table = b.block_table.cpu().numpy()
    used = np.zeros(b.k_pages.shape[0], dtype=bool)
    for s, L in enumerate(b.seq_lens.cpu().numpy()):
        n = -(-int(L) // 64)
        mk = mask[s].cpu().numpy()
        for h in range(2):
            for lp in range(n):
                if mk[h, lp]:
                    used[table[s, lp]] = True
                else:
                    b.k_pages[int(table[s, lp]), h] = float("nan")
                    b.v_pages[int(table[s, lp]), h] = float("nan")
        if L % 64 and n:
            pg = int(table[s, n - 1])
            b.k_pages[pg, :, L % 64:] = float("nan")
            b.v_pages[pg, :, L % 64:] = float("nan")
    unused = torch.from_numpy(np.nonzero(~used)[0]).to(DEV)
    b.k_pages[unused] = float("nan")
    b.v_pages[unused] = float("nan")
    out = fused(b)
    inp = host_inputs(b)
    compare_out(out.cpu().numpy(), oracle.attention(inp["q"], inp["k_pool"], inp["v_pool"],
                                                    inp["block_table"], inp["seq_lens"],
                                                    block_mask=inp["block_mask"], scale=b.scale),
                2e-3, "fused mask edge")
    assert torch.equal(out[2], torch.zeros_like(out[2]))
    assert torch.equal(out[0, 4:], torch.zeros_like(out[0, 4:])), "KV head 1 of request 0 is all masked"


@pytest.mark.parametrize("cfg", ["C2", "C4", "C5", "C5_G8"])
def test_fused_fp8_pages(cfg):
    """8-bit pages: the fused step against the oracle over the dequantized
    pools and against da_micro_attention_fp8 + da_merge."""
    spec = REDUCED[cfg].replace(S=min(REDUCED[cfg].S, 2))
    if cfg == "C4":
        spec = spec.replace(lens=("fixed", 8192))
    announce("fused fp8", cfg)
    b = wl.build(spec, 9, DEV)
    kc, ks = _lib.quantize_rows(b.k_pages)
    vc, vs = _lib.quantize_rows(b.v_pages)
    args = (b.q, kc, ks, vc, vs, b.block_table, b.seq_lens, b.split_bounds, b.block_mask)
    out = _lib.attention_fp8(*args, scale=b.scale)
    MA, m, e = _lib.micro_attention_fp8(*args, scale=b.scale)
    ref = _lib.merge(MA, m, e)
    torch.cuda.synchronize()
    assert max_abs(out, ref) <= 1e-5
    h = wl.host
    kd = oq.dequantize(h(kc), h(ks))
    vd = oq.dequantize(h(vc), h(vs))
    want = oracle.attention(h(b.q), kd, vd, h(b.block_table), h(b.seq_lens),
                            block_mask=None if b.block_mask is None else h(b.block_mask),
                            scale=b.scale)
    compare_out(out.cpu().numpy(), want, 2e-3, f"fused fp8 {cfg}")


@pytest.mark.parametrize("cfg", ["C4", "C5"])
@pytest.mark.slow
def test_fused_full_size_against_two_call(cfg):
    """Full-size workloads in the layout the benchmark times: the fused step
    equals the two-call path (which the full-size sampled parity test pins
    to the oracle) within fp32 rounding."""
    spec = wl.CONFIGS[cfg].replace(layout=wl.PREFERRED_LAYOUT.get(cfg, "page"))
    announce("fused full", cfg)
    b = wl.build(spec, 0, DEV)
    out = fused(b)
    ref = two_call(b)
    assert torch.isfinite(out).all()
    assert max_abs(out, ref) <= 1e-5, f"{cfg}: fused vs two-call"
