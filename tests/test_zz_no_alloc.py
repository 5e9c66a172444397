"""da_attention_noalloc (the step of da_attention with the library's per-GPU
scratch array instead of a workspace) through the C ABI: two calls in a row,
the second on a smaller input, each against da_attention on the same inputs
(the same kernels and partial order: equal within fp32 rounding, 1e-5) and
against the fp64 oracle at the workload tolerance; both forms of the step;
and a shape whose step needs more than the array is refused before launch.
Needs an MI355X and the built libda.so."""

from __future__ import annotations

import sys

import pytest
import torch

from harness import TOL_OUT, compare_out, host_inputs, oracle_out
from long_context_decode_microattention_amd import _lib
from long_context_decode_microattention_amd import workloads as wl

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def announce(*parts):
    print("[gpu-case]", *parts, flush=True)
    sys.stdout.flush()


def _step(fn, b, fuse=0):
    out = fn(b.q, b.k_pages, b.v_pages, b.block_table, b.seq_lens, b.split_bounds, b.block_mask,
             scale=b.scale, pool_layout=b.layout, fuse=fuse)
    torch.cuda.synchronize()
    return out


@pytest.mark.parametrize("fuse", [0, 1, 2])
def test_noalloc_two_calls_against_da_attention(fuse):
    big = wl.build(wl.CONFIGS["C5"].replace(S=2, lens=("fixed", 32768), layout="head"), 4, DEV)
    small = wl.build(wl.CONFIGS["C1"], 4, DEV)
    for b in (big, small):  # the second call is the smaller input
        announce("noalloc", b.spec.name, "fuse", fuse)
        got = _step(_lib.attention_noalloc, b, fuse)
        ref = _step(_lib.attention, b, fuse)
        assert torch.isfinite(got).all()
        assert float((got - ref).abs().max()) <= 1e-5, f"{b.spec.name}: noalloc vs da_attention"
        compare_out(got.cpu().numpy(), oracle_out(host_inputs(b), b.scale), TOL_OUT[b.spec.dtype],
                    f"noalloc {b.spec.name} fuse={fuse}")


def test_noalloc_refuses_a_step_larger_than_its_scratch():
    announce("noalloc refuse")
    S, H, D, b = 64, 64, 128, 32  # 64 * 64 * 32 partials of 130 floats: 68 MB > 32 MiB
    q = torch.zeros((S, H, D), dtype=torch.bfloat16, device=DEV)
    k = torch.zeros((1, H, 16, D), dtype=torch.bfloat16, device=DEV)
    table = torch.zeros((S, 1), dtype=torch.int32, device=DEV)
    lens = torch.ones(S, dtype=torch.int32, device=DEV)
    bounds = torch.zeros((S, 1, b + 1), dtype=torch.int32, device=DEV)
    bounds[:, 0, 1:] = 1
    with pytest.raises(_lib.DaError) as ei:
        _lib.attention_noalloc(q, k, k, table, lens, bounds)
    assert ei.value.status == _lib.DA_ERR_INVALID_ARG
    assert "scratch" in ei.value.message
