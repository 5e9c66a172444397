"""Shared helpers for the GPU tests: run the HIP path through the C ABI, run
the fp64 oracle on host copies of the same seeded inputs, and compare.

Tolerances: max-abs error on the attention output of 1e-5 for fp32 K/V and
2e-3 for bf16 K/V; m_j within 1e-4 * max(1, |m_j|); e_j within 1e-4
relative; MA_j / e_j within the output tolerance.  Empty splits must be
exactly (MA = 0, m = -inf, e = 0).  Integer and index work is bit-exact.
"""

from __future__ import annotations

import numpy as np
import torch

import oracle
from long_context_decode_microattention_amd import _lib
from long_context_decode_microattention_amd import workloads as wl

TOL_OUT = {wl.F32: 1e-5, wl.BF16: 2e-3}


def run_gpu(batch: wl.Batch, chunks: int = 0, workspace=None, schedule: int = 0):
    MA, m, e = _lib.micro_attention(batch.q, batch.k_pages, batch.v_pages, batch.block_table,
                                    batch.seq_lens, batch.split_bounds, batch.block_mask,
                                    scale=batch.scale, chunks=chunks, workspace=workspace,
                                    schedule=schedule, pool_layout=batch.layout)
    out = _lib.merge(MA, m, e)
    torch.cuda.synchronize()
    return out, MA, m, e


def host_inputs(batch: wl.Batch):
    h = wl.host
    return dict(q=h(batch.q), k_pool=h(batch.k_pm), v_pool=h(batch.v_pm),
                block_table=h(batch.block_table), seq_lens=h(batch.seq_lens),
                split_bounds=h(batch.split_bounds),
                block_mask=None if batch.block_mask is None else h(batch.block_mask))


def sub_inputs(batch: wl.Batch, s: int, kv_lo: int, kv_hi: int):
    """Host copies of request s restricted to KV heads [kv_lo, kv_hi) and the
    query heads of their groups, with the request's pages gathered into a
    compact pool (block table renumbered 0..n-1).  Data selection only."""
    sp = batch.spec
    G = sp.G
    L = int(batch.seq_lens[s].item())
    n = -(-L // sp.P)
    pages = batch.block_table[s, :n].long()
    k = batch.k_pm[:, kv_lo:kv_hi].index_select(0, pages).contiguous()
    v = batch.v_pm[:, kv_lo:kv_hi].index_select(0, pages).contiguous()
    q = batch.q[s:s + 1, kv_lo * G:kv_hi * G].contiguous()
    sb = batch.split_bounds[s:s + 1]
    if batch.bounds_per_head:
        sb = sb[:, kv_lo:kv_hi]
    mask = None
    if batch.block_mask is not None:
        mask = batch.block_mask[s:s + 1, kv_lo:kv_hi, :n].contiguous()
    h = wl.host
    return dict(q=h(q), k_pool=h(k), v_pool=h(v),
                block_table=np.arange(n, dtype=np.int32)[None, :],
                seq_lens=np.array([L], dtype=np.int32), split_bounds=h(sb.contiguous()),
                block_mask=None if mask is None else h(mask))


def oracle_out(inp, scale, pairs=None):
    return oracle.attention(inp["q"], inp["k_pool"], inp["v_pool"], inp["block_table"],
                            inp["seq_lens"], block_mask=inp["block_mask"], scale=scale, pairs=pairs)


def oracle_micro(inp, scale, pairs=None):
    return oracle.micro_attention(inp["q"], inp["k_pool"], inp["v_pool"], inp["block_table"],
                                  inp["seq_lens"], inp["split_bounds"], block_mask=inp["block_mask"],
                                  scale=scale, pairs=pairs)


def compare_out(got: np.ndarray, want: np.ndarray, tol: float, what=""):
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    err = float(np.max(np.abs(got.astype(np.float64) - want)))
    assert err <= tol, f"{what}: max-abs error {err:.3e} > {tol:.1e}"
    return err


def compare_partials(MA, m, e, oMA, om, oe, tol: float, what=""):
    MA = MA.astype(np.float64)
    m = m.astype(np.float64)
    e = e.astype(np.float64)
    empty = np.isneginf(om)
    assert np.array_equal(np.isneginf(m), empty), f"{what}: empty-split pattern differs"
    assert np.all(e[empty] == 0) and np.all(MA[empty] == 0), f"{what}: empty split not (0,-inf,0)"
    full = ~empty
    if not np.any(full):
        return
    dm = np.abs(m[full] - om[full]) / np.maximum(1.0, np.abs(om[full]))
    assert np.max(dm) <= 1e-4, f"{what}: m error {np.max(dm):.3e}"
    de = np.abs(e[full] - oe[full]) / oe[full]
    assert np.max(de) <= 1e-4, f"{what}: e relative error {np.max(de):.3e}"
    ratio = MA[full] / e[full][:, None]
    oratio = oMA[full] / oe[full][:, None]
    err = np.max(np.abs(ratio - oratio))
    assert err <= tol, f"{what}: MA/e error {err:.3e} > {tol:.1e}"
