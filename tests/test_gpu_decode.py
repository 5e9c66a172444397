"""Decode-time cache update and reused selection (da_append_kv,
da_split_bounds, the horizon of da_select_pages) through the C ABI against
the fp64 oracles on the same seeded inputs.  Needs an MI355X and the built
libda.so.

Bars: pools, statistics, split bounds and masks are integer / stored-value
work and are compared bit for bit; attention outputs within the workload
tolerance (2e-3 bf16, 1e-5 fp32 K/V).
"""

from __future__ import annotations

import sys

import numpy as np
import pytest
import torch

import oracle
import oracle.decode as odec
import oracle.selector as osel
from harness import TOL_OUT, compare_out
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


def _page_major(stats):
    """Head-major statistics [Hkv, NP, ...] in the oracle's page-major order
    (a transpose, no arithmetic)."""
    return stats.transpose(0, 1).contiguous()


# (spec, logical, steps): lengths put the first appends just before a
# physical-page boundary; shuffled tables with spare pages.  The fp32 case
# fills its cache after 19 of its 24 steps (L + 19 is a whole number of
# pages), so its last 5 appends must change nothing.  Steps never exceed the
# reserve otherwise, so every append lands on a mapped page.
APPEND_CASES = {
    "gqa4_bf16_P64_l16": (wl.CONFIGS["C5"].replace(S=2, lens=("fixed", 64 * 31 + 59), mask=None,
                                                    table="shuffled", extra_pages=3, reserve=20,
                                                    splits=("equal", 2)), 16, 20),
    "mha_f32_D64_P16_l8": (wl.CONFIGS["C1"].replace(S=3, lens=("fixed", 16 * 20 + 13),
                                                    reserve=19, table="shuffled"), 8, 24),
    "mixed_bf16_P16_l16": (wl.CONFIGS["C3"].replace(S=5, Hq=4, Hkv=4, lens=("loguniform", 700),
                                                    reserve=9), 16, 9),
}


@pytest.mark.parametrize("flags_kind", ["all", "upper", "none"])
@pytest.mark.parametrize("name", sorted(APPEND_CASES))
def test_append_matches_oracle(name, flags_kind):
    """Consecutive appends with statistics kept current: after every step the
    pools equal the oracle's pools bit for bit, and the statistics equal the
    oracle's statistics recomputed from scratch on the new contents."""
    spec, logical, steps = APPEND_CASES[name]
    announce("append", name, flags_kind)
    b = wl.build(spec, 0, DEV)
    h = wl.host
    Hkv = spec.Hkv
    flags = None
    if flags_kind == "upper":
        flags = np.array([1 if i >= Hkv // 2 else 0 for i in range(Hkv)], dtype=np.uint8)
    sel_t = None if flags is None else torch.from_numpy(flags).to(DEV)
    lens = b.seq_lens.clone()
    stats = None
    if flags_kind != "none":
        stats = _lib.page_stats(b.k_pages, b.block_table, lens, logical=logical, select_heads=sel_t)
    table = h(b.block_table)
    ok, ov = h(b.k_pages), h(b.v_pages)
    cap = table.shape[1] * spec.P
    for step in range(steps):
        kn, vn = wl.new_tokens(spec, 0, step, DEV)
        _lib.append_kv(kn, vn, b.block_table, lens, b.k_pages, b.v_pages, stats=stats,
                       logical=logical, select_heads=sel_t)
        L_host = h(lens)
        ok, ov = odec.append_kv(ok, ov, table, L_host, h(kn), h(vn))
        lens = torch.clamp(lens + 1, max=cap)
        torch.cuda.synchronize()
        assert np.array_equal(h(b.k_pages), ok), f"{name} step {step}: K pool differs"
        assert np.array_equal(h(b.v_pages), ov), f"{name} step {step}: V pool differs"
        if stats is not None and (step % 5 == 4 or step == steps - 1):
            want = osel.page_stats(ok, table, h(lens), logical=logical)
            got = oracle.to_f64(h(_page_major(stats)))
            on = np.ones(Hkv, dtype=bool) if flags is None else flags.astype(bool)
            assert np.array_equal(got[:, on], want[:, on]), f"{name} step {step}: statistics differ"


@pytest.mark.parametrize("b_splits", [1, 3, 16, 40])
@pytest.mark.parametrize("kind", ["random", "sparse", "empty", "dense_none"])
@pytest.mark.parametrize("max_pages", [300, 8193, 20000])
def test_split_bounds_matches_oracle(kind, b_splits, max_pages):
    """Rows of 300 and 8193 pages (each thread's pages read as one bit
    word) and 20000 pages (more than 64 per thread: read page by page)."""
    announce("split bounds", kind, b_splits, max_pages)
    rng = np.random.default_rng(100 + b_splits)
    S, Hkv, P = 4, 3, 16
    lens = np.array([max_pages * P, 1, 4000, 0], dtype=np.int32)
    if kind == "random":
        mask = (rng.random((S, Hkv, max_pages)) < 0.5).astype(np.uint8)
    elif kind == "sparse":
        mask = (rng.random((S, Hkv, max_pages)) < 0.03).astype(np.uint8)
    else:
        mask = np.zeros((S, Hkv, max_pages), dtype=np.uint8)
    lens_t = torch.from_numpy(lens).to(DEV)
    for hz in (0, 16, 5000):
        if kind == "dense_none":
            got = _lib.split_bounds(None, lens_t, P=P, b=b_splits, horizon=hz, Hkv=Hkv,
                                    max_pages=max_pages)
            want = odec.kept_page_bounds(None, lens, P, b_splits, horizon=hz, Hkv=Hkv,
                                         max_pages=max_pages)
        else:
            got = _lib.split_bounds(torch.from_numpy(mask).to(DEV), lens_t, P=P, b=b_splits,
                                    horizon=hz)
            want = odec.kept_page_bounds(mask, lens, P, b_splits, horizon=hz)
        got = got.cpu().numpy()
        assert np.array_equal(got, want), (
            f"{kind} b={b_splits} horizon={hz}: differs at {np.argwhere(got != want)[:5].tolist()}")


@pytest.mark.parametrize("horizon", [0, 1, 16, 64, 65, 100000])
def test_select_horizon_matches_oracle(horizon):
    announce("select horizon", horizon)
    rng = np.random.default_rng(7 + horizon % 97)
    S, Hkv, P, max_pages = 3, 4, 64, 700
    sc = (rng.standard_normal((S, Hkv, max_pages)) * 30).astype(np.float32)
    lens = np.array([64 * 600 + 1, 64 * 700, 64 * 5 - 1], dtype=np.int32)
    flags = np.array([1, 0, 1, 1], dtype=np.uint8)
    for fl in (None, flags):
        got = _lib.select_pages(torch.from_numpy(sc).to(DEV), torch.from_numpy(lens).to(DEV), P=P,
                                budget=100, keep_first=1, keep_last=2,
                                select_heads=None if fl is None else torch.from_numpy(fl).to(DEV),
                                horizon=horizon).cpu().numpy()
        want = osel.select_pages(sc.astype(np.float64), lens, P, 100, 1, 2, select_heads=fl,
                                 horizon=horizon)
        assert np.array_equal(got, want), f"horizon {horizon}: mask differs"


def test_reused_selection_chunk():
    """One 16-step chunk of the decode loop with a reused selection: page
    statistics once, then scores, top-K (horizon 16) and split bounds once,
    then 16 x (append with statistics, MicroAttention + merge with the
    reused mask and bounds).  Every step's output matches the oracle's
    attention over the oracle-appended cache under the same mask; the final
    statistics equal the oracle's from scratch."""
    chunk = 16
    spec = wl.CONFIGS["C5"].replace(S=2, lens=("fixed", 64 * 60 + 55), reserve=chunk,
                                    table="shuffled", mask=None, splits=("equal", 4))
    announce("reused selection chunk", spec.name)
    b = wl.build(spec, 1, DEV)
    h = wl.host
    P, Hkv, logical = spec.P, spec.Hkv, 16
    flags = np.array([1 if i >= Hkv // 2 else 0 for i in range(Hkv)], dtype=np.uint8)
    sel_t = torch.from_numpy(flags).to(DEV)
    lens = b.seq_lens.clone()
    stats = _lib.page_stats(b.k_pages, b.block_table, lens, logical=logical, select_heads=sel_t)
    scores = _lib.page_scores(b.q, stats, b.block_table, lens, P=P, select_heads=sel_t)
    npg = -(-int(lens[0].item()) // P)
    budget = (npg - 3) // 4
    mask = _lib.select_pages(scores, lens, P=P, budget=budget, keep_first=1, keep_last=2,
                             select_heads=sel_t, horizon=chunk)
    nb = 8
    bounds = _lib.split_bounds(mask, lens, P=P, b=nb, horizon=chunk)
    torch.cuda.synchronize()
    mask_h = mask.cpu().numpy()
    assert np.array_equal(h(bounds), odec.kept_page_bounds(mask_h, h(lens), P, nb, horizon=chunk))
    table = h(b.block_table)
    ok, ov = h(b.k_pages), h(b.v_pages)
    for step in range(chunk):
        kn, vn = wl.new_tokens(spec, 1, step, DEV)
        _lib.append_kv(kn, vn, b.block_table, lens, b.k_pages, b.v_pages, stats=stats,
                       logical=logical, select_heads=sel_t)
        ok, ov = odec.append_kv(ok, ov, table, h(lens), h(kn), h(vn))
        lens += 1
        out = _lib.attention(b.q, b.k_pages, b.v_pages, b.block_table, lens, bounds, mask,
                             scale=b.scale)
        torch.cuda.synchronize()
        want = oracle.attention(h(b.q), ok, ov, table, h(lens), block_mask=mask_h, scale=b.scale)
        compare_out(out.cpu().numpy(), want, TOL_OUT[spec.dtype], f"chunk step {step}")
    want_stats = osel.page_stats(ok, table, h(lens), logical=logical)
    got_stats = oracle.to_f64(h(_page_major(stats)))
    assert np.array_equal(got_stats[:, flags.astype(bool)], want_stats[:, flags.astype(bool)])
