"""Page selection (da_page_stats, da_page_scores, da_select_pages) through the
C ABI against the fp64 selection oracle on the same seeded inputs.  Needs an
MI355X and the built libda.so.

Bars:
* statistics are maxima and minima of stored values, so they are compared
  bit for bit (as float64);
* scores are fp32 sums of D exact products: |gpu - oracle| <= 2 D 2^-24 M,
  where M is the largest sum_d |q_d| max(|kmax_d|, |kmin_d|) over the
  candidates of the page (a bound on recursive fp32 summation error; the max
  over candidates is 1-Lipschitz), and the -inf pattern is exact;
* the mask is an integer decision taken on fp32 scores, so the oracle takes
  it on the GPU's fp32 scores and the two masks must be equal bit for bit;
  the kept set must also be a valid top-K of the oracle's fp64 scores up to
  twice the score tolerance.
"""

from __future__ import annotations

import sys

import numpy as np
import pytest
import torch

import oracle
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


# (spec, logical): head shapes, page sizes and dtypes the selector supports,
# with ragged last pages and last logical pages, shuffled tables with
# unreferenced pages, mixed lengths.
CASES = {
    "c5_gqa4_bf16_P64_l16": (wl.CONFIGS["C5"].replace(S=2, lens=("fixed", 32768 + 37), mask=None,
                                                       table="shuffled", extra_pages=5,
                                                       splits=("equal", 4)), 16),
    "mha_bf16_P16_l8": (wl.CONFIGS["C2"].replace(S=2, Hq=4, Hkv=4, lens=("fixed", 4096 - 3),
                                                 k_scaled=None), 8),
    "mha_f32_D64_P16_l16": (wl.CONFIGS["C1"].replace(lens=("fixed", 1000)), 16),
    "gqa2_f32_D128_P64_l32": (wl.CONFIGS["C5"].replace(S=3, Hq=8, Hkv=4, dtype=wl.F32, mask=None,
                                                        lens=("fixed", 64 * 40 + 33),
                                                        splits=("equal", 2)), 32),
    "gqa8_bf16_D64_P64_l64": (wl.CONFIGS["C5"].replace(S=2, Hq=16, Hkv=2, D=64, mask=None,
                                                        lens=("fixed", 64 * 300 + 1),
                                                        splits=("equal", 2)), 64),
    "mixed_bf16_P16_l16": (wl.CONFIGS["C3"].replace(S=6, Hq=8, Hkv=8, extra_pages=7), 16),
}

SELECTIONS = [
    # (budget fraction of the pages, keep_first, keep_last, select_heads: None | "upper" | "alt")
    (0.25, 1, 2, None),
    (0.25, 1, 2, "upper"),
    (0.5, 0, 0, "alt"),
    (0.0, 3, 1, None),
    (1.0, 0, 0, None),
    (0.1, 1000, 0, "upper"),
]


def _select_flags(kind, Hkv):
    if kind is None:
        return None
    if kind == "upper":
        return np.array([1 if h >= Hkv // 2 else 0 for h in range(Hkv)], dtype=np.uint8)
    if kind == "alt":
        return np.array([h % 2 for h in range(Hkv)], dtype=np.uint8)
    raise ValueError(kind)


def _score_tolerance(q_host, stats64, table, lens, P, logical, D):
    """2 D 2^-24 times the largest candidate magnitude per page (oracle scores
    of |q| against statistics replaced by max(|kmax|, |kmin|))."""
    mag = np.maximum(np.abs(stats64[..., 0, :]), np.abs(stats64[..., 1, :]))
    st_abs = np.stack([mag, mag], axis=-2)
    qa = np.abs(oracle.to_f64(q_host))
    M = osel.page_scores(qa, st_abs, table, lens, P, logical)
    return 2.0 * D * 2.0 ** -24 * np.where(np.isfinite(M), M, 0.0)


def _check_mask_valid(mask, want_scores, tol, lens, P, budget, kf, kl, flags):
    """Every kept non-forced page scores (fp64) at least every dropped one,
    up to twice the score tolerance."""
    S, Hkv, _ = mask.shape
    for s in range(S):
        npg = osel.n_pages(int(lens[s]), P)
        for h in range(Hkv):
            if flags is not None and not flags[h]:
                continue
            lo = min(kf, npg)
            hi = max(npg - kl, lo)
            cand = np.arange(lo, hi)
            if cand.size == 0:
                continue
            kept = cand[mask[s, h, cand] == 1]
            drop = cand[mask[s, h, cand] == 0]
            assert kept.size == min(budget, cand.size), (s, h, kept.size, budget, cand.size)
            if kept.size and drop.size:
                gap = want_scores[s, h, kept].min() - want_scores[s, h, drop].max()
                slack = 2 * max(tol[s, h, kept].max(), tol[s, h, drop].max())
                assert gap >= -slack, f"({s},{h}) kept page scores {gap:.3e} below a dropped one"


def _page_major(stats):
    """The library's head-major statistics [Hkv, NP, ...] in the oracle's
    page-major order [NP, Hkv, ...] (a transpose, no arithmetic)."""
    return stats.transpose(0, 1).contiguous()


def _run_case(name, spec, logical, seed):
    announce("selector", name, "seed", seed)
    b = wl.build(spec, seed, DEV)
    h = wl.host
    P, D, Hkv = spec.P, spec.D, spec.Hkv
    table, lens = h(b.block_table), h(b.seq_lens)

    stats = _lib.page_stats(b.k_pages, b.block_table, b.seq_lens, logical=logical)
    upper = _select_flags("upper", Hkv)
    stats_upper = _lib.page_stats(b.k_pages, b.block_table, b.seq_lens, logical=logical,
                                  select_heads=torch.from_numpy(upper).to(DEV))
    torch.cuda.synchronize()
    want_stats = osel.page_stats(h(b.k_pages), table, lens, logical=logical)
    got_stats = oracle.to_f64(h(_page_major(stats)))
    assert np.array_equal(got_stats, want_stats), f"{name}: statistics differ"
    # heads with flag 0 are not written (the output was allocated as zeros)
    got_upper = oracle.to_f64(h(_page_major(stats_upper)))
    on = upper.astype(bool)
    assert np.array_equal(got_upper[:, on], want_stats[:, on]), f"{name}: selected-head statistics"
    assert not np.any(got_upper[:, ~on]), f"{name}: statistics written for an unselected head"

    tol = _score_tolerance(h(b.q), want_stats, table, lens, P, logical, D)
    q_host = h(b.q)
    for frac, kf, kl, kind in SELECTIONS:
        flags = _select_flags(kind, Hkv)
        sel_t = None if flags is None else torch.from_numpy(flags).to(DEV)
        scores = _lib.page_scores(b.q, stats, b.block_table, b.seq_lens, P=P, select_heads=sel_t)
        npg_max = int(max(osel.n_pages(int(L), P) for L in lens))
        budget = int(frac * npg_max)
        mask = _lib.select_pages(scores, b.seq_lens, P=P, budget=budget, keep_first=kf,
                                 keep_last=kl, select_heads=sel_t)
        torch.cuda.synchronize()
        got = scores.cpu().numpy().astype(np.float64)
        want = osel.page_scores(q_host, want_stats, table, lens, P, logical, select_heads=flags)
        inf_got, inf_want = np.isneginf(got), np.isneginf(want)
        assert np.array_equal(inf_got, inf_want), f"{name}: -inf pattern of the scores differs"
        fin = ~inf_want
        err = np.abs(got[fin] - want[fin])
        assert np.all(err <= tol[fin]), (
            f"{name}: score error {err.max():.3e} > tolerance {tol[fin][np.argmax(err - tol[fin])]:.3e}")
        got_mask = mask.cpu().numpy()
        want_mask = osel.select_pages(got, lens, P, budget, kf, kl, select_heads=flags)
        assert np.array_equal(got_mask, want_mask), (
            f"{name} budget={budget} kf={kf} kl={kl} {kind}: mask differs at "
            f"{np.argwhere(got_mask != want_mask)[:5].tolist()}")
        _check_mask_valid(got_mask, want, tol, lens, P, budget, kf, kl, flags)
    return b, stats


@pytest.mark.parametrize("seed", [0, 1])
@pytest.mark.parametrize("name", sorted(CASES))
def test_selector_parity(name, seed):
    spec, logical = CASES[name]
    _run_case(name, spec, logical, seed)


@pytest.mark.parametrize("max_pages", [5, 1000, 1024, 1025, 2049, 8192 + 77, 20000, 32768 + 1, 65536])
@pytest.mark.parametrize("kind", ["ties", "continuous", "signed_zero"])
def test_select_pages_direct(max_pages, kind):
    """da_select_pages on seeded score arrays: heavy ties, continuous values,
    +0.0 / -0.0 and negative scores, ragged lengths, budgets from 0 to past
    the candidate count; bit-exact against the oracle."""
    announce("select", kind, max_pages)
    S, Hkv, P = 3, 4, 16
    rng = np.random.default_rng(1234 + max_pages)
    if kind == "ties":
        sc = rng.integers(-3, 4, size=(S, Hkv, max_pages)).astype(np.float32)
    elif kind == "continuous":
        sc = (rng.standard_normal((S, Hkv, max_pages)) * 50).astype(np.float32)
    else:
        sc = rng.choice(np.array([0.0, -0.0, 1.0, -1.0], dtype=np.float32), size=(S, Hkv, max_pages))
    lens = np.array([max_pages * P, max(1, (max_pages * P) // 3 - 5), 1], dtype=np.int32)
    sc_t = torch.from_numpy(sc).to(DEV)
    lens_t = torch.from_numpy(lens).to(DEV)
    flags = np.array([1, 0, 1, 1], dtype=np.uint8)
    for budget, kf, kl, fl in [(0, 0, 0, None), (1, 0, 0, None), (max_pages // 4, 1, 2, flags),
                               (max_pages - 1, 0, 1, None), (max_pages, 2, 2, None),
                               (max_pages + 5, 0, 0, flags), (3, max_pages, max_pages, None)]:
        sel_t = None if fl is None else torch.from_numpy(fl).to(DEV)
        got = _lib.select_pages(sc_t, lens_t, P=P, budget=budget, keep_first=kf, keep_last=kl,
                                select_heads=sel_t).cpu().numpy()
        want = osel.select_pages(sc.astype(np.float64), lens, P, budget, kf, kl, select_heads=fl)
        assert np.array_equal(got, want), (
            f"{kind} max_pages={max_pages} budget={budget} kf={kf} kl={kl}: mask differs at "
            f"{np.argwhere(got != want)[:5].tolist()}")


def test_selected_mask_drives_attention():
    """Statistics -> scores -> top-K mask on the upper half of the KV heads,
    then the MicroAttention + merge step over the selected pages with splits
    over the kept pages; the output matches the oracle's attention under the
    same mask (itself checked bit-exact against the oracle's selection)."""
    spec, logical = CASES["c5_gqa4_bf16_P64_l16"]
    announce("selector end-to-end", spec.name)
    b, stats = _run_case("e2e", spec, logical, 0)
    h = wl.host
    P, Hkv = spec.P, spec.Hkv
    flags = _select_flags("upper", Hkv)
    sel_t = torch.from_numpy(flags).to(DEV)
    lens = h(b.seq_lens)
    npg = osel.n_pages(int(lens[0]), P)
    budget = (npg - 3) // 4
    scores = _lib.page_scores(b.q, stats, b.block_table, b.seq_lens, P=P, select_heads=sel_t)
    mask = _lib.select_pages(scores, b.seq_lens, P=P, budget=budget, keep_first=1, keep_last=2,
                             select_heads=sel_t)
    # 8 splits over the kept pages of each (request, KV head)
    mask_h = mask.cpu().numpy()
    nb = 8
    sb = np.zeros((spec.S, Hkv, nb + 1), dtype=np.int32)
    for s in range(spec.S):
        for kvh in range(Hkv):
            kp = np.nonzero(mask_h[s, kvh, :osel.n_pages(int(lens[s]), P)])[0]
            for j in range(1, nb):
                sb[s, kvh, j] = int(kp[(j * len(kp)) // nb]) * P
            sb[s, kvh, nb] = int(lens[s])
    sb_t = torch.from_numpy(sb).to(DEV)
    out = _lib.attention(b.q, b.k_pages, b.v_pages, b.block_table, b.seq_lens, sb_t, mask,
                         scale=b.scale)
    torch.cuda.synchronize()
    want = oracle.attention(h(b.q), h(b.k_pages), h(b.v_pages), h(b.block_table), lens,
                            block_mask=mask_h, scale=b.scale)
    compare_out(out.cpu().numpy(), want, TOL_OUT[spec.dtype], "selected-mask attention")


@pytest.mark.slow
def test_selector_full_c5_sampled():
    """Full-size GQA workload (8 x 512K tokens, 32/8 heads, 64-token pages,
    16-token logical pages) in the launch configuration the benchmark times;
    statistics, scores and mask of sampled (request, KV head) units against
    the oracle run on those units alone."""
    spec = wl.CONFIGS["C5"].replace(layout=wl.PREFERRED_LAYOUT.get("C5", "page"))
    announce("selector full", spec.name, spec.layout)
    b = wl.build(spec, 0, DEV)
    P, G, logical = spec.P, spec.G, 16
    flags = _select_flags("upper", spec.Hkv)
    sel_t = torch.from_numpy(flags).to(DEV)
    stats = _lib.page_stats(b.k_pages, b.block_table, b.seq_lens, logical=logical,
                            pool_layout=b.layout)
    scores = _lib.page_scores(b.q, stats, b.block_table, b.seq_lens, P=P, select_heads=sel_t)
    npg = -(-spec.max_len // P)  # pages holding each request's tokens
    budget = (npg - 3) // 4
    mask = _lib.select_pages(scores, b.seq_lens, P=P, budget=budget, keep_first=1, keep_last=2,
                             select_heads=sel_t)
    torch.cuda.synchronize()
    h = wl.host
    for s, kvh in [(0, 5), (7, 6), (3, 1)]:
        announce("unit", s, kvh)
        L = int(b.seq_lens[s].item())
        n = osel.n_pages(L, P)
        pages = b.block_table[s, :n].long()
        k = h(b.k_pm[:, kvh:kvh + 1].index_select(0, pages).contiguous())
        q = h(b.q[s:s + 1, kvh * G:(kvh + 1) * G].contiguous())
        table = np.arange(n, dtype=np.int32)[None, :]
        lens = np.array([L], dtype=np.int32)
        want_stats = osel.page_stats(k, table, lens, logical=logical)
        got_stats = oracle.to_f64(h(_page_major(stats[kvh:kvh + 1].index_select(1, pages))))
        assert np.array_equal(got_stats, want_stats), f"unit ({s},{kvh}): statistics differ"
        fl = flags[kvh:kvh + 1]
        want = osel.page_scores(q, want_stats, table, lens, P, logical, select_heads=fl)
        got = scores[s:s + 1, kvh:kvh + 1].cpu().numpy().astype(np.float64)
        # table columns past the request's pages (spare capacity) score -inf
        assert np.all(np.isneginf(got[..., n:])), f"unit ({s},{kvh}): spare pages scored"
        got = got[..., :n]
        assert np.array_equal(np.isneginf(got), np.isneginf(want))
        tol = _score_tolerance(q, want_stats, table, lens, P, logical, spec.D)
        fin = ~np.isneginf(want)
        assert np.all(np.abs(got[fin] - want[fin]) <= tol[fin]), f"unit ({s},{kvh}): scores"
        got_mask = mask[s:s + 1, kvh:kvh + 1].cpu().numpy()
        assert not np.any(got_mask[..., n:]), f"unit ({s},{kvh}): spare pages kept"
        got_mask = got_mask[..., :n]
        want_mask = osel.select_pages(got, lens, P, budget, 1, 2, select_heads=fl)
        assert np.array_equal(got_mask, want_mask), f"unit ({s},{kvh}): mask differs"
        _check_mask_valid(got_mask, want, tol, lens, P, budget, 1, 2, fl)
