"""HIP path (through the C ABI) against the fp64 oracle on the same seeded
inputs.  Needs an MI355X and the built libda.so."""

from __future__ import annotations

import sys

import numpy as np
import pytest
import torch

from harness import (TOL_OUT, compare_out, compare_partials, host_inputs, oracle_micro,
                     oracle_out, run_gpu, sub_inputs)
from long_context_decode_microattention_amd import _lib
from long_context_decode_microattention_amd import workloads as wl

pytestmark = pytest.mark.gpu

DEV = "cuda:0"

# Reduced copies of the five workloads: same head shapes, page sizes, split
# rules and structure (shuffled tables, scaled rows, sinks, masks, ragged
# lengths), sized so the oracle finishes every output in seconds.
REDUCED = {
    "C1": wl.CONFIGS["C1"],
    "C2": wl.CONFIGS["C2"].replace(S=2),
    "C3": wl.CONFIGS["C3"].replace(S=6, Hq=8, Hkv=8),
    "C4": wl.CONFIGS["C4"].replace(Hq=8, Hkv=8, lens=("fixed", 32768)),
    "C5": wl.CONFIGS["C5"].replace(S=2, lens=("fixed", 32768)),
    # eight query heads per KV head: the dense value product over bf16 pages
    "C5_G8": wl.CONFIGS["C5"].replace(S=1, Hq=64, lens=("fixed", 16384 + 50)),
}


def announce(*parts):
    print("[gpu-case]", *parts, flush=True)
    sys.stdout.flush()


@pytest.fixture(autouse=True)
def _free_memory():
    yield
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


@pytest.mark.parametrize("seed", [0, 1, 2])
@pytest.mark.parametrize("cfg", sorted(REDUCED))
def test_reduced_config_parity(cfg, seed):
    spec = REDUCED[cfg]
    announce("reduced", cfg, "seed", seed)
    b = wl.build(spec, seed, DEV)
    out, MA, m, e = run_gpu(b)
    inp = host_inputs(b)
    tol = TOL_OUT[spec.dtype]
    compare_out(out.cpu().numpy(), oracle_out(inp, b.scale), tol, f"{cfg}/{seed} out")
    oMA, om, oe = oracle_micro(inp, b.scale)
    compare_partials(MA.cpu().numpy(), m.cpu().numpy(), e.cpu().numpy(), oMA, om, oe, tol,
                     f"{cfg}/{seed} partials")


@pytest.mark.parametrize("chunks", [1, 3, 7])
@pytest.mark.parametrize("cfg", ["C2", "C3", "C4", "C5"])
def test_forced_chunks_parity(cfg, chunks):
    """Splits cut into a forced number of page-range chunks (folded back by
    the combine kernel) give the same partials and outputs within tolerance."""
    spec = REDUCED[cfg]
    announce("chunks", cfg, chunks)
    b = wl.build(spec, 4, DEV)
    out, MA, m, e = run_gpu(b, chunks=chunks)
    inp = host_inputs(b)
    tol = TOL_OUT[spec.dtype]
    compare_out(out.cpu().numpy(), oracle_out(inp, b.scale), tol, f"{cfg} chunks={chunks}")
    oMA, om, oe = oracle_micro(inp, b.scale)
    compare_partials(MA.cpu().numpy(), m.cpu().numpy(), e.cpu().numpy(), oMA, om, oe, tol,
                     f"{cfg} chunks={chunks} partials")


@pytest.mark.parametrize("chunks", [0, 3])
@pytest.mark.parametrize("cfg", sorted(REDUCED))
def test_persistent_schedule_parity(cfg, chunks):
    """Persistent workgroups claiming items from the work queue (forced)."""
    spec = REDUCED[cfg]
    announce("persistent", cfg, chunks)
    b = wl.build(spec, 9, DEV)
    out, MA, m, e = run_gpu(b, chunks=chunks, schedule=2)
    inp = host_inputs(b)
    tol = TOL_OUT[spec.dtype]
    compare_out(out.cpu().numpy(), oracle_out(inp, b.scale), tol, f"{cfg} persistent")
    oMA, om, oe = oracle_micro(inp, b.scale)
    compare_partials(MA.cpu().numpy(), m.cpu().numpy(), e.cpu().numpy(), oMA, om, oe, tol,
                     f"{cfg} persistent partials")


@pytest.mark.parametrize("chunks", [0, 3])
@pytest.mark.parametrize("cfg,splits", [("C2", ("equal", 5)), ("C2", ("equal", 13)),
                                        ("C3", ("chunk", 3000)), ("C1", ("equal", 1))])
def test_persistent_queues_any_split_count(cfg, splits, chunks):
    """The persistent launch's per-XCD queues split the items by split index
    modulo 8: split counts that leave queues empty or uneven (1, 5, 11, 13
    splits) still hand out every item exactly once."""
    spec = REDUCED[cfg].replace(splits=splits)
    announce("persistent queues", cfg, splits, chunks)
    b = wl.build(spec, 12, DEV)
    out, MA, m, e = run_gpu(b, chunks=chunks, schedule=2)
    inp = host_inputs(b)
    tol = TOL_OUT[spec.dtype]
    compare_out(out.cpu().numpy(), oracle_out(inp, b.scale), tol, f"{cfg} {splits} persistent")
    oMA, om, oe = oracle_micro(inp, b.scale)
    compare_partials(MA.cpu().numpy(), m.cpu().numpy(), e.cpu().numpy(), oMA, om, oe, tol,
                     f"{cfg} {splits} persistent partials")


@pytest.mark.parametrize("cfg", sorted(REDUCED))
def test_one_workgroup_per_item_parity(cfg):
    """Without a workspace the launch is one workgroup per item (no work
    queue, no chunks): same results within tolerance."""
    spec = REDUCED[cfg]
    announce("no-workspace", cfg)
    b = wl.build(spec, 6, DEV)
    out, MA, m, e = run_gpu(b, workspace=False)
    inp = host_inputs(b)
    tol = TOL_OUT[spec.dtype]
    compare_out(out.cpu().numpy(), oracle_out(inp, b.scale), tol, f"{cfg} no workspace")
    oMA, om, oe = oracle_micro(inp, b.scale)
    compare_partials(MA.cpu().numpy(), m.cpu().numpy(), e.cpu().numpy(), oMA, om, oe, tol,
                     f"{cfg} no workspace partials")


def test_work_queue_reused_across_calls():
    """The persistent launch's counter is reset on the stream before every
    call: repeated calls on one workspace, with shapes that change between
    them, keep giving the same results."""
    announce("queue-reuse")
    ws = torch.zeros(1 << 24, dtype=torch.uint8, device=DEV)
    batches = [wl.build(REDUCED[c], 8, DEV) for c in ("C3", "C5", "C2")]
    first = []
    for b in batches:
        first.append(run_gpu(b, workspace=ws, schedule=2)[0].clone())
    for _ in range(2):
        for b, ref in zip(batches, first):
            assert torch.equal(run_gpu(b, workspace=ws, schedule=2)[0], ref)
    ref3 = oracle_out(host_inputs(batches[0]), batches[0].scale)
    compare_out(first[0].cpu().numpy(), ref3, 2e-3, "queue reuse C3")


# Full-size workloads: outputs sampled at (request, KV-head range) units the
# oracle computes one by one.
FULL_SAMPLES = {
    "C2": [(0, 0, 1), (15, 31, 32), (7, 13, 14)],
    "C3": None,  # chosen from the drawn lengths: longest, shortest, median
    "C4": [(0, 0, 1), (0, 31, 32)],
    "C5": [(0, 0, 1), (7, 7, 8), (3, 0, 8)],  # (3, 0, 8): every KV head of one request, dense and masked
}


@pytest.mark.slow
@pytest.mark.parametrize("cfg", ["C2", "C3", "C4", "C5"])
def test_full_size_sampled(cfg):
    spec = wl.CONFIGS[cfg].replace(layout=wl.PREFERRED_LAYOUT.get(cfg, "page"))
    announce("full", cfg, spec.layout)
    b = wl.build(spec, 0, DEV)
    out, MA, m, e = run_gpu(b)
    samples = FULL_SAMPLES[cfg]
    if samples is None:
        lens = b.seq_lens.cpu().numpy()
        order = np.argsort(lens)
        samples = [(int(order[-1]), 0, 1), (int(order[0]), 39, 40), (int(order[len(order) // 2]), 20, 21)]
    tol = TOL_OUT[spec.dtype]
    G = spec.G
    for s, lo, hi in samples:
        inp = sub_inputs(b, s, lo, hi)
        want = oracle_out(inp, b.scale)[0]
        got = out[s, lo * G:hi * G].cpu().numpy()
        compare_out(got, want, tol, f"{cfg} s={s} kv[{lo},{hi})")
        oMA, om, oe = oracle_micro(inp, b.scale)
        compare_partials(MA[s:s + 1, lo * G:hi * G].cpu().numpy(), m[s:s + 1, lo * G:hi * G].cpu().numpy(),
                         e[s:s + 1, lo * G:hi * G].cpu().numpy(), oMA, om, oe, tol,
                         f"{cfg} s={s} partials")
    del b, out, MA, m, e


# ---------------------------------------------------------------------------
# bit-exact indexing probes
# ---------------------------------------------------------------------------

def _splitmix(x: np.ndarray) -> np.ndarray:
    x = (x + np.uint64(0x9E3779B97F4A7C15)) & np.uint64(0xFFFFFFFFFFFFFFFF)
    z = x
    z = ((z ^ (z >> np.uint64(30))) * np.uint64(0xBF58476D1CE4E5B9)) & np.uint64(0xFFFFFFFFFFFFFFFF)
    z = ((z ^ (z >> np.uint64(27))) * np.uint64(0x94D049BB133111EB)) & np.uint64(0xFFFFFFFFFFFFFFFF)
    return z ^ (z >> np.uint64(31))


def fingerprint(S, Hkv, L, D):
    """bits[s, kvh, t, c] in {0, 1}: bit c of a hash of (s, kvh, t)."""
    s = np.arange(S, dtype=np.uint64)[:, None, None]
    h = np.arange(Hkv, dtype=np.uint64)[None, :, None]
    t = np.arange(L, dtype=np.uint64)[None, None, :]
    key = (s << np.uint64(40)) | (h << np.uint64(32)) | t
    words = [_splitmix(key + np.uint64(w) * np.uint64(0x1000000000000)) for w in range(-(-D // 64))]
    bits = np.zeros((S, Hkv, L, D), dtype=np.float32)
    for c in range(D):
        bits[..., c] = ((words[c // 64] >> np.uint64(c % 64)) & np.uint64(1)).astype(np.float32)
    return bits


def _fill_pool_from_logical(b: wl.Batch, values: np.ndarray, target: torch.Tensor):
    """values [S, Hkv, L, D] by logical token -> pool slots through the table."""
    sp = b.spec
    table = b.block_table.cpu().numpy()
    lens = b.seq_lens.cpu().numpy()
    host = torch.zeros(target.shape, dtype=torch.float32)
    for s in range(sp.S):
        L = int(lens[s])
        t = np.arange(L)
        pages = torch.from_numpy(table[s, t // sp.P].astype(np.int64))
        slots = torch.from_numpy((t % sp.P).astype(np.int64))
        for h in range(sp.Hkv):
            host[pages, h, slots] = torch.from_numpy(values[s, h, :L])
    target.copy_(host.to(target.dtype))


@pytest.mark.parametrize("schedule", [1, 2])
@pytest.mark.parametrize("chunks", [0, 5])
@pytest.mark.parametrize("cfg", ["C1", "C3", "C5"])
def test_fingerprint_counts_bit_exact(cfg, chunks, schedule):
    """q = 0 makes every weight exp(0) = 1: m_j = 0, e_j = kept-token count and
    MA_j[c] = number of kept tokens whose fingerprint has bit c set -- exact
    integers, compared bitwise with numpy counts."""
    spec = REDUCED[cfg].replace(S=min(REDUCED[cfg].S, 3))
    announce("fingerprint", cfg, chunks, schedule)
    b = wl.build(spec, 5, DEV)
    b.q.zero_()
    sp = b.spec
    L = int(b.seq_lens.max().item())
    bits = fingerprint(sp.S, sp.Hkv, L, sp.D)
    _fill_pool_from_logical(b, bits, b.v_pages)
    _, MA, m, e = run_gpu(b, chunks=chunks, schedule=schedule)
    MA, m, e = MA.cpu().numpy(), m.cpu().numpy(), e.cpu().numpy()
    lens = b.seq_lens.cpu().numpy()
    sb = b.split_bounds.cpu().numpy()
    mask = None if b.block_mask is None else b.block_mask.cpu().numpy()
    for s in range(sp.S):
        for h in range(sp.Hq):
            kvh = h // sp.G
            row = sb[s, kvh if b.bounds_per_head else 0]
            for j in range(b.max_splits):
                lo, hi = max(int(row[j]), 0), min(int(row[j + 1]), int(lens[s]))
                t = np.arange(lo, hi) if hi > lo else np.zeros(0, dtype=np.int64)
                if mask is not None and t.size:
                    t = t[mask[s, kvh, t // sp.P] != 0]
                want_e = np.float32(t.size)
                want_MA = bits[s, kvh, t].sum(axis=0).astype(np.float32) if t.size else np.zeros(sp.D, np.float32)
                assert e[s, h, j] == want_e, (s, h, j, e[s, h, j], want_e)
                assert np.array_equal(MA[s, h, j], want_MA), (s, h, j)
                if t.size:
                    assert m[s, h, j] == 0.0
                else:
                    assert np.isneginf(m[s, h, j])


def test_shuffled_table_bitwise_equal_identity():
    """The same logical cache stored under an identity table and under a
    shuffled table (pool permuted to match) gives bitwise-equal results."""
    spec = REDUCED["C4"].replace(Hq=4, Hkv=4, lens=("fixed", 16384 + 37))
    announce("shuffle-bitwise")
    a = wl.build(spec, 3, DEV)
    n = a.k_pm.shape[0]
    perm = torch.randperm(n, generator=torch.Generator().manual_seed(9)).to(DEV)
    inv = torch.empty_like(perm)
    inv[perm] = torch.arange(n, device=DEV)
    table2 = perm[a.block_table.long()].to(torch.int32)  # logical page -> new location
    k2 = torch.empty_like(a.k_pages)
    v2 = torch.empty_like(a.v_pages)
    k2[perm] = a.k_pages
    v2[perm] = a.v_pages
    out1, MA1, m1, e1 = run_gpu(a)
    MA2, m2, e2 = _lib.micro_attention(a.q, k2, v2, table2, a.seq_lens, a.split_bounds, None, scale=a.scale)
    out2 = _lib.merge(MA2, m2, e2)
    torch.cuda.synchronize()
    for x, y in ((out1, out2), (MA1, MA2), (m1, m2), (e1, e2)):
        assert torch.equal(x, y)


@pytest.mark.parametrize("G", [1, 2, 4, 8])
def test_gqa_probe_exact(G):
    """K = 0 and V = KV-head id + 1: query head h must output h // G + 1 exactly."""
    Hkv = 4
    spec = wl.Spec("gqa probe", S=2, Hq=Hkv * G, Hkv=Hkv, D=128, P=16, dtype=wl.BF16,
                   lens=("fixed", 300), splits=("equal", 3))
    announce("gqa", G)
    b = wl.build(spec, 1, DEV)
    b.k_pages.zero_()
    for h in range(Hkv):
        b.v_pages[:, h] = float(h + 1)
    out, *_ = run_gpu(b)
    want = (torch.arange(spec.Hq, device=DEV) // G + 1).float()
    assert torch.equal(out, want[None, :, None].expand_as(out))


@pytest.mark.parametrize("cfg", ["C1", "C3", "C5"])
def test_nan_poison_never_read(cfg):
    """NaN in every slot no split may read (tail of a partial last page,
    masked pages, pages the table does not name): results stay finite and
    match the oracle."""
    spec = REDUCED[cfg].replace(S=min(REDUCED[cfg].S, 3), extra_pages=5)
    if cfg == "C1":
        spec = spec.replace(lens=("fixed", 1000), splits=("equal", 4))
    announce("nan-poison", cfg)
    b = wl.build(spec, 7, DEV)
    sp = b.spec
    table = b.block_table.cpu().numpy()
    lens = b.seq_lens.cpu().numpy()
    used = np.zeros(b.k_pm.shape[0], dtype=bool)
    for s in range(sp.S):
        n = -(-int(lens[s]) // sp.P)
        used[table[s, :n]] = True
        tail = int(lens[s]) % sp.P
        if tail:
            pg = int(table[s, n - 1])
            b.k_pages[pg, :, tail:] = float("nan")
            b.v_pages[pg, :, tail:] = float("nan")
        if b.block_mask is not None:
            mk = b.block_mask[s].cpu().numpy()
            for h in range(sp.Hkv):
                for lp in np.nonzero(mk[h, :n] == 0)[0]:
                    b.k_pages[int(table[s, lp]), h] = float("nan")
                    b.v_pages[int(table[s, lp]), h] = float("nan")
    unused = torch.from_numpy(np.nonzero(~used)[0]).to(DEV)
    assert unused.numel() >= 5
    b.k_pages[unused] = float("nan")
    b.v_pages[unused] = float("nan")
    out, MA, m, e = run_gpu(b)
    inp = host_inputs(b)
    compare_out(out.cpu().numpy(), oracle_out(inp, b.scale), TOL_OUT[sp.dtype], f"poison {cfg}")
    assert torch.isfinite(MA).all() and torch.isfinite(e).all()


# ---------------------------------------------------------------------------
# split invariance and separate ("remote") calls
# ---------------------------------------------------------------------------

def _random_bounds(rng, L, b):
    kind = rng.integers(0, 3)
    if kind == 0:  # uniform cuts, mid-page
        cuts = np.sort(rng.integers(0, L + 1, size=b - 1))
    elif kind == 1:  # one-token splits at the start, rest in one
        cuts = np.minimum(np.arange(1, b), L)
    else:  # empty splits (repeated cuts)
        cuts = np.sort(rng.choice([0, L // 3, L // 3, L], size=b - 1))
    return np.concatenate([[0], cuts, [L]]).astype(np.int32)


@pytest.mark.parametrize("b_splits", [1, 3, 8, 17])
def test_split_invariance_and_order(b_splits):
    spec = wl.Spec("split invariance", S=3, Hq=8, Hkv=2, D=128, P=16, dtype=wl.BF16,
                   lens=("fixed", 1111), table="shuffled", splits=("equal", 1), extra_pages=3)
    announce("split-invariance", b_splits)
    base = wl.build(spec, 11, DEV)
    ref = oracle_out(host_inputs(base), base.scale)
    rng = np.random.default_rng(b_splits)
    lens = base.seq_lens.cpu().numpy()
    sb = np.stack([_random_bounds(rng, int(L), b_splits) for L in lens])[:, None, :]
    sbt = torch.from_numpy(sb).to(DEV)
    MA, m, e = _lib.micro_attention(base.q, base.k_pages, base.v_pages, base.block_table,
                                    base.seq_lens, sbt, None, scale=base.scale)
    out = _lib.merge(MA, m, e)
    compare_out(out.cpu().numpy(), ref, 2e-3, f"b={b_splits}")
    perm = torch.from_numpy(rng.permutation(b_splits)).to(DEV)
    out_p = _lib.merge(MA[:, :, perm].contiguous(), m[:, :, perm].contiguous(), e[:, :, perm].contiguous())
    compare_out(out_p.cpu().numpy(), ref, 2e-3, f"b={b_splits} permuted")


def test_separate_calls_with_separate_pools_merge():
    """Two calls over disjoint token ranges, each with its own pool and table
    (the splits another instance would hold), concatenated and merged, equal
    a single call and the oracle."""
    spec = wl.Spec("remote halves", S=2, Hq=8, Hkv=8, D=128, P=64, dtype=wl.BF16,
                   lens=("fixed", 64 * 40 + 17), splits=("equal", 4))
    announce("remote-halves")
    b = wl.build(spec, 13, DEV)
    L = int(b.seq_lens[0].item())
    cut_page = 23
    cut = cut_page * spec.P
    n = -(-L // spec.P)
    tabA = torch.zeros_like(b.block_table)
    tabB = torch.zeros_like(b.block_table)
    pools = []
    for s in range(spec.S):
        tabA[s, :cut_page] = torch.arange(s * cut_page, (s + 1) * cut_page, dtype=torch.int32)
        tabB[s, cut_page:n] = torch.arange(s * (n - cut_page), (s + 1) * (n - cut_page), dtype=torch.int32)
    idxA = torch.cat([b.block_table[s, :cut_page] for s in range(spec.S)]).long()
    idxB = torch.cat([b.block_table[s, cut_page:n] for s in range(spec.S)]).long()
    kA, vA = b.k_pages[idxA].contiguous(), b.v_pages[idxA].contiguous()
    kB, vB = b.k_pages[idxB].contiguous(), b.v_pages[idxB].contiguous()
    sbA = torch.tensor([[[0, cut // 2, cut]]] * spec.S, dtype=torch.int32, device=DEV)
    sbB = torch.tensor([[[cut, cut + 100, L]]] * spec.S, dtype=torch.int32, device=DEV)
    pA = _lib.micro_attention(b.q, kA, vA, tabA, b.seq_lens, sbA, None, scale=b.scale)
    pB = _lib.micro_attention(b.q, kB, vB, tabB, b.seq_lens, sbB, None, scale=b.scale)
    cat = [torch.cat([x, y], dim=2).contiguous() for x, y in zip(pA, pB)]
    out = _lib.merge(*cat)
    single, *_ = run_gpu(b)
    ref = oracle_out(host_inputs(b), b.scale)
    compare_out(out.cpu().numpy(), ref, 2e-3, "remote halves")
    compare_out(single.cpu().numpy(), ref, 2e-3, "single call")


# ---------------------------------------------------------------------------
# stability and edge shapes
# ---------------------------------------------------------------------------

def test_large_scores_stable():
    """K rows scaled x100 (scores near 100, far past exp overflow in fp32
    without the max shift) stay finite and within tolerance."""
    spec = REDUCED["C2"].replace(S=2, Hq=4, Hkv=4, k_scaled=(0.05, 100.0))
    announce("stability")
    b = wl.build(spec, 21, DEV)
    out, MA, m, e = run_gpu(b)
    assert torch.isfinite(out).all() and torch.isfinite(MA).all() and torch.isfinite(e).all()
    assert float(m.max()) > 50.0
    inp = host_inputs(b)
    compare_out(out.cpu().numpy(), oracle_out(inp, b.scale), 2e-3, "x100")
    oMA, om, oe = oracle_micro(inp, b.scale)
    compare_partials(MA.cpu().numpy(), m.cpu().numpy(), e.cpu().numpy(), oMA, om, oe, 2e-3, "x100")


EDGE = []
for dtype in (wl.F32, wl.BF16):
    for D in (64, 128):
        for P in (16, 64):
            for G in (1, 4, 8):
                EDGE.append((dtype, D, P, G))
# the other page sizes built (32, 128, 256 tokens: 2 to 16 slabs per page)
EDGE += [(wl.BF16, 128, 32, 4), (wl.BF16, 64, 128, 2), (wl.BF16, 128, 256, 4),
         (wl.BF16, 128, 256, 1), (wl.F32, 64, 256, 8)]


@pytest.mark.parametrize("dtype,D,P,G", EDGE)
def test_edge_shapes(dtype, D, P, G):
    """Lengths 1, P-1, P, P+1 and a longer ragged one in one batch, three
    splits each, shuffled table; every (dtype, D, P, G) the library builds."""
    Hkv = 2
    lens = [1, P - 1, P, P + 1, 5 * P + 3]
    spec = wl.Spec(f"edge {dtype} {D} {P} {G}", S=len(lens), Hq=Hkv * G, Hkv=Hkv, D=D, P=P,
                   dtype=dtype, lens=("fixed", max(lens)), table="shuffled", splits=("equal", 3),
                   extra_pages=2)
    announce("edge", dtype, D, P, G)
    b = wl.build(spec, 17, DEV)
    b.seq_lens.copy_(torch.tensor(lens, dtype=torch.int32))
    sb = np.stack([[[(L * j) // 3 for j in range(4)]] for L in lens]).astype(np.int32)
    b.split_bounds = torch.from_numpy(sb).to(DEV)
    out, MA, m, e = run_gpu(b)
    inp = host_inputs(b)
    tol = TOL_OUT[dtype]
    compare_out(out.cpu().numpy(), oracle_out(inp, b.scale), tol, "edge out")
    oMA, om, oe = oracle_micro(inp, b.scale)
    compare_partials(MA.cpu().numpy(), m.cpu().numpy(), e.cpu().numpy(), oMA, om, oe, tol, "edge")


def test_all_masked_but_one_page_and_empty_requests():
    spec = wl.Spec("mask edge", S=3, Hq=8, Hkv=2, D=128, P=64, dtype=wl.BF16,
                   lens=("fixed", 64 * 9 + 5), splits=("equal", 4))
    announce("mask-edge")
    b = wl.build(spec, 23, DEV)
    mask = torch.zeros((3, 2, b.block_table.shape[1]), dtype=torch.uint8, device=DEV)
    mask[0, 0, 4] = 1          # one page kept
    mask[1, 1, 9] = 1          # only the partial last page kept
    mask[2, :, :] = 1          # dense
    b.block_mask = mask
    b.seq_lens[2] = 0          # empty request: every split empty
    out, MA, m, e = run_gpu(b)
    inp = host_inputs(b)
    compare_out(out.cpu().numpy(), oracle_out(inp, b.scale), 2e-3, "mask edge")
    oMA, om, oe = oracle_micro(inp, b.scale)
    compare_partials(MA.cpu().numpy(), m.cpu().numpy(), e.cpu().numpy(), oMA, om, oe, 2e-3, "mask edge")
    assert torch.equal(out[2], torch.zeros_like(out[2]))


def test_check_inputs_counts_violations():
    spec = REDUCED["C3"]
    announce("check-inputs")
    b = wl.build(spec, 0, DEV)
    NP = b.k_pm.shape[0]
    assert _lib.check_inputs(b.block_table, b.seq_lens, NP, spec.P) == 0
    bad = b.block_table.clone()
    lens = b.seq_lens.cpu().numpy()
    s = int(np.argmax(lens))
    bad[s, 0] = NP
    bad[s, 1] = -1
    bad_lens = b.seq_lens.clone()
    bad_lens[0] = spec.max_pages * spec.P + 1
    assert _lib.check_inputs(bad, b.seq_lens, NP, spec.P) == 2
    assert _lib.check_inputs(b.block_table, bad_lens, NP, spec.P) >= 1
