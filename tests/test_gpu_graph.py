"""A decode step captured once in a HIP graph (torch.cuda.CUDAGraph) and
replayed, through the C ABI: append of the step's K/V rows (with page
statistics), seq_lens + 1, MicroAttention with the chunk's reused mask and
split bounds, merge -- as two calls, or as the fused single launch whose
group counters must return to zero for the next replay.  Every replay is
checked bit for bit against the same step run eagerly on the same state:
the kernels are deterministic (one
workgroup owns each item or chunk, whatever order the work queue hands them
out in), so a replay must reproduce the eager bits exactly.  Between
replays the program does eager work of its own and synchronizes, and the
work-queue counter the persistent schedule uses is cleared by a kernel of
the graph, not a memset node.  Needs an MI355X and the built libda.so.
"""

from __future__ import annotations

import sys

import pytest
import torch

from long_context_decode_microattention_amd import _lib
from long_context_decode_microattention_amd import workloads as wl

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
STEPS = 12

# (spec, logical page of the statistics): the GQA matrix-core kernel over a
# selected mask, and the vector kernel over fp32 16-token pages with no mask.
SPECS = {
    "gqa4_bf16_P64": (wl.CONFIGS["C5"].replace(S=2, lens=("fixed", 64 * 60 + 55), reserve=STEPS,
                                               table="shuffled", mask=None, splits=("equal", 4)), 16),
    "mha_f32_D64_P16": (wl.CONFIGS["C1"].replace(S=3, lens=("fixed", 16 * 40 + 9), reserve=STEPS,
                                                 table="shuffled"), 16),
}
# (schedule, chunks): library choice; persistent workgroups on the work
# queue; forced page-range chunks (partials combined by a second kernel)
SCHEDULES = [(0, 0), (2, 0), (1, 3)]


def announce(*parts):
    print("[gpu-case]", *parts, flush=True)
    sys.stdout.flush()


@pytest.fixture(autouse=True)
def _free_memory():
    yield
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


@pytest.mark.parametrize("fused", [False, True], ids=["two_call", "fused"])
@pytest.mark.parametrize("schedule,chunks", SCHEDULES)
@pytest.mark.parametrize("name", list(SPECS))
def test_graph_replay_matches_eager(name, schedule, chunks, fused):
    spec, logical = SPECS[name]
    announce("graph replay", name, f"schedule={schedule} chunks={chunks} fused={fused}")
    b = wl.build(spec, 3, DEV)
    P, Hkv = spec.P, spec.Hkv
    sel = torch.tensor([1 if i >= Hkv // 2 else 0 for i in range(Hkv)], dtype=torch.uint8,
                       device=DEV)
    lens0 = b.seq_lens.clone()
    stats = _lib.page_stats(b.k_pages, b.block_table, lens0, logical=logical, select_heads=sel)
    if spec.dtype == wl.BF16:
        scores = _lib.page_scores(b.q, stats, b.block_table, lens0, P=P, select_heads=sel)
        npg = -(-int(lens0[0].item()) // P)
        mask = _lib.select_pages(scores, lens0, P=P, budget=(npg - 3) // 4, keep_first=1,
                                 keep_last=2, select_heads=sel, horizon=STEPS)
    else:
        mask = None
    bounds = _lib.split_bounds(mask, lens0, P=P, b=8, horizon=STEPS, Hkv=Hkv,
                               max_pages=b.block_table.shape[1])
    toks = [wl.new_tokens(spec, 3, step, DEV) for step in range(STEPS)]
    init = [t.clone() for t in (b.k_pages, b.v_pages, stats)]

    lens = lens0.clone()
    kn, vn = torch.empty_like(toks[0][0]), torch.empty_like(toks[0][1])
    S, Hq, D = b.q.shape
    MA = torch.empty((S, Hq, 8, D), dtype=torch.float32, device=DEV)
    m = torch.empty((S, Hq, 8), dtype=torch.float32, device=DEV)
    e = torch.empty((S, Hq, 8), dtype=torch.float32, device=DEV)
    out = torch.empty((S, Hq, D), dtype=torch.float32, device=DEV)

    sh = _lib.shape_of(b.q, b.k_pages, b.block_table, bounds, b.scale, chunks, schedule)
    # workspaces of the graph's own (the binding's cached ones may be replaced)
    fws = torch.zeros(_lib.attention_workspace_size(sh)[0], dtype=torch.uint8, device=DEV)
    mws = torch.empty(max(16, _lib.workspace_size(sh)), dtype=torch.uint8, device=DEV)

    def step():
        _lib.append_kv(kn, vn, b.block_table, lens, b.k_pages, b.v_pages, stats=stats,
                       logical=logical, select_heads=sel)
        lens.add_(1)
        if fused:  # one launch: partials and merge (group counters in fws)
            _lib.attention(b.q, b.k_pages, b.v_pages, b.block_table, lens, bounds, mask,
                           scale=b.scale, out=out, schedule=schedule, chunks=chunks,
                           workspace=fws)
        else:
            _lib.micro_attention(b.q, b.k_pages, b.v_pages, b.block_table, lens, bounds, mask,
                                 scale=b.scale, out=(MA, m, e), schedule=schedule, chunks=chunks,
                                 workspace=mws)
            _lib.merge(MA, m, e, out=out)

    def restore():
        for t, t0 in zip((b.k_pages, b.v_pages, stats), init):
            t.copy_(t0)
        lens.copy_(lens0)

    # eager reference, step by step
    want = []
    for i in range(STEPS):
        kn.copy_(toks[i][0])
        vn.copy_(toks[i][1])
        step()
        want.append(out.clone())
    want_state = [t.clone() for t in (b.k_pages, b.v_pages, stats)]
    torch.cuda.synchronize()

    # warm-up on a side stream, then capture from the restored state
    restore()
    kn.copy_(toks[0][0])
    vn.copy_(toks[0][1])
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    restore()
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    torch.cuda.synchronize()
    assert torch.equal(lens, lens0), "capture must not run the step"

    noise = torch.empty(1 << 20, device=DEV)
    for i in range(STEPS):
        kn.copy_(toks[i][0])
        vn.copy_(toks[i][1])
        out.fill_(float("nan"))
        graph.replay()
        torch.cuda.synchronize()
        # the program's own eager work between replays
        noise.normal_()
        MA.fill_(float("nan"))
        _ = noise.sum().item()
        assert torch.equal(out, want[i]), f"replay {i}: output differs from the eager step"
        assert torch.equal(lens, lens0 + i + 1), f"replay {i}: seq_lens"
    for got, ref, what in zip((b.k_pages, b.v_pages, stats), want_state, ("K", "V", "stats")):
        assert torch.equal(got, ref), f"{what} after {STEPS} replays differs from the eager steps"
    counters = _lib.attention_workspace_size(sh)[1]
    assert int(fws[:counters].count_nonzero()) == 0, "group counters left non-zero"
