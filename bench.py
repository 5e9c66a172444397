#!/usr/bin/env python3
"""Decode-step benchmark of split-KV attention on one MI355X.

A step is one pass of the whole path over one batch: da_micro_attention
(MicroAttention partials for every request, query head and split) followed by
da_merge (aggregation into the attention output), on inputs already resident
in HBM.  The headline workload is the single 1M-token request (LLaMA-2-7B /
LWM shape, 32 heads, D=128, bf16 K/V, 64-token pages, 32 splits); the
batched GQA + block-sparse workload (8 x 512K, 32/8 heads) is reported beside
it.  Prints ONE JSON line on stdout.

Metric: effective KV-read GB/s = algorithmic bytes / step time, where the
algorithmic bytes are 2 * D * sizeof(elem) per kept token per KV head (every
kept K and V row read once).  roofline.achieved uses the same bytes over the
average duration of the MicroAttention kernel alone, timed with HIP events on
the stream the kernels run on.
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "split-KV decode attention: effective KV-read GB/s vs HBM peak; µs/step"
HBM_PEAK_GBPS = 8000.0  # MI355X HBM3E, published


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def measured_traffic(key, group=None):
    """HBM bytes per launch of a workload's kernel from the committed
    rocprofv3 counter summary (FETCH_SIZE + WRITE_SIZE, scaled by a 1 GiB
    copy), or None when the kernel sources changed since those counters were
    taken.  group None = the MicroAttention kernels, "selector" = the page
    selection kernels."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if group is not None:
        rec = rec.get(group, {})
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "long_context_decode_microattention_amd", "csrc")
    for name in rec.get("files", []):
        with open(os.path.join(csrc, name), "rb") as f:
            h.update(f.read())
    if h.hexdigest() != rec.get("kernel_sources_sha256"):
        return None
    w = rec.get("workloads", {}).get(key)
    return None if w is None else int(w["traffic_bytes"])


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="C4", help="headline workload (C1..C5)")
    ap.add_argument("--secondary", default="C5,C4_fp8,C5_fp8,C4_fp4,C5_fp4,C1,C2,C3",
                    help="comma list reported beside it ('_fp8' / '_fp4': over 8- / 4-bit "
                         "pages; ':dense' / ':masked': only the dense or only the masked KV "
                         "heads of C5), or ''")
    ap.add_argument("--seed", default="0",
                    help="seed(s) of the synthetic inputs, comma list; one record per (workload, seed)")
    ap.add_argument("--settle", type=float, default=1.0,
                    help="seconds of untimed steps per workload before the warm-up steps")
    ap.add_argument("--flush-mib", type=int, default=1024,
                    help="MiB written between the timed steps of workloads that fit in the caches' reach")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-workers", type=int, default=0,
                    help="oracle worker processes (0: one per core this process may run on)")
    ap.add_argument("--no-ceiling", action="store_true", help="skip the streaming-read ceiling")
    ap.add_argument("--chunks", type=int, default=3,
                    help="timed 16-step chunks of the decode loop with a reused selection")
    ap.add_argument("--no-selector", action="store_true",
                    help="skip the page-selection timing on the block-sparse workload")
    return ap.parse_args()


# Workloads whose pools are small enough that the last-level caches could
# keep part of them between steps: timed with a cache flush between steps
# (outside the timed region) and reported as the median step.
FLUSHED = {"C1", "C2", "C3"}


def _settle(step, seconds):
    """Untimed steps for `seconds`: the GPU's clocks and the pools' address
    translations reach their steady state under sustained load (the first
    ~0.3 s of a fresh process measured 3-5% slower)."""
    import torch

    t0 = time.perf_counter()
    while time.perf_counter() - t0 < seconds:
        for _ in range(8):
            step()
        torch.cuda.synchronize()


def _median(x):
    s = sorted(x)
    n = len(s)
    return s[n // 2] if n % 2 else 0.5 * (s[n // 2 - 1] + s[n // 2])


def time_workload(key, steps, warmup, dev, seed=0, settle=1.0, flush_mib=0):
    """Times the decode step of workload `key`; a "_fp8" / "_fp4" suffix runs
    it over 8- / 4-bit pages made from the workload's bf16 pools by
    da_quantize_rows / da_quantize_rows_fp4 (quantization is untimed: it
    belongs to the cache write).  A ":dense" / ":masked" suffix keeps only
    the KV heads a block-masked workload leaves dense, or only those it masks
    (the others' mask rows are cleared, so their items hold no pages and
    their bytes are not counted): the two halves of the step, measured
    apart.  With
    flush_mib > 0 a buffer of that size is overwritten before every timed
    step (outside the events) and the step time is the median; otherwise the
    steps run back to back and the step time is their mean."""
    import torch

    from long_context_decode_microattention_amd import _lib
    from long_context_decode_microattention_amd import workloads as wl

    name, _, heads = key.partition(":")
    bits = 8 if name.endswith("_fp8") else 4 if name.endswith("_fp4") else 16
    fp8 = bits < 16
    base = name[:-4] if fp8 else name
    spec = wl.CONFIGS[base].replace(layout=wl.PREFERRED_LAYOUT.get(base, "page"))
    t0 = time.time()
    b = wl.build(spec, seed, dev)
    torch.cuda.synchronize()
    log(f"[bench] built {key} seed {seed} in {time.time() - t0:.1f}s: NP={b.k_pm.shape[0]}")
    S, Hq, D, B = spec.S, spec.Hq, spec.D, b.max_splits
    if heads:
        if spec.mask is None or heads not in ("dense", "masked"):
            raise ValueError(f"{key}: ':dense' / ':masked' need a block-masked workload")
        masked = [h >= spec.Hkv // 2 for h in range(spec.Hkv)]  # the mask covers the upper half
        for h in range(spec.Hkv):
            if masked[h] != (heads == "masked"):
                b.block_mask[:, h, :] = 0
                for s in range(S):
                    b.kept_pages[s * spec.Hkv + h] = b.kept_pages[s * spec.Hkv + h][:0]
    kept = int(b.kept_tokens().sum())
    if fp8:
        quant = _lib.quantize_rows if bits == 8 else _lib.quantize_rows_fp4
        kc, ks = quant(b.k_pages)
        vc, vs = quant(b.v_pages)
        torch.cuda.synchronize()
        b.k_pages = b.v_pages = None  # the bf16 pools are not needed any more
        torch.cuda.empty_cache()
        # a row of D codes of `bits` bits plus its fp32 scale, K and V
        kv_bytes = kept * 2 * (D * bits // 8 + 4)
        micro = _lib.micro_attention_fp8 if bits == 8 else _lib.micro_attention_fp4
        args = (b.q, kc, ks, vc, vs, b.block_table, b.seq_lens, b.split_bounds, b.block_mask)
    else:
        kv_bytes = b.kv_bytes()
        micro = _lib.micro_attention
        args = (b.q, b.k_pages, b.v_pages, b.block_table, b.seq_lens, b.split_bounds, b.block_mask)
    MA = torch.empty((S, Hq, B, D), dtype=torch.float32, device=dev)
    m = torch.empty((S, Hq, B), dtype=torch.float32, device=dev)
    e = torch.empty((S, Hq, B), dtype=torch.float32, device=dev)
    out = torch.empty((S, Hq, D), dtype=torch.float32, device=dev)

    # a plain copy of known size (1 GiB): the yardstick for the HBM byte counters
    src = torch.empty(1 << 28, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    dst.copy_(src)
    del src, dst
    flush = None
    if flush_mib > 0:
        flush = torch.empty(flush_mib << 18, dtype=torch.int32, device=dev)

    def step():
        micro(*args, scale=b.scale, out=(MA, m, e), pool_layout=b.layout)
        _lib.merge(MA, m, e, out=out)

    _settle(step, settle)
    for _ in range(warmup):
        step()
    torch.cuda.synchronize()

    ev = [torch.cuda.Event(enable_timing=True) for _ in range(3 * steps)]
    torch.cuda.synchronize()
    for i in range(steps):
        if flush is not None:
            flush.fill_(i)
        ev[3 * i].record()
        micro(*args, scale=b.scale, out=(MA, m, e), pool_layout=b.layout)
        ev[3 * i + 1].record()
        _lib.merge(MA, m, e, out=out)
        ev[3 * i + 2].record()
    torch.cuda.synchronize()
    micro_ms = [ev[3 * i].elapsed_time(ev[3 * i + 1]) for i in range(steps)]
    merge_ms = [ev[3 * i + 1].elapsed_time(ev[3 * i + 2]) for i in range(steps)]
    step_ms = [ev[3 * i].elapsed_time(ev[3 * i + 2]) for i in range(steps)]
    if flush is None:
        ms_step = ev[0].elapsed_time(ev[-1]) / steps
        avg_micro = sum(micro_ms) / steps
        avg_merge = sum(merge_ms) / steps
    else:
        ms_step = _median(step_ms)
        avg_micro = _median(micro_ms)
        avg_merge = _median(merge_ms)
    assert torch.isfinite(out).all(), "non-finite output"

    # the same step in one launch (da_attention / da_attention_fp8), beside it
    fused = {8: _lib.attention_fp8, 4: _lib.attention_fp4, 16: _lib.attention}[bits]
    out_f = torch.empty_like(out)

    def step_fused():
        fused(*args, scale=b.scale, out=out_f, pool_layout=b.layout)

    for _ in range(max(1, warmup)):
        step_fused()
    torch.cuda.synchronize()
    fev = [torch.cuda.Event(enable_timing=True) for _ in range(2 * steps)]
    for i in range(steps):
        if flush is not None:
            flush.fill_(i)
        fev[2 * i].record()
        step_fused()
        fev[2 * i + 1].record()
    torch.cuda.synchronize()
    if flush is None:
        us_fused = fev[0].elapsed_time(fev[-1]) * 1e3 / steps
    else:
        us_fused = _median([fev[2 * i].elapsed_time(fev[2 * i + 1]) for i in range(steps)]) * 1e3
    fused_diff = float((out_f - out).abs().max())
    assert fused_diff <= 1e-4, f"one-launch step differs from the two calls by {fused_diff}"
    res = dict(
        workload=spec.name + (f" ({heads} KV heads only)" if heads else ""), key=key, seed=seed,
        kv_bytes=kv_bytes, ms_per_step=ms_step,
        us_per_step=ms_step * 1e3, us_micro=avg_micro * 1e3, us_merge=avg_merge * 1e3,
        us_per_step_median=_median(step_ms) * 1e3,
        us_micro_min=min(micro_ms) * 1e3, merge_share=avg_merge / (avg_micro + avg_merge),
        timing=(f"median of {steps} steps, {flush_mib} MiB written between steps" if flush is not None
                else f"mean of {steps} back-to-back steps"),
        GBps=kv_bytes / (ms_step * 1e-3) / 1e9, micro_GBps=kv_bytes / (avg_micro * 1e-3) / 1e9,
        shape=dict(S=S, Hq=Hq, Hkv=spec.Hkv, D=D, P=spec.P, splits=B,
                   kv_dtype={8: "fp8_e4m3+f32 row scale", 4: "fp4_e2m1+f32 row scale"}.get(bits, spec.dtype),
                   pool_layout="[Hkv, NP, P, D]" if spec.layout == "head" else "[NP, Hkv, P, D]",
                   max_len=spec.max_len, block_mask=spec.mask is not None),
        kept_tokens=kept,
        tokens_per_s=kept / (ms_step * 1e-3),
        us_per_step_one_launch=us_fused, one_launch_max_abs_diff=fused_diff,
    )
    res["frac_of_peak"] = res["GBps"] / HBM_PEAK_GBPS
    res["roofline_frac"] = res["micro_GBps"] / HBM_PEAK_GBPS
    b.out = out  # the timed step's output, compared with the oracle's in oracle_check
    return b, res


def sp_key(spec):
    """Workload key (C1..C5) of a spec."""
    from long_context_decode_microattention_amd import workloads as wl

    return next(k for k, v in wl.CONFIGS.items() if v.name == spec.name)


def time_selector(b, steps, warmup, dev, logical=16):
    """Page selection on a block-sparse workload's own pool: statistics of
    every page of the KV heads it masks, once (the prefill-time cost), then per step the
    page scores of the KV heads the workload masks and the top-K mask with
    the workload's own budget (the same kept count as its seeded mask),
    followed by the attention step over the selected pages."""
    import numpy as np
    import torch

    from long_context_decode_microattention_amd import _lib

    sp = b.spec
    _, keep_first, keep_last, frac = sp.mask
    Hkv, P, D = sp.Hkv, sp.P, sp.D
    flags = torch.tensor([1 if h >= Hkv // 2 else 0 for h in range(Hkv)], dtype=torch.uint8,
                         device=dev)
    n_sel = int(flags.sum().item())
    max_pages = sp.max_pages  # table width (includes spare capacity for appends)
    npg = -(-sp.max_len // P)  # pages holding each request's tokens (fixed lengths)
    budget = int(frac * (npg - keep_first - keep_last))
    esize = sp.esize
    NL = P // logical
    stats = torch.zeros((Hkv, b.k_pm.shape[0], NL, 2, D), dtype=b.k_pages.dtype, device=dev)
    scores = torch.empty((sp.S, Hkv, max_pages), dtype=torch.float32, device=dev)
    mask = torch.empty((sp.S, Hkv, max_pages), dtype=torch.uint8, device=dev)
    ev = lambda: torch.cuda.Event(enable_timing=True)  # noqa: E731

    # statistics of the selected KV heads over the whole pool, timed
    for _ in range(max(1, warmup)):
        _lib.page_stats(b.k_pages, b.block_table, b.seq_lens, logical=logical,
                        select_heads=flags, out=stats, pool_layout=b.layout)
    reps = max(3, steps // 4)
    s0, s1 = ev(), ev()
    s0.record()
    for _ in range(reps):
        _lib.page_stats(b.k_pages, b.block_table, b.seq_lens, logical=logical,
                        select_heads=flags, out=stats, pool_layout=b.layout)
    s1.record()
    torch.cuda.synchronize()
    us_stats = s0.elapsed_time(s1) * 1e3 / reps
    # every key row of a selected head read once, its statistics written once
    key_rows = int(b.seq_lens.sum().item()) * n_sel
    stats_bytes = key_rows * D * esize + sp.S * npg * n_sel * NL * 2 * D * esize

    def select():
        _lib.page_scores(b.q, stats, b.block_table, b.seq_lens, P=P, select_heads=flags, out=scores)

    def topk():
        _lib.select_pages(scores, b.seq_lens, P=P, budget=budget, keep_first=keep_first,
                          keep_last=keep_last, select_heads=flags, out=mask)

    for _ in range(warmup):
        select()
        topk()
    torch.cuda.synchronize()
    # each kernel timed over `steps` launches back to back (idempotent calls),
    # so the figure is its own rate, not that of one launch between two events
    e0, e1, e2 = ev(), ev(), ev()
    e0.record()
    for _ in range(steps):
        select()
    e1.record()
    for _ in range(steps):
        topk()
    e2.record()
    torch.cuda.synchronize()
    us_scores = e0.elapsed_time(e1) * 1e3 / steps
    us_topk = e1.elapsed_time(e2) * 1e3 / steps
    # bytes the score kernel must move: the statistics of the selected KV
    # heads' pages below L_s, plus one fp32 score per (request, KV head, page)
    score_bytes = sp.S * n_sel * npg * NL * 2 * D * esize + sp.S * Hkv * max_pages * 4

    # attention over the selected pages: splits over each head's kept pages
    mask_h = mask.cpu().numpy()
    lens = b.seq_lens.cpu().numpy()
    nb = b.max_splits
    sb = np.zeros((sp.S, Hkv, nb + 1), dtype=np.int32)
    kept = 0
    for s in range(sp.S):
        n = -(-int(lens[s]) // P)
        for h in range(Hkv):
            kp = np.nonzero(mask_h[s, h, :n])[0]
            kept += int(np.minimum((kp + 1) * P, lens[s]).sum() - (kp * P).sum())
            for j in range(1, nb):
                sb[s, h, j] = int(kp[(j * len(kp)) // nb]) * P
            sb[s, h, nb] = int(lens[s])
    sb_t = torch.from_numpy(sb).to(dev)
    MA = torch.empty((sp.S, sp.Hq, nb, D), dtype=torch.float32, device=dev)
    m = torch.empty((sp.S, sp.Hq, nb), dtype=torch.float32, device=dev)
    e = torch.empty_like(m)
    out = torch.empty((sp.S, sp.Hq, D), dtype=torch.float32, device=dev)

    def step():
        select()
        topk()
        _lib.micro_attention(b.q, b.k_pages, b.v_pages, b.block_table, b.seq_lens, sb_t, mask,
                             scale=b.scale, out=(MA, m, e), pool_layout=b.layout)
        _lib.merge(MA, m, e, out=out)

    for _ in range(warmup):
        step()
    t0, t1 = ev(), ev()
    t0.record()
    for _ in range(steps):
        step()
    t1.record()
    torch.cuda.synchronize()
    us_step = t0.elapsed_time(t1) * 1e3 / steps
    kv_bytes = kept * 2 * D * esize
    return dict(
        kernel="page_scores_kernel (da_page_scores)", logical_page=logical, selected_kv_heads=n_sel,
        score_traffic=measured_traffic(f"{sp_key(sp)}_page_scores", "selector"),
        stats_traffic=measured_traffic(f"{sp_key(sp)}_page_stats", "selector"),
        budget=budget, keep_first=keep_first, keep_last=keep_last,
        us_page_scores=us_scores, us_select_topk=us_topk,
        score_bytes=score_bytes, score_GBps=score_bytes / (us_scores * 1e-6) / 1e9,
        roofline_frac=score_bytes / (us_scores * 1e-6) / 1e9 / HBM_PEAK_GBPS,
        us_page_stats=us_stats, stats_bytes=stats_bytes,
        stats_GBps=stats_bytes / (us_stats * 1e-6) / 1e9,
        us_step_with_selection=us_step, kv_bytes_selected=kv_bytes,
        step_GBps_kv_only=kv_bytes / (us_step * 1e-6) / 1e9,
    )


def _kept_tokens(mask_h, lens, P):
    """Tokens below L_s on pages the mask keeps, summed over (request, KV head)."""
    import numpy as np

    total = 0
    for s in range(mask_h.shape[0]):
        L = int(lens[s])
        n = -(-L // P)
        for h in range(mask_h.shape[1]):
            kp = np.nonzero(mask_h[s, h, :n])[0]
            total += int((np.minimum((kp + 1) * P, L) - kp * P).sum())
    return total


def time_decode_chunks(b, chunks, dev, logical=16, chunk=16):
    """The decode loop with a reused selection on a block-sparse workload:
    per chunk of `chunk` steps, page scores + top-K (horizon = chunk) + split
    bounds once, then per step: append the new token's K/V (statistics kept
    current), advance seq_lens, MicroAttention with the reused mask and
    bounds, merge.  Statistics are computed once before the first chunk.
    Every chunk starts again from the workload's lengths (the spare capacity
    of the pool holds one chunk's tokens)."""
    import numpy as np
    import torch

    from long_context_decode_microattention_amd import _lib
    from long_context_decode_microattention_amd import workloads as wl

    sp = b.spec
    _, keep_first, keep_last, frac = sp.mask
    Hkv, P, D = sp.Hkv, sp.P, sp.D
    if sp.reserve < chunk:
        raise ValueError(f"{sp.name}: the pool needs {chunk} tokens of spare capacity")
    flags = torch.tensor([1 if h >= Hkv // 2 else 0 for h in range(Hkv)], dtype=torch.uint8,
                         device=dev)
    npg = -(-sp.max_len // P)
    budget = int(frac * (npg - keep_first - keep_last))
    nb = b.max_splits
    lens0 = b.seq_lens.clone()
    lens = lens0.clone()
    stats = _lib.page_stats(b.k_pages, b.block_table, lens, logical=logical, select_heads=flags,
                            pool_layout=b.layout)
    scores = torch.empty((sp.S, Hkv, sp.max_pages), dtype=torch.float32, device=dev)
    mask = torch.empty((sp.S, Hkv, sp.max_pages), dtype=torch.uint8, device=dev)
    bounds = torch.empty((sp.S, Hkv, nb + 1), dtype=torch.int32, device=dev)
    MA = torch.empty((sp.S, sp.Hq, nb, D), dtype=torch.float32, device=dev)
    m = torch.empty((sp.S, sp.Hq, nb), dtype=torch.float32, device=dev)
    e = torch.empty_like(m)
    out = torch.empty((sp.S, sp.Hq, D), dtype=torch.float32, device=dev)
    new = [wl.new_tokens(sp, 0, i, dev) for i in range(chunk)]

    def run_chunk():
        _lib.page_scores(b.q, stats, b.block_table, lens, P=P, select_heads=flags, out=scores)
        _lib.select_pages(scores, lens, P=P, budget=budget, keep_first=keep_first,
                          keep_last=keep_last, select_heads=flags, horizon=chunk, out=mask)
        _lib.split_bounds(mask, lens, P=P, b=nb, horizon=chunk, out=bounds)
        for i in range(chunk):
            _lib.append_kv(new[i][0], new[i][1], b.block_table, lens, b.k_pages, b.v_pages,
                           stats=stats, logical=logical, select_heads=flags, pool_layout=b.layout)
            lens.add_(1)
            _lib.micro_attention(b.q, b.k_pages, b.v_pages, b.block_table, lens, bounds, mask,
                                 scale=b.scale, out=(MA, m, e), pool_layout=b.layout)
            _lib.merge(MA, m, e, out=out)

    ms = []
    for c in range(chunks + 1):  # the first chunk is a warm-up
        lens.copy_(lens0)
        torch.cuda.synchronize()
        t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        t0.record()
        run_chunk()
        t1.record()
        torch.cuda.synchronize()
        if c:
            ms.append(t0.elapsed_time(t1))
    assert torch.isfinite(out).all(), "non-finite output"
    mask_h = mask.cpu().numpy()
    L0 = lens0.cpu().numpy().astype(np.int64)
    kv_bytes = sum(_kept_tokens(mask_h, L0 + i + 1, P) for i in range(chunk)) * 2 * D * sp.esize
    us_chunk = sum(ms) / len(ms) * 1e3
    return dict(chunk_steps=chunk, chunks_timed=chunks, us_per_chunk=us_chunk,
                us_per_step=us_chunk / chunk, kv_bytes_per_chunk=kv_bytes,
                GBps=kv_bytes / (us_chunk * 1e-6) / 1e9,
                frac_of_peak=kv_bytes / (us_chunk * 1e-6) / 1e9 / HBM_PEAK_GBPS,
                step="append + micro_attention + merge per step; page scores + top-K + split "
                     "bounds once per chunk")


def read_ceiling(b):
    """Streaming-read rate over the workload's own K and V pools."""
    import torch

    from long_context_decode_microattention_amd import _lib

    sink = None
    bufs = (b.k_pages, b.v_pages)
    for buf in bufs:  # warm
        sink = _lib.stream_read(buf, sink)
    torch.cuda.synchronize()
    s, t = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    reps = 3
    s.record()
    for _ in range(reps):
        for buf in bufs:
            _lib.stream_read(buf, sink)
    t.record()
    torch.cuda.synchronize()
    nbytes = sum(x.numel() * x.element_size() for x in bufs) * reps
    return nbytes / (s.elapsed_time(t) * 1e-3) / 1e9


# ---------------------------------------------------------------------------
# the oracle on the host's cores
# ---------------------------------------------------------------------------
#
# A pool of worker processes is forked at start-up, before anything touches
# the GPU, so the workers hold no GPU state.  For a check, the workload's K and
# V pools are copied into memory-mapped files in shared memory; each task is
# one (request, KV head) unit, for which a worker runs oracle.attention over
# its query heads through the real block table and mask, gathering from the
# mapped pools.  Every worker runs one BLAS thread: one process per core.

_POOL = None
_POOL_N = 0


def _worker_init():
    for v in ("OMP_NUM_THREADS", "OPENBLAS_NUM_THREADS", "MKL_NUM_THREADS", "BLIS_NUM_THREADS"):
        os.environ[v] = "1"


def _unit_task(a):
    """One (request, KV head) unit through the fp64 oracle; returns (s, kvh,
    out [G, D] float64, seconds)."""
    import numpy as np

    import oracle

    t0 = time.perf_counter()
    dt = np.dtype(a["dtype"])
    kp = np.memmap(a["k_path"], dtype=dt, mode="r", shape=tuple(a["pool_shape"]))
    vp = np.memmap(a["v_path"], dtype=dt, mode="r", shape=tuple(a["pool_shape"]))
    kvh = a["kvh"]
    if a["head_major"]:  # [Hkv, NP, P, D] -> the head's [NP, 1, P, D]
        kv, vv = kp[kvh][:, None], vp[kvh][:, None]
    else:
        kv, vv = kp[:, kvh:kvh + 1], vp[:, kvh:kvh + 1]
    mask = None if a["mask"] is None else a["mask"][None, None]
    out = oracle.attention(a["q"][None], kv, vv, a["table"][None],
                           np.array([a["L"]], dtype=np.int32), block_mask=mask, scale=a["scale"])
    del kp, vp
    return a["s"], kvh, out[0], time.perf_counter() - t0


def start_pool(n):
    """Fork the oracle workers (call before the GPU is touched)."""
    global _POOL, _POOL_N
    import multiprocessing as mp

    _POOL = mp.get_context("fork").Pool(n, initializer=_worker_init)
    _POOL_N = n


def stop_pool():
    global _POOL
    if _POOL is not None:
        _POOL.close()
        _POOL.join()
        _POOL = None


def _shm_dir():
    return "/dev/shm" if os.path.isdir("/dev/shm") else __import__("tempfile").gettempdir()


def oracle_check(b, label, units=None, one_core_units=0):
    """The fp64 oracle over the given (request, KV head) units of batch b
    (all units when None) on the worker pool, compared with the timed step's
    output b.out.  Returns the wall time on the pool's cores, the oracle's
    effective GB/s over the same algorithmic bytes, the largest deviation of
    the GPU output, and (one_core_units > 0) the same oracle run on one core,
    unit after unit, over the first units."""
    import numpy as np
    import torch

    from long_context_decode_microattention_amd import workloads as wl

    sp = b.spec
    G = sp.G
    h = wl.host
    kept = b.kept_tokens()
    lens = b.seq_lens.cpu().numpy()
    table = b.block_table.cpu().numpy()
    mask = None if b.block_mask is None else b.block_mask.cpu().numpy()
    q = h(b.q)
    got_all = b.out.double().cpu().numpy()
    if units is None:
        units = [(s, kvh) for s in range(sp.S) for kvh in range(sp.Hkv)]
    # the pools into shared memory (untimed: a copy of the workload's input)
    tag = f"da_bench_{os.getpid()}_{label.replace('/', '_')}"
    kpath = os.path.join(_shm_dir(), tag + "_k")
    vpath = os.path.join(_shm_dir(), tag + "_v")
    npdt = np.uint16 if b.k_pages.dtype == torch.bfloat16 else np.float32
    shape = tuple(b.k_pages.shape)
    try:
        for src, path in ((b.k_pages, kpath), (b.v_pages, vpath)):
            mm = np.memmap(path, dtype=npdt, mode="w+", shape=shape)
            dst = torch.from_numpy(mm.view(np.int16) if npdt == np.uint16 else mm)
            step = max(1, shape[0] // 16)
            for i in range(0, shape[0], step):  # in slices: no host copy of the whole pool
                sl = src[i:i + step]
                dst[i:i + step].copy_(sl.view(torch.int16) if npdt == np.uint16 else sl)
            mm.flush()
            del mm, dst
        tasks = []
        for s, kvh in units:
            L = int(lens[s])
            npg = -(-L // sp.P)
            tasks.append(dict(
                s=s, kvh=kvh, k_path=kpath, v_path=vpath, pool_shape=shape, dtype=np.dtype(npdt).str,
                head_major=b.layout == "head", q=q[s, kvh * G:(kvh + 1) * G].copy(),
                table=table[s, :max(npg, 1)].copy(), L=L,
                mask=None if mask is None else mask[s, kvh, :max(npg, 1)].copy(), scale=b.scale))
        order = sorted(range(len(tasks)), key=lambda i: -int(kept[tasks[i]["s"], tasks[i]["kvh"]]))
        t0 = time.perf_counter()
        results = _POOL.map(_unit_task, [tasks[i] for i in order], chunksize=1)
        wall = time.perf_counter() - t0
        one = None
        if one_core_units > 0:
            secs, nb = 0.0, 0
            for tsk in tasks[:one_core_units]:
                _, _, _, sec = _POOL.apply(_unit_task, (tsk,))
                secs += sec
                nb += int(kept[tsk["s"], tsk["kvh"]]) * 2 * sp.D * sp.esize
            one = dict(value=nb / secs / 1e9, unit="GB/s", cores=1, seconds=round(secs, 3),
                       units=f"{min(one_core_units, len(tasks))} (request, KV head) unit(s)")
    finally:
        for path in (kpath, vpath):
            if os.path.exists(path):
                os.remove(path)
    err = 0.0
    for s, kvh, want, _ in results:
        got = got_all[s, kvh * G:(kvh + 1) * G]
        err = max(err, float(np.max(np.abs(got - want))))
    nbytes = sum(int(kept[s, kvh]) for s, kvh in units) * 2 * sp.D * sp.esize
    tol = 1e-5 if sp.dtype == wl.F32 else 2e-3
    assert err <= tol, f"{label}: timed step differs from the oracle by {err:.3e} (> {tol})"
    return dict(units=f"{len(units)}/{sp.S * sp.Hkv}", workers=_POOL_N, wall_s=round(wall, 3),
                GBps=nbytes / wall / 1e9, max_abs_err_vs_step=err, tolerance=tol, one_core=one)


def main():
    a = parse()
    if a.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {a.gpus} is not supported "
              f"(the path is single-GPU; multi-GPU sharding is a design note, not built)", file=sys.stderr)
        sys.exit(2)
    seeds = [int(x) for x in str(a.seed).split(",") if x != ""]
    cores = a.cpu_workers or len(os.sched_getaffinity(0))
    if not a.no_cpu_baseline:
        start_pool(cores)  # before the GPU is touched
    try:
        line = run(a, seeds)
    finally:
        stop_pool()
    print(json.dumps(line), flush=True)


def _rounded(r):
    return {k: (round(v, 4) if isinstance(v, float) else v) for k, v in r.items()}


def run(a, seeds):
    import torch

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    from long_context_decode_microattention_amd import _lib

    _lib.load()
    check = not a.no_cpu_baseline

    def flush_for(key):
        return a.flush_mib if key.split(":")[0].split("_")[0] in FLUSHED else 0

    head, cpu, ceiling, head_selector = None, None, None, None
    records = []
    for seed in seeds:
        b, r = time_workload(a.workload, a.steps, a.warmup, dev, seed, a.settle, flush_for(a.workload))
        # an "_fp8" headline keeps only the 8-bit pools; a half (":dense") is not checked
        bf16_pools = b.k_pages is not None and ":" not in a.workload
        if check and bf16_pools:
            oc = oracle_check(b, f"{a.workload}/{seed}", one_core_units=2)
            r["oracle_check"] = oc
        records.append(r)
        if head is None:
            head = r
            ceiling = None if a.no_ceiling or not bf16_pools else read_ceiling(b)
            if check and bf16_pools:
                cpu = dict(value=oc["GBps"], unit="GB/s", cores=oc["workers"], kind="oracle",
                           sample=(f"{sp_key(b.spec)} (all {oc['units']} (request, KV head) units, "
                                   f"{r['kv_bytes'] / 2**30:.2f} GiB of K+V): fp64 numpy "
                                   f"oracle.attention, one process per core, {oc['wall_s']:.1f} s wall"),
                           wall_s=oc["wall_s"], units=oc["units"], one_core=oc["one_core"],
                           max_abs_err_vs_step=oc["max_abs_err_vs_step"], tolerance=oc["tolerance"])
            if b.spec.mask is not None and not a.no_selector and bf16_pools:
                head_selector = time_selector(b, a.steps, a.warmup, dev)
                head_selector["decode_loop"] = time_decode_chunks(b, a.chunks, dev)
        del b
        torch.cuda.empty_cache()
    secondary = {}
    for key in [k for k in a.secondary.split(",") if k and k != a.workload]:
        for seed in seeds:
            b2, r2 = time_workload(key, a.steps, a.warmup, dev, seed, a.settle, flush_for(key))
            r2["traffic"] = measured_traffic(key) if seed == 0 else None
            if check and b2.k_pages is not None and ":" not in key:
                base = key.split("_")[0]
                r2["oracle_check"] = oracle_check(b2, f"{key}/{seed}",
                                                  one_core_units=(10**9 if base in ("C1", "C2") else 0))
            records.append(r2)
            if seed == seeds[0]:
                secondary[key] = r2
                if b2.spec.mask is not None and not a.no_selector and b2.k_pages is not None \
                        and ":" not in key:
                    secondary[key + "_selector"] = time_selector(b2, a.steps, a.warmup, dev)
                    secondary[key + "_selector"]["decode_loop"] = time_decode_chunks(b2, a.chunks, dev)
            del b2
            torch.cuda.empty_cache()

    kv = head["shape"]["kv_dtype"]
    return {
        "metric": METRIC,
        "value": round(head["GBps"], 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": a.steps,
        "warmup": a.warmup,
        "ms_per_step": round(head["ms_per_step"], 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": kv if kv in ("bf16", "f32") else kv.split("_")[0],
        "data": "synthetic",
        "config": {"workload": head["workload"], **head["shape"], "accum_dtype": "f32",
                   "seed": seeds[0], "kv_bytes_per_step": head["kv_bytes"]},
        "us_per_step": round(head["us_per_step"], 2),
        "us_per_step_median": round(head["us_per_step_median"], 2),
        "frac_of_hbm_peak": round(head["frac_of_peak"], 4),
        "roofline": {
            "bound": "hbm",
            "achieved": round(head["micro_GBps"], 2),
            "peak": HBM_PEAK_GBPS,
            "unit": "GB/s",
            "frac": round(head["micro_GBps"] / HBM_PEAK_GBPS, 4),
            "traffic": measured_traffic(a.workload),
            "kernel": "micro_kernel (da_micro_attention)",
            "us_per_launch": round(head["us_micro"], 2),
        },
        "us_merge": round(head["us_merge"], 2),
        "merge_share_of_step": round(head["merge_share"], 5),
        "us_per_step_one_launch": round(head["us_per_step_one_launch"], 2),
        "read_ceiling_GBps": None if ceiling is None else round(ceiling, 1),
        "frac_of_read_ceiling": None if ceiling is None else round(head["GBps"] / ceiling, 4),
        "cpu_baseline": cpu,
        "selector": None if head_selector is None else _rounded(head_selector),
        "secondary": {k: _rounded(r) for k, r in secondary.items()},
        "records": [dict(workload=r["key"], seed=r["seed"], us_per_step=round(r["us_per_step"], 2),
                         GBps=round(r["GBps"], 1), frac_of_peak=round(r["frac_of_peak"], 4),
                         roofline_frac=round(r["roofline_frac"], 4), timing=r["timing"],
                         us_per_step_one_launch=round(r["us_per_step_one_launch"], 2),
                         oracle_max_abs_err=(None if "oracle_check" not in r
                                             else r["oracle_check"]["max_abs_err_vs_step"]))
                    for r in records],
    }


if __name__ == "__main__":
    main()
