"""8-bit (FP8 E4M3) KV pages through the C ABI (da_quantize_rows,
da_micro_attention_fp8) against the fp64 oracles on the same seeded inputs.
Needs an MI355X and the built libda.so.

Bars: codes and scales are integer / fp32-decided work and are compared bit
for bit with the oracle's quantization (both take the rounding decision in
fp32); attention over the quantized pages is compared with the oracle's
attention over the exactly dequantized values at the bf16 tolerance (max-abs
2e-3 on the output; m_j, e_j, MA_j / e_j as for bf16 pages): the GPU reads
the same codes and scales, widens them exactly and accumulates in fp32, so
only the accumulation order differs.
"""

from __future__ import annotations

import sys

import numpy as np
import pytest
import torch

import oracle
import oracle.quant as oq
from harness import compare_out, compare_partials
from long_context_decode_microattention_amd import _lib
from long_context_decode_microattention_amd import workloads as wl

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
TOL = 2e-3


def announce(*parts):
    print("[gpu-case]", *parts, flush=True)
    sys.stdout.flush()


@pytest.fixture(autouse=True)
def _free_memory():
    yield
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def _bits(t):
    return wl.host(t)


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_quantize_rows_bit_exact(dtype, D):
    """Random rows at several magnitudes, an all-zero row, a row with one
    non-zero, rows whose quotients x / s land exactly on E4M3 midpoints, tiny
    and huge magnitudes, negative values that round to zero."""
    announce("quantize", dtype, D)
    rng = np.random.default_rng(D + (dtype == "f32"))
    rows = (rng.standard_normal((300, D)) * rng.choice([1e-20, 1e-3, 1.0, 40.0, 1e20], (300, 1)))
    rows[0] = 0.0
    rows[1] = 0.0
    rows[1, 5] = -3.0
    tie = np.zeros(D)
    tie[:6] = [3.5, 1.0625, 1.1875, -1.0625, 0.5 + 1 / 256, -1e-6]  # y = 448, 136, 152, -136, 65, ~0
    rows[2] = tie
    rows[3] = np.linspace(-1, 1, D)
    x = torch.from_numpy(rows.astype(np.float32))
    if dtype == "bf16":
        x = x.to(torch.bfloat16)
    x = x.to(DEV)
    codes, scales = _lib.quantize_rows(x)
    torch.cuda.synchronize()
    want_c, want_s = oq.quantize_rows(_bits(x))
    got_s = scales.cpu().numpy()
    assert np.array_equal(got_s.view(np.uint32), want_s.view(np.uint32)), "scales differ"
    got_c = codes.cpu().numpy()
    bad = np.argwhere(got_c != want_c)
    assert bad.size == 0, f"codes differ at {bad[:5].tolist()}"


# Reduced workloads with bf16 queries (the fp8 entry point's q type): same
# head shapes, page sizes, split rules and structure as the full ones.
CASES = {
    "C1_bf16": wl.CONFIGS["C1"].replace(dtype=wl.BF16),
    "C2": wl.CONFIGS["C2"].replace(S=2),
    "C3": wl.CONFIGS["C3"].replace(S=6, Hq=8, Hkv=8),
    "C4": wl.CONFIGS["C4"].replace(Hq=8, Hkv=8, lens=("fixed", 32768 + 21)),
    "C5": wl.CONFIGS["C5"].replace(S=2, lens=("fixed", 32768)),
    "C5_G2_D64": wl.CONFIGS["C5"].replace(S=2, Hq=16, D=64, lens=("fixed", 8192 + 7)),
    "C5_G8": wl.CONFIGS["C5"].replace(S=1, Hq=64, lens=("fixed", 8192 + 50)),
    "C5_G8_P32": wl.CONFIGS["C5"].replace(S=1, Hq=64, P=32, lens=("fixed", 8192 + 19)),
    # pages of 32 and 128 tokens (one and four 32-token slabs per page of the
    # grouped-query kernel), splits cut mid-slab, ragged last page
    "C5_P32": wl.CONFIGS["C5"].replace(S=2, P=32, lens=("fixed", 16384 + 13)),
    "C5_P128_G2": wl.CONFIGS["C5"].replace(S=2, Hq=16, P=128, lens=("fixed", 16384 + 77)),
    "C4_G4_P32_mid": wl.CONFIGS["C4"].replace(Hq=8, Hkv=2, P=32, lens=("fixed", 8192 + 21),
                                               splits=("equal", 7)),
    # 64-token pages with splits cut inside a slab (the packed softmax's
    # partial slabs), four and eight query heads per KV head
    "C4_G4_P64_mid": wl.CONFIGS["C4"].replace(Hq=8, Hkv=2, P=64, lens=("fixed", 8192 + 37),
                                               splits=("equal", 7)),
    "C4_G8_P64_mid": wl.CONFIGS["C4"].replace(Hq=16, Hkv=2, P=64, lens=("fixed", 8192 + 37),
                                               splits=("equal", 7)),
    # the largest page size built: 256 tokens (8 slabs of 32 or 16 of 16 per page)
    "C4_P256": wl.CONFIGS["C4"].replace(Hq=4, Hkv=4, P=256, lens=("fixed", 256 * 20 + 77),
                                        splits=("equal", 5)),
    "C5_P256_G4": wl.CONFIGS["C5"].replace(S=1, P=256, lens=("fixed", 256 * 24 + 3)),
}


def _quantized(b):
    """GPU quantization of the batch's pools, checked bit for bit against
    the oracle's; returns the device codes / scales and the host dequantized
    pools (float64) for the oracle's attention."""
    kc, ks = _lib.quantize_rows(b.k_pages)
    vc, vs = _lib.quantize_rows(b.v_pages)
    torch.cuda.synchronize()
    okc, oks = oq.quantize_rows(_bits(b.k_pages))
    ovc, ovs = oq.quantize_rows(_bits(b.v_pages))
    assert np.array_equal(kc.cpu().numpy(), okc) and np.array_equal(vc.cpu().numpy(), ovc)
    assert np.array_equal(ks.cpu().numpy(), oks) and np.array_equal(vs.cpu().numpy(), ovs)
    return (kc, ks, vc, vs), (oq.dequantize(okc, oks), oq.dequantize(ovc, ovs))


def _run(b, dev_q, chunks=0, workspace=None):
    kc, ks, vc, vs = dev_q
    MA, m, e = _lib.micro_attention_fp8(b.q, kc, ks, vc, vs, b.block_table, b.seq_lens,
                                        b.split_bounds, b.block_mask, scale=b.scale, chunks=chunks,
                                        workspace=workspace, pool_layout=b.layout)
    out = _lib.merge(MA, m, e)
    torch.cuda.synchronize()
    return out, MA, m, e


@pytest.mark.parametrize("seed", [0, 1])
@pytest.mark.parametrize("cfg", sorted(CASES))
def test_fp8_attention_parity(cfg, seed):
    spec = CASES[cfg]
    announce("fp8 attention", cfg, "seed", seed)
    b = wl.build(spec, seed, DEV)
    dev_q, (kd, vd) = _quantized(b)
    out, MA, m, e = _run(b, dev_q)
    h = wl.host
    args = (h(b.q), kd, vd, h(b.block_table), h(b.seq_lens))
    mask = None if b.block_mask is None else h(b.block_mask)
    want = oracle.attention(*args, block_mask=mask, scale=b.scale)
    compare_out(out.cpu().numpy(), want, TOL, f"{cfg}/{seed} out")
    oMA, om, oe = oracle.micro_attention(*args, h(b.split_bounds), block_mask=mask, scale=b.scale)
    compare_partials(MA.cpu().numpy(), m.cpu().numpy(), e.cpu().numpy(), oMA, om, oe, TOL,
                     f"{cfg}/{seed} partials")


@pytest.mark.parametrize("chunks", [1, 3, 7])
@pytest.mark.parametrize("cfg", ["C4", "C5"])
def test_fp8_forced_chunks(cfg, chunks):
    spec = CASES[cfg]
    announce("fp8 chunks", cfg, chunks)
    b = wl.build(spec, 2, DEV)
    dev_q, (kd, vd) = _quantized(b)
    ws = torch.empty(1 << 24, dtype=torch.uint8, device=DEV)
    out, *_ = _run(b, dev_q, chunks=chunks, workspace=ws)
    h = wl.host
    mask = None if b.block_mask is None else h(b.block_mask)
    want = oracle.attention(h(b.q), kd, vd, h(b.block_table), h(b.seq_lens), block_mask=mask,
                            scale=b.scale)
    compare_out(out.cpu().numpy(), want, TOL, f"{cfg} chunks={chunks}")


@pytest.mark.parametrize("cfg", ["C4", "C5", "C5_G2_D64"])
def test_fp8_unread_slots_poisoned(cfg):
    """NaN codes (0x7f) and NaN scales in every slot no split reads (past L_s
    in the last page, masked pages, pages no table names): the output must
    not change."""
    spec = CASES[cfg].replace(extra_pages=3, table="shuffled")
    announce("fp8 poison", cfg)
    b = wl.build(spec, 3, DEV)
    (kc, ks, vc, vs), (kd, vd) = _quantized(b)
    h = wl.host
    table, lens = h(b.block_table), h(b.seq_lens)
    mask = None if b.block_mask is None else h(b.block_mask)
    P = spec.P
    read = np.zeros(ks.shape, dtype=bool)  # [NP, Hkv, P]
    for s in range(spec.S):
        L = int(lens[s])
        for lp in range(-(-L // P)):
            for kvh in range(spec.Hkv):
                if mask is not None and not mask[s, kvh, lp]:
                    continue
                n = min(P, L - lp * P)
                read[table[s, lp], kvh, :n] = True
    unread = torch.from_numpy(~read).to(DEV)
    for c in (kc, vc):
        c[unread] = 0x7F
    for sc in (ks, vs):
        sc[unread] = float("nan")
    out, *_ = _run(b, (kc, ks, vc, vs))
    want = oracle.attention(h(b.q), kd, vd, table, lens, block_mask=mask, scale=b.scale)
    compare_out(out.cpu().numpy(), want, TOL, f"{cfg} poisoned")


@pytest.mark.slow
@pytest.mark.parametrize("cfg", ["C4", "C5"])
def test_fp8_full_size_sampled(cfg):
    """Full-size workload quantized on the GPU and run in the launch
    configuration the benchmark times; sampled (request, KV head) units
    against the oracle on those units alone."""
    spec = wl.CONFIGS[cfg].replace(layout=wl.PREFERRED_LAYOUT.get(cfg, "page"))
    announce("fp8 full", cfg, spec.layout)
    b = wl.build(spec, 0, DEV)
    kc, ks = _lib.quantize_rows(b.k_pages)
    vc, vs = _lib.quantize_rows(b.v_pages)
    out, *_ = _run(b, (kc, ks, vc, vs))
    if b.layout == "head":  # page-major views for the host-side selection below
        kc, ks, vc, vs = (t.transpose(0, 1) for t in (kc, ks, vc, vs))
    h = wl.host
    G, P = spec.G, spec.P
    units = [(0, 0), (0, spec.Hkv - 1)] if spec.S == 1 else [(0, 5), (spec.S - 1, 2)]
    for s, kvh in units:
        announce("unit", s, kvh)
        L = int(b.seq_lens[s].item())
        n = -(-L // P)
        pages = b.block_table[s, :n].long()
        sub = lambda t: h(t[:, kvh:kvh + 1].index_select(0, pages).contiguous())  # noqa: E731
        kc_u, vc_u = sub(kc), sub(vc)
        ks_u, vs_u = sub(ks), sub(vs)
        okc, oks = oq.quantize_rows(sub(b.k_pm))
        assert np.array_equal(kc_u, okc) and np.array_equal(ks_u, oks), f"unit ({s},{kvh}) codes"
        q = h(b.q[s:s + 1, kvh * G:(kvh + 1) * G].contiguous())
        mask = None
        if b.block_mask is not None:
            mask = h(b.block_mask[s:s + 1, kvh:kvh + 1, :n].contiguous())
        want = oracle.attention(q, oq.dequantize(kc_u, ks_u), oq.dequantize(vc_u, vs_u),
                                np.arange(n, dtype=np.int32)[None], np.array([L], dtype=np.int32),
                                block_mask=mask, scale=b.scale)
        got = out[s:s + 1, kvh * G:(kvh + 1) * G].cpu().numpy()
        compare_out(got, want, TOL, f"unit ({s},{kvh})")


def _host_append_fp8(codes, scales, table, lens, new_rows):
    """Oracle of an 8-bit append: quantize the new rows, then write codes and
    scales through the table (scales as one-element rows)."""
    import oracle.decode as odec
    c_new, s_new = oq.quantize_rows(new_rows)
    c2, s2 = odec.append_kv(codes, scales[..., None], table, lens, c_new, s_new[..., None])
    return c2, s2[..., 0]


@pytest.mark.parametrize("cfg", ["C4", "C5", "C5_G2_D64"])
def test_append_fp8_matches_oracle(cfg):
    """Consecutive 8-bit appends across a page boundary: after every step the
    code and scale pools equal the oracle's (quantize the new rows, write them
    through the table) bit for bit; the statistics kept from the bf16 key rows
    (upper half of the KV heads) equal the oracle's statistics of the bf16
    cache with the same rows appended."""
    import oracle.decode as odec
    import oracle.selector as osel
    spec = CASES[cfg].replace(reserve=24, table="shuffled", extra_pages=2)
    announce("fp8 append", cfg)
    b = wl.build(spec, 4, DEV)
    (kc, ks, vc, vs), _ = _quantized(b)
    h = wl.host
    table = h(b.block_table)
    okc, oks, ovc, ovs = h(kc), h(ks), h(vc), h(vs)
    ok_bf16 = h(b.k_pages)  # the full-precision keys the statistics follow
    lens = b.seq_lens.clone()
    logical = 16
    flags = np.array([1 if i >= spec.Hkv // 2 else 0 for i in range(spec.Hkv)], dtype=np.uint8)
    sel_t = torch.from_numpy(flags).to(DEV)
    stats = _lib.page_stats(b.k_pages, b.block_table, lens, logical=logical, select_heads=sel_t)
    on = flags.astype(bool)
    for step in range(20):
        kn, vn = wl.new_tokens(spec, 4, step, DEV)
        _lib.append_kv_fp8(kn, vn, b.block_table, lens, kc, ks, vc, vs, stats=stats,
                           logical=logical, select_heads=sel_t)
        L = h(lens)
        okc, oks = _host_append_fp8(okc, oks, table, L, h(kn))
        ovc, ovs = _host_append_fp8(ovc, ovs, table, L, h(vn))
        ok_bf16, _ = odec.append_kv(ok_bf16, ok_bf16, table, L, h(kn), h(kn))
        lens += 1
        torch.cuda.synchronize()
        assert np.array_equal(h(kc), okc) and np.array_equal(h(vc), ovc), f"{cfg} step {step}: codes"
        assert np.array_equal(h(ks), oks) and np.array_equal(h(vs), ovs), f"{cfg} step {step}: scales"
        if step % 7 == 6 or step == 19:
            want = osel.page_stats(ok_bf16, table, h(lens), logical=logical)
            got = oracle.to_f64(h(stats.transpose(0, 1).contiguous()))
            assert np.array_equal(got[:, on], want[:, on]), f"{cfg} step {step}: statistics"


def test_fp8_decode_chunk():
    """16 decode steps over 8-bit pages with a reused mask: split bounds once
    (horizon 16), then per step an 8-bit append and the attention step; every
    step's output matches the oracle's attention over the oracle's pools."""
    import oracle.decode as odec
    chunk = 16
    spec = CASES["C5"].replace(lens=("fixed", 64 * 40 + 57), reserve=chunk)
    announce("fp8 decode chunk")
    b = wl.build(spec, 5, DEV)
    (kc, ks, vc, vs), _ = _quantized(b)
    h = wl.host
    table = h(b.block_table)
    mask = b.block_mask.clone()
    # keep the pages the chunk's tokens open (the horizon of a reused selection)
    L0 = int(b.seq_lens[0].item())
    mask[:, :, L0 // spec.P:-(-(L0 + chunk) // spec.P)] = 1
    lens = b.seq_lens.clone()
    bounds = _lib.split_bounds(mask, lens, P=spec.P, b=8, horizon=chunk)
    okc, oks, ovc, ovs = h(kc), h(ks), h(vc), h(vs)
    mask_h = h(mask)
    for step in range(chunk):
        kn, vn = wl.new_tokens(spec, 5, step, DEV)
        _lib.append_kv_fp8(kn, vn, b.block_table, lens, kc, ks, vc, vs)
        okc, oks = _host_append_fp8(okc, oks, table, h(lens), h(kn))
        ovc, ovs = _host_append_fp8(ovc, ovs, table, h(lens), h(vn))
        lens += 1
        MA, m, e = _lib.micro_attention_fp8(b.q, kc, ks, vc, vs, b.block_table, lens, bounds, mask,
                                            scale=b.scale)
        out = _lib.merge(MA, m, e)
        torch.cuda.synchronize()
        want = oracle.attention(h(b.q), oq.dequantize(okc, oks), oq.dequantize(ovc, ovs), table,
                                h(lens), block_mask=mask_h, scale=b.scale)
        compare_out(out.cpu().numpy(), want, TOL, f"fp8 chunk step {step}")
