"""The C ABI without a GPU: the library loads, exports every function that
include/da.h declares, and rejects bad arguments on the host with the
documented status codes before anything is launched."""

import ctypes
import os

import pytest

from long_context_decode_microattention_amd import _lib
from long_context_decode_microattention_amd import build as da_build


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(_lib.LIB_PATH):
        da_build.build()
    return _lib.load()


def test_exports_every_declared_function(lib):
    names = _lib.header_functions()
    assert {"da_micro_attention", "da_merge", "da_last_error", "da_check_inputs"} <= set(names)
    for n in names:
        assert hasattr(lib, n), f"libda.so does not export {n}"


FAKE = 0x10000  # aligned, never dereferenced: every call below fails validation first


def good_shape(**kw):
    base = dict(S=2, Hq=8, Hkv=2, D=128, P=16, max_pages=4, max_splits=2, bounds_per_head=0,
                dtype=_lib.DA_BF16, scale=0.088, NP=8, chunks=0, schedule=0)
    base.update(kw)
    return _lib.DaShape(**base)


def call_micro(lib, sh, **ptrs):
    args = dict(q=FAKE, k=FAKE, v=FAKE, table=FAKE, lens=FAKE, bounds=FAKE, mask=None,
                MA=FAKE, m=FAKE, e=FAKE, ws=None, ws_bytes=0)
    args.update(ptrs)
    vp = lambda x: None if x is None else ctypes.c_void_p(x)
    return lib.da_micro_attention(None if sh is None else ctypes.byref(sh),
                                  *(vp(args[k]) for k in ("q", "k", "v", "table", "lens", "bounds",
                                                          "mask", "MA", "m", "e", "ws")),
                                  args["ws_bytes"], None)


@pytest.mark.parametrize("case,status", [
    (dict(sh=None), _lib.DA_ERR_INVALID_ARG),
    (dict(shape=dict(S=0)), _lib.DA_ERR_INVALID_ARG),
    (dict(shape=dict(Hq=6, Hkv=4)), _lib.DA_ERR_INVALID_ARG),
    (dict(shape=dict(max_splits=0)), _lib.DA_ERR_INVALID_ARG),
    (dict(shape=dict(scale=0.0)), _lib.DA_ERR_INVALID_ARG),
    (dict(shape=dict(scale=float("inf"))), _lib.DA_ERR_INVALID_ARG),
    (dict(shape=dict(dtype=7)), _lib.DA_ERR_INVALID_ARG),
    (dict(shape=dict(bounds_per_head=2)), _lib.DA_ERR_INVALID_ARG),
    (dict(shape=dict(max_pages=1 << 28, P=16)), _lib.DA_ERR_INVALID_ARG),
    (dict(ptrs=dict(q=None)), _lib.DA_ERR_INVALID_ARG),
    (dict(ptrs=dict(e=None)), _lib.DA_ERR_INVALID_ARG),
    (dict(ptrs=dict(k=FAKE + 8)), _lib.DA_ERR_INVALID_ARG),
    (dict(ptrs=dict(MA=FAKE + 4)), _lib.DA_ERR_INVALID_ARG),
    (dict(ptrs=dict(lens=FAKE + 2)), _lib.DA_ERR_INVALID_ARG),
    (dict(shape=dict(chunks=-1)), _lib.DA_ERR_INVALID_ARG),
    (dict(shape=dict(chunks=65)), _lib.DA_ERR_INVALID_ARG),
    (dict(shape=dict(chunks=4)), _lib.DA_ERR_INVALID_ARG),  # forced chunks, no workspace
    (dict(shape=dict(chunks=4), ptrs=dict(ws=FAKE, ws_bytes=16)), _lib.DA_ERR_INVALID_ARG),
    (dict(ptrs=dict(ws=FAKE + 4, ws_bytes=4096)), _lib.DA_ERR_INVALID_ARG),  # misaligned workspace
    (dict(shape=dict(schedule=3)), _lib.DA_ERR_INVALID_ARG),
    (dict(shape=dict(schedule=2)), _lib.DA_ERR_INVALID_ARG),  # persistent, no workspace
    (dict(shape=dict(D=96)), _lib.DA_ERR_UNSUPPORTED),
    (dict(shape=dict(P=24)), _lib.DA_ERR_UNSUPPORTED),
    (dict(shape=dict(Hq=6, Hkv=2)), _lib.DA_ERR_UNSUPPORTED),
    (dict(shape=dict(Hq=32, Hkv=2)), _lib.DA_ERR_UNSUPPORTED),
], ids=lambda x: str(x))
def test_micro_rejects(lib, case, status):
    sh = None if "sh" in case else good_shape(**case.get("shape", {}))
    got = call_micro(lib, sh, **case.get("ptrs", {}))
    assert got == status, (got, lib.da_last_error())
    assert len(lib.da_last_error()) > 0


def call_fused(lib, sh, **ptrs):
    args = dict(q=FAKE, k=FAKE, v=FAKE, table=FAKE, lens=FAKE, bounds=FAKE, mask=None, out=FAKE,
                ws=FAKE, ws_bytes=1 << 30)
    args.update(ptrs)
    vp = lambda x: None if x is None else ctypes.c_void_p(x)
    return lib.da_attention(None if sh is None else ctypes.byref(sh),
                            *(vp(args[k]) for k in ("q", "k", "v", "table", "lens", "bounds",
                                                    "mask", "out", "ws")),
                            args["ws_bytes"], None)


@pytest.mark.parametrize("case,status", [
    (dict(sh=None), _lib.DA_ERR_INVALID_ARG),
    (dict(shape=dict(S=0)), _lib.DA_ERR_INVALID_ARG),
    (dict(shape=dict(Hq=6, Hkv=4)), _lib.DA_ERR_INVALID_ARG),
    (dict(ptrs=dict(out=None)), _lib.DA_ERR_INVALID_ARG),
    (dict(ptrs=dict(out=FAKE + 2)), _lib.DA_ERR_INVALID_ARG),
    (dict(ptrs=dict(q=None)), _lib.DA_ERR_INVALID_ARG),
    (dict(ptrs=dict(ws=None, ws_bytes=0)), _lib.DA_ERR_INVALID_ARG),   # the fused step needs one
    (dict(ptrs=dict(ws_bytes=64)), _lib.DA_ERR_INVALID_ARG),           # too small
    (dict(ptrs=dict(ws=FAKE + 8)), _lib.DA_ERR_INVALID_ARG),           # misaligned
    (dict(shape=dict(chunks=4), ptrs=dict(ws_bytes=1024)), _lib.DA_ERR_INVALID_ARG),
    (dict(shape=dict(dtype=_lib.DA_FP8_E4M3)), _lib.DA_ERR_INVALID_ARG),
    (dict(shape=dict(fuse=3)), _lib.DA_ERR_INVALID_ARG),
    (dict(shape=dict(fuse=-1)), _lib.DA_ERR_INVALID_ARG),
    (dict(shape=dict(D=96)), _lib.DA_ERR_UNSUPPORTED),
    (dict(shape=dict(Hq=6, Hkv=2)), _lib.DA_ERR_UNSUPPORTED),
], ids=lambda x: str(x))
def test_fused_rejects(lib, case, status):
    sh = None if "sh" in case else good_shape(**case.get("shape", {}))
    got = call_fused(lib, sh, **case.get("ptrs", {}))
    assert got == status, (got, lib.da_last_error())
    assert len(lib.da_last_error()) > 0


def test_fused_fp8_rejects(lib):
    vp = ctypes.c_void_p
    sh = good_shape(dtype=_lib.DA_BF16)  # the 8-bit entry needs DA_FP8_E4M3
    # q, k_codes, k_scales, v_codes, v_scales, table, lens, bounds, mask, out, workspace
    got = lib.da_attention_fp8(ctypes.byref(sh), *([vp(FAKE)] * 8), None, vp(FAKE), vp(FAKE),
                               1 << 30, None)
    assert got == _lib.DA_ERR_INVALID_ARG
    sh = good_shape(dtype=_lib.DA_FP8_E4M3)
    got = lib.da_attention_fp8(ctypes.byref(sh), vp(FAKE), vp(FAKE), None, vp(FAKE), vp(FAKE),
                               vp(FAKE), vp(FAKE), vp(FAKE), None, vp(FAKE), vp(FAKE), 1 << 30, None)
    assert got == _lib.DA_ERR_INVALID_ARG  # NULL k_scales


def test_fused_workspace_size(lib):
    """Counters first (one int32 per (request, KV head), 16-byte aligned),
    then the work-queue counter and the partials of every split and chunk."""
    sh = good_shape()
    n, c = _lib.attention_workspace_size(sh)
    assert c == 16 and n > c
    chunks = 1
    parts = sh.S * sh.Hq * sh.max_splits * chunks
    # with automatic chunks the partials grow with the chunk count
    assert n >= c + 16 + parts * (sh.D + 2) * 4
    sh2 = good_shape(S=37, Hkv=2, Hq=8)
    n2, c2 = _lib.attention_workspace_size(sh2)
    assert c2 == ((37 * 2 * 4 + 15) // 16) * 16
    forced = good_shape(chunks=3)
    n3, _ = _lib.attention_workspace_size(forced)
    assert n3 >= 16 + 16 + forced.S * forced.Hq * forced.max_splits * 3 * (forced.D + 2) * 4
    with pytest.raises(_lib.DaError):
        _lib.attention_workspace_size(good_shape(D=96))


def test_workspace_size(lib):
    n = ctypes.c_size_t(7)
    # few items: the library cuts splits into chunks and needs a workspace
    sh = good_shape(S=1, Hq=32, Hkv=8, max_pages=8192, max_splits=16, P=64)
    assert lib.da_micro_attention_workspace_size(ctypes.byref(sh), ctypes.byref(n)) == _lib.DA_OK
    chunks = 2  # 128 items -> 2048 / 128 = 16 chunks (capped at 16)
    assert n.value > 0
    # many items: no chunks; only the work-queue counters (8 x 64 bytes)
    sh = good_shape(S=64, Hq=40, Hkv=40, max_pages=2048, max_splits=16, P=16)
    assert lib.da_micro_attention_workspace_size(ctypes.byref(sh), ctypes.byref(n)) == _lib.DA_OK
    assert n.value == 512
    # forced chunks: the counter and the three chunk arrays, 16-byte aligned each
    sh = good_shape(S=2, Hq=8, Hkv=2, D=128, max_splits=3, chunks=5)
    assert lib.da_micro_attention_workspace_size(ctypes.byref(sh), ctypes.byref(n)) == _lib.DA_OK
    rows = 2 * 8 * 3 * 5
    align = lambda x: (x + 15) // 16 * 16
    assert n.value == 512 + align(rows * 128 * 4) + 2 * align(rows * 4)
    assert lib.da_micro_attention_workspace_size(ctypes.byref(sh), None) == _lib.DA_ERR_INVALID_ARG
    del chunks


def test_merge_rejects(lib):
    sh = good_shape()
    vp = ctypes.c_void_p
    assert lib.da_merge(None, vp(FAKE), vp(FAKE), vp(FAKE), vp(FAKE), None) == _lib.DA_ERR_INVALID_ARG
    assert lib.da_merge(ctypes.byref(sh), None, vp(FAKE), vp(FAKE), vp(FAKE), None) == _lib.DA_ERR_INVALID_ARG
    bad = good_shape(max_splits=0)
    assert lib.da_merge(ctypes.byref(bad), vp(FAKE), vp(FAKE), vp(FAKE), vp(FAKE), None) == _lib.DA_ERR_INVALID_ARG
    assert lib.da_merge(ctypes.byref(sh), vp(FAKE + 2), vp(FAKE), vp(FAKE), vp(FAKE), None) == _lib.DA_ERR_INVALID_ARG


@pytest.mark.parametrize("case", [
    dict(sh=None),
    dict(shape=dict(max_splits=0)),
    dict(shape=dict(D=0)),
    dict(n_out=0, slot=0),
    dict(n_out=4, slot=4),
    dict(n_out=4, slot=-1),
    dict(ptrs=dict(MA=None)),
    dict(ptrs=dict(m_out=None)),
    dict(ptrs=dict(e_out=FAKE + 2)),
    dict(ptrs=dict(MA_out=FAKE + 1)),
], ids=lambda x: str(x))
def test_merge_partials_rejects(lib, case):
    sh = None if "sh" in case else good_shape(**case.get("shape", {}))
    p = dict(MA=FAKE, m=FAKE, e=FAKE, MA_out=FAKE, m_out=FAKE, e_out=FAKE)
    p.update(case.get("ptrs", {}))
    got = lib.da_merge_partials(None if sh is None else ctypes.byref(sh), _vp(p["MA"]),
                                _vp(p["m"]), _vp(p["e"]), case.get("n_out", 2),
                                case.get("slot", 1), _vp(p["MA_out"]), _vp(p["m_out"]),
                                _vp(p["e_out"]), None)
    assert got == _lib.DA_ERR_INVALID_ARG, lib.da_last_error()
    assert len(lib.da_last_error()) > 0


def test_check_inputs_and_stream_read_reject(lib):
    vp = ctypes.c_void_p
    sh = good_shape()
    assert lib.da_check_inputs(ctypes.byref(sh), None, vp(FAKE), vp(FAKE), None) == _lib.DA_ERR_INVALID_ARG
    assert lib.da_stream_read(None, 16, vp(FAKE), None) == _lib.DA_ERR_INVALID_ARG
    assert lib.da_stream_read(vp(FAKE), 15, vp(FAKE), None) == _lib.DA_ERR_INVALID_ARG
    assert lib.da_stream_read_sink_words() >= 1


def test_binding_refuses_cpu_tensors():
    import torch
    q = torch.zeros(1, 4, 64)
    with pytest.raises((ValueError, TypeError, RuntimeError)):
        _lib.micro_attention(q, torch.zeros(2, 4, 16, 64), torch.zeros(2, 4, 16, 64),
                             torch.zeros(1, 2, dtype=torch.int32), torch.zeros(1, dtype=torch.int32),
                             torch.zeros(1, 1, 2, dtype=torch.int64))


def _vp(x):
    return None if x is None else ctypes.c_void_p(x)


@pytest.mark.parametrize("case,status", [
    (dict(shape=dict(S=0)), _lib.DA_ERR_INVALID_ARG),
    (dict(shape=dict(Hq=6, Hkv=4)), _lib.DA_ERR_INVALID_ARG),
    (dict(shape=dict(dtype=5)), _lib.DA_ERR_INVALID_ARG),
    (dict(shape=dict(D=96)), _lib.DA_ERR_UNSUPPORTED),
    (dict(shape=dict(Hq=6, Hkv=2)), _lib.DA_ERR_UNSUPPORTED),  # G = 3
    (dict(logical=12), _lib.DA_ERR_UNSUPPORTED),
    (dict(logical=32), _lib.DA_ERR_UNSUPPORTED),  # larger than P = 16
    (dict(shape=dict(P=48), logical=16), _lib.DA_ERR_UNSUPPORTED),  # P / logical = 3
    (dict(shape=dict(P=4096), logical=8), _lib.DA_ERR_UNSUPPORTED),  # P / logical = 512
    (dict(ptrs=dict(k=None)), _lib.DA_ERR_INVALID_ARG),
    (dict(ptrs=dict(stats=FAKE + 4)), _lib.DA_ERR_INVALID_ARG),
])
def test_page_stats_rejects(lib, case, status):
    sh = good_shape(**case.get("shape", {}))
    p = dict(k=FAKE, table=FAKE, lens=FAKE, stats=FAKE)
    p.update(case.get("ptrs", {}))
    got = lib.da_page_stats(ctypes.byref(sh), _vp(p["k"]), _vp(p["table"]), _vp(p["lens"]),
                            case.get("logical", 16), None, _vp(p["stats"]), None)
    assert got == status, _lib.load().da_last_error()


@pytest.mark.parametrize("case,status", [
    (dict(shape=dict(NP=0)), _lib.DA_ERR_INVALID_ARG),
    (dict(logical=4), _lib.DA_ERR_UNSUPPORTED),
    (dict(ptrs=dict(q=None)), _lib.DA_ERR_INVALID_ARG),
    (dict(ptrs=dict(q=FAKE + 8)), _lib.DA_ERR_INVALID_ARG),
    (dict(ptrs=dict(scores=FAKE + 2)), _lib.DA_ERR_INVALID_ARG),
])
def test_page_scores_rejects(lib, case, status):
    sh = good_shape(**case.get("shape", {}))
    p = dict(q=FAKE, stats=FAKE, table=FAKE, lens=FAKE, sel=None, scores=FAKE)
    p.update(case.get("ptrs", {}))
    got = lib.da_page_scores(ctypes.byref(sh), _vp(p["q"]), _vp(p["stats"]), _vp(p["table"]),
                             _vp(p["lens"]), case.get("logical", 16), _vp(p["sel"]),
                             _vp(p["scores"]), None)
    assert got == status, _lib.load().da_last_error()


@pytest.mark.parametrize("case,status", [
    (dict(shape=dict(Hkv=0)), _lib.DA_ERR_INVALID_ARG),
    (dict(args=(-1, 0, 0, 0)), _lib.DA_ERR_INVALID_ARG),
    (dict(args=(4, -2, 0, 0)), _lib.DA_ERR_INVALID_ARG),
    (dict(args=(4, 0, -1, 0)), _lib.DA_ERR_INVALID_ARG),
    (dict(args=(4, 0, 0, -1)), _lib.DA_ERR_INVALID_ARG),
    (dict(ptrs=dict(mask=None)), _lib.DA_ERR_INVALID_ARG),
    (dict(ptrs=dict(scores=FAKE + 1)), _lib.DA_ERR_INVALID_ARG),
    (dict(shape=dict(max_pages=65537, P=16)), _lib.DA_ERR_UNSUPPORTED),
])
def test_select_pages_rejects(lib, case, status):
    sh = good_shape(**case.get("shape", {}))
    p = dict(scores=FAKE, lens=FAKE, sel=None, mask=FAKE)
    p.update(case.get("ptrs", {}))
    budget, kf, kl, hz = case.get("args", (4, 1, 1, 0))
    got = lib.da_select_pages(ctypes.byref(sh), _vp(p["scores"]), _vp(p["lens"]), budget, kf, kl,
                              hz, _vp(p["sel"]), _vp(p["mask"]), None)
    assert got == status, _lib.load().da_last_error()


@pytest.mark.parametrize("case,status", [
    (dict(shape=dict(S=0)), _lib.DA_ERR_INVALID_ARG),
    (dict(shape=dict(dtype=7)), _lib.DA_ERR_INVALID_ARG),
    (dict(shape=dict(D=96)), _lib.DA_ERR_UNSUPPORTED),
    (dict(logical=12, ptrs=dict(stats=FAKE)), _lib.DA_ERR_UNSUPPORTED),
    (dict(ptrs=dict(k_new=None)), _lib.DA_ERR_INVALID_ARG),
    (dict(ptrs=dict(v=FAKE + 8)), _lib.DA_ERR_INVALID_ARG),
    (dict(ptrs=dict(stats=FAKE + 4)), _lib.DA_ERR_INVALID_ARG),
    (dict(ptrs=dict(table=FAKE + 2)), _lib.DA_ERR_INVALID_ARG),
])
def test_append_kv_rejects(lib, case, status):
    sh = good_shape(**case.get("shape", {}))
    p = dict(k_new=FAKE, v_new=FAKE, table=FAKE, lens=FAKE, k=FAKE, v=FAKE, sel=None, stats=None)
    p.update(case.get("ptrs", {}))
    got = lib.da_append_kv(ctypes.byref(sh), _vp(p["k_new"]), _vp(p["v_new"]), _vp(p["table"]),
                           _vp(p["lens"]), _vp(p["k"]), _vp(p["v"]), case.get("logical", 16),
                           _vp(p["sel"]), _vp(p["stats"]), None)
    assert got == status, _lib.load().da_last_error()


@pytest.mark.parametrize("case,status", [
    (dict(shape=dict(max_splits=0)), _lib.DA_ERR_INVALID_ARG),
    (dict(shape=dict(Hkv=0)), _lib.DA_ERR_INVALID_ARG),
    (dict(horizon=-1), _lib.DA_ERR_INVALID_ARG),
    (dict(ptrs=dict(out=None)), _lib.DA_ERR_INVALID_ARG),
    (dict(ptrs=dict(lens=FAKE + 1)), _lib.DA_ERR_INVALID_ARG),
])
def test_split_bounds_rejects(lib, case, status):
    sh = good_shape(**case.get("shape", {}))
    p = dict(mask=None, lens=FAKE, out=FAKE)
    p.update(case.get("ptrs", {}))
    got = lib.da_split_bounds(ctypes.byref(sh), _vp(p["mask"]), _vp(p["lens"]),
                              case.get("horizon", 0), _vp(p["out"]), None)
    assert got == status, _lib.load().da_last_error()


@pytest.mark.parametrize("case,status", [
    (dict(shape=dict(dtype=_lib.DA_BF16)), _lib.DA_ERR_INVALID_ARG),  # needs DA_FP8_E4M3
    (dict(shape=dict(D=96)), _lib.DA_ERR_UNSUPPORTED),
    (dict(shape=dict(Hq=6, Hkv=2)), _lib.DA_ERR_UNSUPPORTED),  # G = 3
    (dict(ptrs=dict(ks=None)), _lib.DA_ERR_INVALID_ARG),
    (dict(ptrs=dict(vs=FAKE + 2)), _lib.DA_ERR_INVALID_ARG),
    (dict(ptrs=dict(k=FAKE + 8)), _lib.DA_ERR_INVALID_ARG),
])
def test_micro_attention_fp8_rejects(lib, case, status):
    sh = good_shape(**{"dtype": _lib.DA_FP8_E4M3, **case.get("shape", {})})
    p = dict(q=FAKE, k=FAKE, ks=FAKE, v=FAKE, vs=FAKE, table=FAKE, lens=FAKE, bounds=FAKE,
             mask=None, MA=FAKE, m=FAKE, e=FAKE, ws=None)
    p.update(case.get("ptrs", {}))
    got = lib.da_micro_attention_fp8(ctypes.byref(sh), *[_vp(p[k]) for k in
                                                         ("q", "k", "ks", "v", "vs", "table", "lens",
                                                          "bounds", "mask", "MA", "m", "e", "ws")],
                                     0, None)
    assert got == status, _lib.load().da_last_error()


def test_fp8_dtype_refused_by_the_bf16_entry_point(lib):
    sh = good_shape(dtype=_lib.DA_FP8_E4M3)
    assert call_micro(lib, sh) == _lib.DA_ERR_INVALID_ARG
    n = ctypes.c_size_t(0)
    assert lib.da_micro_attention_workspace_size(ctypes.byref(sh), ctypes.byref(n)) == _lib.DA_OK


@pytest.mark.parametrize("args,status", [
    ((2, 10, 96), _lib.DA_ERR_UNSUPPORTED),
    ((1, -1, 128), _lib.DA_ERR_INVALID_ARG),
    ((5, 10, 128), _lib.DA_ERR_INVALID_ARG),
    ((1, 0, 128), _lib.DA_OK),  # nothing to do
])
def test_quantize_rows_rejects(lib, args, status):
    dtype, rows, D = args
    dtype = _lib.DA_F32 if dtype == 2 else dtype
    got = lib.da_quantize_rows(dtype, rows, D, _vp(FAKE), _vp(FAKE), _vp(FAKE), None)
    assert got == status, _lib.load().da_last_error()


def test_last_error_is_cleared_by_a_successful_call(lib):
    """da_last_error() describes the most recent call: a failure sets it, the
    next call that returns DA_OK leaves it empty (host-side calls only)."""
    lib.da_last_error.restype = ctypes.c_char_p
    assert lib.da_quantize_rows(_lib.DA_BF16, -1, 128, _vp(FAKE), _vp(FAKE), _vp(FAKE),
                                None) == _lib.DA_ERR_INVALID_ARG
    assert len(lib.da_last_error()) > 0
    assert lib.da_quantize_rows(_lib.DA_BF16, 0, 128, _vp(FAKE), _vp(FAKE), _vp(FAKE),
                                None) == _lib.DA_OK
    assert lib.da_last_error() == b""


def test_quantize_rows_misaligned(lib):
    got = lib.da_quantize_rows(_lib.DA_BF16, 4, 128, _vp(FAKE + 8), _vp(FAKE), _vp(FAKE), None)
    assert got == _lib.DA_ERR_INVALID_ARG
    got = lib.da_quantize_rows(_lib.DA_BF16, 4, 128, _vp(FAKE), _vp(FAKE + 4), _vp(FAKE), None)
    assert got == _lib.DA_ERR_INVALID_ARG


@pytest.mark.parametrize("case,status", [
    (dict(shape=dict(S=0)), _lib.DA_ERR_INVALID_ARG),
    (dict(shape=dict(dtype=_lib.DA_FP8_E4M3)), _lib.DA_ERR_INVALID_ARG),
    (dict(shape=dict(D=96)), _lib.DA_ERR_UNSUPPORTED),
    (dict(ptrs=dict(ks=None)), _lib.DA_ERR_INVALID_ARG),
    (dict(ptrs=dict(k_new=FAKE + 8)), _lib.DA_ERR_INVALID_ARG),
    (dict(ptrs=dict(kc=FAKE + 4)), _lib.DA_ERR_INVALID_ARG),
    (dict(ptrs=dict(vs=FAKE + 2)), _lib.DA_ERR_INVALID_ARG),
    (dict(ptrs=dict(stats=FAKE), logical=12), _lib.DA_ERR_UNSUPPORTED),
    (dict(ptrs=dict(stats=FAKE + 8)), _lib.DA_ERR_INVALID_ARG),
])
def test_append_kv_fp8_rejects(lib, case, status):
    sh = good_shape(**case.get("shape", {}))
    p = dict(k_new=FAKE, v_new=FAKE, table=FAKE, lens=FAKE, kc=FAKE, ks=FAKE, vc=FAKE, vs=FAKE)
    p.update(case.get("ptrs", {}))
    got = lib.da_append_kv_fp8(ctypes.byref(sh), *[_vp(p[k]) for k in
                                                   ("k_new", "v_new", "table", "lens", "kc", "ks",
                                                    "vc", "vs")], case.get("logical", 16), None,
                               _vp(p.get("stats")), None)
    assert got == status, _lib.load().da_last_error()


def test_fused_workspace_clean_prefix_bookkeeping():
    """The binding's cached workspace for the one-launch step (host logic,
    CPU tensors): a new buffer is all zero; a call whose counters reach past
    what the previous call left clean gets exactly that range zeroed first;
    a buffer too small is replaced by a larger zeroed one."""
    w = _lib._FusedWorkspace()
    buf = w.get("cpu", 256, 32)
    assert buf.numel() == 256 and int(buf.count_nonzero()) == 0
    buf[32:].fill_(7)          # the call's partials land after its 32 counter bytes
    again = w.get("cpu", 256, 32)
    assert again is buf and int(buf[:32].count_nonzero()) == 0
    assert int((buf[32:] == 7).sum()) == 224   # not touched: this call's counters end at 32
    grown = w.get("cpu", 256, 96)               # more counters, over the old partials
    assert grown is buf
    assert int(buf[:96].count_nonzero()) == 0 and int((buf[96:] == 7).sum()) == 160
    buf[96:].fill_(5)
    small = w.get("cpu", 128, 16)               # fits: same buffer, clean prefix shrinks to 16
    assert small is buf and w.clean == 16
    buf[16:].fill_(3)
    w.get("cpu", 256, 64)
    assert int(buf[:64].count_nonzero()) == 0 and int((buf[64:] == 3).sum()) == 192
    big = w.get("cpu", 1024, 64)                # too small: a fresh zeroed buffer
    assert big is not buf and big.numel() == 1024 and int(big.count_nonzero()) == 0


def _call_quant_step(fn, sh, **ptrs):
    p = dict(q=FAKE, kc=FAKE, ks=FAKE, vc=FAKE, vs=FAKE, table=FAKE, lens=FAKE, bounds=FAKE,
             MA=FAKE, m=FAKE, e=FAKE)
    p.update(ptrs)
    return fn(ctypes.byref(sh), *[_vp(p[k]) for k in ("q", "kc", "ks", "vc", "vs", "table", "lens",
                                                      "bounds")],
              None, _vp(p["MA"]), _vp(p["m"]), _vp(p["e"]), None, 0, None)


@pytest.mark.parametrize("case,status", [
    (dict(shape=dict(dtype=_lib.DA_BF16)), _lib.DA_ERR_INVALID_ARG),       # needs DA_FP4_E2M1
    (dict(shape=dict(dtype=_lib.DA_FP8_E4M3)), _lib.DA_ERR_INVALID_ARG),   # the 8-bit type
    (dict(ptrs=dict(ks=None)), _lib.DA_ERR_INVALID_ARG),
    (dict(ptrs=dict(vs=FAKE + 2)), _lib.DA_ERR_INVALID_ARG),
    (dict(ptrs=dict(kc=FAKE + 8)), _lib.DA_ERR_INVALID_ARG),                # codes 16-byte aligned
    (dict(shape=dict(D=96)), _lib.DA_ERR_UNSUPPORTED),
    (dict(shape=dict(D=64, P=16, Hq=2, Hkv=2)), _lib.DA_ERR_UNSUPPORTED),  # D 64, G 1 needs P >= 32
], ids=lambda x: str(x))
def test_micro_attention_fp4_rejects(lib, case, status):
    sh = good_shape(**{"dtype": _lib.DA_FP4_E2M1, **case.get("shape", {})})
    got = _call_quant_step(lib.da_micro_attention_fp4, sh, **case.get("ptrs", {}))
    assert got == status, (got, lib.da_last_error())


def test_fp8_entry_rejects_fp4_pages(lib):
    sh = good_shape(dtype=_lib.DA_FP4_E2M1)
    assert _call_quant_step(lib.da_micro_attention_fp8, sh) == _lib.DA_ERR_INVALID_ARG
    assert b"DA_FP8_E4M3" in lib.da_last_error()
    sh = good_shape(dtype=_lib.DA_FP4_E2M1)
    assert call_micro(lib, sh) == _lib.DA_ERR_INVALID_ARG  # the bf16 / fp32 entry point


def test_quantize_rows_fp4_rejects(lib):
    assert lib.da_quantize_rows_fp4(_lib.DA_BF16, 4, 96, _vp(FAKE), _vp(FAKE), _vp(FAKE),
                                    None) == _lib.DA_ERR_UNSUPPORTED
    assert lib.da_quantize_rows_fp4(7, 4, 128, _vp(FAKE), _vp(FAKE), _vp(FAKE),
                                    None) == _lib.DA_ERR_INVALID_ARG
    # 4-bit codes only need 4-byte alignment (a lane writes one word), not 8
    assert lib.da_quantize_rows_fp4(_lib.DA_BF16, 4, 128, _vp(FAKE), _vp(FAKE + 2), _vp(FAKE),
                                    None) == _lib.DA_ERR_INVALID_ARG
    assert lib.da_quantize_rows_fp4(_lib.DA_BF16, 0, 128, None, None, None, None) == _lib.DA_OK


def test_fp4_workspace_size_counts_packed_rows(lib):
    """The chunk heuristic prices a 4-bit row at D / 2 + 4 bytes: the same
    shape is cut at most as much as over 8-bit pages."""
    n4, n8 = ctypes.c_size_t(0), ctypes.c_size_t(0)
    sh4 = good_shape(S=8, Hq=32, Hkv=8, max_pages=8193, max_splits=16, P=64, dtype=_lib.DA_FP4_E2M1)
    sh8 = good_shape(S=8, Hq=32, Hkv=8, max_pages=8193, max_splits=16, P=64, dtype=_lib.DA_FP8_E4M3)
    assert lib.da_micro_attention_workspace_size(ctypes.byref(sh4), ctypes.byref(n4)) == _lib.DA_OK
    assert lib.da_micro_attention_workspace_size(ctypes.byref(sh8), ctypes.byref(n8)) == _lib.DA_OK
    assert 0 < n4.value <= n8.value
