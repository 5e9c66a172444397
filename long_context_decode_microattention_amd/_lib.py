"""ctypes binding of libda.so (C ABI in include/da.h).

Argument marshalling only: shapes are read off the tensors, outputs are
allocated with torch (device memory is plumbing here), and every step of the
computation runs in the library's HIP kernels on the current torch stream.
There is no fallback: if the library is missing or a call fails, an
exception is raised.
"""

from __future__ import annotations

import ctypes
import math
import os
import re
from typing import Optional

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libda.so")
HEADER = os.path.join(os.path.dirname(HERE), "include", "da.h")

DA_OK, DA_ERR_INVALID_ARG, DA_ERR_UNSUPPORTED, DA_ERR_HIP = 0, 1, 2, 3
DA_F32, DA_BF16, DA_FP8_E4M3, DA_FP4_E2M1 = 0, 1, 2, 3
STATUS_NAMES = {0: "DA_OK", 1: "DA_ERR_INVALID_ARG", 2: "DA_ERR_UNSUPPORTED", 3: "DA_ERR_HIP"}


class DaShape(ctypes.Structure):
    _fields_ = [
        ("S", ctypes.c_int32),
        ("Hq", ctypes.c_int32),
        ("Hkv", ctypes.c_int32),
        ("D", ctypes.c_int32),
        ("P", ctypes.c_int32),
        ("max_pages", ctypes.c_int32),
        ("max_splits", ctypes.c_int32),
        ("bounds_per_head", ctypes.c_int32),
        ("dtype", ctypes.c_int32),
        ("scale", ctypes.c_float),
        ("NP", ctypes.c_int64),
        ("chunks", ctypes.c_int32),
        ("schedule", ctypes.c_int32),
        ("pool_layout", ctypes.c_int32),
        ("fuse", ctypes.c_int32),
    ]


class DaError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{STATUS_NAMES.get(status, status)}: {message}")
        self.status = status
        self.message = message


_LIB = None
_VP = ctypes.c_void_p


def load() -> ctypes.CDLL:
    """Load libda.so (once) and declare its signatures."""
    global _LIB
    if _LIB is not None:
        return _LIB
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(
            f"{LIB_PATH} is not built; run __graft_entry__.build() (hipcc, gfx950) first")
    lib = ctypes.CDLL(LIB_PATH)
    sp = ctypes.POINTER(DaShape)
    lib.da_micro_attention.argtypes = [sp, _VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP,
                                       _VP, ctypes.c_size_t, _VP]
    lib.da_micro_attention.restype = ctypes.c_int
    lib.da_micro_attention_workspace_size.argtypes = [sp, ctypes.POINTER(ctypes.c_size_t)]
    lib.da_micro_attention_workspace_size.restype = ctypes.c_int
    lib.da_merge.argtypes = [sp, _VP, _VP, _VP, _VP, _VP]
    lib.da_merge.restype = ctypes.c_int
    lib.da_merge_partials.argtypes = [sp, _VP, _VP, _VP, ctypes.c_int32, ctypes.c_int32, _VP, _VP,
                                      _VP, _VP]
    lib.da_merge_partials.restype = ctypes.c_int
    lib.da_check_inputs.argtypes = [sp, _VP, _VP, _VP, _VP]
    lib.da_check_inputs.restype = ctypes.c_int
    lib.da_last_error.argtypes = []
    lib.da_last_error.restype = ctypes.c_char_p
    lib.da_page_stats.argtypes = [sp, _VP, _VP, _VP, ctypes.c_int32, _VP, _VP, _VP]
    lib.da_page_stats.restype = ctypes.c_int
    lib.da_page_scores.argtypes = [sp, _VP, _VP, _VP, _VP, ctypes.c_int32, _VP, _VP, _VP]
    lib.da_page_scores.restype = ctypes.c_int
    lib.da_select_pages.argtypes = [sp, _VP, _VP, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                                    ctypes.c_int32, _VP, _VP, _VP]
    lib.da_select_pages.restype = ctypes.c_int
    lib.da_append_kv.argtypes = [sp, _VP, _VP, _VP, _VP, _VP, _VP, ctypes.c_int32, _VP, _VP, _VP]
    lib.da_append_kv.restype = ctypes.c_int
    lib.da_split_bounds.argtypes = [sp, _VP, _VP, ctypes.c_int32, _VP, _VP]
    lib.da_split_bounds.restype = ctypes.c_int
    lib.da_micro_attention_fp8.argtypes = [sp, _VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP,
                                           _VP, _VP, _VP, ctypes.c_size_t, _VP]
    lib.da_micro_attention_fp8.restype = ctypes.c_int
    lib.da_micro_attention_fp4.argtypes = lib.da_micro_attention_fp8.argtypes
    lib.da_micro_attention_fp4.restype = ctypes.c_int
    lib.da_attention.argtypes = [sp, _VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP, ctypes.c_size_t,
                                 _VP]
    lib.da_attention.restype = ctypes.c_int
    lib.da_attention_fp8.argtypes = [sp, _VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP,
                                     ctypes.c_size_t, _VP]
    lib.da_attention_fp8.restype = ctypes.c_int
    lib.da_attention_fp4.argtypes = lib.da_attention_fp8.argtypes
    lib.da_attention_fp4.restype = ctypes.c_int
    lib.da_attention_noalloc.argtypes = [sp, _VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP]
    lib.da_attention_noalloc.restype = ctypes.c_int
    lib.da_attention_workspace_size.argtypes = [sp, ctypes.POINTER(ctypes.c_size_t),
                                                ctypes.POINTER(ctypes.c_size_t)]
    lib.da_attention_workspace_size.restype = ctypes.c_int
    lib.da_quantize_rows.argtypes = [ctypes.c_int32, ctypes.c_int64, ctypes.c_int32, _VP, _VP, _VP,
                                     _VP]
    lib.da_quantize_rows.restype = ctypes.c_int
    lib.da_quantize_rows_fp4.argtypes = lib.da_quantize_rows.argtypes
    lib.da_quantize_rows_fp4.restype = ctypes.c_int
    lib.da_append_kv_fp8.argtypes = [sp, _VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP, ctypes.c_int32,
                                     _VP, _VP, _VP]
    lib.da_append_kv_fp8.restype = ctypes.c_int
    lib.da_append_kv_fp4.argtypes = lib.da_append_kv_fp8.argtypes
    lib.da_append_kv_fp4.restype = ctypes.c_int
    lib.da_stream_read.argtypes = [_VP, ctypes.c_size_t, _VP, _VP]
    lib.da_stream_read.restype = ctypes.c_int
    lib.da_stream_read_sink_words.argtypes = []
    lib.da_stream_read_sink_words.restype = ctypes.c_size_t
    _LIB = lib
    return lib


def header_functions() -> list:
    """Names of the functions that include/da.h declares."""
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(da_[a-z0-9_]+)\s*\(", text)))


def _check(status: int):
    if status != DA_OK:
        raise DaError(status, load().da_last_error().decode(errors="replace"))


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(device: torch.device):
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _need(t: torch.Tensor, name: str, dtype, device, ndim: int):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a tensor")
    if t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} has dtype {t.dtype}, expected {dtype}")
    if t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dims, has shape {tuple(t.shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


POOL_LAYOUTS = {"page": 0, "head": 1}


def shape_of(q, k_pages, block_table, split_bounds, scale: Optional[float] = None,
             chunks: int = 0, schedule: int = 0, pool_layout: str = "page",
             codes_per_byte: int = 1) -> DaShape:
    """da_shape of a call; pool_layout "page" = pools [NP, Hkv, P, D],
    "head" = [Hkv, NP, P, D] (4-bit code pools: D / 2 bytes per row,
    codes_per_byte = 2)."""
    S, Hq, D = q.shape
    if pool_layout not in POOL_LAYOUTS:
        raise ValueError(f"pool_layout must be one of {sorted(POOL_LAYOUTS)}")
    if pool_layout == "head":
        Hkv, NP, P, D2 = k_pages.shape
    else:
        NP, Hkv, P, D2 = k_pages.shape
    D2 *= codes_per_byte
    if D2 != D:
        raise ValueError(f"head dim of q ({D}) and k_pages ({D2}) differ")
    nbh = split_bounds.shape[1]
    if nbh not in (1, Hkv):
        raise ValueError(f"split_bounds has {nbh} rows per request; expected 1 or Hkv={Hkv}")
    if q.dtype == torch.float32:
        dt = DA_F32
    elif q.dtype == torch.bfloat16:
        dt = DA_BF16
    else:
        raise TypeError(f"unsupported dtype {q.dtype}")
    return DaShape(S=S, Hq=Hq, Hkv=Hkv, D=D, P=P, max_pages=block_table.shape[1],
                   max_splits=split_bounds.shape[2] - 1, bounds_per_head=int(nbh == Hkv and Hkv > 1),
                   dtype=dt, scale=(1.0 / math.sqrt(D)) if scale is None else float(scale), NP=NP,
                   chunks=int(chunks), schedule=int(schedule),
                   pool_layout=POOL_LAYOUTS[pool_layout])


_WORKSPACE = {}


def workspace_size(sh: DaShape) -> int:
    n = ctypes.c_size_t(0)
    _check(load().da_micro_attention_workspace_size(ctypes.byref(sh), ctypes.byref(n)))
    return int(n.value)


def _cached_workspace(device: torch.device, nbytes: int) -> Optional[torch.Tensor]:
    """A per-device scratch tensor of at least nbytes, reused across calls.
    Calls that may overlap on different streams must pass their own."""
    if nbytes == 0:
        return None
    key = (device.type, device.index)
    ws = _WORKSPACE.get(key)
    if ws is None or ws.numel() < nbytes:
        ws = torch.empty(nbytes, dtype=torch.uint8, device=device)
        _WORKSPACE[key] = ws
    return ws


def _paged_args(q, k, v, block_table, seq_lens, split_bounds, block_mask, scale, chunks, schedule,
                pool_layout, k_scales=None, v_scales=None, bits: int = 8) -> DaShape:
    """Checks the arguments every attention entry point shares and returns
    the call's da_shape: bf16 / fp32 pools (k, v as q's dtype), or 8-bit
    pools (k, v uint8 codes with k_scales / v_scales, q bf16)."""
    dev = q.device
    fp8 = k_scales is not None
    _need(q, "q", torch.bfloat16 if fp8 else None, dev, 3)
    _need(k, "k_codes" if fp8 else "k_pages", torch.uint8 if fp8 else q.dtype, dev, 4)
    _need(v, "v_codes" if fp8 else "v_pages", torch.uint8 if fp8 else q.dtype, dev, 4)
    if v.shape != k.shape:
        raise ValueError("the K and V pools differ in shape")
    if fp8:
        for name, t in (("k_scales", k_scales), ("v_scales", v_scales)):
            _need(t, name, torch.float32, dev, 3)
            if tuple(t.shape) != tuple(k.shape[:3]):
                raise ValueError(f"{name} must match the first three dims of the code pools")
    _need(block_table, "block_table", torch.int32, dev, 2)
    _need(seq_lens, "seq_lens", torch.int32, dev, 1)
    _need(split_bounds, "split_bounds", torch.int32, dev, 3)
    if block_mask is not None:
        _need(block_mask, "block_mask", torch.uint8, dev, 3)
    sh = shape_of(q, k, block_table, split_bounds, scale, chunks, schedule, pool_layout,
                  2 if fp8 and bits == 4 else 1)
    if fp8:
        sh.dtype = DA_FP8_E4M3 if bits == 8 else DA_FP4_E2M1
    if block_table.shape[0] != sh.S or seq_lens.shape[0] != sh.S or split_bounds.shape[0] != sh.S:
        raise ValueError("block_table, seq_lens and split_bounds must have S rows")
    if block_mask is not None and tuple(block_mask.shape) != (sh.S, sh.Hkv, sh.max_pages):
        raise ValueError(f"block_mask must be [S, Hkv, max_pages] = {(sh.S, sh.Hkv, sh.max_pages)}")
    return sh


def _partials_out(sh: DaShape, out, dev):
    """(MA, m, e) to write: fresh tensors, or the caller's."""
    if out is None:
        return (torch.empty((sh.S, sh.Hq, sh.max_splits, sh.D), dtype=torch.float32, device=dev),
                torch.empty((sh.S, sh.Hq, sh.max_splits), dtype=torch.float32, device=dev),
                torch.empty((sh.S, sh.Hq, sh.max_splits), dtype=torch.float32, device=dev))
    return out


def _micro_workspace(sh: DaShape, workspace, dev):
    if workspace is False:
        return None
    if workspace is None:
        return _cached_workspace(dev, workspace_size(sh))
    if workspace.device != dev or not workspace.is_contiguous():
        raise ValueError("workspace must be a contiguous tensor on the device of q")
    return workspace


def _step_out(sh: DaShape, out, dev):
    if out is None:
        return torch.empty((sh.S, sh.Hq, sh.D), dtype=torch.float32, device=dev)
    _need(out, "out", torch.float32, dev, 3)
    if tuple(out.shape) != (sh.S, sh.Hq, sh.D):
        raise ValueError("out must be [S, Hq, D]")
    return out


def micro_attention(q, k_pages, v_pages, block_table, seq_lens, split_bounds, block_mask=None,
                    *, scale: Optional[float] = None, out=None, chunks: int = 0,
                    workspace: Optional[torch.Tensor] = None, schedule: int = 0,
                    pool_layout: str = "page"):
    """MicroAttention partials (MA [S,Hq,b,D], m [S,Hq,b], e [S,Hq,b]) via da_micro_attention.

    chunks: 0 lets the library cut splits into page ranges when that balances
    the launch; a positive value forces that many.  workspace: a uint8
    device tensor; None uses a cached per-device one (which a later call
    with a larger shape replaces: a HIP graph must be captured with a
    workspace of its own); False passes none (one workgroup per item, no
    chunks).  schedule: 0 library choice, 1 one workgroup per item, 2
    persistent workgroups on a work queue."""
    dev = q.device
    sh = _paged_args(q, k_pages, v_pages, block_table, seq_lens, split_bounds, block_mask, scale,
                     chunks, schedule, pool_layout)
    MA, m, e = _partials_out(sh, out, dev)
    workspace = _micro_workspace(sh, workspace, dev)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(load().da_micro_attention(
        ctypes.byref(sh), _ptr(q), _ptr(k_pages), _ptr(v_pages), _ptr(block_table), _ptr(seq_lens),
        _ptr(split_bounds), _ptr(block_mask), _ptr(MA), _ptr(m), _ptr(e), _ptr(workspace),
        ws_bytes, _stream(dev)))
    return MA, m, e


def quantize_rows(x, *, out=None):
    """8-bit rows via da_quantize_rows: x [..., D] (bf16 or float32) ->
    (codes uint8 [..., D], scales float32 [...]), OCP FP8 E4M3 codes with one
    scale amax / 448 per row."""
    dev = x.device
    if not isinstance(x, torch.Tensor) or x.device.type != "cuda" or not x.is_contiguous():
        raise ValueError("x must be a contiguous device tensor")
    D = x.shape[-1]
    rows = x.numel() // D
    if out is None:
        codes = torch.empty(x.shape, dtype=torch.uint8, device=dev)
        scales = torch.empty(x.shape[:-1], dtype=torch.float32, device=dev)
    else:
        codes, scales = out
        _need(codes, "codes", torch.uint8, dev, x.dim())
        _need(scales, "scales", torch.float32, dev, x.dim() - 1)
        if codes.shape != x.shape or scales.shape != x.shape[:-1]:
            raise ValueError("codes must match x, scales x without its last dim")
    _check(load().da_quantize_rows(_dtype_code(x), rows, D, _ptr(x), _ptr(codes), _ptr(scales),
                                   _stream(dev)))
    return codes, scales


def quantize_rows_fp4(x, *, out=None):
    """4-bit rows via da_quantize_rows_fp4: x [..., D] (bf16 or float32) ->
    (codes uint8 [..., D / 2], two OCP FP4 E2M1 codes per byte, element 2i in
    the low nibble; scales float32 [...], amax / 6 per row)."""
    dev = x.device
    if not isinstance(x, torch.Tensor) or x.device.type != "cuda" or not x.is_contiguous():
        raise ValueError("x must be a contiguous device tensor")
    D = x.shape[-1]
    if D % 2:
        raise ValueError("D must be even")
    rows = x.numel() // D
    cshape = tuple(x.shape[:-1]) + (D // 2,)
    if out is None:
        codes = torch.empty(cshape, dtype=torch.uint8, device=dev)
        scales = torch.empty(x.shape[:-1], dtype=torch.float32, device=dev)
    else:
        codes, scales = out
        _need(codes, "codes", torch.uint8, dev, x.dim())
        _need(scales, "scales", torch.float32, dev, x.dim() - 1)
        if tuple(codes.shape) != cshape or scales.shape != x.shape[:-1]:
            raise ValueError("codes must be x with D / 2 in its last dim, scales x without it")
    _check(load().da_quantize_rows_fp4(_dtype_code(x), rows, D, _ptr(x), _ptr(codes), _ptr(scales),
                                       _stream(dev)))
    return codes, scales


def micro_attention_fp4(q, k_codes, k_scales, v_codes, v_scales, block_table, seq_lens,
                        split_bounds, block_mask=None, *, scale: Optional[float] = None, out=None,
                        chunks: int = 0, workspace: Optional[torch.Tensor] = None,
                        schedule: int = 0, pool_layout: str = "page"):
    """MicroAttention partials over 4-bit pages via da_micro_attention_fp4:
    q [S, Hq, D] bf16; k_codes / v_codes [NP, Hkv, P, D / 2] uint8 (two E2M1
    codes per byte); scales as micro_attention_fp8."""
    dev = q.device
    sh = _paged_args(q, k_codes, v_codes, block_table, seq_lens, split_bounds, block_mask, scale,
                     chunks, schedule, pool_layout, k_scales, v_scales, bits=4)
    MA, m, e = _partials_out(sh, out, dev)
    workspace = _micro_workspace(sh, workspace, dev)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(load().da_micro_attention_fp4(
        ctypes.byref(sh), _ptr(q), _ptr(k_codes), _ptr(k_scales), _ptr(v_codes), _ptr(v_scales),
        _ptr(block_table), _ptr(seq_lens), _ptr(split_bounds), _ptr(block_mask), _ptr(MA), _ptr(m),
        _ptr(e), _ptr(workspace), ws_bytes, _stream(dev)))
    return MA, m, e


def micro_attention_fp8(q, k_codes, k_scales, v_codes, v_scales, block_table, seq_lens,
                        split_bounds, block_mask=None, *, scale: Optional[float] = None, out=None,
                        chunks: int = 0, workspace: Optional[torch.Tensor] = None,
                        schedule: int = 0, pool_layout: str = "page"):
    """MicroAttention partials over 8-bit pages via da_micro_attention_fp8:
    q [S, Hq, D] bf16; k_codes / v_codes [NP, Hkv, P, D] uint8 E4M3 codes;
    k_scales / v_scales [NP, Hkv, P] float32.  Arguments otherwise as
    micro_attention."""
    dev = q.device
    sh = _paged_args(q, k_codes, v_codes, block_table, seq_lens, split_bounds, block_mask, scale,
                     chunks, schedule, pool_layout, k_scales, v_scales)
    MA, m, e = _partials_out(sh, out, dev)
    workspace = _micro_workspace(sh, workspace, dev)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(load().da_micro_attention_fp8(
        ctypes.byref(sh), _ptr(q), _ptr(k_codes), _ptr(k_scales), _ptr(v_codes), _ptr(v_scales),
        _ptr(block_table), _ptr(seq_lens), _ptr(split_bounds), _ptr(block_mask), _ptr(MA), _ptr(m),
        _ptr(e), _ptr(workspace), ws_bytes, _stream(dev)))
    return MA, m, e


def merge(MA, m, e, *, out=None):
    """Aggregate partials into out [S, Hq, D] float32 via da_merge."""
    dev = MA.device
    _need(MA, "MA", torch.float32, dev, 4)
    _need(m, "m", torch.float32, dev, 3)
    _need(e, "e", torch.float32, dev, 3)
    S, Hq, B, D = MA.shape
    if tuple(m.shape) != (S, Hq, B) or tuple(e.shape) != (S, Hq, B):
        raise ValueError("m and e must be [S, Hq, b]")
    if out is None:
        out = torch.empty((S, Hq, D), dtype=torch.float32, device=dev)
    sh = DaShape(S=S, Hq=Hq, Hkv=1, D=D, P=1, max_pages=1, max_splits=B, bounds_per_head=0,
                 dtype=DA_F32, scale=1.0, NP=1)
    _check(load().da_merge(ctypes.byref(sh), _ptr(MA), _ptr(m), _ptr(e), _ptr(out), _stream(dev)))
    return out


def merge_partials(MA, m, e, *, out=None, slot: int = 0, out_splits: int = 1):
    """Fold the b partials of each (request, head) into one triple written to
    slot `slot` of a gather buffer via da_merge_partials.

    out: (MA_out [S, Hq, out_splits, D], m_out, e_out [S, Hq, out_splits])
    float32 tensors to write into (other slots are left untouched); when
    None, fresh buffers with out_splits slots are allocated.  Returns out."""
    dev = MA.device
    _need(MA, "MA", torch.float32, dev, 4)
    _need(m, "m", torch.float32, dev, 3)
    _need(e, "e", torch.float32, dev, 3)
    S, Hq, B, D = MA.shape
    if tuple(m.shape) != (S, Hq, B) or tuple(e.shape) != (S, Hq, B):
        raise ValueError("m and e must be [S, Hq, b]")
    if out is None:
        out = (torch.zeros((S, Hq, out_splits, D), dtype=torch.float32, device=dev),
               torch.full((S, Hq, out_splits), float("-inf"), dtype=torch.float32, device=dev),
               torch.zeros((S, Hq, out_splits), dtype=torch.float32, device=dev))
    MA_o, m_o, e_o = out
    _need(MA_o, "MA_out", torch.float32, dev, 4)
    _need(m_o, "m_out", torch.float32, dev, 3)
    _need(e_o, "e_out", torch.float32, dev, 3)
    n_out = MA_o.shape[2]
    if (tuple(MA_o.shape) != (S, Hq, n_out, D) or tuple(m_o.shape) != (S, Hq, n_out)
            or tuple(e_o.shape) != (S, Hq, n_out)):
        raise ValueError("out must be ([S, Hq, n, D], [S, Hq, n], [S, Hq, n])")
    sh = DaShape(S=S, Hq=Hq, Hkv=1, D=D, P=1, max_pages=1, max_splits=B, bounds_per_head=0,
                 dtype=DA_F32, scale=1.0, NP=1)
    _check(load().da_merge_partials(ctypes.byref(sh), _ptr(MA), _ptr(m), _ptr(e), n_out, slot,
                                    _ptr(MA_o), _ptr(m_o), _ptr(e_o), _stream(dev)))
    return out


def attention_workspace_size(sh: DaShape):
    """(bytes, counter_bytes) of the fused step's workspace for this shape."""
    n, c = ctypes.c_size_t(0), ctypes.c_size_t(0)
    _check(load().da_attention_workspace_size(ctypes.byref(sh), ctypes.byref(n), ctypes.byref(c)))
    return int(n.value), int(c.value)


class _FusedWorkspace:
    """A per-device workspace for the fused step.  Its first `clean` bytes are
    known to be zero: every completed call leaves its own counters zero and
    may overwrite what lies beyond them with partials, so a call whose
    counters reach past `clean` gets that range zeroed first."""

    def __init__(self):
        self.buf = None
        self.clean = 0

    def get(self, device, nbytes: int, counter_bytes: int) -> torch.Tensor:
        if self.buf is None or self.buf.numel() < nbytes:
            self.buf = torch.zeros(nbytes, dtype=torch.uint8, device=device)
            self.clean = nbytes
        elif self.clean < counter_bytes:
            self.buf[self.clean:counter_bytes].zero_()
        self.clean = counter_bytes
        return self.buf


_FUSED_WORKSPACE = {}


def _fused_workspace(device: torch.device, sh: DaShape, workspace) -> torch.Tensor:
    if workspace is not None:
        if workspace.device != device or not workspace.is_contiguous():
            raise ValueError("workspace must be a contiguous tensor on the device of q")
        return workspace
    nbytes, counter_bytes = attention_workspace_size(sh)
    key = (device.type, device.index)
    return _FUSED_WORKSPACE.setdefault(key, _FusedWorkspace()).get(device, nbytes, counter_bytes)


def attention(q, k_pages, v_pages, block_table, seq_lens, split_bounds, block_mask=None,
              *, scale: Optional[float] = None, out=None, chunks: int = 0, schedule: int = 0,
              workspace: Optional[torch.Tensor] = None, pool_layout: str = "page", fuse: int = 0):
    """One decode step via da_attention: MicroAttention partials and their
    merge into out [S, Hq, D] float32, in one launch or two (fuse: 0 the
    library's choice, 1 one launch, 2 two).  workspace: None uses a
    cached per-device one (replaced by a later call with a larger shape, so
    a HIP graph must be captured with a workspace of its own); a caller's
    own must have been zero-filled once (see da_attention) and must not be
    shared by concurrent calls."""
    dev = q.device
    sh = _paged_args(q, k_pages, v_pages, block_table, seq_lens, split_bounds, block_mask, scale,
                     chunks, schedule, pool_layout)
    sh.fuse = int(fuse)
    out = _step_out(sh, out, dev)
    ws = _fused_workspace(dev, sh, workspace)
    _check(load().da_attention(
        ctypes.byref(sh), _ptr(q), _ptr(k_pages), _ptr(v_pages), _ptr(block_table), _ptr(seq_lens),
        _ptr(split_bounds), _ptr(block_mask), _ptr(out), _ptr(ws), ws.numel(), _stream(dev)))
    return out


def attention_noalloc(q, k_pages, v_pages, block_table, seq_lens, split_bounds, block_mask=None,
                      *, scale: Optional[float] = None, out=None, chunks: int = 0,
                      schedule: int = 0, pool_layout: str = "page", fuse: int = 0):
    """The step of attention via da_attention_noalloc: no workspace, the
    library's per-GPU scratch array instead (calls on one GPU must not
    overlap).  out: [S, Hq, D] float32 (allocated here when None; pass one to
    call without any allocation)."""
    dev = q.device
    sh = _paged_args(q, k_pages, v_pages, block_table, seq_lens, split_bounds, block_mask, scale,
                     chunks, schedule, pool_layout)
    sh.fuse = int(fuse)
    out = _step_out(sh, out, dev)
    _check(load().da_attention_noalloc(
        ctypes.byref(sh), _ptr(q), _ptr(k_pages), _ptr(v_pages), _ptr(block_table), _ptr(seq_lens),
        _ptr(split_bounds), _ptr(block_mask), _ptr(out), _stream(dev)))
    return out


def attention_fp8(q, k_codes, k_scales, v_codes, v_scales, block_table, seq_lens, split_bounds,
                  block_mask=None, *, scale: Optional[float] = None, out=None, chunks: int = 0,
                  schedule: int = 0, workspace: Optional[torch.Tensor] = None,
                  pool_layout: str = "page", fuse: int = 0):
    """One decode step over 8-bit pages via da_attention_fp8 (inputs as
    micro_attention_fp8, output, workspace and fuse as attention)."""
    dev = q.device
    sh = _paged_args(q, k_codes, v_codes, block_table, seq_lens, split_bounds, block_mask, scale,
                     chunks, schedule, pool_layout, k_scales, v_scales)
    sh.fuse = int(fuse)
    out = _step_out(sh, out, dev)
    ws = _fused_workspace(dev, sh, workspace)
    _check(load().da_attention_fp8(
        ctypes.byref(sh), _ptr(q), _ptr(k_codes), _ptr(k_scales), _ptr(v_codes), _ptr(v_scales),
        _ptr(block_table), _ptr(seq_lens), _ptr(split_bounds), _ptr(block_mask), _ptr(out),
        _ptr(ws), ws.numel(), _stream(dev)))
    return out


def attention_fp4(q, k_codes, k_scales, v_codes, v_scales, block_table, seq_lens, split_bounds,
                  block_mask=None, *, scale: Optional[float] = None, out=None, chunks: int = 0,
                  schedule: int = 0, workspace: Optional[torch.Tensor] = None,
                  pool_layout: str = "page", fuse: int = 0):
    """One decode step over 4-bit pages via da_attention_fp4 (inputs as
    micro_attention_fp4, output, workspace and fuse as attention)."""
    dev = q.device
    sh = _paged_args(q, k_codes, v_codes, block_table, seq_lens, split_bounds, block_mask, scale,
                     chunks, schedule, pool_layout, k_scales, v_scales, bits=4)
    sh.fuse = int(fuse)
    out = _step_out(sh, out, dev)
    ws = _fused_workspace(dev, sh, workspace)
    _check(load().da_attention_fp4(
        ctypes.byref(sh), _ptr(q), _ptr(k_codes), _ptr(k_scales), _ptr(v_codes), _ptr(v_scales),
        _ptr(block_table), _ptr(seq_lens), _ptr(split_bounds), _ptr(block_mask), _ptr(out),
        _ptr(ws), ws.numel(), _stream(dev)))
    return out


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return DA_F32
    if t.dtype == torch.bfloat16:
        return DA_BF16
    raise TypeError(f"unsupported dtype {t.dtype}")


def _selector_shape(S, Hq, Hkv, D, P, NP, max_pages, dtype, pool_layout: str = "page") -> DaShape:
    return DaShape(S=S, Hq=Hq, Hkv=Hkv, D=D, P=P, max_pages=max_pages, max_splits=1,
                   bounds_per_head=0, dtype=dtype, scale=1.0, NP=NP,
                   pool_layout=POOL_LAYOUTS[pool_layout])


def _pool_dims(pool, pool_layout: str):
    """(NP, Hkv, P, D) of a pool in the given layout."""
    if pool_layout not in POOL_LAYOUTS:
        raise ValueError(f"pool_layout must be one of {sorted(POOL_LAYOUTS)}")
    a, b, P, D = pool.shape
    return (b, a, P, D) if pool_layout == "head" else (a, b, P, D)


def page_stats(k_pages, block_table, seq_lens, *, logical: int = 16, select_heads=None,
               out=None, pool_layout: str = "page"):
    """Per-logical-page key maxima and minima [Hkv, NP, P // logical, 2, D]
    (dtype of k_pages, head-major) via da_page_stats.  Pages that no table row names
    below L_s, and KV heads whose select_heads flag is 0, are left as they
    are in ``out`` (zeros when it is allocated here)."""
    dev = k_pages.device
    _need(k_pages, "k_pages", None, dev, 4)
    _need(block_table, "block_table", torch.int32, dev, 2)
    _need(seq_lens, "seq_lens", torch.int32, dev, 1)
    NP, Hkv, P, D = _pool_dims(k_pages, pool_layout)
    if select_heads is not None:
        _need(select_heads, "select_heads", torch.uint8, dev, 1)
        if select_heads.shape[0] != Hkv:
            raise ValueError("select_heads must have Hkv entries")
    if P % logical:
        raise ValueError(f"logical={logical} does not divide P={P}")
    if out is None:
        out = torch.zeros((Hkv, NP, P // logical, 2, D), dtype=k_pages.dtype, device=dev)
    else:
        _need(out, "out", k_pages.dtype, dev, 5)
        if tuple(out.shape) != (Hkv, NP, P // logical, 2, D):
            raise ValueError("out must be [Hkv, NP, P // logical, 2, D]")
    sh = _selector_shape(block_table.shape[0], Hkv, Hkv, D, P, NP, block_table.shape[1],
                         _dtype_code(k_pages), pool_layout)
    _check(load().da_page_stats(ctypes.byref(sh), _ptr(k_pages), _ptr(block_table), _ptr(seq_lens),
                                int(logical), _ptr(select_heads), _ptr(out), _stream(dev)))
    return out


def page_scores(q, stats, block_table, seq_lens, *, P: int, select_heads=None, out=None):
    """Physical-page scores [S, Hkv, max_pages] float32 via da_page_scores:
    the largest statistics bound over the group's query heads and the
    page's logical pages; -inf past L_s and for unselected KV heads."""
    dev = q.device
    _need(q, "q", None, dev, 3)
    _need(stats, "stats", q.dtype, dev, 5)
    _need(block_table, "block_table", torch.int32, dev, 2)
    _need(seq_lens, "seq_lens", torch.int32, dev, 1)
    if select_heads is not None:
        _need(select_heads, "select_heads", torch.uint8, dev, 1)
    S, Hq, D = q.shape
    Hkv, NP, NL, two, D2 = stats.shape
    if two != 2 or D2 != D or P % NL:
        raise ValueError("stats must be [Hkv, NP, P // logical, 2, D]")
    if select_heads is not None and select_heads.shape[0] != Hkv:
        raise ValueError("select_heads must have Hkv entries")
    max_pages = block_table.shape[1]
    if out is None:
        out = torch.empty((S, Hkv, max_pages), dtype=torch.float32, device=dev)
    else:
        _need(out, "out", torch.float32, dev, 3)
    sh = _selector_shape(S, Hq, Hkv, D, P, NP, max_pages, _dtype_code(q))
    _check(load().da_page_scores(ctypes.byref(sh), _ptr(q), _ptr(stats), _ptr(block_table),
                                 _ptr(seq_lens), int(P // NL), _ptr(select_heads), _ptr(out),
                                 _stream(dev)))
    return out


def select_pages(scores, seq_lens, *, P: int, budget: int, keep_first: int = 0,
                 keep_last: int = 0, select_heads=None, horizon: int = 0, out=None):
    """Block mask [S, Hkv, max_pages] uint8 via da_select_pages: forced first
    and last pages plus the ``budget`` best-scoring others, and the pages the
    next ``horizon`` appended tokens open."""
    dev = scores.device
    _need(scores, "scores", torch.float32, dev, 3)
    _need(seq_lens, "seq_lens", torch.int32, dev, 1)
    if select_heads is not None:
        _need(select_heads, "select_heads", torch.uint8, dev, 1)
    S, Hkv, max_pages = scores.shape
    if select_heads is not None and select_heads.shape[0] != Hkv:
        raise ValueError("select_heads must have Hkv entries")
    if out is None:
        out = torch.empty((S, Hkv, max_pages), dtype=torch.uint8, device=dev)
    else:
        _need(out, "out", torch.uint8, dev, 3)
    sh = _selector_shape(S, Hkv, Hkv, 1, P, 1, max_pages, DA_F32)
    _check(load().da_select_pages(ctypes.byref(sh), _ptr(scores), _ptr(seq_lens), int(budget),
                                  int(keep_first), int(keep_last), int(horizon), _ptr(select_heads),
                                  _ptr(out), _stream(dev)))
    return out


def append_kv(k_new, v_new, block_table, seq_lens, k_pages, v_pages, *, stats=None,
              logical: int = 16, select_heads=None, pool_layout: str = "page"):
    """Write each request's new K/V rows ([S, Hkv, D]) at position seq_lens[s]
    of the paged pools in place via da_append_kv, keeping ``stats`` (head-major
    statistics, or None) current.  seq_lens is not advanced."""
    dev = k_pages.device
    _need(k_pages, "k_pages", None, dev, 4)
    _need(v_pages, "v_pages", k_pages.dtype, dev, 4)
    if v_pages.shape != k_pages.shape:
        raise ValueError("k_pages and v_pages differ in shape")
    NP, Hkv, P, D = _pool_dims(k_pages, pool_layout)
    S = block_table.shape[0]
    for name, t in (("k_new", k_new), ("v_new", v_new)):
        _need(t, name, k_pages.dtype, dev, 3)
        if tuple(t.shape) != (S, Hkv, D):
            raise ValueError(f"{name} must be [S, Hkv, D] = {(S, Hkv, D)}")
    _need(block_table, "block_table", torch.int32, dev, 2)
    _need(seq_lens, "seq_lens", torch.int32, dev, 1)
    if seq_lens.shape[0] != S:
        raise ValueError("seq_lens must have S entries")
    if stats is not None:
        _need(stats, "stats", k_pages.dtype, dev, 5)
        if tuple(stats.shape) != (Hkv, NP, P // logical, 2, D):
            raise ValueError("stats must be [Hkv, NP, P // logical, 2, D]")
    if select_heads is not None:
        _need(select_heads, "select_heads", torch.uint8, dev, 1)
        if select_heads.shape[0] != Hkv:
            raise ValueError("select_heads must have Hkv entries")
    sh = _selector_shape(S, Hkv, Hkv, D, P, NP, block_table.shape[1], _dtype_code(k_pages),
                         pool_layout)
    _check(load().da_append_kv(ctypes.byref(sh), _ptr(k_new), _ptr(v_new), _ptr(block_table),
                               _ptr(seq_lens), _ptr(k_pages), _ptr(v_pages), int(logical),
                               _ptr(select_heads), _ptr(stats), _stream(dev)))


def append_kv_fp8(k_new, v_new, block_table, seq_lens, k_codes, k_scales, v_codes, v_scales, *,
                  stats=None, logical: int = 16, select_heads=None, pool_layout: str = "page"):
    """Quantize each request's new K/V rows ([S, Hkv, D], bf16 or float32)
    and write their codes and scales at position seq_lens[s] of the 8-bit
    pools in place via da_append_kv_fp8, keeping ``stats`` (head-major
    statistics in the rows' dtype, or None) current from the full-precision
    key rows.  seq_lens is not advanced."""
    _append_quantized(8, k_new, v_new, block_table, seq_lens, k_codes, k_scales, v_codes, v_scales,
                      stats, logical, select_heads, pool_layout)


def append_kv_fp4(k_new, v_new, block_table, seq_lens, k_codes, k_scales, v_codes, v_scales, *,
                  stats=None, logical: int = 16, select_heads=None, pool_layout: str = "page"):
    """append_kv_fp8 for 4-bit pools (codes [NP, Hkv, P, D / 2]) via
    da_append_kv_fp4."""
    _append_quantized(4, k_new, v_new, block_table, seq_lens, k_codes, k_scales, v_codes, v_scales,
                      stats, logical, select_heads, pool_layout)


def _append_quantized(bits, k_new, v_new, block_table, seq_lens, k_codes, k_scales, v_codes,
                      v_scales, stats, logical, select_heads, pool_layout):
    dev = k_codes.device
    _need(k_codes, "k_codes", torch.uint8, dev, 4)
    _need(v_codes, "v_codes", torch.uint8, dev, 4)
    if v_codes.shape != k_codes.shape:
        raise ValueError("k_codes and v_codes differ in shape")
    NP, Hkv, P, D = _pool_dims(k_codes, pool_layout)
    D *= 8 // bits  # 4-bit pools hold two codes per byte
    for name, t in (("k_scales", k_scales), ("v_scales", v_scales)):
        _need(t, name, torch.float32, dev, 3)
        if tuple(t.shape) != tuple(k_codes.shape[:3]):
            raise ValueError(f"{name} must match the first three dims of the code pools")
    S = block_table.shape[0]
    for name, t in (("k_new", k_new), ("v_new", v_new)):
        _need(t, name, k_new.dtype, dev, 3)
        if tuple(t.shape) != (S, Hkv, D):
            raise ValueError(f"{name} must be [S, Hkv, D] = {(S, Hkv, D)}")
    _need(block_table, "block_table", torch.int32, dev, 2)
    _need(seq_lens, "seq_lens", torch.int32, dev, 1)
    if stats is not None:
        _need(stats, "stats", k_new.dtype, dev, 5)
        if tuple(stats.shape) != (Hkv, NP, P // logical, 2, D):
            raise ValueError("stats must be [Hkv, NP, P // logical, 2, D]")
    if select_heads is not None:
        _need(select_heads, "select_heads", torch.uint8, dev, 1)
    sh = _selector_shape(S, Hkv, Hkv, D, P, NP, block_table.shape[1], _dtype_code(k_new),
                         pool_layout)
    fn = load().da_append_kv_fp8 if bits == 8 else load().da_append_kv_fp4
    _check(fn(ctypes.byref(sh), _ptr(k_new), _ptr(v_new), _ptr(block_table), _ptr(seq_lens),
              _ptr(k_codes), _ptr(k_scales), _ptr(v_codes), _ptr(v_scales), int(logical),
              _ptr(select_heads), _ptr(stats), _stream(dev)))


def split_bounds(block_mask, seq_lens, *, P: int, b: int, horizon: int = 0, Hkv=None,
                 max_pages=None, out=None):
    """Per-head split bounds [S, Hkv, b + 1] int32 over the kept pages via
    da_split_bounds (block_mask None = every page kept; then Hkv and
    max_pages are required)."""
    dev = seq_lens.device
    _need(seq_lens, "seq_lens", torch.int32, dev, 1)
    S = seq_lens.shape[0]
    if block_mask is not None:
        _need(block_mask, "block_mask", torch.uint8, dev, 3)
        S2, Hkv, max_pages = block_mask.shape
        if S2 != S:
            raise ValueError("block_mask must have S rows")
    elif Hkv is None or max_pages is None:
        raise ValueError("Hkv and max_pages are required without a block mask")
    if out is None:
        out = torch.empty((S, Hkv, b + 1), dtype=torch.int32, device=dev)
    else:
        _need(out, "out", torch.int32, dev, 3)
        if tuple(out.shape) != (S, Hkv, b + 1):
            raise ValueError("out must be [S, Hkv, b + 1]")
    sh = DaShape(S=S, Hq=Hkv, Hkv=Hkv, D=1, P=P, max_pages=max_pages, max_splits=b,
                 bounds_per_head=1, dtype=DA_F32, scale=1.0, NP=1)
    _check(load().da_split_bounds(ctypes.byref(sh), _ptr(block_mask), _ptr(seq_lens), int(horizon),
                                  _ptr(out), _stream(dev)))
    return out


def check_inputs(block_table, seq_lens, NP: int, P: int) -> int:
    """Number of invalid seq_lens / block-table entries (synchronises)."""
    dev = block_table.device
    _need(block_table, "block_table", torch.int32, dev, 2)
    _need(seq_lens, "seq_lens", torch.int32, dev, 1)
    err = torch.zeros(1, dtype=torch.int32, device=dev)
    sh = DaShape(S=block_table.shape[0], Hq=1, Hkv=1, D=1, P=P, max_pages=block_table.shape[1],
                 max_splits=1, bounds_per_head=0, dtype=DA_F32, scale=1.0, NP=NP)
    _check(load().da_check_inputs(ctypes.byref(sh), _ptr(block_table), _ptr(seq_lens), _ptr(err),
                                  _stream(dev)))
    return int(err.item())


def stream_read(buf: torch.Tensor, sink: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Read every byte of ``buf`` once (HBM read-rate measurement)."""
    if sink is None:
        sink = torch.zeros(int(load().da_stream_read_sink_words()), dtype=torch.int32, device=buf.device)
    _check(load().da_stream_read(_ptr(buf), buf.numel() * buf.element_size(), _ptr(sink),
                                 _stream(buf.device)))
    return sink
