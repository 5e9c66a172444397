"""Seeded synthetic inputs for split-KV decode attention.

This module only builds inputs: query vectors, a paged K/V pool, block
tables, sequence lengths, split bounds and block masks, drawn from seeded
generators.  It holds none of the attention arithmetic and is shared by the
tests, the benchmark and the oracle checks, which all see the same tensors.

Workload shapes follow the model and context scales the pages use:
LLaMA-2-7B/13B (Infinite-LLM page, experiments), LWM-1M-Text on the
LLaMA-2-7B shape at 1M tokens (LoongServe page, experiment setup), LLaMA-3-8B
with 64-token physical pages and block masks at 512K context (LServe blog
page, sections 2.2.2 and 4.1).  The traces and datasets those pages measure on
are not used; every value here is i.i.d. N(0, 1) noise or a seeded structure
(shuffled tables, scaled rows, sinks, masks) of stated shape.
"""

from __future__ import annotations

import dataclasses
import math
import zlib
from dataclasses import dataclass, field
from typing import Optional

import numpy as np
import torch

F32 = "f32"
BF16 = "bf16"
TORCH_DTYPE = {F32: torch.float32, BF16: torch.bfloat16}


@dataclass(frozen=True)
class Spec:
    """Shape and structure of one workload.

    lens      -- ("fixed", L) or ("loguniform", L_max): per-request context.
    table     -- "identity" (request s owns pages s*max_pages ...) or
                 "shuffled" (one random permutation over the whole pool).
    splits    -- ("equal", b), ("chunk", tokens) or ("kept_pages", b).
    k_scaled  -- (fraction of K rows per (request, KV head), factor) or None.
    sink      -- (tokens, cosine) of request-prefix keys aligned to q, or None.
    mask      -- ("lserve", keep_first, keep_last, fraction) applied to the
                 upper half of the KV heads, or None.
    reserve   -- tokens of spare capacity per request: the block table maps
                 pages up to ceil((L_s + reserve) / P), so decode steps can
                 append that many tokens.
    layout    -- "page": pools [NP, Hkv, P, D]; "head": [Hkv, NP, P, D] (each
                 KV head's pages contiguous).  The values at (page, head,
                 slot) are the same either way.
    """

    name: str
    S: int
    Hq: int
    Hkv: int
    D: int
    P: int
    dtype: str
    lens: tuple
    table: str = "identity"
    splits: tuple = ("equal", 1)
    k_scaled: Optional[tuple] = None
    sink: Optional[tuple] = None
    mask: Optional[tuple] = None
    extra_pages: int = 0
    reserve: int = 0
    layout: str = "page"

    @property
    def G(self) -> int:
        return self.Hq // self.Hkv

    @property
    def esize(self) -> int:
        return 4 if self.dtype == F32 else 2

    @property
    def max_len(self) -> int:
        return int(self.lens[1])

    @property
    def max_pages(self) -> int:
        return -(-(self.max_len + self.reserve) // self.P)

    def replace(self, **kw) -> "Spec":
        return dataclasses.replace(self, **kw)


# The five workloads.  Sizes are the full ones; tests use reduced copies.
CONFIGS = {
    "C1": Spec("C1 tiny fp32 MHA", S=1, Hq=4, Hkv=4, D=64, P=16, dtype=F32,
               lens=("fixed", 1024), splits=("equal", 4)),
    "C2": Spec("C2 LLaMA-2-7B layer, batch 16, 4K, bf16", S=16, Hq=32, Hkv=32, D=128, P=16,
               dtype=BF16, lens=("fixed", 4096), table="shuffled", splits=("equal", 8),
               k_scaled=(0.01, 8.0)),
    "C3": Spec("C3 LLaMA-2-13B shape, 64 mixed lengths up to 32K, bf16", S=64, Hq=40, Hkv=40,
               D=128, P=16, dtype=BF16, lens=("loguniform", 32768), table="shuffled",
               splits=("chunk", 2048)),
    "C4": Spec("C4 one 1M-token request, LLaMA-2-7B/LWM shape, bf16", S=1, Hq=32, Hkv=32,
               D=128, P=64, dtype=BF16, lens=("fixed", 1 << 20), splits=("equal", 32),
               sink=(4, 0.9)),
    "C5": Spec("C5 LLaMA-3-8B GQA 32/8, batch 8, 512K, half the KV heads block-sparse, bf16",
               S=8, Hq=32, Hkv=8, D=128, P=64, dtype=BF16, lens=("fixed", 1 << 19),
               splits=("kept_pages", 16), mask=("lserve", 1, 2, 0.25), reserve=16),
}


# Pool layout each full-size workload is measured with: head-major pools
# read 2.7% faster on the GQA block-sparse workload (its dense heads stream
# contiguous runs and its masked heads read ascending tiles of one head's
# run) and 0.7% faster on the 1M-token one (2426 against 2443 us in one
# process), where each split then reads one contiguous run instead of
# 16 KiB tiles 512 KiB apart; on the 16-token-page batches (a random
# table) the two layouts measured equal.
PREFERRED_LAYOUT = {"C5": "head", "C4": "head"}


@dataclass
class Batch:
    spec: Spec
    seed: int
    q: torch.Tensor            # [S, Hq, D]
    k_pages: torch.Tensor      # [NP, Hkv, P, D]
    v_pages: torch.Tensor      # [NP, Hkv, P, D]
    block_table: torch.Tensor  # [S, max_pages] int32
    seq_lens: torch.Tensor     # [S] int32
    split_bounds: torch.Tensor  # [S, 1 or Hkv, b+1] int32
    block_mask: Optional[torch.Tensor]  # [S, Hkv, max_pages] uint8 or None
    scale: float
    kept_pages: list = field(default_factory=list)  # per (s, kvh): sorted kept logical pages (np.int64)
    layout: str = "page"

    @property
    def k_pm(self) -> torch.Tensor:
        """K pool as a page-major view [NP, Hkv, P, D] whatever the layout."""
        return self.k_pages.transpose(0, 1) if self.layout == "head" else self.k_pages

    @property
    def v_pm(self) -> torch.Tensor:
        """V pool as a page-major view [NP, Hkv, P, D] whatever the layout."""
        return self.v_pages.transpose(0, 1) if self.layout == "head" else self.v_pages

    @property
    def max_splits(self) -> int:
        return int(self.split_bounds.shape[2]) - 1

    @property
    def bounds_per_head(self) -> bool:
        return int(self.split_bounds.shape[1]) != 1

    def kept_tokens(self) -> np.ndarray:
        """[S, Hkv] number of tokens in [0, L_s) on kept pages."""
        sp = self.spec
        lens = self.seq_lens.cpu().numpy().astype(np.int64)
        out = np.zeros((sp.S, sp.Hkv), dtype=np.int64)
        for s in range(sp.S):
            for h in range(sp.Hkv):
                pages = self.kept_pages[s * sp.Hkv + h]
                full = np.minimum((pages + 1) * sp.P, lens[s]) - pages * sp.P
                out[s, h] = int(np.clip(full, 0, None).sum())
        return out

    def kv_bytes(self) -> int:
        """Algorithmic bytes: every kept token is read once as a K row and a V row."""
        return int(self.kept_tokens().sum()) * 2 * self.spec.D * self.spec.esize


def _seed_for(seed: int, spec: Spec, tag: str) -> int:
    """Independent 63-bit sub-stream seed per (seed, workload, tensor)."""
    h = zlib.crc32(f"{spec.name}|{tag}".encode())
    return (int(seed) * 0x9E3779B97F4A7C15 + h) & ((1 << 63) - 1)


def _gen(seed: int, spec: Spec, tag: str, device) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(_seed_for(seed, spec, tag))
    return g


def _np_rng(seed: int, spec: Spec, tag: str) -> np.random.Generator:
    return np.random.default_rng(_seed_for(seed, spec, tag))


def _lengths(spec: Spec, seed: int) -> np.ndarray:
    kind, L = spec.lens
    if kind == "fixed":
        return np.full(spec.S, int(L), dtype=np.int64)
    if kind == "loguniform":
        u = _np_rng(seed, spec, "lens").random(spec.S)
        return np.clip(np.round(np.exp(u * math.log(L))), 1, L).astype(np.int64)
    raise ValueError(kind)


def _normal_pool(shape, dtype, g, device, chunk_pages: int = 256) -> torch.Tensor:
    """N(0,1) pool, drawn page-chunk by page-chunk so peak memory stays small."""
    out = torch.empty(shape, dtype=TORCH_DTYPE[dtype], device=device)
    for p0 in range(0, shape[0], chunk_pages):
        p1 = min(p0 + chunk_pages, shape[0])
        x = torch.randn((p1 - p0,) + tuple(shape[1:]), generator=g, device=device, dtype=torch.float32)
        out[p0:p1].copy_(x)
    return out


def build(spec: Spec, seed: int = 0, device="cpu") -> Batch:
    """Draw one batch of the workload on ``device``."""
    device = torch.device(device)
    S, Hkv, P, D = spec.S, spec.Hkv, spec.P, spec.D
    lens = _lengths(spec, seed)
    n_log = [-(-int(L) // P) for L in lens]
    max_pages = spec.max_pages
    n_cap = [min(max_pages, -(-(int(L) + spec.reserve) // P)) for L in lens]  # mapped pages

    # block table
    table = np.zeros((S, max_pages), dtype=np.int32)
    if spec.table == "identity":
        NP = S * max_pages
        for s in range(S):
            table[s, :n_cap[s]] = s * max_pages + np.arange(n_cap[s])
    elif spec.table == "shuffled":
        NP = int(sum(n_cap))
        perm = _np_rng(seed, spec, "table").permutation(NP + spec.extra_pages)[:NP]
        off = 0
        for s in range(S):
            table[s, :n_cap[s]] = perm[off:off + n_cap[s]]
            off += n_cap[s]
    else:
        raise ValueError(spec.table)
    NP += spec.extra_pages

    # q, K, V
    qg = _gen(seed, spec, "q", device)
    q = torch.randn((S, spec.Hq, D), generator=qg, device=device, dtype=torch.float32).to(TORCH_DTYPE[spec.dtype])
    k_pages = _normal_pool((NP, Hkv, P, D), spec.dtype, _gen(seed, spec, "k", device), device)
    v_pages = _normal_pool((NP, Hkv, P, D), spec.dtype, _gen(seed, spec, "v", device), device)
    table_t = torch.from_numpy(table)

    # 1% of K rows per (request, KV head) scaled by a power of two (exact)
    if spec.k_scaled is not None:
        frac, factor = spec.k_scaled
        rng = _np_rng(seed, spec, "k_scaled")
        rows_p, rows_h, rows_s = [], [], []
        for s in range(S):
            n = int(round(frac * lens[s]))
            for h in range(Hkv):
                t = rng.choice(int(lens[s]), size=n, replace=False)
                rows_p.append(table[s, t // P])
                rows_s.append(t % P)
                rows_h.append(np.full(n, h))
        pi = torch.from_numpy(np.concatenate(rows_p).astype(np.int64)).to(device)
        hi = torch.from_numpy(np.concatenate(rows_h).astype(np.int64)).to(device)
        si = torch.from_numpy(np.concatenate(rows_s).astype(np.int64)).to(device)
        k_pages[pi, hi, si] = (k_pages[pi, hi, si].float() * factor).to(k_pages.dtype)

    # sink prefix: keys with cosine `cos` to the query that reads them
    if spec.sink is not None:
        n_sink, cos = spec.sink
        g = _gen(seed, spec, "sink", device)
        for s in range(S):
            for h in range(Hkv):
                qh = q[s, h * spec.G].float()
                qhat = qh / qh.norm()
                for t in range(min(n_sink, int(lens[s]))):
                    r = torch.randn(D, generator=g, device=device)
                    u = torch.randn(D, generator=g, device=device)
                    u = u - (u @ qhat) * qhat
                    u = u / u.norm()
                    k = r.norm() * (cos * qhat + math.sqrt(1.0 - cos * cos) * u)
                    k_pages[int(table[s, t // P]), h, t % P] = k.to(k_pages.dtype)

    # block mask: upper half of the KV heads keep first/last pages + a fraction
    kept = []
    mask_np = None
    if spec.mask is not None:
        _, keep_first, keep_last, frac = spec.mask
        rng = _np_rng(seed, spec, "mask")
        mask_np = np.zeros((S, Hkv, max_pages), dtype=np.uint8)
        for s in range(S):
            n = n_log[s]
            for h in range(Hkv):
                if h < Hkv // 2:
                    mask_np[s, h, :n] = 1
                    continue
                mask_np[s, h, :min(keep_first, n)] = 1
                mask_np[s, h, max(n - keep_last, 0):n] = 1
                middle = np.arange(keep_first, max(n - keep_last, keep_first))
                k = int(math.floor(frac * len(middle)))
                if k:
                    mask_np[s, h, rng.choice(middle, size=k, replace=False)] = 1
    for s in range(S):
        for h in range(Hkv):
            if mask_np is None:
                kept.append(np.arange(n_log[s], dtype=np.int64))
            else:
                kept.append(np.nonzero(mask_np[s, h, :n_log[s]])[0].astype(np.int64))

    # split bounds
    kind, arg = spec.splits
    if kind == "equal":
        b = int(arg)
        sb = np.zeros((S, 1, b + 1), dtype=np.int32)
        for s in range(S):
            sb[s, 0] = [(int(lens[s]) * j) // b for j in range(b + 1)]
    elif kind == "chunk":
        b = -(-spec.max_len // int(arg))
        sb = np.zeros((S, 1, b + 1), dtype=np.int32)
        for s in range(S):
            sb[s, 0] = [min(int(arg) * j, int(lens[s])) for j in range(b + 1)]
    elif kind == "kept_pages":
        b = int(arg)
        sb = np.zeros((S, Hkv, b + 1), dtype=np.int32)
        for s in range(S):
            for h in range(Hkv):
                kp = kept[s * Hkv + h]
                for j in range(b):
                    sb[s, h, j] = 0 if j == 0 else int(kp[(j * len(kp)) // b]) * P
                sb[s, h, b] = int(lens[s])
    else:
        raise ValueError(kind)

    if spec.layout == "head":  # [Hkv, NP, P, D], copied one head at a time
        k_pages, v_pages = _head_major(k_pages), _head_major(v_pages)
    elif spec.layout != "page":
        raise ValueError(spec.layout)
    return Batch(
        spec=spec, seed=seed, q=q, k_pages=k_pages, v_pages=v_pages,
        block_table=table_t.to(device), seq_lens=torch.from_numpy(lens.astype(np.int32)).to(device),
        split_bounds=torch.from_numpy(sb).to(device),
        block_mask=None if mask_np is None else torch.from_numpy(mask_np).to(device),
        scale=1.0 / math.sqrt(D), kept_pages=kept, layout=spec.layout,
    )


def _head_major(pool: torch.Tensor) -> torch.Tensor:
    NP, Hkv, P, D = pool.shape
    out = torch.empty((Hkv, NP, P, D), dtype=pool.dtype, device=pool.device)
    for h in range(Hkv):
        out[h].copy_(pool[:, h])
    return out


def new_tokens(spec: Spec, seed: int, step: int, device="cpu"):
    """Key and value rows [S, Hkv, D] of the token appended at decode step
    `step`: i.i.d. N(0, 1) in the workload's dtype, one seeded sub-stream per
    (seed, workload, step)."""
    g = _gen(seed, spec, f"new_tokens/{step}", torch.device(device))
    shape = (spec.S, spec.Hkv, spec.D)
    k = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
    v = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
    return k.to(TORCH_DTYPE[spec.dtype]), v.to(TORCH_DTYPE[spec.dtype])


def host(t: Optional[torch.Tensor]):
    """numpy copy of a tensor for the oracle: bf16 as its uint16 bit pattern."""
    if t is None:
        return None
    t = t.detach().cpu().contiguous()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()
