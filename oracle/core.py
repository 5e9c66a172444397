"""Plain fp64 CPU oracle for decode attention over a paged KV cache.

TEST INFRASTRUCTURE ONLY.  Only the test suite, ``__graft_entry__.smoke()`` and
the ``cpu_baseline`` leg of ``bench.py`` may import this module.  The product
path (the HIP library and its Python binding) never imports, calls or links
anything here, and this module imports nothing from the product package.

Everything is computed in float64 with numpy, in the order the defining
equations state.  No blocking, fusion or reordering beyond what those equations
say.  Sources (all on the Infinite-LLM page, "Infinite-LLM: Efficient LLM
Service for Long Context with DistAttention and Distributed KVCache"):

* standard attention with a global max -- section 方法细节 (method details),
  paragraph "分布式注意力机制的通信挑战", equations for m_g and Attention(Q,K,V);
* MicroAttention -- same section, paragraph "DistAttention 的等价数学变换",
  equations for m_j, e_j and MA_j;
* aggregation of b partials -- same section, paragraph "结果聚合与通信开销降低",
  equations for m_g, e_g and Attention.

Block-sparse page skipping follows the LServe blog page ("LLM长序列服务优化：
LServe的块稀疏注意力技术"), section 2.1.1: the KV history is cut into
fixed-size blocks and only selected blocks are loaded and computed.

Readings where the pages are silent (each is also listed with its reason in the
design notes):

* scores are scaled, s_i = scale * (q . k_i), scale = 1/sqrt(D) unless given;
* the query for q head h reads KV head h // G with G = Hq / Hkv;
* a split is the logical token range [sb_j, sb_{j+1}) intersected with
  [0, L_s); masked pages are removed from it; an empty split is the triple
  (MA = 0, m = -inf, e = 0), and if every split is empty the output is 0;
* bf16 inputs are given as their uint16 bit patterns and widened exactly.

Parity status: every function here is pinned by ``tests/test_oracle.py``
(closed forms, a 50-digit decimal brute force, the split identities, the
compacted-mask equivalence, the GQA probe) and by the hand-derived worked
example in ``tests/golden/``.
"""

from __future__ import annotations

import numpy as np

NEG_INF = -np.inf


# ---------------------------------------------------------------------------
# element conversion
# ---------------------------------------------------------------------------

def to_f64(x) -> np.ndarray:
    """Widen an input array to float64 exactly.

    A bfloat16 value is the upper 16 bits of an IEEE-754 binary32 value, so a
    uint16 bit pattern widens by placing it in the high half of a 32-bit word.
    float32 and float64 arrays widen directly.
    """
    a = np.asarray(x)
    if a.dtype == np.uint16:
        return (a.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)
    if a.dtype in (np.float32, np.float64):
        return a.astype(np.float64)
    raise TypeError(f"unsupported element type {a.dtype}")


def default_scale(head_dim: int) -> float:
    """Scaled dot-product reading of the score: 1/sqrt(D)."""
    return 1.0 / np.sqrt(float(head_dim))


# ---------------------------------------------------------------------------
# the plain definition over a contiguous token set
# ---------------------------------------------------------------------------

def scores(q, K, scale: float) -> np.ndarray:
    """s_i = scale * (q . k_i) for every row k_i of K."""
    q64 = to_f64(q)
    K64 = to_f64(K)
    return (K64 @ q64) * float(scale)


def attention_tokens(q, K, V, scale: float) -> np.ndarray:
    """Standard attention of one query over the rows of K and V.

    Global-max form: m_g = max_i s_i and
    out = sum_i exp(s_i - m_g) V_i / sum_j exp(s_j - m_g).
    An empty token set gives the zero vector (empty-split reading).
    """
    V64 = to_f64(V)
    if V64.shape[0] == 0:
        return np.zeros(V64.shape[1], dtype=np.float64)
    s = scores(q, K, scale)
    m_g = s.max()
    w = np.exp(s - m_g)
    return (w[:, None] * V64).sum(axis=0) / w.sum()


def micro_tokens(q, K, V, scale: float):
    """MicroAttention over the rows of K and V (one split).

    m_j = max_i s_i, e_j = sum_i exp(s_i - m_j), MA_j = sum_i exp(s_i - m_j) V_i.
    Returns (MA_j, m_j, e_j); an empty split gives (0, -inf, 0).
    """
    V64 = to_f64(V)
    if V64.shape[0] == 0:
        return np.zeros(V64.shape[1], dtype=np.float64), NEG_INF, 0.0
    s = scores(q, K, scale)
    m_j = s.max()
    w = np.exp(s - m_j)
    return (w[:, None] * V64).sum(axis=0), float(m_j), float(w.sum())


# ---------------------------------------------------------------------------
# paged KV cache
# ---------------------------------------------------------------------------

def kept_tokens(seq_len: int, page_size: int, t_begin: int, t_end: int,
                mask_row=None) -> np.ndarray:
    """Logical token ids of [t_begin, t_end) intersected with [0, seq_len),
    in increasing order, with every token of a page whose mask entry is 0
    removed."""
    lo = max(int(t_begin), 0)
    hi = min(int(t_end), int(seq_len))
    if hi <= lo:
        return np.zeros(0, dtype=np.int64)
    t = np.arange(lo, hi, dtype=np.int64)
    if mask_row is not None:
        keep = np.asarray(mask_row)[t // page_size] != 0
        t = t[keep]
    return t


def gather(pool, block_table_row, kv_head: int, tokens: np.ndarray, page_size: int):
    """Rows of one KV head for the given logical tokens of one request.

    The pool is laid out [physical page, KV head, slot, D]; logical token t
    lives in physical page block_table_row[t // P] at slot t % P.
    """
    tokens = np.asarray(tokens, dtype=np.int64)
    phys = np.asarray(block_table_row, dtype=np.int64)[tokens // page_size]
    slot = tokens % page_size
    return np.asarray(pool)[phys, kv_head, slot, :]


def kv_head_of(h: int, Hq: int, Hkv: int) -> int:
    """KV head read by query head h: consecutive grouping, h // (Hq / Hkv)."""
    return h // (Hq // Hkv)


def _dims(q, k_pool):
    q = np.asarray(q)
    k_pool = np.asarray(k_pool)
    S, Hq, D = q.shape
    Hkv = k_pool.shape[1]
    if Hq % Hkv != 0:
        raise ValueError("Hq must be a multiple of Hkv")
    return S, Hq, Hkv, D, k_pool.shape[2]


def attention(q, k_pool, v_pool, block_table, seq_lens, block_mask=None,
              scale: float | None = None, pairs=None) -> np.ndarray:
    """Unsplit attention out[s, h, :] for every request s and query head h.

    q [S, Hq, D]; k_pool, v_pool [NP, Hkv, P, D]; block_table [S, max_pages];
    seq_lens [S]; block_mask [S, Hkv, max_pages] or None.  ``pairs`` limits
    the work to the listed (s, h) pairs; the other rows stay NaN.
    """
    S, Hq, Hkv, D, P = _dims(q, k_pool)
    sc = default_scale(D) if scale is None else float(scale)
    out = np.full((S, Hq, D), np.nan, dtype=np.float64)
    todo = [(s, h) for s in range(S) for h in range(Hq)] if pairs is None else pairs
    for s, h in todo:
        kvh = kv_head_of(h, Hq, Hkv)
        mrow = None if block_mask is None else np.asarray(block_mask)[s, kvh]
        t = kept_tokens(int(seq_lens[s]), P, 0, int(seq_lens[s]), mrow)
        K = gather(k_pool, block_table[s], kvh, t, P)
        V = gather(v_pool, block_table[s], kvh, t, P)
        out[s, h] = attention_tokens(np.asarray(q)[s, h], K, V, sc)
    return out


def micro_attention(q, k_pool, v_pool, block_table, seq_lens, split_bounds,
                    block_mask=None, scale: float | None = None, pairs=None):
    """MicroAttention partials for every (request, query head, split).

    split_bounds is [S, 1, b+1] (one set of bounds per request) or
    [S, Hkv, b+1] (one set per KV head).  Returns MA [S, Hq, b, D],
    m [S, Hq, b], e [S, Hq, b]; rows outside ``pairs`` stay NaN.
    """
    S, Hq, Hkv, D, P = _dims(q, k_pool)
    sb = np.asarray(split_bounds)
    nbh, b = sb.shape[1], sb.shape[2] - 1
    if nbh not in (1, Hkv):
        raise ValueError("split_bounds must have 1 or Hkv rows per request")
    sc = default_scale(D) if scale is None else float(scale)
    MA = np.full((S, Hq, b, D), np.nan, dtype=np.float64)
    m = np.full((S, Hq, b), np.nan, dtype=np.float64)
    e = np.full((S, Hq, b), np.nan, dtype=np.float64)
    todo = [(s, h) for s in range(S) for h in range(Hq)] if pairs is None else pairs
    for s, h in todo:
        kvh = kv_head_of(h, Hq, Hkv)
        row = sb[s, kvh if nbh == Hkv else 0]
        mrow = None if block_mask is None else np.asarray(block_mask)[s, kvh]
        for j in range(b):
            t = kept_tokens(int(seq_lens[s]), P, int(row[j]), int(row[j + 1]), mrow)
            K = gather(k_pool, block_table[s], kvh, t, P)
            V = gather(v_pool, block_table[s], kvh, t, P)
            MA[s, h, j], m[s, h, j], e[s, h, j] = micro_tokens(np.asarray(q)[s, h], K, V, sc)
    return MA, m, e


# ---------------------------------------------------------------------------
# aggregation
# ---------------------------------------------------------------------------

def _weights(m, axis):
    """exp(m_j - m_g) with m_g = max_j m_j; 0 for empty partials (m_j = -inf)."""
    m = np.asarray(m, dtype=np.float64)
    m_g = np.max(m, axis=axis, keepdims=True)
    safe = np.where(np.isneginf(m_g), 0.0, m_g)
    w = np.where(np.isneginf(m), 0.0, np.exp(m - safe))
    return m_g, w


def merge(MA, m, e) -> np.ndarray:
    """Aggregate b partials into attention (last two axes of MA are [b, D]).

    m_g = max_j m_j, e_g = sum_j e_j exp(m_j - m_g),
    out = sum_j MA_j exp(m_j - m_g) / e_g.  All-empty input gives 0.
    """
    MA = np.asarray(MA, dtype=np.float64)
    e = np.asarray(e, dtype=np.float64)
    _, w = _weights(m, axis=-1)
    e_g = (e * w).sum(axis=-1)
    num = (MA * w[..., None]).sum(axis=-2)
    den = np.where(e_g > 0, e_g, 1.0)[..., None]
    return np.where((e_g > 0)[..., None], num / den, 0.0)


def merge_partials(MA, m, e):
    """Aggregate b partials into one partial triple (MA', m', e') that is again
    a MicroAttention result over the union of the token sets: m' = m_g,
    e' = e_g, MA' = sum_j MA_j exp(m_j - m_g).  The split axis is the last
    axis of m and e, and the second-last axis of MA."""
    MA = np.asarray(MA, dtype=np.float64)
    e = np.asarray(e, dtype=np.float64)
    m_g, w = _weights(m, axis=-1)
    return (MA * w[..., None]).sum(axis=-2), m_g[..., 0], (e * w).sum(axis=-1)
