"""Plain CPU oracle for the decode-time cache update and the reuse of a page
selection across a chunk of decode steps.

TEST INFRASTRUCTURE ONLY.  Only the test suite, ``__graft_entry__.smoke()`` and
the ``cpu_baseline`` leg of ``bench.py`` may import this module.  The product
path never imports, calls or links anything here, and this module imports
nothing from the product package.

Sources:

* LServe blog page ("LLM长序列服务优化：LServe的块稀疏注意力技术"), section
  3.1.2: the logical-page statistics are computed when the KV cache is
  written, so they add no decode latency.  Here the statistics after a write
  are, by definition, the statistics of the new cache contents; the oracle
  recomputes them from scratch with ``oracle.selector.page_stats`` on the
  pool that ``append_kv`` returns, which is what an in-place update must
  reproduce.
* The same page, section 2.2.2 (reusable page selector): decoding is cut into
  chunks of a fixed number of tokens (16 in the example); the full page
  selection runs only at the start of a chunk and its result is reused
  inside the chunk.  ``oracle.selector.select_pages(..., horizon=...)`` keeps
  the pages the chunk's appended tokens will open.
* Infinite-LLM page, 方法细节: the sequence is cut into sub-blocks whose
  partial results are merged; the split rule used here gives each of b
  splits an equal share (to within one page) of a head's kept pages, which
  is the workload statement's "b splits over the kept pages".

Parity status: ``append_kv`` and ``kept_page_bounds`` are pinned by
``tests/test_decode_oracle.py`` (a brute-force gather of every token after the
write, untouched rows, the full-cache case, hand-derived bounds in
``tests/golden/decode_worked.json``, the balance and coverage properties of
the split rule, planted mistakes).
"""

from __future__ import annotations

import numpy as np


def append_kv(k_pool, v_pool, block_table, seq_lens, k_new, v_new):
    """Pools after writing token t = seq_lens[s] of every request s.

    k_pool, v_pool: [NP, Hkv, P, D] (any dtype; copied, not modified).
    k_new, v_new:   [S, Hkv, D], same dtype.
    For each request with 0 <= t < max_pages * P, every KV head's new key row
    goes to page block_table[s, t // P], slot t % P, and likewise the value
    row.  Requests whose cache is full are left unchanged.  Returns the new
    (k_pool, v_pool).
    """
    k = np.array(k_pool, copy=True)
    v = np.array(v_pool, copy=True)
    table = np.asarray(block_table)
    lens = np.asarray(seq_lens)
    P = k.shape[2]
    max_pages = table.shape[1]
    for s in range(lens.shape[0]):
        t = int(lens[s])
        if t < 0 or t >= max_pages * P:
            continue
        phys = int(table[s, t // P])
        k[phys, :, t % P, :] = np.asarray(k_new)[s]
        v[phys, :, t % P, :] = np.asarray(v_new)[s]
    return k, v


def kept_page_bounds(block_mask, seq_lens, P: int, b: int, horizon: int = 0, Hkv=None,
                     max_pages=None) -> np.ndarray:
    """Split bounds [S, Hkv, b + 1] (int) over the kept pages.

    For request s the pages considered are those below
    ceil(E / P) with E = min(L_s + horizon, max_pages * P); kept pages are
    those with block_mask[s, h, page] != 0 (every page when block_mask is
    None).  With K kept pages, kept[0] < ... < kept[K-1]:
        bound[0] = 0, bound[b] = E,
        bound[j] = P * kept[floor(j K / b)] if floor(j K / b) < K, else E,
    so split j holds kept pages of ordinals floor(j K / b) .. floor((j+1) K / b) - 1.
    """
    lens = np.asarray(seq_lens)
    S = lens.shape[0]
    if block_mask is not None:
        mask = np.asarray(block_mask)
        _, Hkv, max_pages = mask.shape
    out = np.zeros((S, Hkv, b + 1), dtype=np.int64)
    for s in range(S):
        E = min(int(lens[s]) + horizon, max_pages * P)
        n = -(-E // P)
        for h in range(Hkv):
            if block_mask is None:
                kept = list(range(n))
            else:
                kept = [lp for lp in range(n) if mask[s, h, lp] != 0]
            K = len(kept)
            out[s, h, 0] = 0
            out[s, h, b] = E
            for j in range(1, b):
                o = (j * K) // b
                out[s, h, j] = P * kept[o] if o < K else E
    return out
