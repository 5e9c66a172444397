"""The benchmark's oracle leg on the CPU: the forked worker pool, the
memory-mapped pools and the per-(request, KV head) tasks give the same
outputs as calling the oracle directly, for page- and head-major pools, with
and without a block mask; a wrong output is caught."""

from __future__ import annotations

import os
import sys

import numpy as np
import pytest
import torch

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import bench  # noqa: E402
import oracle  # noqa: E402
from long_context_decode_microattention_amd import workloads as wl  # noqa: E402


@pytest.fixture(scope="module")
def pool():
    bench.start_pool(2)
    yield
    bench.stop_pool()


def _direct(b):
    h = wl.host
    return oracle.attention(h(b.q), h(b.k_pm), h(b.v_pm), h(b.block_table), h(b.seq_lens),
                            block_mask=h(b.block_mask), scale=b.scale)


@pytest.mark.parametrize("cfg,layout", [("C1", "page"), ("C3", "page"), ("C5", "head"), ("C5", "page")])
def test_pool_matches_direct_oracle(pool, cfg, layout):
    small = {
        "C1": wl.CONFIGS["C1"],
        "C3": wl.CONFIGS["C3"].replace(S=3, Hq=4, Hkv=4, lens=("loguniform", 3000)),
        "C5": wl.CONFIGS["C5"].replace(S=2, lens=("fixed", 64 * 40 + 5)),
    }[cfg].replace(layout=layout)
    b = wl.build(small, 0, "cpu")
    want = _direct(b)
    b.out = torch.from_numpy(want.astype(np.float32))
    res = bench.oracle_check(b, f"test_{cfg}_{layout}", one_core_units=2)
    assert res["units"] == f"{small.S * small.Hkv}/{small.S * small.Hkv}"
    assert res["max_abs_err_vs_step"] <= 1e-6
    assert res["one_core"]["cores"] == 1 and res["one_core"]["value"] > 0
    assert not [f for f in os.listdir(bench._shm_dir()) if f.startswith(f"da_bench_{os.getpid()}_")]


def test_pool_catches_a_wrong_output(pool):
    b = wl.build(wl.CONFIGS["C1"], 0, "cpu")
    out = _direct(b)
    out[0, 2, 5] += 1e-3  # one element of query head 2 (KV head 2) off by more than 1e-5
    b.out = torch.from_numpy(out)
    with pytest.raises(AssertionError, match="differs from the oracle"):
        bench.oracle_check(b, "test_wrong")
