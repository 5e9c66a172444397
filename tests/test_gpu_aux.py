"""Measurement helper and device validation on the GPU: da_stream_read over
whole and ragged buffer sizes (a partial last 1 KiB block, sizes below one
block) completes and leaves the sink untouched."""

import sys

import pytest
import torch

from long_context_decode_microattention_amd import _lib

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


@pytest.mark.parametrize("nbytes", [16, 1008, 1024, 1040, 64 * 1024 + 48, (3 << 20) + 16, 64 << 20])
def test_stream_read_sizes(nbytes):
    print("[gpu-case] stream_read", nbytes, flush=True)
    sys.stdout.flush()
    buf = torch.ones(nbytes // 4, dtype=torch.int32, device=DEV)
    sink = torch.zeros(int(_lib.load().da_stream_read_sink_words()), dtype=torch.int32, device=DEV)
    _lib.stream_read(buf, sink)
    torch.cuda.synchronize()
    assert int(sink.abs().sum()) == 0
