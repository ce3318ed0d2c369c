"""GPU: the benchmark's reference streaming kernel (libhgref.so) moves what it
claims: the shards into the written rows, the previously written rows to the
output, then arms them -- checked on a small and a ragged size."""

from __future__ import annotations

import ctypes

import pytest
import torch

from tp_vocab_logits_amd import _lib

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
ARMED = -(1 << 31)


@pytest.mark.parametrize("vectors,grid", [(1, 1), (5000, 7), (65536, 1024)])
def test_stream_ref_moves_the_bytes(vectors, grid):
    print(f"[gpu] stream ref vectors={vectors} grid={grid}", flush=True)
    g = torch.Generator(device=DEV).manual_seed(vectors)
    n = vectors * 4
    src = torch.randint(-(1 << 31), 1 << 31, (n,), dtype=torch.int64, device=DEV, generator=g).to(torch.int32)
    box_r = torch.randint(-(1 << 31), 1 << 31, (n,), dtype=torch.int64, device=DEV, generator=g).to(torch.int32)
    box_w = torch.zeros(n, dtype=torch.int32, device=DEV)
    out = torch.zeros(n, dtype=torch.int32, device=DEV)
    before = box_r.clone()
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    assert _lib.ref().hgref_stream(src.data_ptr(), box_w.data_ptr(), box_r.data_ptr(), out.data_ptr(),
                                   vectors, grid, stream) == 0
    torch.cuda.synchronize()
    assert torch.equal(box_w, src)
    assert torch.equal(out, before)
    assert bool((box_r == ARMED).all())
    assert _lib.ref().hgref_stream(None, box_w.data_ptr(), box_r.data_ptr(), out.data_ptr(),
                                   vectors, grid, stream) == -1
