"""GPU: hg_gather_static, the gather that allocates nothing (its mailbox and
parity live in the library's static device array), called through the C ABI
and checked bit for bit against hg_gather, the context entry point, and the
CPU oracle on the same inputs: calls in a row with shrinking inputs (the
second smaller than the first, then another vocabulary width), the size
limit, and replays of captured calls."""

from __future__ import annotations

import ctypes

import numpy as np
import pytest
import torch

from oracle import gather as og
from tp_vocab_logits_amd import _lib
from tp_vocab_logits_amd import synthetic as syn
from tp_vocab_logits_amd.head_gather import HeadGather

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def note(msg: str) -> None:
    print(f"[gpu] {msg}", flush=True)


def inputs(tp: int, shard: int, m: int, k: int) -> np.ndarray:
    s = syn.shard_set(syn.WORKLOADS["spec"], k, rows=m, tp=tp, shard=shard)
    syn.inject_sentinel_words(s, 0.01, 500 + k)
    return s


def gather_static(shards: torch.Tensor, out: torch.Tensor) -> int:
    tp, m, shard = (int(v) for v in shards.shape)
    step = m * shard * 2
    ptrs = _lib.pointer_array([shards.data_ptr() + r * step for r in range(tp)])
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    return _lib.lib().hg_gather_static(tp, shard, ptrs, m, ctypes.c_void_p(out.data_ptr()), stream)


def test_static_gather_matches_the_context_gather():
    # decode geometry at 8 rows (2.6 MB of the 8 MiB parity), then one row,
    # then a different vocabulary width (TP=2, V=4096): every call's output
    # equals hg_gather's on the same inputs, and the oracle's
    cases = [(8, 20480, 8, 0), (8, 20480, 1, 1), (2, 2048, 1, 2), (8, 20480, 3, 3)]
    for tp, shard, m, k in cases:
        note(f"static gather tp={tp} shard={shard} m={m}")
        s = inputs(tp, shard, m, k)
        d = syn.to_torch_bf16(s, DEV)
        hg = HeadGather(tp, shard, m, device=DEV)
        want = hg(d)
        out = torch.empty((m, tp * shard), dtype=torch.bfloat16, device=DEV)
        assert gather_static(d, out) == _lib.HG_OK
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), want.view(torch.int16)), (tp, shard, m)
        assert np.array_equal(syn.from_torch_bf16(out), og.gather_definition(list(s)))
        hg.close()


def test_static_gather_size_limit_and_arguments():
    lib = _lib.lib()
    tp, shard = 8, 20480
    rows = _lib.HG_STATIC_PARITY_BYTES // (tp * shard * 2)  # 25 rows of V=163840
    d = torch.zeros((tp, rows + 1, shard), dtype=torch.bfloat16, device=DEV)
    out = torch.empty((rows + 1, tp * shard), dtype=torch.bfloat16, device=DEV)
    assert gather_static(d, out) == _lib.HG_ESIZE
    assert b"static" in lib.hg_last_error_detail()
    ptrs = _lib.pointer_array([d.data_ptr()] * tp)
    s = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    assert lib.hg_gather_static(tp, shard, ptrs, 0, ctypes.c_void_p(out.data_ptr()), s) == _lib.HG_EDECLINE
    assert lib.hg_gather_static(1, shard, ptrs, 1, ctypes.c_void_p(out.data_ptr()), s) == _lib.HG_EINVAL
    assert lib.hg_gather_static(tp, 12, ptrs, 1, ctypes.c_void_p(out.data_ptr()), s) == _lib.HG_EINVAL
    # the largest call that fits is served
    s_big = inputs(tp, shard, rows, 7)
    db = syn.to_torch_bf16(s_big, DEV)
    ob = torch.empty((rows, tp * shard), dtype=torch.bfloat16, device=DEV)
    assert gather_static(db, ob) == _lib.HG_OK
    torch.cuda.synchronize()
    assert np.array_equal(syn.from_torch_bf16(ob), og.gather_definition(list(s_big)))


def test_static_gather_replays_from_a_graph():
    tp, shard = 4, 1024
    note("static gather under graph capture")
    ms = [2, 1]
    static_in = [syn.to_torch_bf16(inputs(tp, shard, m, 20 + m), DEV) for m in ms]
    static_out = [torch.empty((m, tp * shard), dtype=torch.bfloat16, device=DEV) for m in ms]
    for i in range(2):  # eager first (the first call on the device may not be captured)
        assert gather_static(static_in[i], static_out[i]) == _lib.HG_OK
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for i in range(2):
            assert gather_static(static_in[i], static_out[i]) == _lib.HG_OK
    for rep in range(4):
        sets = [inputs(tp, shard, m, 40 + 10 * rep + m) for m in ms]
        for i in range(2):
            static_in[i].copy_(syn.to_torch_bf16(sets[i], DEV))
        graph.replay()
        torch.cuda.synchronize()
        for i in range(2):
            assert np.array_equal(syn.from_torch_bf16(static_out[i]), og.gather_definition(list(sets[i]))), (rep, i)
        # eager call between replays
        e = inputs(tp, shard, 3, 90 + rep)
        eo = torch.empty((3, tp * shard), dtype=torch.bfloat16, device=DEV)
        assert gather_static(syn.to_torch_bf16(e, DEV), eo) == _lib.HG_OK
        torch.cuda.synchronize()
        assert np.array_equal(syn.from_torch_bf16(eo), og.gather_definition(list(e)))
