"""GPU: device-side parity and graph capture.

With the parity kept in device memory, gathers captured into a HIP graph are
served (instead of declined) and every replay alternates the parity. Each
replay is checked against the oracle -- outputs, both mailbox parities and the
parity -- with eager work on the same context between replays."""

from __future__ import annotations

import numpy as np
import pytest
import torch

from oracle import gather as og
from tp_vocab_logits_amd import _lib
from tp_vocab_logits_amd import synthetic as syn
from tp_vocab_logits_amd.head_gather import HeadGather, HgError

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def note(msg: str) -> None:
    print(f"[gpu] {msg}", flush=True)


def bits(t: torch.Tensor) -> np.ndarray:
    return syn.from_torch_bf16(t)


def dev(b: np.ndarray) -> torch.Tensor:
    return syn.to_torch_bf16(b, DEV)


def make(tp, shard, cap) -> HeadGather:
    hg = HeadGather(tp, shard, cap, device=DEV)
    hg.set_poll_limit(1 << 20)
    return hg


def assert_state(hg, sim):
    assert hg.parity == sim.parity
    for p in (0, 1):
        assert np.array_equal(bits(hg.mailbox(p)), sim.mailbox_bf16(p)), p


def inputs(tp, shard, m, k, frac=0.02):
    s = syn.shard_set("spec", k, rows=m, tp=tp, shard=shard)
    syn.inject_sentinel_words(s, frac, 300 + k)
    return s


def test_eager_calls_with_device_parity():
    tp, shard, cap = 4, 512, 3
    note(f"device parity eager tp={tp} shard={shard} cap={cap}")
    hg, sim = make(tp, shard, cap), og.MailboxSim(tp, shard, cap)
    s0 = inputs(tp, shard, 2, 0)
    hg(dev(s0)), sim.gather(list(s0))           # host parity: now 1
    hg.set_device_parity(True)
    assert_state(hg, sim)
    for n in range(7):
        m = 1 + n % cap
        s = inputs(tp, shard, m, n + 1)
        if n % 3 == 2:
            assert hg.push(dev(s)) and sim.push(list(s)) == og.OK
            out = hg.collect(m)
            status, want = sim.collect(m)
        else:
            out = hg(dev(s))
            status, want = sim.gather(list(s))
        assert status == og.OK and np.array_equal(bits(out), want), n
        assert_state(hg, sim)
    hg.set_device_parity(False)                 # back to host parity
    assert hg.parity == sim.parity
    s = inputs(tp, shard, 1, 50)
    out = hg(dev(s))
    status, want = sim.gather(list(s))
    assert status == og.OK and np.array_equal(bits(out), want)
    assert_state(hg, sim)
    assert hg.poll_status() == _lib.HG_OK


@pytest.mark.parametrize("calls", [1, 2, 3])
def test_graph_of_fused_gathers_replays(calls):
    tp, shard, cap, m = 8, 2048, 4, 4
    note(f"graph of {calls} fused gathers, device parity")
    hg, sim = make(tp, shard, cap), og.MailboxSim(tp, shard, cap)
    hg.set_device_parity(True)
    static_in = [dev(inputs(tp, shard, m, 100 + c)) for c in range(calls)]
    static_out = [torch.empty((m, tp * shard), dtype=torch.bfloat16, device=DEV) for _ in range(calls)]
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for c in range(calls):
            hg(static_in[c], out=static_out[c])
    # capturing recorded the launches without running them: state unchanged
    assert_state(hg, sim)
    for rep in range(6):
        sets = [inputs(tp, shard, m, 1000 * rep + c) for c in range(calls)]
        for c in range(calls):
            static_in[c].copy_(dev(sets[c]))
        graph.replay()
        torch.cuda.synchronize()
        for c in range(calls):
            status, want = sim.gather(list(sets[c]))
            assert status == og.OK and np.array_equal(bits(static_out[c]), want), (rep, c)
        assert_state(hg, sim)
        # eager work on the same context between replays
        s = inputs(tp, shard, 1 + rep % cap, 5000 + rep)
        out = hg(dev(s))
        status, want = sim.gather(list(s))
        assert status == og.OK and np.array_equal(bits(out), want)
        assert_state(hg, sim)
    assert hg.poll_status() == _lib.HG_OK


def test_graph_of_split_push_collect():
    tp, shard, cap, m = 3, 264, 2, 2
    note("graph of split push + collect, device parity")
    hg, sim = make(tp, shard, cap), og.MailboxSim(tp, shard, cap)
    hg.set_device_parity(True)
    static_in = dev(inputs(tp, shard, m, 7))
    static_out = torch.empty((m, tp * shard), dtype=torch.bfloat16, device=DEV)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        assert hg.push(static_in)
        hg.collect(m, out=static_out)
    for rep in range(5):
        s = inputs(tp, shard, m, 70 + rep)
        static_in.copy_(dev(s))
        graph.replay()
        torch.cuda.synchronize()
        status, want = sim.gather(list(s))
        assert status == og.OK and np.array_equal(bits(static_out), want), rep
        assert_state(hg, sim)
    assert hg.poll_status() == _lib.HG_OK


@pytest.mark.parametrize("m", [3, 130])
def test_graph_of_producer_gather(m):
    # 3 rows: the 8 x 1 product; 130: the 4 x 2 product, whose epilogue reads
    # the device parity too
    tp, shard, hidden = 2, 256, 192
    cap = m
    note(f"graph of lm_head producer + gather, device parity, m={m}")
    hg, sim = make(tp, shard, cap), og.MailboxSim(tp, shard, cap)
    hg.set_device_parity(True)
    x = dev(syn.random_bf16((m, hidden), 0.5, 1))
    w = dev(syn.random_bf16((tp, shard, hidden), 0.5, 2))
    shards = torch.empty((tp, m, shard), dtype=torch.bfloat16, device=DEV)
    out = torch.empty((m, tp * shard), dtype=torch.bfloat16, device=DEV)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        hg.gemm_gather(x, w, out=out, shards_out=shards)
    for rep in range(4):
        x.copy_(dev(syn.random_bf16((m, hidden), 0.5, 10 + rep)))
        graph.replay()
        torch.cuda.synchronize()
        status, want = sim.gather(list(bits(shards)))
        assert status == og.OK and np.array_equal(bits(out), want), rep
        assert_state(hg, sim)


def test_host_parity_still_declines_capture_and_mode_switch_rules():
    tp, shard, cap = 2, 64, 2
    note("host parity declines capture; mode switch rules")
    hg = make(tp, shard, cap)
    s = dev(inputs(tp, shard, 1, 3))
    assert hg.push(s)
    with pytest.raises(HgError):
        hg.set_device_parity(True)  # a split push is pending
    hg.collect(1)
    assert hg.parity == 1
    hg.set_device_parity(True)
    assert hg.parity == 1
    hg.set_device_parity(False)
    assert hg.parity == 1


@pytest.mark.parametrize("tp,shard,cap", [(4, 1024, 4), (8, 20480, 8), (2, 8, 3)])
def test_graph_replays_across_grid_sizes(tp, shard, cap):
    """The parity slots are laid out per wave of the launch that completes a
    call: the layout changes with the grid, from one workgroup (TP=2, S=8) to
    hundreds (TP=8, V=163840 at cap rows), between the calls of one replay."""
    note(f"graph replays across grid sizes tp={tp} shard={shard} cap={cap}")
    hg, sim = make(tp, shard, cap), og.MailboxSim(tp, shard, cap)
    hg.set_device_parity(True)
    ms = [1, cap, 2]
    static_in = [dev(inputs(tp, shard, m, 600 + m)) for m in ms]
    static_out = [torch.empty((m, tp * shard), dtype=torch.bfloat16, device=DEV) for m in ms]
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        hg(static_in[0], out=static_out[0])        # fused
        assert hg.push(static_in[1])               # split
        hg.collect(ms[1], out=static_out[1])
        hg(static_in[2], out=static_out[2])        # fused
    for rep in range(4):
        sets = [inputs(tp, shard, m, 700 + 10 * rep + m) for m in ms]
        for c in range(3):
            static_in[c].copy_(dev(sets[c]))
        graph.replay()
        torch.cuda.synchronize()
        for c in range(3):
            status, want = sim.gather(list(sets[c]))
            assert status == og.OK and np.array_equal(bits(static_out[c]), want), (rep, c)
        assert_state(hg, sim)
        s = inputs(tp, shard, 1 + rep % cap, 800 + rep)  # eager call between replays
        out = hg(dev(s))
        status, want = sim.gather(list(s))
        assert status == og.OK and np.array_equal(bits(out), want)
        assert_state(hg, sim)
    assert hg.poll_status() == _lib.HG_OK
