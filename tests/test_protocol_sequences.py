"""GPU: every sequence of three calls on one context, against the oracle's
protocol simulator -- fused gathers at 1 and cap rows, declines (no rows, too
many rows, host parity under graph capture), split push + collect, a push by
the two ranks separately, and re-arm -- with outputs, parity and both mailbox
parities compared after each sequence, with the parity kept on the host and
on the device. TP=2, S=16, cap=2."""

from __future__ import annotations

import itertools

import numpy as np
import pytest
import torch

from oracle import gather as og
from tp_vocab_logits_amd import _lib
from tp_vocab_logits_amd import synthetic as syn
from tp_vocab_logits_amd.head_gather import HeadGather

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
TP, SHARD, CAP = 2, 16, 2
OPS = [("gather", 1, "fused"), ("gather", 2, "fused"), ("decline", 0, "fused"),
       ("decline", 3, "fused"), ("decline", 1, "capture"), ("split", 1, "split"),
       ("split", 2, "split"), ("split", 1, "ranks"), ("arm", 0, "arm")]


def bits(t: torch.Tensor) -> np.ndarray:
    return syn.from_torch_bf16(t)


def dev(b: np.ndarray) -> torch.Tensor:
    return syn.to_torch_bf16(b, DEV)


@pytest.mark.parametrize("device_parity", [False, True], ids=["host-parity", "device-parity"])
@pytest.mark.parametrize("first", range(len(OPS)), ids=[f"{o[0]}{o[1]}-{o[2]}" for o in OPS])
def test_all_three_call_sequences(first, device_parity):
    """With the parity on the host a captured call declines (stock result,
    parity kept); with device-side parity it is served on replay."""
    print(f"[gpu] sequences starting with {OPS[first]}, device parity {device_parity}", flush=True)
    hg = HeadGather(TP, SHARD, CAP, device=DEV)
    hg.set_poll_limit(1 << 20)
    hg.set_device_parity(device_parity)
    k = 0
    for rest in itertools.product(range(len(OPS)), repeat=2):
        seq = (first,) + rest
        hg.arm()
        sim = og.MailboxSim(TP, SHARD, CAP)
        for i in seq:
            kind, m, how = OPS[i]
            if how == "arm":
                hg.arm()
                sim.arm()
                continue
            k += 1
            s = syn.shard_set("spec", 50000 + 100 * first + k, rows=m, tp=TP, shard=SHARD)
            syn.inject_sentinel_words(s, 0.1, 60000 + 100 * first + k)
            if how == "fused":
                got = hg(dev(s))
                status, want = sim.gather(list(s))
            elif how == "capture":
                static_in = dev(s)
                out = torch.empty((m, TP * SHARD), dtype=torch.bfloat16, device=DEV)
                g = torch.cuda.CUDAGraph()
                with torch.cuda.graph(g):
                    hg(static_in, out=out)
                g.replay()
                torch.cuda.synchronize()
                got = out
                status, want = sim.gather(list(s), capturing=not device_parity)
            elif how == "split":
                assert hg.push(dev(s)) and sim.push(list(s)) == og.OK
                got = hg.collect(m)
                status, want = sim.collect(m)
            else:
                d = dev(s)
                assert hg.push_ranks(d, [1]) and sim.push_ranks(list(s), [1]) == og.OK
                assert hg.push_ranks(d, [0]) and sim.push_ranks(list(s), [0]) == og.OK
                got = hg.collect(m)
                status, want = sim.collect(m)
            served = kind != "decline" or (how == "capture" and device_parity)
            assert status == (og.OK if served else og.DECLINE), seq
            assert np.array_equal(bits(got), want), (seq, i)
        assert hg.parity == sim.parity, seq
        for p in (0, 1):
            assert np.array_equal(bits(hg.mailbox(p)), sim.mailbox_bf16(p)), (seq, p)
    assert hg.poll_status() == _lib.HG_OK
    hg.close()
