"""GPU: random sequences of mixed calls on one context, call by call against
the oracle's protocol simulator, on a ragged small geometry and on the decode
geometry.

Each sequence interleaves fused gathers, split and partial pushes, declined
calls (no rows, too many rows), producer + gather calls, vocab-slice changes,
switches between host and device parity, graphs captured in device mode and
replayed with new data, and re-arms. After every call the output is compared
with the simulator's (sliced to the current vocab); the parity and both
mailbox parities are compared every few calls and at the end."""

from __future__ import annotations

import random

import numpy as np
import pytest
import torch

from oracle import gather as og
from tp_vocab_logits_amd import _lib
from tp_vocab_logits_amd import synthetic as syn
from tp_vocab_logits_amd.head_gather import HeadGather

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
# (tp, shard, cap, hidden): a ragged geometry (36 vectors per shard row, so
# chunks end mid-segment) and the decode geometry (TP=8, V=163840)
SMALL = (3, 288, 4, 40)
DECODE = (8, 20480, 8, 64)


def note(msg: str) -> None:
    print(f"[gpu] {msg}", flush=True)


def bits(t: torch.Tensor) -> np.ndarray:
    return syn.from_torch_bf16(t)


def dev(b: np.ndarray) -> torch.Tensor:
    return syn.to_torch_bf16(b, DEV)


class Run:
    def __init__(self, seed: int, geometry=SMALL):
        self.tp, self.shard, self.cap, self.hidden = geometry
        self.v = self.tp * self.shard
        self.rng = random.Random(seed)
        self.seed = seed
        self.k = 0
        self.hg = HeadGather(self.tp, self.shard, self.cap, device=DEV)
        self.hg.set_poll_limit(1 << 20)
        self.sim = og.MailboxSim(self.tp, self.shard, self.cap)
        self.vocab = self.v
        self.device_mode = False
        self.w = dev(syn.random_bf16((self.tp, self.shard, self.hidden), 0.5, 7000 + seed))

    def inputs(self, m: int) -> np.ndarray:
        self.k += 1
        s = syn.shard_set("spec", 10000 * self.seed + self.k, rows=m, tp=self.tp, shard=self.shard)
        syn.inject_sentinel_words(s, 0.05, 20000 * self.seed + self.k)
        return s

    def expect(self, got: torch.Tensor, want: np.ndarray, what: str) -> None:
        assert np.array_equal(bits(got), og.slice_vocab(want, self.vocab)), what

    def check_state(self, what: str) -> None:
        assert self.hg.parity == self.sim.parity, what
        for p in (0, 1):
            assert np.array_equal(bits(self.hg.mailbox(p)), self.sim.mailbox_bf16(p)), (what, p)
        assert self.hg.poll_status() == _lib.HG_OK, what

    # -- operations ---------------------------------------------------------
    def fused(self):
        m = self.rng.randint(1, self.cap)
        s = self.inputs(m)
        got = self.hg(dev(s))
        status, want = self.sim.gather(list(s))
        assert status == og.OK
        self.expect(got, want, f"fused m={m}")

    def declined(self):
        m = self.rng.choice([0, self.cap + 1, self.cap + 2])
        s = self.inputs(m)
        got = self.hg(dev(s))
        status, want = self.sim.gather(list(s))
        assert status == og.DECLINE
        self.expect(got, want, f"declined m={m}")

    def split(self):
        m = self.rng.randint(1, self.cap)
        s = self.inputs(m)
        assert self.hg.push(dev(s)) and self.sim.push(list(s)) == og.OK
        got = self.hg.collect(m)
        status, want = self.sim.collect(m)
        assert status == og.OK
        self.expect(got, want, f"split m={m}")

    def partial(self):
        m = self.rng.randint(1, self.cap)
        s = self.inputs(m)
        ranks = list(range(self.tp))
        self.rng.shuffle(ranks)
        cut = self.rng.randint(1, self.tp - 1)
        for part in (ranks[:cut], ranks[cut:]):
            assert self.hg.push_ranks(dev(s), part)
            assert self.sim.push_ranks(list(s), part) == og.OK
        got = self.hg.collect(m)
        status, want = self.sim.collect(m)
        assert status == og.OK
        self.expect(got, want, f"partial m={m} ranks={ranks[:cut]}|{ranks[cut:]}")

    def producer(self):
        m = self.rng.randint(1, self.cap)
        x = dev(syn.random_bf16((m, self.hidden), 0.5, 30000 * self.seed + self.k))
        self.k += 1
        shards = torch.empty((self.tp, m, self.shard), dtype=torch.bfloat16, device=DEV)
        got = self.hg.gemm_gather(x, self.w, shards_out=shards)
        status, want = self.sim.gather(list(bits(shards)))
        assert status == og.OK
        self.expect(got, want, f"producer m={m}")

    def vocab_change(self):
        v = self.v
        self.vocab = self.rng.choice([v, v - 1, v - 8, 8 * self.rng.randint(1, v // 8), self.rng.randint(1, v)])
        self.hg.set_vocab(self.vocab)

    def mode_switch(self):
        self.device_mode = not self.device_mode
        self.hg.set_device_parity(self.device_mode)

    def graph(self):
        if not self.device_mode:
            self.mode_switch()
        calls = self.rng.randint(1, 3)
        ms = [self.rng.randint(1, self.cap) for _ in range(calls)]
        static_in = [dev(self.inputs(m)) for m in ms]
        static_out = [torch.empty((m, self.vocab), dtype=torch.bfloat16, device=DEV) for m in ms]
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for c in range(calls):
                self.hg(static_in[c], out=static_out[c])
        for rep in range(self.rng.randint(1, 3)):
            sets = [self.inputs(m) for m in ms]
            for c in range(calls):
                static_in[c].copy_(dev(sets[c]))
            g.replay()
            torch.cuda.synchronize()
            for c in range(calls):
                status, want = self.sim.gather(list(sets[c]))
                assert status == og.OK
                self.expect(static_out[c], want, f"graph call {c} replay {rep}")

    def arm(self):
        self.hg.arm()
        self.sim.arm()


OPS = [("fused", 6), ("declined", 2), ("split", 3), ("partial", 3), ("producer", 2),
       ("vocab_change", 2), ("mode_switch", 2), ("graph", 2), ("arm", 1)]


@pytest.mark.parametrize("seed,geometry", [(s, SMALL) for s in range(1, 33)]
                         + [(s, DECODE) for s in range(101, 105)],
                         ids=lambda v: "x".join(map(str, v)) if isinstance(v, tuple) else str(v))
def test_random_mixed_sequence(seed, geometry):
    run = Run(seed, geometry)
    names = [n for n, wgt in OPS for _ in range(wgt)]
    for i in range(100):
        op = run.rng.choice(names)
        note(f"seed {seed} {geometry} step {i}: {op} (vocab {run.vocab}, device parity {run.device_mode})")
        getattr(run, op)()
        if i % 5 == 4:
            run.check_state(f"seed {seed} after step {i} ({op})")
    run.check_state(f"seed {seed} end")
    run.hg.close()
