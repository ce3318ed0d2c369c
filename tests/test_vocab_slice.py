"""GPU: the padded-vocab slice folded into the copy step.

Served calls write ``[M, vocab]``, the first ``vocab`` columns of each gathered
row, and must equal the oracle's slice of its gathered logits bit for bit,
while the mailbox protocol (push, poll, re-arm, parity) is unchanged. Every
output lives inside a larger buffer whose tail is a guard pattern, so a store
past ``M * vocab`` elements is caught."""

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
GUARD = 4096  # BF16 elements after the output
GUARD_BITS = 0x7FC1


def note(msg: str) -> None:
    print(f"[gpu] {msg}", flush=True)


def bits(t: torch.Tensor) -> np.ndarray:
    return syn.from_torch_bf16(t)


def dev(b: np.ndarray) -> torch.Tensor:
    return syn.to_torch_bf16(b, DEV)


def guarded_out(m: int, vocab: int):
    """A ``[m, vocab]`` output at the start of a buffer that ends in a guard."""
    flat = dev(np.full(m * vocab + GUARD, GUARD_BITS, np.uint16))
    return flat, flat[: m * vocab].view(m, vocab)


def assert_guard(flat: torch.Tensor, m: int, vocab: int) -> None:
    tail = bits(flat[m * vocab:])
    assert np.all(tail == GUARD_BITS), "store past the sliced output"


def assert_state(hg, sim):
    assert hg.parity == sim.parity
    for p in (0, 1):
        assert np.array_equal(bits(hg.mailbox(p)), sim.mailbox_bf16(p)), p
    assert hg.poll_status() == _lib.HG_OK


def inputs(tp, shard, m, k, frac=0.02):
    s = syn.shard_set("spec", k, rows=m, tp=tp, shard=shard)
    syn.inject_sentinel_words(s, frac, 700 + k)
    return s


TP, SHARD, CAP = 3, 264, 3  # 33 vectors per shard: ragged chunks
V = TP * SHARD
VOCABS = [V, V - 8, V - 1, V - 7, 777, SHARD + 3, SHARD, 530, 9, 8, 1]


@pytest.mark.parametrize("vocab", VOCABS)
def test_fused_gather_slices(vocab):
    note(f"fused gather vocab={vocab} of V={V}")
    hg, sim = HeadGather(TP, SHARD, CAP, device=DEV, vocab=vocab), og.MailboxSim(TP, SHARD, CAP)
    hg.set_poll_limit(1 << 20)
    for n in range(5):
        m = 1 + n % CAP
        s = inputs(TP, SHARD, m, n)
        flat, out = guarded_out(m, vocab)
        got = hg(dev(s), out=out)
        status, want = sim.gather(list(s))
        assert status == og.OK
        assert np.array_equal(bits(got), og.slice_vocab(want, vocab)), n
        assert_guard(flat, m, vocab)
        assert_state(hg, sim)


@pytest.mark.parametrize("vocab", [V - 1, 530, V])
def test_split_push_collect_slices(vocab):
    note(f"split push/collect vocab={vocab}")
    hg, sim = HeadGather(TP, SHARD, CAP, device=DEV, vocab=vocab), og.MailboxSim(TP, SHARD, CAP)
    hg.set_poll_limit(1 << 20)
    for n in range(4):
        m = CAP - n % CAP
        s = inputs(TP, SHARD, m, 40 + n)
        assert hg.push(dev(s)) and sim.push(list(s)) == og.OK
        flat, out = guarded_out(m, vocab)
        hg.collect(m, out=out)
        status, want = sim.collect(m)
        assert status == og.OK and np.array_equal(bits(out), og.slice_vocab(want, vocab)), n
        assert_guard(flat, m, vocab)
        assert_state(hg, sim)


def test_vocab_change_between_calls_and_argument_rules():
    note("vocab changes between calls; argument rules")
    hg, sim = HeadGather(TP, SHARD, CAP, device=DEV), og.MailboxSim(TP, SHARD, CAP)
    hg.set_poll_limit(1 << 20)
    for n, vocab in enumerate([V, 17, V - 3, 264, V]):
        hg.set_vocab(vocab)
        assert _lib.lib().hg_vocab(hg.handle) == vocab
        s = inputs(TP, SHARD, 2, 80 + n)
        got = hg(dev(s))
        assert tuple(got.shape) == (2, vocab)
        status, want = sim.gather(list(s))
        assert status == og.OK and np.array_equal(bits(got), og.slice_vocab(want, vocab))
        assert_state(hg, sim)
    for bad in (0, -1, V + 1):
        with pytest.raises(HgError):
            hg.set_vocab(bad)
    assert hg.vocab == V


def test_declined_calls_return_the_sliced_stock_gather():
    vocab = V - 5
    note(f"declined calls, vocab={vocab}")
    hg = HeadGather(TP, SHARD, CAP, device=DEV, vocab=vocab)
    s = inputs(TP, SHARD, CAP + 1, 90)
    got = hg(dev(s))  # m > cap: declined, stock path, no rewrite
    assert np.array_equal(bits(got), og.slice_vocab(og.stock_concat(list(s)), vocab))
    assert hg.parity == 0
    s1 = inputs(TP, SHARD, 1, 91)
    graph_out = torch.empty((1, vocab), dtype=torch.bfloat16, device=DEV)
    static_in = dev(s1)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):  # host parity: declined under capture
        hg(static_in, out=graph_out)
    g.replay()
    torch.cuda.synchronize()
    assert np.array_equal(bits(graph_out), og.slice_vocab(og.stock_concat(list(s1)), vocab))
    assert hg.parity == 0


@pytest.mark.parametrize("m", [3, 130])
def test_producer_gather_slices(m):
    # 3 rows: the 8 x 1 product; 130 rows: the 4 x 2 product's epilogue push
    tp, shard, hidden = 2, 256, 64
    cap = m + 1
    for vocab in (505, 496, 2 * shard):
        note(f"producer + gather m={m} vocab={vocab}")
        hg, sim = HeadGather(tp, shard, cap, device=DEV, vocab=vocab), og.MailboxSim(tp, shard, cap)
        hg.set_poll_limit(1 << 20)
        x = dev(syn.random_bf16((m, hidden), 0.5, vocab))
        w = dev(syn.random_bf16((tp, shard, hidden), 0.5, vocab + 1))
        shards = torch.empty((tp, m, shard), dtype=torch.bfloat16, device=DEV)
        flat, out = guarded_out(m, vocab)
        hg.gemm_gather(x, w, out=out, shards_out=shards)
        status, want = sim.gather(list(bits(shards)))
        assert status == og.OK and np.array_equal(bits(out), og.slice_vocab(want, vocab))
        assert_guard(flat, m, vocab)
        assert_state(hg, sim)


def test_graph_replays_with_device_parity_and_slice():
    tp, shard, cap, m, vocab = 8, 2048, 4, 4, 8 * 2048 - 11
    note(f"graph of 2 sliced fused gathers, vocab={vocab}")
    hg, sim = HeadGather(tp, shard, cap, device=DEV, vocab=vocab), og.MailboxSim(tp, shard, cap)
    hg.set_poll_limit(1 << 20)
    hg.set_device_parity(True)
    static_in = [dev(inputs(tp, shard, m, 300 + c)) for c in range(2)]
    static_out = [torch.empty((m, vocab), dtype=torch.bfloat16, device=DEV) for _ in range(2)]
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for c in range(2):
            hg(static_in[c], out=static_out[c])
    for rep in range(4):
        sets = [inputs(tp, shard, m, 400 + 10 * rep + c) for c in range(2)]
        for c in range(2):
            static_in[c].copy_(dev(sets[c]))
        g.replay()
        torch.cuda.synchronize()
        for c in range(2):
            status, want = sim.gather(list(sets[c]))
            assert status == og.OK
            assert np.array_equal(bits(static_out[c]), og.slice_vocab(want, vocab)), (rep, c)
        assert_state(hg, sim)


@pytest.mark.parametrize("name,vocab", [("decode", 163837), ("spec", 163832), ("fused", 163833)])
def test_full_size_slices(name, vocab):
    w = syn.WORKLOADS[name]
    note(f"full size {name}: tp={w.tp} V={w.vocab} m={w.rows} vocab={vocab}")
    hg, sim = HeadGather(w.tp, w.shard, w.cap, device=DEV, vocab=vocab), og.MailboxSim(w.tp, w.shard, w.cap)
    hg.set_poll_limit(1 << 22)
    for k in range(3):
        s = syn.shard_set(w, k)
        syn.inject_sentinel_words(s, 0.001, 800 + k)
        flat, out = guarded_out(w.rows, vocab)
        hg(dev(s), out=out)
        status, want = sim.gather(list(s))
        assert status == og.OK and np.array_equal(bits(out), og.slice_vocab(want, vocab)), k
        assert_guard(flat, w.rows, vocab)
    assert_state(hg, sim)
    hg.close()


def test_graph_keeps_its_captured_width_after_set_vocab():
    # a call captured at one width replays at that width after the context's
    # vocabulary changed; eager calls take the new width; the parity keeps
    # alternating across both
    tp, shard, cap, m = 3, 264, 2, 2
    v_cap, v_new = 3 * 264 - 9, 530
    note(f"graph width {v_cap} kept after set_vocab({v_new})")
    hg, sim = HeadGather(tp, shard, cap, device=DEV, vocab=v_cap), og.MailboxSim(tp, shard, cap)
    hg.set_poll_limit(1 << 20)
    hg.set_device_parity(True)
    static_in = dev(inputs(tp, shard, m, 400))
    flat, static_out = guarded_out(m, v_cap)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        hg(static_in, out=static_out)
    hg.set_vocab(v_new)
    for rep in range(3):
        s = inputs(tp, shard, m, 410 + rep)
        static_in.copy_(dev(s))
        g.replay()
        torch.cuda.synchronize()
        status, want = sim.gather(list(s))
        assert status == og.OK
        assert np.array_equal(bits(static_out), og.slice_vocab(want, v_cap)), rep
        assert_guard(flat, m, v_cap)
        e = inputs(tp, shard, 1, 420 + rep)
        got = hg(dev(e))
        status, want = sim.gather(list(e))
        assert status == og.OK and np.array_equal(bits(got), og.slice_vocab(want, v_new)), rep
    assert_state(hg, sim)
