"""GPU parity: the HIP path through the C ABI against the CPU oracle, bit for
bit -- gathered logits, both mailbox parities and the parity bit -- on the
seeded workloads (tiny, decode, spec, batched, fused-size gather), ragged
geometries, every launch shape, declines, graph capture, the split variant's
intermediate mailbox, partial pushes with a bounded poll, and long random
call sequences."""

from __future__ import annotations

import numpy as np
import pytest
import torch

from oracle import gather as og
from tp_vocab_logits_amd import _lib
from tp_vocab_logits_amd import synthetic as syn
from tp_vocab_logits_amd.head_gather import HeadGather, HgError, stock_gather

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
POLL_LIMIT = 1 << 20  # a visibility bug then shows as a timeout within seconds


def note(msg: str) -> None:
    print(f"[gpu] {msg}", flush=True)


def bits(t: torch.Tensor) -> np.ndarray:
    return syn.from_torch_bf16(t)


def dev(b: np.ndarray) -> torch.Tensor:
    return syn.to_torch_bf16(b, DEV)


def make(tp: int, shard: int, cap: int, **tuning) -> HeadGather:
    hg = HeadGather(tp, shard, cap, device=DEV)
    hg.set_poll_limit(POLL_LIMIT)
    for knob, value in tuning.items():
        hg.set_tuning(getattr(_lib, "TUNE_" + knob.upper()), value)
    return hg


def assert_state(hg: HeadGather, sim: og.MailboxSim) -> None:
    assert hg.parity == sim.parity
    for p in (0, 1):
        assert np.array_equal(bits(hg.mailbox(p)), sim.mailbox_bf16(p)), f"mailbox parity {p}"


def assert_no_timeout(hg: HeadGather) -> None:
    assert hg.poll_status() == _lib.HG_OK


def run_lockstep(hg, sim, sets, calls, variant, mailbox_every=1):
    dev_sets = [dev(s) for s in sets]
    for n in range(calls):
        k = n % len(sets)
        m = sets[k].shape[1]
        if variant == "fused":
            out = hg(dev_sets[k])
        else:
            assert hg.push(dev_sets[k])
            out = hg.collect(m)
        status, want = sim.gather(list(sets[k]))
        assert status == og.OK
        assert np.array_equal(bits(out), want), f"call {n}"
        if mailbox_every and n % mailbox_every == 0:
            assert_state(hg, sim)
    assert_no_timeout(hg)
    assert_state(hg, sim)


@pytest.mark.parametrize("variant", ["fused", "split"])
def test_tiny_four_calls(variant):
    w = syn.WORKLOADS["tiny"]
    note(f"tiny tp={w.tp} V={w.vocab} m={w.rows} cap={w.cap} {variant}")
    sets = [syn.shard_set(w, k) for k in range(w.pool)]
    hg, sim = make(w.tp, w.shard, w.cap), og.MailboxSim(w.tp, w.shard, w.cap)
    assert_state(hg, sim)
    run_lockstep(hg, sim, sets, w.calls, variant)


@pytest.mark.parametrize("tp,shard,cap,m", [(2, 2048, 1, 1), (3, 24, 3, 2), (8, 520, 4, 3)])
def test_split_intermediate_mailbox(tp, shard, cap, m):
    note(f"split intermediate tp={tp} shard={shard} cap={cap} m={m}")
    w = syn.WORKLOADS["decode"]
    hg, sim = make(tp, shard, cap), og.MailboxSim(tp, shard, cap)
    for k in range(3):
        s = syn.shard_set(w, k, rows=m, tp=tp, shard=shard)
        syn.inject_sentinel_words(s, 0.05, 77 + k)
        assert hg.push(dev(s)) and sim.push(list(s)) == og.OK
        assert_state(hg, sim)  # rows 0..m-1 of the current parity hold the rewritten words
        out = hg.collect(m)
        status, want = sim.collect(m)
        assert status == og.OK and np.array_equal(bits(out), want)
        assert_state(hg, sim)
    assert_no_timeout(hg)


GEOMETRIES = [(2, 8, 3), (3, 24, 3), (8, 8, 2), (5, 520, 3), (8, 2056, 3), (2, 4104, 2),
              (4, 64 * 8 * 8, 2), (64, 16, 2)]


# (push, poll, re-arm) flavours of the kernels
MODES = [(0, 0, 0), (2, 1, 1), (3, 2, 0), (1, 1, 1)]


@pytest.mark.parametrize("modes", MODES, ids=lambda m: "push%d-poll%d-rearm%d" % m)
@pytest.mark.parametrize("vpt", [1, 2, 4, 8])
@pytest.mark.parametrize("tp,shard,cap", GEOMETRIES)
def test_ragged_geometries_all_vpt(tp, shard, cap, vpt, modes):
    note(f"ragged tp={tp} shard={shard} cap={cap} vpt={vpt} modes={modes}")
    w = syn.WORKLOADS["spec"]
    ms = [1, cap, max(1, cap - 1), cap, 1]
    sets = []
    for i, m in enumerate(ms):
        s = syn.shard_set(w, i, rows=m, tp=tp, shard=shard)
        syn.inject_sentinel_words(s, 0.03, 99 + i)
        sets.append(s)
    for variant in ("fused", "split"):
        hg = make(tp, shard, cap, fused_vpt=vpt, split_vpt=vpt, push_mode=modes[0],
                  poll_mode=modes[1], rearm_mode=modes[2])
        sim = og.MailboxSim(tp, shard, cap)
        for n, s in enumerate(sets):
            if variant == "fused":
                out = hg(dev(s))
            else:
                assert hg.push(dev(s))
                out = hg.collect(s.shape[1])
            status, want = sim.gather(list(s))
            assert status == og.OK and np.array_equal(bits(out), want), (variant, n)
            assert_state(hg, sim)
        assert_no_timeout(hg)


@pytest.mark.parametrize("block", [64, 256, 1024])
@pytest.mark.parametrize("push,poll", [(p, q) for p in range(4) for q in range(3)])
@pytest.mark.parametrize("grid,skew", [(0, 1), (1, 1), (3, 1), (7, 2), (0, 3), (7, 7), (5, 100000),
                                       (0, 0)])
def test_fused_launch_shapes(block, push, poll, grid, skew):
    """Every poll ownership: grid 1 (one workgroup polls its own pushes), small
    grids with many tiles per workgroup, skews that cross workgroups and XCDs
    (a skew that is a multiple of the grid makes every workgroup poll its own
    pushes), and both ways of publishing the push."""
    note(f"fused shapes block={block} push={push} poll={poll} grid={grid} skew={skew}")
    tp, shard, cap = 8, 2048, 4
    hg = make(tp, shard, cap, fused_block=block, push_mode=push, poll_mode=poll, fused_grid=grid,
              poll_skew=skew, rearm_mode=(push + poll) % 2)
    sim = og.MailboxSim(tp, shard, cap)
    w = syn.WORKLOADS["spec"]
    sets = [syn.shard_set(w, k, rows=m, tp=tp, shard=shard) for k, m in enumerate([4, 1, 3, 4])]
    run_lockstep(hg, sim, sets, 6, "fused")


@pytest.mark.parametrize("block", [64, 128, 512, 1024])
@pytest.mark.parametrize("vpt", [1, 2, 4])
def test_split_launch_shapes(block, vpt):
    """The split variant's push and collect kernels at every block size and
    vectors per lane, on a ragged geometry (36 vectors per shard row)."""
    note(f"split shapes block={block} vpt={vpt}")
    tp, shard, cap = 3, 288, 4
    hg = make(tp, shard, cap, split_block=block, split_vpt=vpt)
    sim = og.MailboxSim(tp, shard, cap)
    w = syn.WORKLOADS["spec"]
    sets = [syn.shard_set(w, k, rows=m, tp=tp, shard=shard) for k, m in enumerate([4, 1, 3, 2])]
    for s in sets:
        syn.inject_sentinel_words(s, 0.05, 11 + s.shape[1])
    run_lockstep(hg, sim, sets, 6, "split")


def test_decode_1000_back_to_back():
    w = syn.WORKLOADS["decode"]
    note(f"decode tp={w.tp} V={w.vocab} m={w.rows} cap={w.cap} calls={w.calls}")
    sets = [syn.shard_set(w, k) for k in range(w.pool)]
    want = [dev(og.gather_definition(list(s))) for s in sets]
    dsets = [dev(s) for s in sets]
    hg = make(w.tp, w.shard, w.cap)
    outs = torch.empty((w.calls, w.rows, w.vocab), dtype=torch.bfloat16, device=DEV)
    for n in range(w.calls):
        hg(dsets[n % w.pool], out=outs[n])
    torch.cuda.synchronize()
    for n in range(w.calls):
        assert torch.equal(outs[n].view(torch.int16), want[n % w.pool].view(torch.int16)), n
    assert hg.parity == w.calls % 2
    sim = og.MailboxSim(w.tp, w.shard, w.cap)
    sim.parity = w.calls % 2
    assert_state(hg, sim)
    assert_no_timeout(hg)


def test_spec_1000_calls_mailbox_after_each():
    w = syn.WORKLOADS["spec"]
    note(f"spec tp={w.tp} V={w.vocab} m={w.rows} cap={w.cap} calls={w.calls}")
    sets = [syn.shard_set(w, k) for k in range(w.pool)]
    want = [dev(og.gather_definition(list(s))) for s in sets]
    dsets = [dev(s) for s in sets]
    hg = make(w.tp, w.shard, w.cap)
    armed = torch.full((w.cap, w.vocab // 2), og.SENT_WORD - (1 << 32), dtype=torch.int32, device=DEV)
    for n in range(w.calls):
        p = hg.parity
        assert p == n % 2
        out = hg(dsets[n % w.pool])
        assert torch.equal(out.view(torch.int16), want[n % w.pool].view(torch.int16)), n
        for q in (0, 1):
            assert torch.equal(hg.mailbox(q).view(torch.int32), armed), (n, q)
    assert hg.parity == 0
    assert_no_timeout(hg)


@pytest.mark.parametrize("variant", ["fused", "split"])
def test_batched_special_rows(variant):
    w = syn.WORKLOADS["batched"]
    note(f"batched tp={w.tp} V={w.vocab} m={w.rows} cap={w.cap} {variant}")
    sets = [syn.shard_set(w, k) for k in range(w.pool)]
    hg, sim = make(w.tp, w.shard, w.cap), og.MailboxSim(w.tp, w.shard, w.cap)
    run_lockstep(hg, sim, sets, 2 * w.pool + 1, variant, mailbox_every=3)
    # the alternating (+0,-0) row arrives as all +0; the other signed-zero rows unchanged
    out = hg(dev(sets[0])) if variant == "fused" else (hg.push(dev(sets[0])), hg.collect(w.rows))[1]
    b = bits(out)
    assert np.all(b[33] == 0) and np.all(b[1] == 0) and np.all(b[17] == 0x8000)
    assert np.all(b[49, 0::2] == 0x8000) and np.all(b[49, 1::2] == 0)


def test_fused_size_gather_m256():
    w = syn.WORKLOADS["fused"]
    note(f"m=256 gather tp={w.tp} V={w.vocab} cap={w.cap}")
    sets = [syn.shard_set(w, k) for k in range(2)]
    for s in sets:
        syn.inject_sentinel_words(s, 0.001, 4242)
    hg, sim = make(w.tp, w.shard, w.cap), og.MailboxSim(w.tp, w.shard, w.cap)
    run_lockstep(hg, sim, sets, 3, "fused", mailbox_every=2)
    run_lockstep(hg, sim, sets, 2, "split", mailbox_every=0)


def test_declines_take_the_stock_path():
    tp, shard, cap = 4, 64, 3
    note(f"declines tp={tp} shard={shard} cap={cap}")
    hg, sim = make(tp, shard, cap), og.MailboxSim(tp, shard, cap)
    w = syn.WORKLOADS["tiny"]
    s1 = syn.shard_set(w, 0, rows=1, tp=tp, shard=shard)
    syn.inject_sentinel_words(s1, 0.2, 5)
    hg(dev(s1)), sim.gather(list(s1))  # parity 1 now
    for m in (0, cap + 1, cap + 5):
        s = syn.shard_set(w, 1, rows=m, tp=tp, shard=shard)
        if m:
            syn.inject_sentinel_words(s, 0.2, 6)
        out = hg(dev(s))
        status, want = sim.gather(list(s))
        assert status == og.DECLINE
        assert np.array_equal(bits(out), want)  # the stock result keeps the sentinel words
        assert_state(hg, sim)
    # wrong dtype / width also take the stock path
    f32 = torch.randn(tp, 2, shard, device=DEV)
    assert torch.equal(hg(f32), torch.cat(list(f32), dim=1))
    narrow = dev(syn.shard_set(w, 2, rows=2, tp=tp, shard=shard - 8))
    assert torch.equal(hg(narrow).view(torch.int16), torch.cat(list(narrow), dim=1).view(torch.int16))
    assert_state(hg, sim)
    assert_no_timeout(hg)


def test_stock_gather_kernel():
    note("stock gather kernel")
    w = syn.WORKLOADS["batched"]
    for tp, shard, m in [(1, 8, 3), (8, 20480, 64), (3, 24, 5), (64, 16, 2)]:
        s = syn.shard_set(w, 0, rows=m, tp=tp, shard=shard)
        out = stock_gather(dev(s), tp)
        assert np.array_equal(bits(out), og.stock_concat(list(s)))


@pytest.mark.parametrize("dtype,width", [(torch.float32, 4), (torch.float32, 12), (torch.int8, 48),
                                         (torch.float64, 2), (torch.float16, 24), (torch.float32, 3)])
def test_stock_gather_moves_bytes_of_any_dtype(dtype, width):
    # rows of a multiple of 16 bytes run in the library kernel, the rest in torch.cat;
    # both give the rank-order concatenation, byte for byte
    note(f"stock gather dtype={dtype} width={width}")
    tp, m = 3, 5
    g = torch.Generator().manual_seed(width)
    raw = torch.randint(0, 256, (tp, m, width * torch.empty((), dtype=dtype).element_size()),
                        dtype=torch.uint8, generator=g)
    shards = raw.view(dtype).to(DEV)
    out = stock_gather(shards, tp)
    want = np.concatenate([raw[r].numpy() for r in range(tp)], axis=1)
    assert np.array_equal(out.cpu().view(torch.uint8).numpy(), want)
    with pytest.raises(ValueError):
        stock_gather(shards.cpu(), tp)


def test_graph_capture_declines_to_stock():
    tp, shard, cap = 2, 2048, 1
    note("graph capture decline")
    hg, sim = make(tp, shard, cap), og.MailboxSim(tp, shard, cap)
    w = syn.WORKLOADS["tiny"]
    static_in = dev(syn.shard_set(w, 0))
    side = torch.cuda.Stream(device=DEV)
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        stock_gather(static_in, tp)  # warm-up outside capture
    torch.cuda.current_stream().wait_stream(side)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        static_out = hg(static_in)
    assert hg.parity == 0
    for k in range(1, 4):
        s = syn.shard_set(w, k)
        static_in.copy_(dev(s))
        graph.replay()
        torch.cuda.synchronize()
        assert np.array_equal(bits(static_out), og.stock_concat(list(s)))
        # eager work between replays, served by the fused kernel
        out = hg(dev(s))
        status, want = sim.gather(list(s))
        assert status == og.OK and np.array_equal(bits(out), want)
    assert_state(hg, sim)
    assert_no_timeout(hg)


def test_split_state_errors():
    tp, shard, cap = 2, 64, 2
    note("split state errors")
    hg = make(tp, shard, cap)
    s = dev(syn.shard_set("tiny", 0, rows=1, tp=tp, shard=shard))
    with pytest.raises(HgError):
        hg.collect(1)
    assert hg.push(s)
    with pytest.raises(HgError):
        hg.push(s)
    with pytest.raises(HgError):
        hg(s)
    with pytest.raises(HgError):
        hg.collect(2)
    hg.collect(1)
    assert hg.parity == 1
    assert hg.push(s)
    hg.arm()
    assert hg.parity == 0
    with pytest.raises(HgError):
        hg.collect(1)
    assert_no_timeout(hg)


def test_partial_push_and_bounded_poll():
    tp, shard, cap, m = 8, 2048, 2, 2
    note("partial push + bounded poll timeout")
    hg, sim = make(tp, shard, cap), og.MailboxSim(tp, shard, cap)
    w = syn.WORKLOADS["spec"]
    s = syn.shard_set(w, 0, rows=m, tp=tp, shard=shard)
    d = dev(s)
    # ranks arrive in three separate pushes, in a scrambled order
    for grp in ([5, 0], [7, 2, 3], [1, 4, 6]):
        assert hg.push_ranks(d, grp)
        assert sim.push_ranks(list(s), grp) == og.OK
        assert_state(hg, sim)
    out = hg.collect(m)
    status, want = sim.collect(m)
    assert status == og.OK and np.array_equal(bits(out), want)
    assert_no_timeout(hg)
    # rank 3 never pushes: the bounded poll gives up, the call still completes
    hg.set_poll_limit(64)
    missing = 3
    ranks = [r for r in range(tp) if r != missing]
    assert hg.push_ranks(d, ranks) and sim.push_ranks(list(s), ranks) == og.OK
    out = hg.collect(m)
    status, want = sim.collect(m)
    assert status == og.ETIMEOUT
    assert hg.poll_status() == _lib.HG_ETIMEOUT
    assert np.array_equal(bits(out), want)
    assert_state(hg, sim)
    # and the context keeps working
    hg.set_poll_limit(POLL_LIMIT)
    run_lockstep(hg, sim, [s], 3, "fused")


def test_random_call_sequence_10k():
    tp, shard, cap = 8, 256, 8
    note(f"random sequence 10k tp={tp} shard={shard} cap={cap}")
    rng = np.random.default_rng(2024)
    w = syn.WORKLOADS["spec"]
    pool = {m: [syn.shard_set(w, k, rows=m, tp=tp, shard=shard) for k in range(3)]
            for m in range(0, cap + 2)}
    for m, sets in pool.items():
        for k, s in enumerate(sets):
            if m:
                syn.inject_sentinel_words(s, 0.01, 1000 * m + k)
    dpool = {m: [dev(s) for s in sets] for m, sets in pool.items()}
    hg, sim = make(tp, shard, cap), og.MailboxSim(tp, shard, cap)
    for n in range(10_000):
        m = int(rng.integers(0, cap + 2))
        k = int(rng.integers(0, 3))
        variant = "fused" if rng.random() < 0.7 else "split"
        if variant == "fused" or not (1 <= m <= cap):
            out = hg(dpool[m][k])
            status, want = sim.gather(list(pool[m][k]))
        else:
            assert hg.push(dpool[m][k]) and sim.push(list(pool[m][k])) == og.OK
            out = hg.collect(m)
            status, want = sim.collect(m)
        assert np.array_equal(bits(out), want), n
        assert hg.parity == sim.parity
        if n % 1000 == 0:
            assert_state(hg, sim)
    assert_state(hg, sim)
    assert_no_timeout(hg)
