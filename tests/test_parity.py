"""GPU parity: the HIP path through the C ABI against the CPU oracle, bit for
bit -- gathered logits, both mailbox parities and the parity bit -- on the
seeded workloads (tiny, decode, spec, batched, fused-size gather), ragged
geometries, row counts that span one to several tiles per workgroup and both
vector widths, declines, graph capture, the split variant's intermediate
mailbox, partial pushes with a bounded poll, and long random call
sequences."""

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


def make(tp: int, shard: int, cap: int) -> HeadGather:
    hg = HeadGather(tp, shard, cap, device=DEV)
    hg.set_poll_limit(POLL_LIMIT)
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


# (tp, shard, cap): ragged segment tails, one rank of 8 vectors up to 64 ranks,
# and caps large enough for two vectors per lane (above 4 vectors per lane
# slot of the whole chip: 262144 vectors at 256 CUs)
GEOMETRIES = [(2, 8, 3), (3, 24, 3), (8, 8, 2), (5, 520, 3), (8, 2056, 3), (2, 4104, 2),
              (4, 64 * 8 * 8, 2), (64, 16, 2), (8, 2056, 160), (5, 4104, 130)]


@pytest.mark.parametrize("tp,shard,cap", GEOMETRIES)
def test_ragged_geometries(tp, shard, cap):
    note(f"ragged tp={tp} shard={shard} cap={cap}")
    w = syn.WORKLOADS["spec"]
    ms = [1, cap, max(1, cap - 1), cap, 1]
    sets = []
    for i, m in enumerate(ms):
        s = syn.shard_set(w, i, rows=m, tp=tp, shard=shard)
        syn.inject_sentinel_words(s, 0.03, 99 + i)
        sets.append(s)
    for variant in ("fused", "split"):
        hg = make(tp, shard, cap)
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


@pytest.mark.parametrize("m", [1, 2, 5, 31, 33, 127, 128, 129, 200, 256])
def test_fused_grids_from_one_tile_to_several_per_workgroup(m):
    """Row counts from one tile (a single workgroup polling its own pushes) to
    several tiles per workgroup (tiles past four resident workgroups per CU):
    TP=8, S=2048 gives 32 chunks of 64 vectors per row at one vector per lane,
    so m = 200 makes 1600 tiles of four chunks for at most 1024 workgroups."""
    tp, shard, cap = 8, 2048, 256
    note(f"fused grids tp={tp} shard={shard} m={m}")
    hg, sim = make(tp, shard, cap), og.MailboxSim(tp, shard, cap)
    assert hg.fused_grid_limit(m) >= 1
    w = syn.WORKLOADS["spec"]
    sets = [syn.shard_set(w, k, rows=m, tp=tp, shard=shard) for k in range(2)]
    for k, st in enumerate(sets):
        syn.inject_sentinel_words(st, 0.01, 300 + m + k)
    run_lockstep(hg, sim, sets, 3, "fused", mailbox_every=3)
    run_lockstep(hg, sim, sets, 2, "split", mailbox_every=2)


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
    f32_narrow = torch.randn(tp, 2, shard - 5, device=DEV)
    assert torch.equal(hg(f32_narrow), torch.cat(list(f32_narrow), dim=1))
    narrow = dev(syn.shard_set(w, 2, rows=2, tp=tp, shard=shard - 8))
    assert torch.equal(hg(narrow).view(torch.int16), torch.cat(list(narrow), dim=1).view(torch.int16))
    assert_state(hg, sim)
    assert_no_timeout(hg)


def test_stock_gather_kernel():
    note("stock gather kernel")
    w = syn.WORKLOADS["batched"]
    for tp, shard, m in [(1, 8, 3), (8, 20480, 64), (3, 24, 5), (64, 16, 2), (3, 7, 4), (2, 1, 3),
                         (8, 20480, 256)]:
        s = syn.shard_set(w, 0, rows=m, tp=tp, shard=shard)
        out = stock_gather(dev(s), tp)
        assert np.array_equal(bits(out), og.stock_concat(list(s))), (tp, shard, m)


@pytest.mark.parametrize("tp,shard,m,vocab", [(8, 2048, 3, 16000), (8, 2048, 3, 16001),
                                              (3, 24, 5, 1), (3, 24, 5, 72), (3, 7, 4, 20),
                                              (8, 20480, 4, 163000)])
def test_stock_gather_keeps_the_vocabulary(tp, shard, m, vocab):
    """The stock path's padded-vocab slice runs in the library's kernel: the
    first `vocab` columns of the rank-order concatenation, row stride vocab."""
    note(f"stock gather vocab tp={tp} shard={shard} m={m} vocab={vocab}")
    w = syn.WORKLOADS["batched"]
    s = syn.shard_set(w, 1, rows=m, tp=tp, shard=shard)
    out = stock_gather(dev(s), tp, vocab=vocab)
    assert tuple(out.shape) == (m, vocab)
    assert np.array_equal(bits(out), og.slice_vocab(og.stock_concat(list(s)), vocab))


@pytest.mark.parametrize("dtype,width", [(torch.float32, 4), (torch.float32, 12), (torch.int8, 48),
                                         (torch.float64, 2), (torch.float16, 24), (torch.float32, 3),
                                         (torch.int8, 6)])
def test_stock_gather_moves_bytes_of_any_dtype(dtype, width):
    # rows of a multiple of 16 bytes move in 16-byte vectors, other even byte
    # widths element by element, both in the library kernel; both give the
    # rank-order concatenation, byte for byte
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


def test_stock_gather_refuses_odd_byte_rows():
    odd = torch.zeros((2, 3, 5), dtype=torch.int8, device=DEV)
    with pytest.raises(ValueError):
        stock_gather(odd, 2)


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
