"""Pins of the CPU oracle against facts that do not come from the oracle.

Each ``check_*`` function raises ``AssertionError`` when the oracle modules it
is given disagree with something the pages or mathematics fix. They take the
modules as arguments so ``test_oracle_mutants.py`` can run them against
deliberately broken copies of the oracle (a plausible mistake must trip at
least one check), while ``test_oracle_pins.py`` runs them against the real one.

Independent sources used here, never the oracle itself:

* torch's own BF16 conversion and raw memory reinterpretation (the sentinel
  bit pattern, the 32-bit packing order, float values for -0 == +0);
* numpy's ``concatenate`` / ``stack`` for the rank-order and NCCL layouts;
* the hand-worked fixtures in ``tests/golden/`` (derived by hand from the
  page's rules, see each file's header);
* exhaustive enumeration on tiny sizes, closed forms and invariants.
"""

from __future__ import annotations

import itertools
import os

import numpy as np
import torch

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ---------------------------------------------------------------------------
# independent helpers
# ---------------------------------------------------------------------------

def torch_sentinel() -> int:
    """The BF16 pair (+0, -0) as torch lays it out in memory, read as int32."""
    t = torch.tensor([0.0, -0.0], dtype=torch.bfloat16)
    return int(t.view(torch.int32).item()) & 0xFFFFFFFF


def torch_words(elems: np.ndarray) -> np.ndarray:
    """32-bit words of contiguous BF16 rows, by reinterpreting memory in torch."""
    t = torch.from_numpy(np.ascontiguousarray(elems, dtype=np.uint16).view(np.int16))
    return t.view(torch.int32).numpy().view(np.uint32)


def torch_floats(elems: np.ndarray) -> np.ndarray:
    """BF16 bit patterns -> float32 values through torch's BF16 type."""
    t = torch.from_numpy(np.ascontiguousarray(elems, dtype=np.uint16).view(np.int16))
    return t.view(torch.bfloat16).to(torch.float32).numpy()


def rand_bits(rng: np.random.Generator, shape) -> np.ndarray:
    """Finite BF16 patterns from N(0, 1) values (no exact zeros in practice)."""
    v = torch.from_numpy(rng.standard_normal(size=shape).astype(np.float32))
    return v.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def force_pairs(bits: np.ndarray, rng: np.random.Generator, count: int) -> None:
    """Force ``count`` random aligned element pairs of ``[tp, m, s]`` to (+0, -0)."""
    flat = bits.reshape(-1)
    pos = rng.choice(flat.size // 2, size=count, replace=False)
    flat[2 * pos] = 0x0000
    flat[2 * pos + 1] = 0x8000


def read_golden(name: str) -> dict:
    rows: dict = {}
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if not line:
                continue
            key, *rest = line.split()
            rows.setdefault(key, []).append(rest)
    return rows


# ---------------------------------------------------------------------------
# gather pins
# ---------------------------------------------------------------------------

def check_sentinel_constant(g) -> None:
    sent = torch_sentinel()
    assert sent == 0x80000000
    assert g.SENT_WORD == sent
    assert int(g.pack_words(np.array([0x0000, 0x8000], np.uint16))[0]) == sent
    # the reversed pair (-0, +0) and the pair (-0, -0) are not the sentinel
    assert int(g.pack_words(np.array([0x8000, 0x0000], np.uint16))[0]) != sent
    assert int(g.pack_words(np.array([0x8000, 0x8000], np.uint16))[0]) != sent


def check_packing(g) -> None:
    rng = np.random.default_rng(11)
    elems = rng.integers(0, 1 << 16, size=(5, 64), dtype=np.uint16)
    assert np.array_equal(g.pack_words(elems), torch_words(elems))
    assert np.array_equal(g.unpack_words(torch_words(elems)), elems)


def check_golden_gather(g) -> None:
    gd = read_golden("gather_tp2_s8_m2.txt")
    tp, shard, m = int(gd["tp"][0][0]), int(gd["width"][0][0]), int(gd["rows"][0][0])
    shards = np.zeros((tp, m, shard), np.uint16)
    for r, row, *vals in gd["shard"]:
        shards[int(r), int(row)] = [int(v, 16) for v in vals]
    want = np.zeros((m, tp * shard), np.uint16)
    for row, *vals in gd["out"]:
        want[int(row)] = [int(v, 16) for v in vals]
    assert np.array_equal(g.gather_definition(list(shards)), want)
    sim = g.MailboxSim(tp, shard, m)
    assert sim.push(list(shards)) == g.OK
    # after the push, parity 0 rows 0..m-1 hold exactly the rewritten output words
    assert np.array_equal(sim.box[0, :m], torch_words(want))
    status, out = sim.collect(m)
    assert status == g.OK and np.array_equal(out, want)
    assert np.all(sim.box == torch_sentinel())


def check_layout_nccl(g) -> None:
    rng = np.random.default_rng(12)
    for tp, m, s in [(2, 1, 8), (3, 5, 16), (8, 4, 24), (4, 2, 40)]:
        shards = rand_bits(rng, (tp, m, s))
        assert not np.any(torch_words(shards) == torch_sentinel())
        # NCCL's all-gather fills [TP, M, S]; the copy to [M, V] puts rank r at columns r*S
        nccl = np.stack(list(shards)).transpose(1, 0, 2).reshape(m, tp * s)
        assert np.array_equal(g.gather_definition(list(shards)), nccl)
        assert np.array_equal(g.stock_concat(list(shards)), nccl)
    # element-by-element brute force on a tiny case
    shards = rand_bits(rng, (3, 2, 8))
    out = g.gather_definition(list(shards))
    for r in range(3):
        for row in range(2):
            for j in range(8):
                assert out[row, r * 8 + j] == shards[r, row, j]


def check_value_equivalence_and_xor(g) -> None:
    rng = np.random.default_rng(13)
    sent = torch_sentinel()
    for tp, m, s, forced in [(2, 3, 16, 10), (8, 4, 32, 100), (4, 1, 8, 16)]:
        shards = rand_bits(rng, (tp, m, s))
        force_pairs(shards, rng, forced)
        cat = np.concatenate(list(shards), axis=1)
        out = g.gather_definition(list(shards))
        # same values to a sampler: -0 == +0, everything else identical
        assert np.array_equal(torch_floats(out), torch_floats(cat))
        diff = torch_words(out) ^ torch_words(cat)
        at_sent = torch_words(cat) == sent
        assert int(at_sent.sum()) >= forced
        assert np.all((diff != 0) == at_sent)
        assert np.all(diff[at_sent] == sent)
        # on sentinel-free input the output is the concatenation, bit for bit
        clean = rand_bits(rng, (tp, m, s))
        assert np.array_equal(g.gather_definition(list(clean)), np.concatenate(list(clean), axis=1))


def check_exhaustive_tiny(g) -> None:
    """TP=2, S=8, one row: every assignment of the 8 words over the alphabet
    {(+0,+0), (+0,-0), (-0,-0), (-0,+0)} -- 4^8 = 65536 cases, one per row."""
    alphabet = np.array([[0x0000, 0x0000], [0x0000, 0x8000], [0x8000, 0x8000], [0x8000, 0x0000]],
                        np.uint16)
    idx = np.indices((4,) * 8).reshape(8, -1).T               # [65536, 8] word choices
    rows = alphabet[idx].reshape(-1, 16)                      # [65536, 16] elements
    shards = [rows[:, :8].copy(), rows[:, 8:].copy()]
    out = g.gather_definition(shards)
    # word choice 1 is the only one that changes, and it becomes (+0, +0)
    want = alphabet[np.where(idx == 1, 0, idx)].reshape(-1, 16)
    assert np.array_equal(out, want)
    sim = g.MailboxSim(2, 8, rows.shape[0])
    status, got = sim.gather(shards)
    assert status == g.OK and np.array_equal(got, want)


def check_protocol(g) -> None:
    """Randomised multi-call sequences through the simulator: served calls give
    the definition, declines give the stock concat and keep the parity, the
    mailbox is all-sentinel after every call, parity = served calls mod 2, and
    the split push leaves exactly rows 0..m-1 of the current parity filled."""
    rng = np.random.default_rng(14)
    sent = torch_sentinel()
    for tp, s, cap in [(2, 8, 1), (3, 16, 2), (4, 24, 3), (8, 8, 3), (2, 16, 2)]:
        sim = g.MailboxSim(tp, s, cap)
        served = 0
        for _ in range(24):
            m = int(rng.integers(1 if cap == 1 else 0, cap + 2))
            shards = rand_bits(rng, (tp, m, s)) if m > 0 else np.zeros((tp, 0, s), np.uint16)
            if m > 0:
                force_pairs(shards, rng, min(3, tp * m * s // 2))
            stock = np.concatenate(list(shards), axis=1)
            ok = 1 <= m <= cap
            if rng.random() < 0.5:
                status, out = sim.gather(list(shards))
            else:
                status = sim.push(list(shards))
                if status == g.OK:
                    box = sim.box.copy()
                    words = torch_words(g.gather_definition(list(shards)))
                    assert np.array_equal(box[served % 2, :m], words)
                    assert np.all(box[served % 2, m:] == sent)
                    assert np.all(box[1 - served % 2] == sent)
                    status, out = sim.collect(m)
                else:
                    out = stock
            if ok:
                assert status == g.OK
                assert np.array_equal(out, g.gather_definition(list(shards)))
                served += 1
            else:
                assert status == g.DECLINE
                assert np.array_equal(out, stock)
            assert sim.parity == served % 2
            assert np.all(sim.box == sent)
        # a capturing stream declines without touching the state
        if cap >= 1:
            shards = rand_bits(rng, (tp, 1, s))
            p = sim.parity
            status, out = sim.gather(list(shards), capturing=True)
            assert status == g.DECLINE and sim.parity == p
            assert np.array_equal(out, np.concatenate(list(shards), axis=1))
        # split-variant state errors
        shards = rand_bits(rng, (tp, 1, s))
        assert sim.collect(1)[0] == g.ESTATE
        assert sim.push(list(shards)) == g.OK
        assert sim.push(list(shards)) == g.ESTATE
        assert sim.gather(list(shards))[0] == g.ESTATE
        if cap >= 2:
            assert sim.collect(2)[0] == g.ESTATE
        p = sim.parity
        assert sim.collect(1)[0] == g.OK and sim.parity == 1 - p
        # arm resets parity and clears a pending push
        assert sim.push(list(shards)) == g.OK
        sim.arm()
        assert sim.parity == 0 and sim.pending is None and np.all(sim.box == sent)


def check_partial_push(g) -> None:
    """Ranks pushing separately: disjoint rank sets accumulate into one call;
    a collect with a rank missing gives up (ETIMEOUT) with that rank's columns
    still the sentinel, and re-arms and flips like any call."""
    rng = np.random.default_rng(15)
    sent = torch_sentinel()
    for tp, s, cap, m in [(2, 8, 1, 1), (4, 16, 3, 2), (8, 24, 2, 2), (3, 8, 4, 4)]:
        sim = g.MailboxSim(tp, s, cap)
        shards = rand_bits(rng, (tp, m, s))
        force_pairs(shards, rng, min(4, tp * m * s // 2))
        want = g.gather_definition(list(shards))
        # all ranks, in a shuffled order of disjoint groups
        order = rng.permutation(tp)
        groups = np.array_split(order, min(3, tp))
        for grp in groups:
            assert sim.push_ranks(list(shards), [int(r) for r in grp]) == g.OK
        assert sim.push_ranks(list(shards), [int(order[0])]) == g.ESTATE  # rank pushes twice
        status, out = sim.collect(m)
        assert status == g.OK and np.array_equal(out, want) and sim.parity == 1
        assert np.all(sim.box == sent)
        # one rank missing: the poll gives up
        missing = int(rng.integers(0, tp))
        assert sim.push_ranks(list(shards), [r for r in range(tp) if r != missing]) == g.OK
        status, out = sim.collect(m)
        assert status == g.ETIMEOUT and sim.parity == 0
        cols = slice(missing * s, (missing + 1) * s)
        assert np.all(torch_words(np.ascontiguousarray(out[:, cols])) == sent)
        keep = np.ones(tp * s, bool)
        keep[cols] = False
        assert np.array_equal(out[:, keep], want[:, keep])
        assert np.all(sim.box == sent)
        # a second push with another row count joins no pending call
        if cap >= 2:
            assert sim.push_ranks(list(shards[:, :1]), [0]) == g.OK
            assert sim.push_ranks(list(shards[:, :2]), [1]) == g.ESTATE
            sim.arm()


def check_create_rules(g) -> None:
    for shard in range(0, 65):
        assert g.create_ok(2, shard, 1) == (shard >= 8 and shard % 8 == 0), shard
    for tp in range(0, 5):
        assert g.create_ok(tp, 8, 1) == (tp >= 2)
    assert not g.create_ok(2, 8, 0)
    assert g.create_ok(8, 20480, 256)


def check_vocab_slice(g) -> None:
    """The padded-vocab slice against the hand-worked golden output: its first
    columns in order, nothing reordered, the full width an exact copy."""
    gd = read_golden("gather_tp2_s8_m2.txt")
    tp, shard, m = int(gd["tp"][0][0]), int(gd["width"][0][0]), int(gd["rows"][0][0])
    want = np.zeros((m, tp * shard), np.uint16)
    for row, *vals in gd["out"]:
        want[int(row)] = [int(v, 16) for v in vals]
    for vocab in (1, 3, 8, 9, 15, tp * shard):
        got = g.slice_vocab(want, vocab)
        assert got.shape == (m, vocab)
        for i in range(m):
            for j in range(vocab):
                assert got[i, j] == want[i, j], (vocab, i, j)
    for bad in (0, tp * shard + 1):
        try:
            g.slice_vocab(want, bad)
        except ValueError:
            continue
        raise AssertionError(f"vocab {bad} accepted")


# The call kinds of the exhaustive sequences: (name, rows, how). `cap` is 2.
SEQ_OPS = [("gather", 1, "fused"), ("gather", 2, "fused"), ("decline", 0, "fused"),
           ("decline", 3, "fused"), ("decline", 1, "capture"), ("split", 1, "split"),
           ("split", 2, "split"), ("split", 1, "ranks"), ("arm", 0, "arm")]


def check_protocol_sequences(g) -> None:
    """Every sequence of three calls from SEQ_OPS on TP=2, S=8, cap=2, each on
    fresh random data with forced sentinel pairs: a served call gives the
    definition, a declined one the unrewritten concat; the parity is the
    number of served calls since the last arm, mod 2; after a push exactly
    rows 0..m-1 of the current parity hold the rewritten words; after every
    call the whole mailbox is the sentinel again."""
    tp, s, cap = 2, 8, 2
    sent = torch_sentinel()
    rng = np.random.default_rng(31)
    for seq in itertools.product(range(len(SEQ_OPS)), repeat=3):
        sim = g.MailboxSim(tp, s, cap)
        served = 0
        for k in seq:
            kind, m, how = SEQ_OPS[k]
            if how == "arm":
                sim.arm()
                served = 0
            else:
                shards = rand_bits(rng, (tp, m, s))
                if m > 0:
                    force_pairs(shards, rng, min(2, tp * m * s // 2))
                want = g.gather_definition(list(shards)) if m > 0 else None
                if how == "fused":
                    status, out = sim.gather(list(shards))
                elif how == "capture":
                    status, out = sim.gather(list(shards), capturing=True)
                else:
                    if how == "split":
                        assert sim.push(list(shards)) == g.OK
                    else:
                        assert sim.push_ranks(list(shards), [1]) == g.OK
                        assert sim.push_ranks(list(shards), [0]) == g.OK
                    box = sim.box.copy()
                    assert np.array_equal(box[served % 2, :m], torch_words(want))
                    assert np.all(box[served % 2, m:] == sent)
                    assert np.all(box[1 - served % 2] == sent)
                    status, out = sim.collect(m)
                if kind == "decline":
                    assert status == g.DECLINE, seq
                    assert np.array_equal(out, np.concatenate(list(shards), axis=1)), seq
                else:
                    assert status == g.OK, seq
                    assert np.array_equal(out, want), seq
                    served += 1
            assert sim.parity == served % 2, seq
            assert np.all(sim.box == sent), seq


GATHER_CHECKS = [check_sentinel_constant, check_packing, check_golden_gather, check_layout_nccl,
                 check_value_equivalence_and_xor, check_exhaustive_tiny, check_protocol,
                 check_protocol_sequences, check_partial_push, check_create_rules,
                 check_vocab_slice]


# ---------------------------------------------------------------------------
# lm_head product pins
# ---------------------------------------------------------------------------

def check_gemm_golden(gm) -> None:
    gd = read_golden("lm_head_h3_s4_m2.txt")
    x = np.array([[int(v, 16) for v in r[1:]] for r in gd["x"]], np.uint16)
    w = np.array([[int(v, 16) for v in r[1:]] for r in gd["w"]], np.uint16)
    want = np.array([[float(v) for v in r[1:]] for r in gd["out"]])
    assert np.array_equal(gm.lm_head_shard(x, w), want)
    for m in range(2):
        for s in range(4):
            assert gm.lm_head_entry(x, w, m, s) == want[m, s]


def check_gemm_one_hot(gm) -> None:
    """X rows one-hot (1.0 at column j_i): row i of the shard is column j_i of
    W_r. Non-square sizes expose a transposed operand."""
    rng = np.random.default_rng(21)
    m, h, s = 5, 7, 3
    w = rand_bits(rng, (s, h))
    cols = [3, 0, 6, 3, 1]
    x = np.zeros((m, h), np.uint16)
    for i, j in enumerate(cols):
        x[i, j] = 0x3F80  # BF16 1.0
    out = gm.lm_head_shard(x, w)
    wf = torch_floats(w).astype(np.float64)
    for i, j in enumerate(cols):
        assert np.array_equal(out[i], wf[:, j])


def check_gemm_closed_forms(gm) -> None:
    h = 64
    # X = 1, W[s, h] = (s+1)/8  ->  out[m, s] = h (s+1) / 8
    x = np.full((2, h), 0x3F80, np.uint16)
    w = np.stack([np.full(h, torch.tensor((s + 1) / 8, dtype=torch.bfloat16).view(torch.int16).item(),
                          np.int16).view(np.uint16) for s in range(5)])
    out = gm.lm_head_shard(x, w)
    assert np.array_equal(out, np.tile(np.array([h * (s + 1) / 8 for s in range(5)]), (2, 1)))
    # X[m, k] = -(m+1), W[s, k] = (-1)^k (s+1): an alternating sum over even h is 0
    xm = torch.tensor([[-(m + 1.0)] * h for m in range(3)], dtype=torch.bfloat16)
    ws = torch.tensor([[(s + 1.0) * (-1) ** k for k in range(h)] for s in range(4)], dtype=torch.bfloat16)
    xb = xm.view(torch.int16).numpy().view(np.uint16)
    wb = ws.view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(gm.lm_head_shard(xb, wb), np.zeros((3, 4)))
    # same with odd h: the sum is the first term, -(m+1)(s+1)
    out = gm.lm_head_shard(xb[:, : h - 1], wb[:, : h - 1])
    assert np.array_equal(out, -np.outer(np.arange(1, 4), np.arange(1, 5)).astype(np.float64))


def check_gemm_library(gm) -> None:
    """Random tiny product against torch's float64 matmul of torch-converted inputs."""
    rng = np.random.default_rng(22)
    x, w = rand_bits(rng, (6, 40)), rand_bits(rng, (9, 40))
    ref = (torch.from_numpy(torch_floats(x)).double() @ torch.from_numpy(torch_floats(w)).double().T).numpy()
    assert np.allclose(gm.lm_head_shard(x, w), ref, rtol=1e-12, atol=1e-12)
    for m, s in [(0, 0), (5, 8), (3, 4)]:
        assert abs(gm.lm_head_entry(x, w, m, s) - ref[m, s]) <= 1e-12 * max(1.0, abs(ref[m, s]))


def check_bf16_rounding(gm) -> None:
    """Round-to-nearest-even onto BF16, against torch's float32 -> bfloat16
    conversion (a library routine) over every class of float32 input."""
    rng = np.random.default_rng(23)
    bits = rng.integers(0, 1 << 32, size=200_000, dtype=np.uint64).astype(np.uint32)
    # exact ties (low half 0x8000) on even and odd upper halves, values one ulp
    # either side of a tie, the overflow boundary, subnormals, zeros, infinities
    ties = (rng.integers(0, 1 << 16, size=20_000, dtype=np.uint32) << 16) | 0x8000
    near = np.concatenate([ties - 1, ties + 1])
    special = np.array([0x7F7F8000, 0x7F7F7FFF, 0x7F7FFFFF, 0xFF7F8000, 0x00000001, 0x00008000,
                        0x00018000, 0x807F8000, 0x00000000, 0x80000000, 0x7F800000, 0xFF800000,
                        0x3F808000, 0x3F818000], np.uint32)
    allbits = np.concatenate([bits, ties, near, special])
    f32 = allbits.view(np.float32)
    with np.errstate(invalid="ignore"):  # signalling-NaN patterns warn when widened
        f64 = f32.astype(np.float64)
    got = gm.round_to_bf16(f64)
    want = torch.from_numpy(f32.copy()).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    nan = np.isnan(f32)
    assert np.array_equal(got[~nan], want[~nan])
    assert np.all((got[nan] & 0x7FFF) > 0x7F80)


def check_rel_frobenius_golden(gm) -> None:
    """The relative Frobenius error against the hand-worked cases of
    ``tests/golden/rel_frobenius_error.txt`` (exact ratios of norms worked out
    by hand), and its symmetry under a common sign flip."""
    gd = read_golden("rel_frobenius_error.txt")
    shapes = {r[0]: (int(r[1]), int(r[2])) for r in gd["shape"]}
    exact = {r[0]: np.array([float(v) for v in r[1:]]).reshape(shapes[r[0]]) for r in gd["exact"]}
    approx = {r[0]: np.array([int(v, 16) for v in r[1:]], np.uint16).reshape(shapes[r[0]])
              for r in gd["approx"]}
    want = {r[0]: int(r[1]) / int(r[2]) for r in gd["err"]}
    assert set(want) == set(exact) == set(approx)
    for case, w in want.items():
        got = gm.relative_frobenius_error(approx[case], exact[case])
        assert abs(got - w) <= 1e-15 * max(w, 1.0), (case, got, w)
        # -A against -E: the same distance over the same norm
        neg = approx[case] ^ np.uint16(0x8000)
        got = gm.relative_frobenius_error(neg, -exact[case])
        assert abs(got - w) <= 1e-15 * max(w, 1.0), (case, "negated", got, w)


GEMM_CHECKS = [check_gemm_golden, check_gemm_one_hot, check_gemm_closed_forms, check_gemm_library,
               check_bf16_rounding, check_rel_frobenius_golden]
