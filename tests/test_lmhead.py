"""GPU: the MFMA lm_head shard product (the producer of the fused workload)
against the float64 oracle, and the producer + gather path bit-exact to the
oracle applied to the product's own BF16 shards, mailbox state included."""

from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle_pins as pins
from oracle import gather as og
from oracle import gemm as ogemm
from tp_vocab_logits_amd import _lib
from tp_vocab_logits_amd import synthetic as syn
from tp_vocab_logits_amd.head_gather import HeadGather, HgError, lmhead

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def note(msg: str) -> None:
    print(f"[gpu] {msg}", flush=True)


def dev(b: np.ndarray) -> torch.Tensor:
    return syn.to_torch_bf16(b, DEV)


def bits(t: torch.Tensor) -> np.ndarray:
    return syn.from_torch_bf16(t)


def rand_bits(shape, sigma, seed):
    return syn.random_bf16(shape, sigma, seed)


def assert_close_to_oracle(got_bits: np.ndarray, x_bits: np.ndarray, w_bits: np.ndarray) -> None:
    """Tolerance from the arithmetic: the kernel sums H = hidden products in
    fp32 (error at most gamma * sum|x*w| with gamma = 2 * H * 2^-24, twice the
    classic n*u bound since the summation order inside the matrix cores is not
    specified) and rounds the sum to BF16 (relative error at most 2^-8). Also
    the relative Frobenius error of the whole shard must stay within 1e-2."""
    ref = ogemm.lm_head_shard(x_bits, w_bits)
    absum = np.abs(ogemm.bf16_to_f64(x_bits)) @ np.abs(ogemm.bf16_to_f64(w_bits)).T
    gamma = 2.0 * x_bits.shape[1] * 2.0 ** -24
    bound = 2.0 ** -8 * (np.abs(ref) + gamma * absum) + gamma * absum
    got = ogemm.bf16_to_f64(got_bits)
    bad = np.abs(got - ref) > bound
    assert not bad.any(), f"{int(bad.sum())} entries outside the bound; worst {np.max(np.abs(got - ref))}"
    if np.linalg.norm(ref) > 0:
        assert ogemm.relative_frobenius_error(got_bits, ref) <= 1e-2


def test_one_hot_rows_select_weight_columns_exactly():
    tp, shard, hidden, m = 2, 64, 136, 5
    note(f"lmhead one-hot tp={tp} shard={shard} hidden={hidden} m={m}")
    w = rand_bits((tp, shard, hidden), 1.0, 1)
    cols = [0, 7, 135, 64, 9]
    x = np.zeros((m, hidden), np.uint16)
    for i, j in enumerate(cols):
        x[i, j] = 0x3F80  # BF16 1.0
    out = bits(lmhead(dev(x), dev(w), tp, shard))
    for r in range(tp):
        for i, j in enumerate(cols):
            assert np.array_equal(out[r, i], w[r, :, j]), (r, i)


def test_hand_worked_golden_product():
    note("lmhead golden (padded to shard 32, hidden 8)")
    gd = pins.read_golden("lm_head_h3_s4_m2.txt")
    x3 = np.array([[int(v, 16) for v in r[1:]] for r in gd["x"]], np.uint16)
    w3 = np.array([[int(v, 16) for v in r[1:]] for r in gd["w"]], np.uint16)
    want = np.array([[float(v) for v in r[1:]] for r in gd["out"]])
    x = np.zeros((2, 8), np.uint16)
    x[:, :3] = x3
    w = np.zeros((1, 32, 8), np.uint16)
    w[0, :4, :3] = w3
    out = ogemm.bf16_to_f64(bits(lmhead(dev(x), dev(w), 1, 32)))
    assert np.array_equal(out[0, :, :4], want)
    assert np.all(out[0, :, 4:] == 0)


@pytest.mark.parametrize("tp,shard,hidden,m", [
    (1, 32, 8, 1), (2, 64, 72, 3), (3, 288, 136, 17), (8, 96, 512, 256), (2, 512, 1032, 300),
    (5, 160, 64, 255), (64, 32, 64, 2), (2, 256, 40, 7), (2, 640, 256, 31), (2, 640, 256, 32),
    (2, 640, 256, 33), (1, 960, 192, 63), (1, 960, 192, 64), (1, 960, 192, 65),
    (3, 320, 200, 129), (4, 352, 264, 257), (2, 320, 7168, 4), (1, 1280, 128, 511)])
def test_ragged_sizes_against_oracle(tp, shard, hidden, m):
    note(f"lmhead ragged tp={tp} shard={shard} hidden={hidden} m={m}")
    x = rand_bits((m, hidden), 0.5, 10 + m)
    w = rand_bits((tp, shard, hidden), 0.5, 20 + hidden)
    out = bits(lmhead(dev(x), dev(w), tp, shard))
    for r in range(tp):
        assert_close_to_oracle(out[r], x, w[r])


@pytest.mark.parametrize("tp,shard,hidden", [(3, 96, 200), (2, 320, 7168)])
def test_rows_do_not_depend_on_row_count(tp, shard, hidden):
    """Below 128 rows one wave layout computes the product, from 128 rows on
    another; both run each 32 x 32 output block as the same chain of MFMAs
    over K, so a row's bits must not depend on how many rows the call has."""
    note(f"lmhead rows vs row count tp={tp} shard={shard} hidden={hidden}")
    x = dev(rand_bits((256, hidden), 0.5, 91))
    w = dev(rand_bits((tp, shard, hidden), 0.5, 92))
    full = lmhead(x, w, tp, shard)
    for m in (1, 5, 127, 128, 200):
        part = lmhead(x[:m].contiguous(), w, tp, shard)
        assert torch.equal(part.view(torch.int16), full[:, :m].view(torch.int16)), m


def test_lmhead_argument_rules():
    note("lmhead argument rules")
    x = dev(rand_bits((4, 64), 1.0, 3))
    with pytest.raises(HgError):  # shard % 32 != 0
        lmhead(x, dev(rand_bits((2, 48, 64), 1.0, 4)), 2, 48)
    with pytest.raises(HgError):  # hidden % 8 != 0
        lmhead(dev(rand_bits((4, 60), 1.0, 3)), dev(rand_bits((2, 64, 60), 1.0, 4)), 2, 64)
    empty = lmhead(dev(rand_bits((0, 64), 1.0, 3)), dev(rand_bits((2, 64, 64), 1.0, 4)), 2, 64)
    assert tuple(empty.shape) == (2, 0, 64)


def test_full_size_producer_gather_m256():
    w_ = syn.WORKLOADS["fused"]
    tp, shard, hidden, m = w_.tp, w_.shard, w_.hidden, w_.rows
    note(f"fused producer+gather tp={tp} V={w_.vocab} m={m} hidden={hidden}")
    x = syn.hidden_states(w_)
    wd = torch.empty((tp, shard, hidden), dtype=torch.bfloat16, device=DEV)
    w_host = []
    for r in range(tp):
        wr = syn.head_weight_shard(w_, r)
        w_host.append(wr)
        wd[r].copy_(dev(wr))
    xd = dev(x)
    hg = HeadGather(tp, shard, w_.cap, device=DEV)
    hg.set_poll_limit(1 << 20)
    sim = og.MailboxSim(tp, shard, w_.cap)
    shards = torch.empty((tp, m, shard), dtype=torch.bfloat16, device=DEV)
    out = hg.gemm_gather(xd, wd, shards_out=shards)
    # the gather is bit-exact to the oracle applied to the product's own shards
    sb = bits(shards)
    status, want = sim.gather(list(sb))
    assert status == og.OK and np.array_equal(bits(out), want)
    assert hg.parity == 1 and hg.poll_status() == _lib.HG_OK
    for p in (0, 1):
        assert np.array_equal(bits(hg.mailbox(p)), sim.mailbox_bf16(p))
    # the product itself, rank by rank, against the float64 oracle
    for r in range(tp):
        assert_close_to_oracle(sb[r], x, w_host[r])
    # deterministic: the standalone product and a second producer call agree
    # bit for bit
    again = lmhead(xd, wd, tp, shard)
    assert torch.equal(again.view(torch.int16), shards.view(torch.int16))
    out2 = hg.gemm_gather(xd, wd)
    assert torch.equal(out2.view(torch.int16), out.view(torch.int16))
    assert hg.parity == 0 and hg.poll_status() == _lib.HG_OK
    hg.close()


def test_producer_gather_declines_and_state():
    tp, shard, hidden = 2, 64, 64
    note("producer+gather declines")
    hg = HeadGather(tp, shard, 4, device=DEV)
    x = dev(rand_bits((5, hidden), 1.0, 1))
    w = dev(rand_bits((tp, shard, hidden), 1.0, 2))
    with pytest.raises(HgError):
        hg.gemm_gather(x, w)  # 5 rows > cap 4: declined
    assert hg.parity == 0
    s = dev(rand_bits((tp, 1, shard), 1.0, 3))
    assert hg.push(s)
    with pytest.raises(HgError):
        hg.gemm_gather(x[:2], w)  # a split push is pending
    hg.collect(1)
    sim = og.MailboxSim(tp, shard, 4)
    sim.gather(list(bits(s)))
    shards = torch.empty((tp, 3, shard), dtype=torch.bfloat16, device=DEV)
    out = hg.gemm_gather(x[:3].contiguous(), w, shards_out=shards)
    status, want = sim.gather(list(bits(shards)))
    assert status == og.OK and np.array_equal(bits(out), want) and hg.parity == sim.parity
    hg.close()


@pytest.mark.parametrize("m", [1, 5, 40, 130, 300])
def test_producer_gather_repeated_calls(m):
    # hg_gemm_gather five times in a row: the shards it keeps equal the
    # standalone product's bit for bit, the gather of them is bit-exact to the
    # oracle's, and the parity alternates
    tp, shard, hidden, cap = 3, 96, 136, 320
    note(f"producer repeated calls m={m}")
    x = dev(rand_bits((m, hidden), 0.5, 70 + m))
    w = dev(rand_bits((tp, shard, hidden), 0.5, 80 + m))
    hg = HeadGather(tp, shard, cap, device=DEV)
    hg.set_poll_limit(1 << 20)
    sim = og.MailboxSim(tp, shard, cap)
    ref = lmhead(x, w, tp, shard)
    for n in range(5):
        shards = torch.empty((tp, m, shard), dtype=torch.bfloat16, device=DEV)
        out = hg.gemm_gather(x, w, shards_out=shards)
        assert torch.equal(shards.view(torch.int16), ref.view(torch.int16)), n
        status, want = sim.gather(list(bits(shards)))
        assert status == og.OK and np.array_equal(bits(out), want), n
        assert hg.parity == sim.parity
    assert hg.poll_status() == _lib.HG_OK
    for p in (0, 1):
        assert np.array_equal(bits(hg.mailbox(p)), sim.mailbox_bf16(p))
    hg.close()


def test_producer_epilogue_rewrites_a_sentinel_product():
    """A product word equal to the sentinel pair (+0, -0) must reach the
    mailbox as (+0, +0): otherwise the collect polls it until it gives up.
    Column 0 of rank 0 has an all-zero weight row (its logit is +0); column 1
    has one weight -2^-70 against x = 2^-70 in row 1, a product of -2^-140,
    which rounds to BF16 -0 (below half the smallest BF16 subnormal, 2^-134)."""
    tp, shard, hidden, cap, m = 2, 64, 72, 4, 3
    note("producer epilogue: sentinel product word")
    rng_x = rand_bits((m, hidden), 0.5, 5)
    w = rand_bits((tp, shard, hidden), 0.5, 6)
    w[0, 0, :] = 0x0000                      # column 0: +0 logits
    w[0, 1, :] = 0x0000
    w[0, 1, 0] = 0x9C80                      # -2^-70
    rng_x[1, 0] = 0x1C80                     # +2^-70
    assert ogemm.bf16_to_f64(np.array([0x9C80], np.uint16))[0] == -(2.0 ** -70)
    x, wd = dev(rng_x), dev(w)
    shards = lmhead(x, wd, tp, shard)
    word = int(bits(shards)[0, 1, 0]) | (int(bits(shards)[0, 1, 1]) << 16)
    assert word == og.SENT_WORD, hex(word)   # the product itself is the sentinel pair
    hg = HeadGather(tp, shard, cap, device=DEV)
    hg.set_poll_limit(1 << 16)
    sim = og.MailboxSim(tp, shard, cap)
    kept = torch.empty((tp, m, shard), dtype=torch.bfloat16, device=DEV)
    out = hg.gemm_gather(x, wd, shards_out=kept)
    assert torch.equal(kept.view(torch.int16), shards.view(torch.int16))  # kept as computed
    got = bits(out)
    assert got[1, 0] == 0 and got[1, 1] == 0                              # rewritten to (+0, +0)
    status, want = sim.gather(list(bits(kept)))
    assert status == og.OK and np.array_equal(got, want)
    assert hg.poll_status() == _lib.HG_OK
    hg.close()


def test_producer_gather_refuses_overlaps():
    """hg_gemm_gather refuses (HG_EINVAL, nothing enqueued, parity unchanged)
    a shard copy overlapping the mailbox or the output, an output overlapping
    a weight block, and hidden states overlapping the mailbox."""
    import ctypes

    tp, shard, hidden, cap, m = 2, 64, 72, 4, 3
    note("producer+gather overlap checks")
    lib = _lib.lib()
    hg = HeadGather(tp, shard, cap, device=DEV)
    x = dev(rand_bits((m, hidden), 0.5, 1))
    w = dev(rand_bits((tp, shard, hidden), 0.5, 2))
    out = torch.empty((m, tp * shard), dtype=torch.bfloat16, device=DEV)
    kept = torch.empty((tp, m, shard), dtype=torch.bfloat16, device=DEV)
    box, nbytes = ctypes.c_void_p(), ctypes.c_size_t()
    assert lib.hg_mailbox(hg.handle, 0, ctypes.byref(box), ctypes.byref(nbytes)) == _lib.HG_OK
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    P = _lib.pointer_array
    wp = P([w[r].data_ptr() for r in range(tp)])
    kp = [kept[r].data_ptr() for r in range(tp)]

    def call(xp, outp, keep):
        return lib.hg_gemm_gather(hg.handle, ctypes.c_void_p(xp), wp, hidden, m, ctypes.c_void_p(outp),
                                  keep, stream)

    assert call(x.data_ptr(), out.data_ptr(), P([box.value, kp[1]])) == _lib.HG_EINVAL  # copy on mailbox
    assert call(x.data_ptr(), out.data_ptr(), P([kp[0], out.data_ptr()])) == _lib.HG_EINVAL  # copy on out
    assert call(x.data_ptr(), w[1].data_ptr(), P(kp)) == _lib.HG_EINVAL  # out on a weight block
    assert call(box.value, out.data_ptr(), P(kp)) == _lib.HG_EINVAL  # x on the mailbox
    assert hg.parity == 0
    # and the well-formed call still runs and is served
    assert call(x.data_ptr(), out.data_ptr(), P(kp)) == _lib.HG_OK
    sim = og.MailboxSim(tp, shard, cap)
    status, want = sim.gather(list(bits(kept)))
    assert status == og.OK and np.array_equal(bits(out), want) and hg.parity == 1
    hg.close()
