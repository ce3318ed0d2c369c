"""GPU: the largest calls, where the addressing changes.

The 128-bit coherent push and poll address the rows of a call through a
buffer resource with 32-bit byte offsets. Between 2 GiB and 4 GiB of rows the
offsets pass 2^31; from 4 GiB on the library switches to 64-bit atomic
accesses through pointers. One case sits in each band, TP=8, V=163840:
9830 rows (3.22 GB per call) and 13200 rows (4.33 GB), fused and split, two
calls each (both parities), with 32-bit random words and injected sentinels.

Every row of the output is checked against the CPU oracle
(``oracle.gather.gather_definition``), 1024 rows at a time; the used rows of
the mailbox must be re-armed and the parity must alternate."""

from __future__ import annotations

import numpy as np
import pytest
import torch

from oracle import gather as og
from tp_vocab_logits_amd import _lib
from tp_vocab_logits_amd import synthetic as syn
from tp_vocab_logits_amd.head_gather import HeadGather

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
TP, SHARD = 8, 20480
V = TP * SHARD
ROW_BYTES = V * 2
SENT = -(1 << 31)  # 0x80000000 as int32


def note(msg: str) -> None:
    print(f"[gpu] {msg}", flush=True)


def words_input(m: int, seed: int) -> torch.Tensor:
    """[TP, m, S] BF16 whose 32-bit words are seeded random patterns, with
    0.1 % of the words set to the sentinel."""
    g = torch.Generator(device=DEV)
    g.manual_seed(seed)
    w = torch.randint(-(1 << 31), 1 << 31, (TP, m, SHARD // 2), dtype=torch.int64, device=DEV,
                      generator=g).to(torch.int32)
    flat = w.view(-1)
    n = flat.numel() // 1000
    idx = torch.randint(0, flat.numel(), (n,), device=DEV, generator=g)
    flat[idx] = SENT
    return w.view(torch.bfloat16)


def check_all_rows_against_oracle(out: torch.Tensor, shards: torch.Tensor, chunk: int = 1024):
    m = out.shape[0]
    for r0 in range(0, m, chunk):
        r1 = min(m, r0 + chunk)
        want = og.gather_definition(list(syn.from_torch_bf16(shards[:, r0:r1, :])))
        got = syn.from_torch_bf16(out[r0:r1])
        if not np.array_equal(got, want):
            bad = np.argwhere(got != want)[0]
            raise AssertionError(f"row {r0 + bad[0]} column {bad[1]} differs from the oracle")


@pytest.mark.parametrize("variant", ["fused", "split"])
@pytest.mark.parametrize("m", [9830, 13200], ids=["2-4GiB", "over-4GiB"])
def test_largest_calls(m, variant):
    assert (m * ROW_BYTES >= 1 << 31) and (m != 9830 or m * ROW_BYTES < 1 << 32)
    note(f"large rows m={m} ({m * ROW_BYTES / 1e9:.2f} GB per call) variant={variant}")
    hg = HeadGather(TP, SHARD, m, device=DEV)
    hg.set_poll_limit(1 << 20)
    for call in range(2):
        shards = words_input(m, 1000 * m + call)
        assert hg.parity == call % 2
        if variant == "fused":
            out = hg(shards)
        else:
            assert hg.push(shards)
            out = hg.collect(m)
        torch.cuda.synchronize()
        assert hg.poll_status() == _lib.HG_OK
        check_all_rows_against_oracle(out, shards)
        del out, shards
        used = hg.mailbox(call % 2).view(torch.int32)
        assert bool((used == SENT).all()), f"mailbox parity {call % 2} not re-armed"
        del used
    assert hg.parity == 0
    hg.close()
    torch.cuda.empty_cache()
