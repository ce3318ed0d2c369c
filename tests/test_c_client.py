"""GPU: the C ABI from a plain C program (tests/c_client/hg_client.c: no
Python, no torch, only include/hg.h and the HIP runtime), checked against the
CPU oracle's protocol simulator: every output, the final parity and both
mailbox parities, bit for bit, fused and split; and the allocation-free
hg_gather_static against the oracle's definition."""

from __future__ import annotations

import os
import subprocess

import numpy as np
import pytest

from oracle import gather as og
from tp_vocab_logits_amd import synthetic as syn

pytestmark = pytest.mark.gpu

CLIENT = os.path.join(os.path.dirname(os.path.abspath(__file__)), "c_client", "hg_client")


def note(msg: str) -> None:
    print(f"[gpu] {msg}", flush=True)


@pytest.mark.parametrize("workload,tp,shard,cap,m,calls,variant", [
    ("tiny", 2, 2048, 1, 1, 4, 0),
    ("decode", 8, 20480, 8, 1, 5, 0),
    ("spec", 8, 20480, 8, 4, 3, 1),
    ("spec", 3, 288, 4, 3, 5, 0),
    ("batched", 5, 40, 6, 6, 4, 1),
    ("decode", 8, 20480, 8, 1, 3, 2),
    ("spec", 3, 288, 4, 3, 4, 2),
])
def test_c_client_against_oracle(tmp_path, workload, tp, shard, cap, m, calls, variant):
    if not os.path.exists(CLIENT):
        pytest.fail("tests/c_client/hg_client is missing: run __graft_entry__.build() first")
    note(f"C client {workload} tp={tp} shard={shard} cap={cap} m={m} calls={calls} "
         f"{['fused', 'split', 'static'][variant]}")
    sets = []
    for k in range(calls):
        s = syn.shard_set(workload, k, rows=m, tp=tp, shard=shard)
        syn.inject_sentinel_words(s, 0.05, 77 + k)
        sets.append(s)
    src, dst = tmp_path / "in.bin", tmp_path / "out.bin"
    with open(src, "wb") as f:
        f.write(np.array([tp, shard, cap, m, calls, variant], dtype=np.int32).tobytes())
        for s in sets:
            f.write(np.ascontiguousarray(s).tobytes())
    res = subprocess.run([CLIENT, str(src), str(dst)], capture_output=True, text=True, timeout=120)
    assert res.returncode == 0, res.stderr
    raw = open(dst, "rb").read()
    v = tp * shard
    sim = og.MailboxSim(tp, shard, cap)
    off = 0
    for k, s in enumerate(sets):
        n = m * v * 2
        got = np.frombuffer(raw[off:off + n], dtype=np.uint16).reshape(m, v)
        off += n
        if variant == 0:
            status, want = sim.gather(list(s))
        elif variant == 2:  # the static entry point: the context stays as created
            status, want = og.OK, og.gather_definition(list(s))
        else:
            assert sim.push(list(s)) == og.OK
            status, want = sim.collect(m)
        assert status == og.OK and np.array_equal(got, want), f"call {k}"
    parity = int(np.frombuffer(raw[off:off + 4], dtype=np.int32)[0])
    off += 4
    assert parity == sim.parity
    for p in (0, 1):
        n = cap * v * 2
        box = np.frombuffer(raw[off:off + n], dtype=np.uint16).reshape(cap, v)
        off += n
        assert np.array_equal(box, sim.mailbox_bf16(p)), f"mailbox parity {p}"
    assert off == len(raw)
