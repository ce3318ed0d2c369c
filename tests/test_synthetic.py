"""The seeded input recipe (no GPU): sizes, exact sentinel counts, special
rows and determinism."""

import numpy as np
import pytest

from tp_vocab_logits_amd import synthetic as syn

SENT_LOW, SENT_HIGH = 0x0000, 0x8000


def _sentinel_words(bits):
    return int(np.sum((bits[..., 0::2] == SENT_LOW) & (bits[..., 1::2] == SENT_HIGH)))


@pytest.mark.parametrize("name,expected", [("tiny", 41), ("decode", 82), ("spec", 328)])
def test_sentinel_counts(name, expected):
    w = syn.WORKLOADS[name]
    bits = syn.shard_set(w, 0)
    assert bits.shape == (w.tp, w.rows, w.shard) and bits.dtype == np.uint16
    # N(0, sigma) draws essentially never give an exact (+0, -0) pair by themselves
    assert _sentinel_words(bits) == expected


def test_batched_special_rows_and_count():
    w = syn.WORKLOADS["batched"]
    bits = syn.shard_set(w, 1)
    assert bits.shape == (8, 64, 20480)
    assert np.all(bits[:, 1, :] == 0x0000)
    assert np.all(bits[:, 17, :] == 0x8000)
    assert np.all(bits[:, 33, 0::2] == 0x0000) and np.all(bits[:, 33, 1::2] == 0x8000)
    assert np.all(bits[:, 49, 0::2] == 0x8000) and np.all(bits[:, 49, 1::2] == 0x0000)
    others = np.delete(bits, [1, 17, 33, 49], axis=1)
    # 52429 forced words overall, minus the ones that landed on overwritten rows
    n = _sentinel_words(others)
    assert 52429 * 56 // 64 - 1500 < n <= 52429


def test_deterministic_and_distinct_sets():
    a0 = syn.shard_set("decode", 0)
    assert np.array_equal(a0, syn.shard_set("decode", 0))
    assert not np.array_equal(a0, syn.shard_set("decode", 1))


def test_overrides_and_torch_roundtrip():
    bits = syn.shard_set("spec", 3, rows=3, tp=4, shard=40)
    assert bits.shape == (4, 3, 40)
    t = syn.to_torch_bf16(bits)
    assert np.array_equal(syn.from_torch_bf16(t), bits)


def test_gemm_inputs_shape():
    x = syn.hidden_states("fused", rows=4, hidden=64)
    wr = syn.head_weight_shard("fused", 3, shard=16, hidden=64)
    assert x.shape == (4, 64) and wr.shape == (16, 64)
    assert not np.array_equal(wr, syn.head_weight_shard("fused", 2, shard=16, hidden=64))
