"""Oracle: the vocab-parallel lm_head shard product that feeds the gather.

TEST INFRASTRUCTURE ONLY (see the package docstring).

What it computes. The gather's input is the output of the vocab-parallel
lm_head: each rank holds the rows ``r*S .. (r+1)*S`` of the ``[V, H]`` head
weight (``install_logits_gather`` on the API page takes the shard width from
``weight.shape[0]``) and produces its ``[M, S]`` logits shard as ``X @ W_r^T``
(API page, module description: the lm_head's ``[M, V/TP]`` shards; PR 55021,
Test Result: the gather overlaps the tail of the LM-head GEMM). The pages do
not fix the arithmetic precision of the product; the oracle computes it in
float64 from the exact BF16 inputs, and the comparison tolerance lives in the
tests.

``round_to_bf16`` is the IEEE-754 round-to-nearest-even onto the BF16 grid
(1 sign bit, 8 exponent bits with bias 127, 7 stored fraction bits), written
from the format's definition.
"""

from __future__ import annotations

import numpy as np


def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    """BF16 bit patterns -> exact float64 values (a BF16 pattern is the upper
    half of the float32 with the same value)."""
    bits = np.asarray(bits, dtype=np.uint16)
    return (bits.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


def lm_head_shard(x_bits: np.ndarray, w_bits: np.ndarray) -> np.ndarray:
    """One rank's logits shard in float64: ``X @ W_r^T``.

    ``x_bits``: ``[M, H]`` BF16 patterns (the hidden states).
    ``w_bits``: ``[S, H]`` BF16 patterns (this rank's rows of the head weight).
    Returns ``[M, S]`` float64; entry ``(m, s)`` is ``sum_h X[m, h] * W_r[s, h]``.
    """
    x = bf16_to_f64(x_bits)
    w = bf16_to_f64(w_bits)
    if x.ndim != 2 or w.ndim != 2 or x.shape[1] != w.shape[1]:
        raise ValueError(f"shape mismatch: X {x.shape}, W_r {w.shape}")
    return x @ w.T


def lm_head_entry(x_bits: np.ndarray, w_bits: np.ndarray, m: int, s: int) -> float:
    """A single logit ``(m, s)`` of one rank's shard, as an exactly rounded
    float64 sum of the ``H`` exact products (``math.fsum``)."""
    import math

    x = bf16_to_f64(np.asarray(x_bits)[m])
    w = bf16_to_f64(np.asarray(w_bits)[s])
    return math.fsum((x * w).tolist())


def round_to_bf16(values) -> np.ndarray:
    """Round real values to the nearest BF16, ties to even; returns uint16 bits.

    Finite values at or beyond the overflow threshold become infinities; NaN
    becomes the quiet NaN ``0x7FC0`` with the input's sign.
    """
    v = np.asarray(values, dtype=np.float64)
    sign = np.signbit(v)
    a = np.abs(v)
    out = np.zeros(v.shape, dtype=np.uint16)

    nan = np.isnan(v)
    finite = np.isfinite(v)
    # Quantum (unit in the last place) of the BF16 binade holding |v|: 8
    # significant bits for normals (|v| >= 2^-126), fixed 2^-133 below.
    with np.errstate(divide="ignore"):
        _, e2 = np.frexp(np.where(finite & (a > 0), a, 1.0))  # a = f * 2^e2, f in [0.5, 1)
    exponent = np.maximum(e2 - 1, -126)
    quantum = np.ldexp(1.0, exponent - 7)
    rounded = np.where(finite, np.rint(np.where(finite, a, 0.0) / quantum) * quantum, 0.0)
    overflow = finite & (rounded >= 2.0 ** 128)
    as_f32 = np.where(overflow | ~finite, 0.0, rounded).astype(np.float32)
    bits = (as_f32.view(np.uint32) >> np.uint32(16)).astype(np.uint16)
    out[...] = bits
    out[overflow | (np.isinf(v))] = np.uint16(0x7F80)
    out[nan] = np.uint16(0x7FC0)
    out = np.where(sign, out | np.uint16(0x8000), out).astype(np.uint16)
    return out


def relative_frobenius_error(approx_bits: np.ndarray, exact: np.ndarray) -> float:
    """``||approx - exact||_F / ||exact||_F`` with ``approx`` given as BF16 bits:
    the root of the summed squared differences over the root of the summed
    squared exact values. This is the reading taken for the fused producer
    workload's "within 1e-2 relative error of the exact product" (the pages fix
    no tolerance for the product that feeds the gather)."""
    approx = bf16_to_f64(approx_bits)
    exact = np.asarray(exact, dtype=np.float64)
    return float(np.linalg.norm(approx - exact) / np.linalg.norm(exact))
