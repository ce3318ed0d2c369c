"""Seeded synthetic inputs for the logits gather and its lm_head producer.

This module only draws inputs: it holds none of the gather's arithmetic (no
packing, no sentinel rewrite, no concatenation), so both the HIP path and the
CPU oracle can be fed from it without sharing method code.

Values are BF16 bit patterns in ``numpy.uint16`` arrays. Draws use
``torch.Generator`` on the CPU, so the same seed gives the same bits on every
machine.

Workloads (sizes of a Kimi-K3 TP8 decode step: V = 163840 vocab entries split
over 8 ranks, one to 256 rows):

======== == ====== === === ===== ========= ==== ======
name     TP V      M   cap sigma sentinels seed hidden
======== == ====== === === ===== ========= ==== ======
tiny     2  4096   1   1   1     2 %       0    -
decode   8  163840 1   8   3     0.1 %     1    -
spec     8  163840 4   8   3     0.1 %     2    -
batched  8  163840 64  64  3     1 % + special rows  3  -
fused    8  163840 256 256 0.02  none      4    7168
======== == ====== === === ===== ========= ==== ======

Recipe for one gather input set ``k`` of a workload with seed ``s``:

1. ``torch.Generator().manual_seed(s + 1000*k)`` draws ``randn([TP, M, S])``
   in float32, scaled by sigma, converted to BF16 (round to nearest even).
2. A second generator, seeded ``s + 500 + 1000*k``, picks exactly
   ``round(fraction * TP*M*S/2)`` distinct word positions (a word = the BF16
   elements ``2j, 2j+1`` of one shard row) through ``randperm`` and sets each to
   the pair (+0, -0): element ``2j`` = ``0x0000``, element ``2j+1`` = ``0x8000``.
3. ``batched`` then overwrites four whole rows across every rank: row 1 all
   +0, row 17 all -0, row 33 alternating +0/-0, row 49 alternating -0/+0.

The fused workload draws ``X [M, hidden]`` (seed ``s``) and the head weight one
rank at a time (``W_r [S, hidden]``, seed ``s + 100 + r``), both ``N(0, 0.02)``
rounded to BF16.
"""

from __future__ import annotations

from dataclasses import dataclass

import numpy as np
import torch


@dataclass(frozen=True)
class Workload:
    name: str
    tp: int
    vocab: int
    rows: int          # M, rows gathered per call
    cap: int           # mailbox rows per parity
    sigma: float
    sentinel_fraction: float
    seed: int
    calls: int         # calls in one run of the workload
    pool: int          # distinct input sets cycled over the calls
    special_rows: tuple[int, ...] = ()
    hidden: int = 0    # lm_head input width (fused workload only)

    @property
    def shard(self) -> int:
        return self.vocab // self.tp


WORKLOADS: dict[str, Workload] = {
    "tiny": Workload("tiny", 2, 4096, 1, 1, 1.0, 0.02, 0, calls=4, pool=4),
    "decode": Workload("decode", 8, 163840, 1, 8, 3.0, 0.001, 1, calls=1000, pool=8),
    "spec": Workload("spec", 8, 163840, 4, 8, 3.0, 0.001, 2, calls=1000, pool=8),
    "batched": Workload("batched", 8, 163840, 64, 64, 3.0, 0.01, 3, calls=64, pool=4,
                        special_rows=(1, 17, 33, 49)),
    "fused": Workload("fused", 8, 163840, 256, 256, 0.02, 0.0, 4, calls=8, pool=1, hidden=7168),
}

# BF16 bit patterns used by the recipe.
_POS_ZERO = 0x0000
_NEG_ZERO = 0x8000


def _bf16_bits(t: torch.Tensor) -> np.ndarray:
    return t.to(torch.bfloat16).contiguous().view(torch.int16).numpy().view(np.uint16)


def random_bf16(shape, sigma: float, seed: int) -> np.ndarray:
    """``N(0, sigma)`` drawn in float32 and rounded to BF16, as uint16 bits."""
    g = torch.Generator().manual_seed(int(seed))
    return _bf16_bits(torch.randn(tuple(shape), generator=g, dtype=torch.float32) * sigma)


def shard_set(w: Workload | str, k: int = 0, rows: int | None = None,
              tp: int | None = None, shard: int | None = None) -> np.ndarray:
    """Input set ``k`` of a workload: ``[TP, M, S]`` uint16 BF16 bits.

    ``rows``, ``tp`` and ``shard`` override the workload's sizes (same recipe),
    for smaller parity cases.
    """
    if isinstance(w, str):
        w = WORKLOADS[w]
    tp = w.tp if tp is None else tp
    m = w.rows if rows is None else rows
    s = w.shard if shard is None else shard
    bits = random_bf16((tp, m, s), w.sigma, w.seed + 1000 * k)
    inject_sentinel_words(bits, w.sentinel_fraction, w.seed + 500 + 1000 * k)
    for i, row in enumerate(w.special_rows):
        if row < m:
            fill_special_row(bits, row, i)
    return bits


def inject_sentinel_words(bits: np.ndarray, fraction: float, seed: int) -> int:
    """Force exactly ``round(fraction * words)`` distinct words to the pair
    (+0, -0), in place. Returns the number of words forced."""
    tp, m, s = bits.shape
    words = tp * m * (s // 2)
    count = int(round(fraction * words))
    if count == 0:
        return 0
    g = torch.Generator().manual_seed(int(seed))
    pos = torch.randperm(words, generator=g)[:count].numpy()
    flat = bits.reshape(-1)
    flat[2 * pos] = _POS_ZERO
    flat[2 * pos + 1] = _NEG_ZERO
    return count


def fill_special_row(bits: np.ndarray, row: int, kind: int) -> None:
    """Overwrite row ``row`` of every rank with one of four signed-zero
    patterns: 0 all +0, 1 all -0, 2 alternating +0/-0, 3 alternating -0/+0."""
    if kind == 0:
        bits[:, row, :] = _POS_ZERO
    elif kind == 1:
        bits[:, row, :] = _NEG_ZERO
    elif kind == 2:
        bits[:, row, 0::2] = _POS_ZERO
        bits[:, row, 1::2] = _NEG_ZERO
    elif kind == 3:
        bits[:, row, 0::2] = _NEG_ZERO
        bits[:, row, 1::2] = _POS_ZERO
    else:
        raise ValueError(f"unknown special row kind {kind}")


def hidden_states(w: Workload | str, rows: int | None = None, hidden: int | None = None) -> np.ndarray:
    """Fused workload: ``X [M, hidden]`` BF16 bits."""
    if isinstance(w, str):
        w = WORKLOADS[w]
    return random_bf16((w.rows if rows is None else rows, w.hidden if hidden is None else hidden),
                       w.sigma, w.seed)


def head_weight_shard(w: Workload | str, rank: int, shard: int | None = None,
                      hidden: int | None = None) -> np.ndarray:
    """Fused workload: rank ``rank``'s head-weight rows ``W_r [S, hidden]``."""
    if isinstance(w, str):
        w = WORKLOADS[w]
    return random_bf16((w.shard if shard is None else shard, w.hidden if hidden is None else hidden),
                       w.sigma, w.seed + 100 + rank)


def to_torch_bf16(bits: np.ndarray, device=None) -> torch.Tensor:
    """uint16 BF16 bits -> a ``torch.bfloat16`` tensor (optionally moved)."""
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16)
    return t.to(device) if device is not None else t


def from_torch_bf16(t: torch.Tensor) -> np.ndarray:
    """A ``torch.bfloat16`` tensor -> uint16 BF16 bits on the host."""
    return t.detach().to("cpu").contiguous().view(torch.int16).numpy().view(np.uint16)
