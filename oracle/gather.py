"""Oracle: the Lamport-mailbox logits gather, written plainly on the CPU (numpy).

TEST INFRASTRUCTURE ONLY (see the package docstring): never imported by the
product path, and sharing no code with it.

Data model. A BF16 value is handled as its 16-bit pattern (``uint16``). A
*word* is a pair of adjacent BF16 elements ``(2k, 2k+1)`` of one shard row,
packed little-endian into 32 bits: element ``2k`` is the low half and element
``2k+1`` the high half. This is the 32-bit view of a contiguous BF16 row that
``HeadGather.__call__`` takes of the shard and of the output before launching
the kernel (API page, ``HeadGather.__call__`` source).

What the method computes (API page, module description and ``HeadGather``
class description): each of ``tp`` ranks holds a ``[M, S]`` BF16 shard of the
vocab-parallel lm_head output; the result is ``[M, V]`` with ``V = tp * S`` and
rank ``r`` at columns ``r * S`` (NCCL's all-gather layout). Bytes move
unchanged, except the sentinel pair -- BF16 ``+0`` followed by BF16 ``-0`` --
which arrives as ``+0, +0``. The module description notes both pairs carry the
same values for sampling.

Readings taken where the pages leave a step open:

* The sentinel pair in element order is (+0, -0); as a little-endian word that
  is ``0x80000000``. Only a word exactly equal to it is rewritten, to ``0``.
* The rewrite happens when the word is pushed into the mailbox, so the mailbox
  holds rewritten words.
* Mailbox rows at or beyond ``M`` are never touched by a call.
* The served row counts are ``1 .. cap``.
* A declined call returns the stock result -- the plain rank-order
  concatenation, not rewritten -- and leaves the parity unchanged, because the
  printed ``__call__`` returns ``stock(logits)`` before it flips the parity.
* Parity starts at 0 at construction; ``arm`` (re-arming both parities) also
  resets it to 0.
* ``tp == 1`` is refused (``install_logits_gather`` source declines it); a shard
  must be a positive multiple of 8 elements (``_install_gather`` source refuses
  ``shard % 8``; a zero shard is refused here as well).
* Split variant: ``push`` fills the current parity and leaves it pending;
  ``collect`` of the same row count completes the call and flips the parity.
  Any other order is a state error. Ranks may push separately
  (``push_ranks``), as each rank of a real TP group pushes its own fragment;
  a collect while some rank has not pushed is a poll that never completes: a
  bounded poll gives up (``ETIMEOUT``), its output keeps the sentinel words it
  read, and the rows are re-armed and the parity flipped as for any call.
"""

from __future__ import annotations

import numpy as np

#: The sentinel word: BF16 +0 (0x0000) in the low half, BF16 -0 (0x8000) in
#: the high half (API page, module description: the pair (+0, -0)).
SENT_WORD = 0x80000000

#: Status values of the protocol simulator, mirroring the C boundary.
OK, DECLINE, EINVAL, ETIMEOUT, ESTATE = 0, 1, -1, -4, -5


# ---------------------------------------------------------------------------
# Word packing (the 32-bit view of a BF16 row)
# ---------------------------------------------------------------------------

def pack_words(elems: np.ndarray) -> np.ndarray:
    """``[..., 2n]`` uint16 BF16 patterns -> ``[..., n]`` uint32 words.

    Word ``k`` = element ``2k`` in bits 0..15 and element ``2k+1`` in bits
    16..31 (little-endian 32-bit view of the row).
    """
    elems = np.asarray(elems, dtype=np.uint16)
    if elems.shape[-1] % 2:
        raise ValueError("a row of BF16 elements must have even length to pack into words")
    low = elems[..., 0::2].astype(np.uint32)
    high = elems[..., 1::2].astype(np.uint32)
    return low | (high << np.uint32(16))


def unpack_words(words: np.ndarray) -> np.ndarray:
    """Inverse of :func:`pack_words`: ``[..., n]`` uint32 -> ``[..., 2n]`` uint16."""
    words = np.asarray(words, dtype=np.uint32)
    out = np.empty(words.shape[:-1] + (2 * words.shape[-1],), dtype=np.uint16)
    out[..., 0::2] = (words & np.uint32(0xFFFF)).astype(np.uint16)
    out[..., 1::2] = (words >> np.uint32(16)).astype(np.uint16)
    return out


def rewrite_sentinel(words: np.ndarray) -> np.ndarray:
    """The substitution applied to every pushed word: a word equal to the
    sentinel pair (+0, -0) becomes (+0, +0); every other word is unchanged
    (API page, ``HeadGather`` class description)."""
    words = np.asarray(words, dtype=np.uint32)
    return np.where(words == np.uint32(SENT_WORD), np.uint32(0), words).astype(np.uint32)


# ---------------------------------------------------------------------------
# The plain definition of the result
# ---------------------------------------------------------------------------

def stock_concat(shards) -> np.ndarray:
    """The stock all-gather result: the shards concatenated in rank order along
    the vocab axis, bytes untouched (API page, module description: NCCL's ring
    all-gather followed by a copy to ``[M, V]``)."""
    shards = [np.asarray(s, dtype=np.uint16) for s in shards]
    return np.concatenate(shards, axis=1)


def gather_definition(shards) -> np.ndarray:
    """The gathered logits of one served call, as BF16 bit patterns ``[M, V]``.

    Rank order concatenation (rank ``r`` at columns ``r * S``), then every
    sentinel word replaced by zero (API page, module description and
    ``HeadGather`` class description).
    """
    return unpack_words(rewrite_sentinel(pack_words(stock_concat(shards))))


def slice_vocab(out, vocab: int) -> np.ndarray:
    """The padded-vocab slice taken after the gather (PR page, Purpose: the
    gather keeps its semantics, the slice to the real vocabulary included):
    the first ``vocab`` columns of every gathered row, as a new ``[M, vocab]``
    array. ``1 <= vocab <= V``."""
    out = np.asarray(out, dtype=np.uint16)
    if not 1 <= vocab <= out.shape[1]:
        raise ValueError(f"vocab {vocab} outside 1..{out.shape[1]}")
    return out[:, :vocab].copy()


# ---------------------------------------------------------------------------
# Construction rules
# ---------------------------------------------------------------------------

def create_ok(tp: int, shard: int, cap: int) -> bool:
    """Whether a gather object may be built for these sizes.

    * ``tp >= 2``: ``install_logits_gather`` declines a TP of 1.
    * ``shard`` a multiple of 8 BF16 elements: ``_install_gather`` refuses any
      other shard width. A zero shard is refused too (nothing to gather).
    * ``cap >= 1``: the mailbox holds ``cap`` rows per parity
      (``HeadGather.__init__``: cap is the largest served row count).
    """
    return tp >= 2 and shard >= 8 and shard % 8 == 0 and cap >= 1


# ---------------------------------------------------------------------------
# Step-by-step simulator of the two-parity mailbox protocol
# ---------------------------------------------------------------------------

class MailboxSim:
    """The gather object's state and calls, step by step.

    State (API page, ``HeadGather.__init__`` source and class description):
    a mailbox of ``2`` parities x ``cap`` rows x ``V/2`` words, every word
    armed with the sentinel, and a parity bit starting at 0.

    A served call on parity ``p`` (API page, module description):

    1. push: for every rank ``r`` and row ``m < M``, the rank's shard row
       (as words, sentinel rewritten) lands in mailbox row ``m`` at word
       columns ``r * S/2 .. (r+1) * S/2``;
    2. poll: every word of rows ``0 .. M-1`` is read until it is not the
       sentinel (in this sequential model one read suffices; a sentinel left
       after the push would be a protocol error);
    3. copy: the polled rows are the output ``[M, V]``;
    4. re-arm: rows ``0 .. M-1`` of parity ``p`` are set back to the sentinel.

    The parity flips once per served call (``HeadGather.__call__`` source).
    """

    def __init__(self, tp: int, shard: int, cap: int):
        if not create_ok(tp, shard, cap):
            raise ValueError(f"invalid gather sizes tp={tp} shard={shard} cap={cap}")
        self.tp, self.shard, self.cap = tp, shard, cap
        self.vocab = tp * shard
        self.words_per_row = self.vocab // 2
        self.box = np.empty((2, cap, self.words_per_row), dtype=np.uint32)
        self.parity = 0
        self.pending: tuple[int, int] | None = None  # (m, parity) of a split push
        self.pushed: set[int] = set()                # ranks that pushed into it
        self.arm()

    # -- state ------------------------------------------------------------
    def arm(self) -> None:
        """Both parities back to all-sentinel, parity 0, no pending push."""
        self.box[...] = np.uint32(SENT_WORD)
        self.parity = 0
        self.pending = None
        self.pushed = set()

    def served(self, m: int, capturing: bool = False) -> bool:
        """Eligibility of a call (``HeadGather.__call__`` source): the row count
        must be one of the served ones (here ``1 .. cap``) and the stream must
        not be capturing a graph."""
        return 1 <= m <= self.cap and not capturing

    # -- the four steps ----------------------------------------------------
    def _push(self, p: int, shards, m: int, ranks=None) -> None:
        half = self.shard // 2
        for r in (range(self.tp) if ranks is None else sorted(ranks)):
            rows = np.asarray(shards[r], dtype=np.uint16)
            if rows.shape != (m, self.shard):
                raise ValueError(f"rank {r} shard has shape {rows.shape}, expected {(m, self.shard)}")
            self.box[p, :m, r * half:(r + 1) * half] = rewrite_sentinel(pack_words(rows))

    def _poll(self, p: int, m: int, bounded: bool = False) -> np.ndarray:
        rows = self.box[p, :m, :].copy()
        if not bounded and np.any(rows == np.uint32(SENT_WORD)):
            raise AssertionError("a polled word is still the sentinel after the push")
        return rows

    def _rearm(self, p: int, m: int) -> None:
        self.box[p, :m, :] = np.uint32(SENT_WORD)

    # -- calls -------------------------------------------------------------
    def gather(self, shards, capturing: bool = False):
        """One call of the fused gather. Returns ``(status, out)``.

        ``status`` is ``OK`` for a served call (``out`` is the gathered
        ``[M, V]`` BF16 patterns) or ``DECLINE`` (``out`` is the stock result
        and no state changed). A call while a split push is pending is a state
        error (``ESTATE``, ``out`` None).
        """
        m = int(np.asarray(shards[0]).shape[0])
        if self.pending is not None:
            return ESTATE, None
        if not self.served(m, capturing):
            return DECLINE, stock_concat(shards)
        p = self.parity
        self.parity ^= 1
        self._push(p, shards, m)
        words = self._poll(p, m)
        self._rearm(p, m)
        return OK, unpack_words(words)

    def push(self, shards, capturing: bool = False) -> int:
        """Split variant, first half: every rank pushes into the current parity."""
        return self.push_ranks(shards, range(self.tp), capturing)

    def push_ranks(self, shards, ranks, capturing: bool = False) -> int:
        """Split variant: the listed ranks push their fragments into the
        current parity (``shards[r]`` is read only for those ranks). Pushes of
        disjoint rank sets with the same row count accumulate into one pending
        call; a rank pushing twice, or another row count, is a state error."""
        ranks = set(int(r) for r in ranks)
        m = int(np.asarray(shards[min(ranks)]).shape[0]) if ranks else 0
        if not ranks or any(r < 0 or r >= self.tp for r in ranks):
            return EINVAL
        if self.pending is not None and (self.pending[0] != m or ranks & self.pushed):
            return ESTATE
        if not self.served(m, capturing):
            return DECLINE
        p = self.parity if self.pending is None else self.pending[1]
        self._push(p, shards, m, ranks)
        self.pending = (m, p)
        self.pushed |= ranks
        return OK

    def collect(self, m: int, capturing: bool = False):
        """Split variant, second half: poll, copy, re-arm, flip the parity.
        Returns ``(status, out)``; ``ETIMEOUT`` when some rank never pushed."""
        if capturing:
            return DECLINE, None
        if self.pending is None or self.pending[0] != m:
            return ESTATE, None
        _, p = self.pending
        complete = len(self.pushed) == self.tp
        words = self._poll(p, m, bounded=not complete)
        self._rearm(p, m)
        self.pending = None
        self.pushed = set()
        self.parity ^= 1
        return (OK if complete else ETIMEOUT), unpack_words(words)

    def mailbox_bf16(self, parity: int) -> np.ndarray:
        """Mailbox of one parity as ``[cap, V]`` BF16 patterns."""
        return unpack_words(self.box[parity])
