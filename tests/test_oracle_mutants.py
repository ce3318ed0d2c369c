"""Plant plausible mistakes in the CPU oracle and check that its pins catch
every one of them (no GPU). Each mutant is patched into the oracle module for
the duration of one test only."""

import numpy as np
import pytest

import oracle_pins as pins
from oracle import gather, gemm


def _pack_swapped(elems):
    e = np.asarray(elems, dtype=np.uint16)
    return (e[..., 1::2].astype(np.uint32)) | (e[..., 0::2].astype(np.uint32) << np.uint32(16))


def _unpack_swapped(words):
    w = np.asarray(words, dtype=np.uint32)
    out = np.empty(w.shape[:-1] + (2 * w.shape[-1],), np.uint16)
    out[..., 1::2] = (w & 0xFFFF).astype(np.uint16)
    out[..., 0::2] = (w >> 16).astype(np.uint16)
    return out


def _rewrite_any_neg_zero_high(words):
    w = np.asarray(words, dtype=np.uint32)
    return np.where((w >> 16) == 0x8000, w & np.uint32(0xFFFF), w).astype(np.uint32)


def _rewrite_to_neg_pair(words):
    w = np.asarray(words, dtype=np.uint32)
    return np.where(w == 0x80000000, np.uint32(0x80008000), w).astype(np.uint32)


def _rewrite_nothing(words):
    return np.asarray(words, dtype=np.uint32).copy()


def _concat_reversed(shards):
    return np.concatenate([np.asarray(s, np.uint16) for s in shards][::-1], axis=1)


def _concat_rank_major(shards):
    st = np.stack([np.asarray(s, np.uint16) for s in shards])  # [tp, m, s]
    return st.reshape(st.shape[1], -1)                          # missing transpose


def _create_ok_mod4(tp, shard, cap):
    return tp >= 2 and shard >= 4 and shard % 4 == 0 and cap >= 1


def _create_ok_tp1(tp, shard, cap):
    return tp >= 1 and shard >= 8 and shard % 8 == 0 and cap >= 1


class _SimNoFlip(gather.MailboxSim):
    def gather(self, shards, capturing=False):
        status, out = super().gather(shards, capturing)
        if status == gather.OK:
            self.parity ^= 1
        return status, out


class _SimFlipOnDecline(gather.MailboxSim):
    def gather(self, shards, capturing=False):
        status, out = super().gather(shards, capturing)
        if status == gather.DECLINE:
            self.parity ^= 1
        return status, out


class _SimNoRearm(gather.MailboxSim):
    def _rearm(self, p, m):
        pass


class _SimPushWrongColumns(gather.MailboxSim):
    def _push(self, p, shards, m):
        # element offsets used as word offsets: rank r lands at word r*S instead of r*S/2
        half = self.shard // 2
        for r in range(self.tp):
            w = gather.rewrite_sentinel(gather.pack_words(np.asarray(shards[r], np.uint16)))
            lo = (r * self.shard) % self.words_per_row
            self.box[p, :m, lo:lo + half] = w


class _SimPushAllRows(gather.MailboxSim):
    def _push(self, p, shards, m):
        super()._push(p, shards, m)
        if m < self.cap:
            self.box[p, m:, :] = 0


class _SimPushOtherParity(gather.MailboxSim):
    def push(self, shards, capturing=False):
        self.parity ^= 1
        status = super().push(shards, capturing)
        self.parity ^= 1
        return status


class _SimServesCapAndOne(gather.MailboxSim):
    def served(self, m, capturing=False):
        return 1 <= m <= self.cap + 1 and not capturing


class _SimIgnoresCapture(gather.MailboxSim):
    def served(self, m, capturing=False):
        return 1 <= m <= self.cap


class _SimArmKeepsParity(gather.MailboxSim):
    def arm(self):
        p = getattr(self, "parity", 0)
        super().arm()
        self.parity = p


class _SimCollectIgnoresMissing(gather.MailboxSim):
    def collect(self, m, capturing=False):
        self.pushed = set(range(self.tp)) if self.pending is not None else self.pushed
        return super().collect(m, capturing)


class _SimPartialPushAll(gather.MailboxSim):
    def push_ranks(self, shards, ranks, capturing=False):
        ranks = set(int(r) for r in ranks)
        status = super().push_ranks(shards, ranks, capturing)
        if status == gather.OK:
            m, p = self.pending
            self._push(p, shards, m)
        return status


def _lm_head_untransposed(x_bits, w_bits):
    x, w = gemm.bf16_to_f64(x_bits), gemm.bf16_to_f64(w_bits)
    return x @ w.reshape(w.shape[1], w.shape[0])


def _lm_head_dropped_term(x_bits, w_bits):
    x, w = gemm.bf16_to_f64(x_bits), gemm.bf16_to_f64(w_bits)
    return x[:, 1:] @ w[:, 1:].T


def _lm_head_wrong_sign(x_bits, w_bits):
    x, w = gemm.bf16_to_f64(x_bits), gemm.bf16_to_f64(w_bits)
    return np.abs(x) @ w.T


def _lm_head_half(x_bits, w_bits):
    x, w = gemm.bf16_to_f64(x_bits).astype(np.float16), gemm.bf16_to_f64(w_bits).astype(np.float16)
    return (x.astype(np.float32) @ w.T.astype(np.float32)).astype(np.float64)


def _round_truncate(values):
    v = np.asarray(values, dtype=np.float64).astype(np.float32)
    return (v.view(np.uint32) >> 16).astype(np.uint16)


def _round_ties_away(values):
    v = np.asarray(values, dtype=np.float64).astype(np.float32)
    return ((v.view(np.uint32) + np.uint32(0x8000)) >> 16).astype(np.uint16)


def _bf16_to_f64_wrong_shift(bits):
    b = np.asarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(15)).view(np.float32).astype(np.float64)


def _rel_err_squared(approx_bits, exact):
    approx = gemm.bf16_to_f64(approx_bits)
    exact = np.asarray(exact, dtype=np.float64)
    return float(np.sum((approx - exact) ** 2) / np.sum(exact ** 2))


def _rel_err_over_approx(approx_bits, exact):
    approx = gemm.bf16_to_f64(approx_bits)
    exact = np.asarray(exact, dtype=np.float64)
    return float(np.linalg.norm(approx - exact) / np.linalg.norm(approx))


def _rel_err_max_abs(approx_bits, exact):
    approx = gemm.bf16_to_f64(approx_bits)
    exact = np.asarray(exact, dtype=np.float64)
    return float(np.max(np.abs(approx - exact)) / np.max(np.abs(exact)))


def _slice_tail(out, vocab):
    out = np.asarray(out, np.uint16)
    return out[:, out.shape[1] - vocab:].copy()


def _slice_one_short(out, vocab):
    out = np.asarray(out, np.uint16)
    if not 1 <= vocab <= out.shape[1]:
        raise ValueError("vocab")
    keep = out[:, :vocab].copy()
    keep[:, -1] = 0
    return keep


MUTANTS = [
    ("vocab slice keeps the last columns", gather, {"slice_vocab": _slice_tail}),
    ("vocab slice drops its last column", gather, {"slice_vocab": _slice_one_short}),
    ("pack high/low swapped", gather, {"pack_words": _pack_swapped, "unpack_words": _unpack_swapped}),
    ("sentinel constant (-0,+0)", gather, {"SENT_WORD": 0x00008000}),
    ("rewrites any word with -0 high half", gather, {"rewrite_sentinel": _rewrite_any_neg_zero_high}),
    ("rewrites sentinel to (-0,-0)", gather, {"rewrite_sentinel": _rewrite_to_neg_pair}),
    ("no rewrite at all", gather, {"rewrite_sentinel": _rewrite_nothing}),
    ("ranks concatenated in reverse", gather, {"stock_concat": _concat_reversed}),
    ("rank-major layout without transpose", gather, {"stock_concat": _concat_rank_major}),
    ("create accepts shard % 4", gather, {"create_ok": _create_ok_mod4}),
    ("create accepts tp == 1", gather, {"create_ok": _create_ok_tp1}),
    ("parity never flips", gather, {"MailboxSim": _SimNoFlip}),
    ("decline flips parity", gather, {"MailboxSim": _SimFlipOnDecline}),
    ("no re-arm", gather, {"MailboxSim": _SimNoRearm}),
    ("push at element offsets", gather, {"MailboxSim": _SimPushWrongColumns}),
    ("push touches rows >= M", gather, {"MailboxSim": _SimPushAllRows}),
    ("split push into the other parity", gather, {"MailboxSim": _SimPushOtherParity}),
    ("serves cap + 1 rows", gather, {"MailboxSim": _SimServesCapAndOne}),
    ("serves under graph capture", gather, {"MailboxSim": _SimIgnoresCapture}),
    ("arm keeps the parity", gather, {"MailboxSim": _SimArmKeepsParity}),
    ("collect ignores a missing rank", gather, {"MailboxSim": _SimCollectIgnoresMissing}),
    ("partial push writes every rank", gather, {"MailboxSim": _SimPartialPushAll}),
    ("lm_head weight not transposed", gemm, {"lm_head_shard": _lm_head_untransposed}),
    ("lm_head drops a term", gemm, {"lm_head_shard": _lm_head_dropped_term}),
    ("lm_head loses a sign", gemm, {"lm_head_shard": _lm_head_wrong_sign}),
    ("lm_head in half precision", gemm, {"lm_head_shard": _lm_head_half}),
    ("bf16 rounding truncates", gemm, {"round_to_bf16": _round_truncate}),
    ("bf16 rounding ties away", gemm, {"round_to_bf16": _round_ties_away}),
    ("bf16 decode shifted wrong", gemm, {"bf16_to_f64": _bf16_to_f64_wrong_shift}),
    ("relative error squared", gemm, {"relative_frobenius_error": _rel_err_squared}),
    ("relative error over the approximation's norm", gemm,
     {"relative_frobenius_error": _rel_err_over_approx}),
    ("relative error as a max-norm ratio", gemm, {"relative_frobenius_error": _rel_err_max_abs}),
]


@pytest.mark.parametrize("name,module,patch", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_mutant_is_caught(name, module, patch, monkeypatch):
    for attr, value in patch.items():
        monkeypatch.setattr(module, attr, value)
    checks = pins.GATHER_CHECKS if module is gather else pins.GEMM_CHECKS
    caught = []
    for check in checks:
        try:
            check(module)
        except Exception as exc:  # an AssertionError, or the mutant breaking a shape contract
            caught.append((check.__name__, type(exc).__name__))
    assert caught, f"mutant '{name}' passed every pin"
