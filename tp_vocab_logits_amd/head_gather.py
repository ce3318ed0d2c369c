"""``HeadGather``: the vocab-parallel lm_head's logits gather ``[M, V/TP] x TP
-> [M, V]`` (BF16) on a two-parity Lamport mailbox, through libhg.so.

Mirrors the gather object on the vLLM API documentation page
``vllm.models.kimi_k3.nvidia.specialized_decode.runtime.logits_gather``
(``HeadGather`` class): construction allocates and arms the mailbox; a call
with a served row count (1..cap) and BF16 shards of the right width, outside
graph capture, is served by one kernel launch and flips the parity; any other
call takes the stock gather (rank-order concatenation, bytes unchanged).

Torch provides the device memory and the stream (the current stream of the
context's device); the wrapper only marshals pointers.
"""

from __future__ import annotations

import ctypes
from typing import Sequence

import torch

from . import _lib
from ._lib import HG_EDECLINE, HG_OK, HgError, check, lib, pointer_array

__all__ = ["HeadGather", "HgError", "lmhead", "stock_gather"]


def _stream_handle(device: torch.device) -> ctypes.c_void_p:
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _shard_pointers(shards, tp: int) -> tuple[list[int], int, int, torch.device, torch.dtype]:
    """Device pointers of the TP shards (a ``[TP, M, S]`` tensor or a sequence
    of ``[M, S]`` tensors), plus M, S, the device and the dtype."""
    if isinstance(shards, torch.Tensor):
        if shards.dim() != 3 or shards.shape[0] != tp:
            raise ValueError(f"expected a [TP={tp}, M, S] tensor, got {tuple(shards.shape)}")
        if not shards.is_contiguous():
            raise ValueError("the stacked shard tensor must be contiguous")
        m, s = int(shards.shape[1]), int(shards.shape[2])
        step = m * s * shards.element_size()
        base = shards.data_ptr()
        return [base + r * step for r in range(tp)], m, s, shards.device, shards.dtype
    shards = list(shards)
    if len(shards) != tp:
        raise ValueError(f"expected {tp} shards, got {len(shards)}")
    m, s = (int(x) for x in shards[0].shape)
    for t in shards:
        if t.dim() != 2 or tuple(t.shape) != (m, s) or not t.is_contiguous():
            raise ValueError("every shard must be a contiguous [M, S] tensor of one shape")
        if t.dtype != shards[0].dtype or t.device != shards[0].device:
            raise ValueError("shards must share dtype and device")
    return [t.data_ptr() for t in shards], m, s, shards[0].device, shards[0].dtype


def stock_gather(shards: torch.Tensor | Sequence[torch.Tensor], tp: int,
                 out: torch.Tensor | None = None, vocab: int | None = None) -> torch.Tensor:
    """The stock gather: rank-order concatenation ``[M, TP*S]``, bytes
    unchanged (the single-device share of an all-gather followed by the copy to
    ``[M, V]``), of which the library's kernel writes the first ``vocab``
    columns (default: all). The shards must be on a CUDA device and their rows
    a whole number of 2-byte units (any dtype: the concatenation only moves
    bytes)."""
    ptrs, m, s, device, dtype = _shard_pointers(shards, tp)
    if device.type != "cuda":
        raise ValueError(f"shards must be on a CUDA device, got {device}")
    cols = tp * s if vocab is None else int(vocab)
    if not 1 <= cols <= tp * s:
        raise ValueError(f"vocab must lie in 1..{tp * s}, got {cols}")
    if out is None:
        out = torch.empty((m, cols), dtype=dtype, device=device)
    elif out.dtype != dtype or tuple(out.shape) != (m, cols) or not out.is_contiguous():
        raise ValueError(f"out must be a contiguous {dtype} [{m}, {cols}] tensor")
    esize = torch.empty((), dtype=dtype).element_size()
    if (s * esize) % 2 or (cols * esize) % 2:
        raise ValueError("the stock gather moves 2-byte units: row widths in bytes must be even")
    if m == 0:
        return out
    with torch.cuda.device(device):
        # the kernel counts widths in 2-byte units
        check(lib().hg_stock_gather(tp, s * esize // 2, pointer_array(ptrs), m,
                                    ctypes.c_void_p(out.data_ptr()), cols * esize // 2,
                                    _stream_handle(device)),
              "hg_stock_gather")
    return out


def _weight_pointers(w, tp: int, shard: int, hidden: int) -> list[int]:
    """Pointers of the TP head-weight blocks: a ``[TP*S, H]`` (or ``[TP, S, H]``)
    tensor, or a sequence of TP ``[S, H]`` tensors."""
    if isinstance(w, torch.Tensor):
        if w.dtype != torch.bfloat16 or not w.is_contiguous() or w.numel() != tp * shard * hidden:
            raise ValueError(f"head weight must be a contiguous BF16 [{tp * shard}, {hidden}] tensor")
        step = shard * hidden * w.element_size()
        return [w.data_ptr() + r * step for r in range(tp)]
    w = list(w)
    if len(w) != tp:
        raise ValueError(f"expected {tp} weight blocks, got {len(w)}")
    for t in w:
        if t.dtype != torch.bfloat16 or tuple(t.shape) != (shard, hidden) or not t.is_contiguous():
            raise ValueError(f"every weight block must be a contiguous BF16 [{shard}, {hidden}] tensor")
    return [t.data_ptr() for t in w]


def lmhead(x: torch.Tensor, w, tp: int, shard: int,
           shards_out: torch.Tensor | None = None) -> torch.Tensor:
    """The lm_head shard product ``[TP, M, S] = X @ W_r^T`` per rank (BF16 in,
    fp32 accumulate, BF16 out), in the library's MFMA kernel."""
    if x.dtype != torch.bfloat16 or x.dim() != 2 or not x.is_contiguous():
        raise ValueError("x must be a contiguous BF16 [M, H] tensor")
    m, hidden = (int(v) for v in x.shape)
    wp = _weight_pointers(w, tp, shard, hidden)
    if shards_out is None:
        shards_out = torch.empty((tp, m, shard), dtype=torch.bfloat16, device=x.device)
    elif (shards_out.dtype != torch.bfloat16 or tuple(shards_out.shape) != (tp, m, shard)
          or not shards_out.is_contiguous()):
        raise ValueError(f"shards_out must be a contiguous BF16 [{tp}, {m}, {shard}] tensor")
    step = m * shard * 2
    op = [shards_out.data_ptr() + r * step for r in range(tp)]
    with torch.cuda.device(x.device):
        check(lib().hg_lmhead(tp, shard, ctypes.c_void_p(x.data_ptr()), pointer_array(wp), hidden, m,
                              pointer_array(op), _stream_handle(x.device)), "hg_lmhead")
    return shards_out


class HeadGather:
    """One gather context: ``tp`` virtual ranks of ``shard`` BF16 columns, up to
    ``cap`` rows per call, on ``device`` (default: the current CUDA device).
    ``vocab`` (default ``tp * shard``) is the real vocabulary: outputs are
    ``[M, vocab]``, the padded-vocab slice of each gathered row, taken inside
    the copy step (``hg_set_vocab``); declined calls return the same slice of
    the stock gather."""

    def __init__(self, tp: int, shard: int, cap: int, device: torch.device | int | None = None,
                 vocab: int | None = None):
        if device is None:
            index = torch.cuda.current_device()
        elif isinstance(device, int):
            index = device
        else:
            d = torch.device(device)
            index = d.index if d.index is not None else torch.cuda.current_device()
        self.device = torch.device("cuda", index)
        self.tp, self.shard, self.cap = int(tp), int(shard), int(cap)
        self.width = self.tp * self.shard  # V, the padded vocabulary
        self._h = ctypes.c_void_p()
        with torch.cuda.device(self.device):
            check(lib().hg_create(self.tp, self.shard, self.cap, ctypes.byref(self._h)), "hg_create")
        self.vocab = self.width
        if vocab is not None:
            self.set_vocab(vocab)

    def set_vocab(self, vocab: int) -> None:
        """Output columns per row from the next call on (1..V)."""
        check(lib().hg_set_vocab(self._h, int(vocab)), "hg_set_vocab")
        self.vocab = int(vocab)

    # -- lifetime ----------------------------------------------------------
    def close(self) -> None:
        if self._h:
            with torch.cuda.device(self.device):
                check(lib().hg_destroy(self._h), "hg_destroy")
            self._h = ctypes.c_void_p()

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    # -- calls -------------------------------------------------------------
    def _eligible(self, ptrs_m_s_dev_dt) -> bool:
        _, m, s, device, dtype = ptrs_m_s_dev_dt
        return dtype == torch.bfloat16 and s == self.shard and device == self.device

    def _out(self, m: int, out: torch.Tensor | None) -> torch.Tensor:
        if out is None:
            return torch.empty((m, self.vocab), dtype=torch.bfloat16, device=self.device)
        if out.dtype != torch.bfloat16 or tuple(out.shape) != (m, self.vocab) or not out.is_contiguous():
            raise ValueError(f"out must be a contiguous BF16 [{m}, {self.vocab}] tensor")
        return out

    def _stock(self, shards, s: int, out: torch.Tensor | None) -> torch.Tensor:
        """The stock gather; shards of this context's width keep the
        vocabulary's columns like a served call (the library's stock kernel
        writes only those)."""
        return stock_gather(shards, self.tp, out, self.vocab if s == self.shard else None)

    def __call__(self, shards, out: torch.Tensor | None = None) -> torch.Tensor:
        """Gather ``[M, S]`` x TP -> ``[M, vocab]``. Served calls run the fused
        kernel and flip the parity; declined calls return the stock gather."""
        info = _shard_pointers(shards, self.tp)
        ptrs, m = info[0], info[1]
        if not self._eligible(info):
            return self._stock(shards, info[2], out)
        out = self._out(m, out)
        with torch.cuda.device(self.device):
            rc = lib().hg_gather(self._h, pointer_array(ptrs), m, ctypes.c_void_p(out.data_ptr()),
                                 _stream_handle(self.device))
        if rc == HG_EDECLINE:
            return self._stock(shards, info[2], out)
        check(rc, "hg_gather")
        return out

    def push(self, shards) -> bool:
        """Split variant, first half. Returns False when declined."""
        info = _shard_pointers(shards, self.tp)
        if not self._eligible(info):
            return False
        with torch.cuda.device(self.device):
            rc = lib().hg_push(self._h, pointer_array(info[0]), info[1], _stream_handle(self.device))
        return check(rc, "hg_push") == HG_OK

    def push_ranks(self, shards, ranks) -> bool:
        """Split variant, partial push by the listed ranks only (``shards`` must
        still hold TP entries; the others are not read). False when declined."""
        info = _shard_pointers(shards, self.tp)
        if not self._eligible(info):
            return False
        mask = 0
        for r in ranks:
            mask |= 1 << int(r)
        with torch.cuda.device(self.device):
            rc = lib().hg_push_ranks(self._h, pointer_array(info[0]), info[1], mask,
                                     _stream_handle(self.device))
        return check(rc, "hg_push_ranks") == HG_OK

    def collect(self, m: int, out: torch.Tensor | None = None) -> torch.Tensor:
        """Split variant, second half: the gathered ``[m, vocab]`` logits."""
        out = self._out(m, out)
        with torch.cuda.device(self.device):
            rc = lib().hg_collect(self._h, m, ctypes.c_void_p(out.data_ptr()),
                                  _stream_handle(self.device))
        if rc == HG_EDECLINE:
            raise HgError(_lib.HG_ESTATE, "hg_collect declined (stream capturing)")
        check(rc, "hg_collect")
        return out

    def gemm_gather(self, x: torch.Tensor, w, out: torch.Tensor | None = None,
                    shards_out: torch.Tensor | None = None) -> torch.Tensor:
        """Producer + gather: the lm_head product ``X @ W_r^T`` with its
        epilogue pushing into the mailbox, then poll/copy/re-arm. ``w`` is the
        ``[TP*S, H]`` head weight (or TP ``[S, H]`` blocks). When given,
        ``shards_out`` ``[TP, M, S]`` also receives the product's BF16 shards.
        Raises on a declined call (no stock producer exists here)."""
        if x.dtype != torch.bfloat16 or x.dim() != 2 or not x.is_contiguous():
            raise ValueError("x must be a contiguous BF16 [M, H] tensor")
        m, hidden = (int(v) for v in x.shape)
        wp = _weight_pointers(w, self.tp, self.shard, hidden)
        out = self._out(m, out)
        op = None
        if shards_out is not None:
            if (shards_out.dtype != torch.bfloat16 or tuple(shards_out.shape) != (self.tp, m, self.shard)
                    or not shards_out.is_contiguous()):
                raise ValueError("shards_out must be a contiguous BF16 [TP, M, S] tensor")
            step = m * self.shard * 2
            op = pointer_array([shards_out.data_ptr() + r * step for r in range(self.tp)])
        with torch.cuda.device(self.device):
            rc = lib().hg_gemm_gather(self._h, ctypes.c_void_p(x.data_ptr()), pointer_array(wp), hidden,
                                      m, ctypes.c_void_p(out.data_ptr()), op,
                                      _stream_handle(self.device))
        if rc == HG_EDECLINE:
            raise HgError(_lib.HG_EINVAL, "hg_gemm_gather declined (rows outside 1..cap or capturing)")
        check(rc, "hg_gemm_gather")
        return out

    def arm(self) -> None:
        with torch.cuda.device(self.device):
            check(lib().hg_arm(self._h, _stream_handle(self.device)), "hg_arm")

    # -- state -------------------------------------------------------------
    @property
    def parity(self) -> int:
        return check(lib().hg_parity(self._h), "hg_parity")

    def mailbox(self, parity: int) -> torch.Tensor:
        """A copy of one parity of the mailbox as ``[cap, V]`` BF16 (stream-ordered)."""
        dst = torch.empty((self.cap, self.width), dtype=torch.bfloat16, device=self.device)
        with torch.cuda.device(self.device):
            check(lib().hg_copy_mailbox(self._h, parity, ctypes.c_void_p(dst.data_ptr()),
                                        _stream_handle(self.device)), "hg_copy_mailbox")
        return dst

    def set_device_parity(self, enable: bool) -> None:
        """Keep the parity in device memory so calls can be captured into a
        graph and replayed (see ``hg_set_device_parity``)."""
        with torch.cuda.device(self.device):
            check(lib().hg_set_device_parity(self._h, 1 if enable else 0, _stream_handle(self.device)),
                  "hg_set_device_parity")

    def set_poll_limit(self, spins: int) -> None:
        check(lib().hg_set_poll_limit(self._h, int(spins)), "hg_set_poll_limit")

    def poll_status(self) -> int:
        """HG_OK, or HG_ETIMEOUT if a bounded poll gave up since the last check."""
        with torch.cuda.device(self.device):
            rc = lib().hg_poll_status(self._h, _stream_handle(self.device))
        if rc == _lib.HG_ETIMEOUT:
            return rc
        return check(rc, "hg_poll_status")

    def fused_grid_limit(self, m: int) -> int:
        with torch.cuda.device(self.device):
            return check(lib().hg_fused_grid_limit(self._h, int(m)), "hg_fused_grid_limit")

    @property
    def handle(self) -> ctypes.c_void_p:
        return self._h
