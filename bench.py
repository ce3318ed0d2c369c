#!/usr/bin/env python3
"""Benchmark of the one-shot Lamport-mailbox logits gather on one MI355X.

Prints ONE JSON line. The timed step is one decode gather -- TP=8 virtual
ranks, V=163840, M=1 row, mailbox cap 8 -- issued K times back to back on one
stream with every input already resident in HBM (8 input sets cycled, K
distinct outputs); ``value`` is microseconds per gather from HIP events around
the K calls. The same run measures the M=256 gather (the bandwidth half of the
metric) on three rotating buffer sets, so each call's inputs were evicted from
the 256 MB Infinity Cache by the two calls before it, and reports its
algorithmic bandwidth against the 8 TB/s HBM peak in ``roofline``. The CPU
oracle is timed on a bounded sample of the same inputs (``cpu_baseline``) and
its results double as the check of the GPU outputs; a mismatch aborts the run.

Algorithmic bytes per gather: 5 * M * V * 2 (shard read, mailbox push write,
mailbox poll read, output write, re-arm write).

The JSON line also carries ``decode_graph``: the same K decode gathers
captured into one HIP graph, with the parity kept in device memory, replayed
and timed per gather; and ``decode_split``: the same gathers through the split
variant (push, then collect).

Modes: default (the JSON line); ``--pmc-probe`` runs only a plain 256 MiB copy
and the M=256 fused gather a few times, for ``rocprofv3 --pmc`` counter runs;
``--gemm-probe`` runs only the M=256 lm_head product (``--gemm-probe-calls`` times, 3 by
default), likewise;
``--graph-only`` runs only the graph-replay leg (checked against the oracle),
for a kernel trace of it.
"""

from __future__ import annotations

import argparse
import ctypes
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "µs per logits gather at M=1 (V=163840, TP=8) + achieved HBM GB/s at M=256"
HBM_PEAK_GBPS = 8000.0
COUNTERS = os.path.join(ROOT, "profiles", "fused_gather_m256_counters.json")
# rocprofv3 kernel traces of this benchmark's M=1 decode gather: the eager
# legs (bench.py --no-cpu --no-graph) and the graph-replay leg
# (bench.py --graph-only), reduced to the fused kernel's median duration
M1_TRACES = {"eager": os.path.join(ROOT, "profiles", "gather_kernels_decode_m1_and_m256.json"),
             "graph": os.path.join(ROOT, "profiles", "fused_gather_decode_m1_graph_replay.json")}


def log(msg: str) -> None:
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def kernel_source_hash() -> str:
    """Hash of the sources that fix the gather kernels and their launch shapes
    (the one the counter summary in profiles/ records)."""
    from tp_vocab_logits_amd.profiling import kernel_source_hash as h

    return h()


def current_profiles(paths: dict, counters: str, variant: str, source_hash: str):
    """The committed profile summaries that still describe the current kernel
    sources: the M=1 fused gather's kernel times per leg (JSON files of
    ``paths``, keyed by leg) and the M=256 traffic per launch from the counter
    summary ``counters`` (for ``variant``). A summary taken on other sources
    (another hash) is left out; a missing file too."""
    m1 = {}
    for leg, path in paths.items():
        if os.path.exists(path):
            with open(path) as f:
                t = json.load(f)
            if t.get("kernel_source_sha256_16") == source_hash:
                m1[leg] = t
    traffic = None
    if os.path.exists(counters):
        with open(counters) as f:
            c = json.load(f)
        if c.get("kernel_source_sha256_16") == source_hash and c.get("variant") == variant:
            traffic = c.get("traffic_bytes_per_launch")
    return m1, traffic


def parse_args():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=1000, help="timed M=1 gathers")
    ap.add_argument("--warmup", type=int, default=100, help="untimed M=1 gathers first")
    ap.add_argument("--large-steps", type=int, default=60, help="timed M=256 gathers")
    ap.add_argument("--variant", choices=["fused", "split"], default="fused")
    ap.add_argument("--no-cpu", action="store_true", help="skip the cpu_baseline leg")
    ap.add_argument("--pmc-probe", action="store_true")
    ap.add_argument("--gemm-probe", action="store_true",
                    help="run only the M=256 lm_head product, --gemm-probe-calls times back to back")
    ap.add_argument("--gemm-probe-calls", type=int, default=3,
                    help="products the --gemm-probe run launches")
    ap.add_argument("--no-graph", dest="graph", action="store_false",
                    help="skip the graph-replay leg of the M=1 decode gather")
    ap.add_argument("--graph-only", action="store_true",
                    help="run only the graph-replay leg (for a kernel trace of it), check it, exit")
    ap.add_argument("--producer-steps", type=int, default=20,
                    help="timed M=256 lm_head producer + gather calls (0: skip)")
    return ap.parse_args()


class Timer:
    """HIP events on the stream the kernels are launched on."""

    def __init__(self, torch, stream):
        self.torch, self.stream = torch, stream

    def __enter__(self):
        self.torch.cuda.synchronize()
        self.t0 = self.torch.cuda.Event(enable_timing=True)
        self.t1 = self.torch.cuda.Event(enable_timing=True)
        self.t0.record(self.stream)
        return self

    def __exit__(self, *exc):
        self.t1.record(self.stream)
        self.t1.synchronize()
        self.torch.cuda.synchronize()
        self.ms = self.t0.elapsed_time(self.t1)


def main() -> int:
    args = parse_args()
    if args.gpus != 1:
        print(json.dumps({"error": f"--gpus {args.gpus}: this benchmark runs on one GPU only; "
                          "the TP ranks are virtual ranks inside that GPU"}))
        return 2

    import numpy as np
    import torch

    from tp_vocab_logits_amd import _lib
    from tp_vocab_logits_amd import synthetic as syn
    from tp_vocab_logits_amd.head_gather import HeadGather

    if not torch.cuda.is_available():
        log("no GPU visible")
        return 3
    lib = _lib.lib()
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream(dev)
    sh = ctypes.c_void_p(stream.cuda_stream)

    # the per-call entry points through the fast-call binding: plain integers
    # (handle, host-array address, rows, device address, stream)
    fast = _lib.fast()
    shi = stream.cuda_stream

    def call_fn(hg, variant):
        h = hg.handle.value
        if variant == "fused":
            g = fast.gather
            return lambda ptrs, m, out: g(h, ptrs, m, out, shi)
        push, collect = fast.push, fast.collect

        def split(ptrs, m, out):
            rc = push(h, ptrs, m, shi)
            return rc if rc else collect(h, m, out, shi)
        return split

    if args.gemm_probe:
        wl = syn.WORKLOADS["fused"]
        xg = torch.randn(wl.rows, wl.hidden, device=dev).mul_(0.02).to(torch.bfloat16)
        wg = torch.randn(wl.tp, wl.shard, wl.hidden, device=dev).mul_(0.02).to(torch.bfloat16)
        sg = torch.empty((wl.tp, wl.rows, wl.shard), dtype=torch.bfloat16, device=dev)
        wptrs = _lib.pointer_array([wg[r].data_ptr() for r in range(wl.tp)])
        sptrs = _lib.pointer_array([sg[r].data_ptr() for r in range(wl.tp)])
        for _ in range(args.gemm_probe_calls):
            rc = lib.hg_lmhead(wl.tp, wl.shard, ctypes.c_void_p(xg.data_ptr()), wptrs, wl.hidden,
                               wl.rows, sptrs, sh)
            if rc:
                raise _lib.HgError(rc, "hg_lmhead")
        torch.cuda.synchronize()
        log(f"gemm probe done: {args.gemm_probe_calls} x lm_head X[256,7168] @ W[163840,7168]^T")
        return 0

    # ---------------- M=256 inputs (three rotation sets) --------------------
    wl = syn.WORKLOADS["fused"]
    big_sets = []
    for k in range(3):
        b = syn.shard_set(wl, k)
        syn.inject_sentinel_words(b, 0.001, 9000 + k)
        big_sets.append(b)
    big_dev = [syn.to_torch_bf16(b, dev) for b in big_sets]
    big_out = [torch.empty((wl.rows, wl.vocab), dtype=torch.bfloat16, device=dev) for _ in range(3)]
    big_ptrs = [_lib.pointer_array([t[r].data_ptr() for r in range(wl.tp)]) for t in big_dev]
    big_outp = [ctypes.c_void_p(o.data_ptr()) for o in big_out]
    big_addr = [ctypes.addressof(a) for a in big_ptrs]
    big_oaddr = [o.data_ptr() for o in big_out]
    hg_big = HeadGather(wl.tp, wl.shard, wl.cap, device=dev)
    big_bytes = 5 * wl.rows * wl.vocab * 2

    if args.pmc_probe:
        src = torch.empty(256 << 20, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        fn = call_fn(hg_big, "fused")
        for _ in range(3):
            dst.copy_(src)
        for n in range(6):
            assert fn(big_addr[n % 3], wl.rows, big_oaddr[n % 3]) == 0
        torch.cuda.synchronize()
        log("pmc probe done: 3 x 256 MiB copy, 6 x M=256 fused gather")
        return 0

    # ---------------- decode: M=1, the timed step --------------------------
    wd = syn.WORKLOADS["decode"]
    dec_sets = [syn.shard_set(wd, k) for k in range(wd.pool)]
    dec_dev = [syn.to_torch_bf16(b, dev) for b in dec_sets]
    dec_ptrs = [_lib.pointer_array([t[r].data_ptr() for r in range(wd.tp)]) for t in dec_dev]
    hg = HeadGather(wd.tp, wd.shard, wd.cap, device=dev)
    n_out = max(args.steps, 1)
    outs = torch.empty((n_out, wd.rows, wd.vocab), dtype=torch.bfloat16, device=dev)
    dec_addr = [ctypes.addressof(a) for a in dec_ptrs]
    out_addr = [outs[n].data_ptr() for n in range(n_out)]
    fn = call_fn(hg, args.variant)

    # ---------------- decode, captured: the same K gathers replayed from a graph
    # (parity kept in device memory so that every replay alternates it)
    def graph_leg():
        hg_g = HeadGather(wd.tp, wd.shard, wd.cap, device=dev)
        hg_g.set_device_parity(True)
        g_outs = torch.empty((n_out, wd.rows, wd.vocab), dtype=torch.bfloat16, device=dev)
        g_ptrs = [ctypes.c_void_p(g_outs[n].data_ptr()) for n in range(n_out)]
        side = torch.cuda.Stream(device=dev)
        side.wait_stream(stream)
        graph = torch.cuda.CUDAGraph()
        rc = 0
        with torch.cuda.graph(graph, stream=side):
            gs = ctypes.c_void_p(side.cuda_stream)
            for n in range(args.steps):
                rc |= lib.hg_gather(hg_g.handle, dec_ptrs[n % wd.pool], wd.rows, g_ptrs[n], gs)
        if rc:
            raise _lib.HgError(-abs(rc), "graph capture")
        graph.replay()
        torch.cuda.synchronize()
        log(f"decode graph replay of {args.steps} captured gathers")
        with Timer(torch, stream) as t_g:
            graph.replay()
        return t_g.ms * 1000.0 / args.steps, hg_g, g_outs

    if args.graph_only:
        from oracle import gather as og

        us, hg_g, g_outs = graph_leg()
        got = g_outs[: wd.pool].cpu().contiguous().view(torch.int16).numpy().view(np.uint16)
        for k in range(min(wd.pool, args.steps)):
            if not np.array_equal(got[k], og.gather_definition(list(dec_sets[k]))):
                log(f"FAIL: graph-replayed decode output of call {k} differs from the oracle")
                return 1
        if hg_g.parity != 0 or hg_g.poll_status() != _lib.HG_OK:
            log("FAIL: device parity or poll status after the graph replays")
            return 1
        log(f"graph-only: {us:.3f} us per captured M=1 gather; outputs match the oracle")
        return 0

    log(f"decode warmup {args.warmup}")
    for n in range(args.warmup):
        rc = fn(dec_addr[n % wd.pool], wd.rows, out_addr[n % n_out])
        if rc:
            raise _lib.HgError(rc, "warmup")
    log(f"decode timed {args.steps} gathers ({args.variant})")
    rcs = 0
    with Timer(torch, stream) as t_dec:
        for n in range(args.steps):
            rcs |= fn(dec_addr[n % wd.pool], wd.rows, out_addr[n])
    if rcs:
        raise _lib.HgError(-abs(rcs), "timed decode loop")
    us_m1 = t_dec.ms * 1000.0 / args.steps

    us_graph = None
    if args.variant == "fused" and args.graph:
        us_graph, hg_g, g_outs = graph_leg()

    # ---------------- decode, split variant: push + collect per gather ------
    us_split = None
    if args.variant == "fused":
        hg_s = HeadGather(wd.tp, wd.shard, wd.cap, device=dev)
        s_outs = torch.empty((n_out, wd.rows, wd.vocab), dtype=torch.bfloat16, device=dev)
        s_addr = [s_outs[n].data_ptr() for n in range(n_out)]
        fs = call_fn(hg_s, "split")
        for n in range(args.warmup):
            if fs(dec_addr[n % wd.pool], wd.rows, s_addr[n % n_out]):
                raise _lib.HgError(-1, "split warmup")
        log(f"decode timed {args.steps} split gathers (push + collect)")
        with Timer(torch, stream) as t_split:
            for n in range(args.steps):
                rcs |= fs(dec_addr[n % wd.pool], wd.rows, s_addr[n])
        if rcs:
            raise _lib.HgError(-abs(rcs), "timed split loop")
        us_split = t_split.ms * 1000.0 / args.steps

    # ---------------- M=256 gather: cold (rotating) and back-to-back -------
    fn_big = call_fn(hg_big, args.variant)
    for n in range(6):
        assert fn_big(big_addr[n % 3], wl.rows, big_oaddr[n % 3]) == 0
    log(f"M=256 timed {args.large_steps} gathers, 3 rotating sets")
    with Timer(torch, stream) as t_cold:
        for n in range(args.large_steps):
            rcs |= fn_big(big_addr[n % 3], wl.rows, big_oaddr[n % 3])
    with Timer(torch, stream) as t_hot:
        for n in range(args.large_steps):
            rcs |= fn_big(big_addr[0], wl.rows, big_oaddr[0])
    if rcs:
        raise _lib.HgError(-abs(rcs), "timed M=256 loop")
    us_cold = t_cold.ms * 1000.0 / args.large_steps
    us_hot = t_hot.ms * 1000.0 / args.large_steps
    gbps_cold = big_bytes / (us_cold * 1e-6) / 1e9
    gbps_hot = big_bytes / (us_hot * 1e-6) / 1e9

    # ---------------- the same bytes through a plain streaming kernel -------
    # (read the shards, write mailbox-sized rows, read rows back, write an
    # output, re-arm the rows; no compare, no poll), on the same rotating
    # shard sets, cold: the practical ceiling of this read/write mix here
    ref = _lib.ref()
    props = torch.cuda.get_device_properties(dev)
    row_vectors = wl.rows * wl.vocab * 2 // 16
    ref_boxes = [torch.empty(wl.rows * wl.vocab, dtype=torch.bfloat16, device=dev) for _ in range(2)]
    ref_outs = [torch.empty(wl.rows * wl.vocab, dtype=torch.bfloat16, device=dev) for _ in range(3)]

    def ref_call(n):
        return ref.hgref_stream(big_dev[n % 3].data_ptr(), ref_boxes[n % 2].data_ptr(),
                                ref_boxes[(n + 1) % 2].data_ptr(), ref_outs[n % 3].data_ptr(),
                                row_vectors, 4 * props.multi_processor_count, sh)
    for n in range(6):
        rcs |= ref_call(n)
    log(f"M=256 plain streaming reference, {args.large_steps} calls, 3 rotating sets")
    with Timer(torch, stream) as t_ref:
        for n in range(args.large_steps):
            rcs |= ref_call(n)
    if rcs:
        raise _lib.HgError(-abs(rcs), "reference streaming loop")
    us_ref = t_ref.ms * 1000.0 / args.large_steps
    del ref_boxes, ref_outs

    # ---------------- the other workloads: tiny, spec (M=4), batched (M=64) --
    # back-to-back eager calls on their own input pools; outputs of each pool
    # set are checked in the cpu_baseline leg
    others = {}
    other_runs = {}
    for name, calls in (("tiny", 200), ("spec", 500), ("batched", 200)):
        w = syn.WORKLOADS[name]
        sets = [syn.shard_set(w, k) for k in range(w.pool)]
        sd = [syn.to_torch_bf16(b, dev) for b in sets]
        sp = [_lib.pointer_array([t[r].data_ptr() for r in range(w.tp)]) for t in sd]
        sa = [ctypes.addressof(a) for a in sp]
        so = torch.empty((w.pool, w.rows, w.vocab), dtype=torch.bfloat16, device=dev)
        soa = [so[k].data_ptr() for k in range(w.pool)]
        hw = HeadGather(w.tp, w.shard, w.cap, device=dev)
        fw = call_fn(hw, args.variant)
        for n in range(20):
            rcs |= fw(sa[n % w.pool], w.rows, soa[n % w.pool])
        with Timer(torch, stream) as t_o:
            for n in range(calls):
                rcs |= fw(sa[n % w.pool], w.rows, soa[n % w.pool])
        if rcs:
            raise _lib.HgError(-abs(rcs), f"{name} loop")
        us = t_o.ms * 1000.0 / calls
        nbytes = 5 * w.rows * w.vocab * 2
        others[name] = {"workload": f"TP={w.tp}, V={w.vocab}, M={w.rows}, cap={w.cap}, "
                                    f"{w.pool} input sets cycled, back-to-back calls",
                        "us_per_gather": round(us, 3),
                        "gbps_algorithmic": round(nbytes / (us * 1e-6) / 1e9, 1)}
        other_runs[name] = (sets, so, hw)

    # ---------------- A/B: the stock path on the same inputs ----------------
    # (rank-order concatenation, no mailbox: the decline path's single-device
    # share; it reads and writes M*V*2 bytes once each)
    stock_fn = fast.stock
    s_small = torch.empty((wd.pool, wd.rows, wd.vocab), dtype=torch.bfloat16, device=dev)
    s_small_p = [s_small[k].data_ptr() for k in range(wd.pool)]
    s_big = [torch.empty((wl.rows, wl.vocab), dtype=torch.bfloat16, device=dev) for _ in range(3)]
    s_big_p = [o.data_ptr() for o in s_big]
    for n in range(args.warmup):
        rcs |= stock_fn(wd.tp, wd.shard, dec_addr[n % wd.pool], wd.rows, s_small_p[n % wd.pool],
                        wd.vocab, shi)
    with Timer(torch, stream) as t_sd:
        for n in range(args.steps):
            rcs |= stock_fn(wd.tp, wd.shard, dec_addr[n % wd.pool], wd.rows, s_small_p[n % wd.pool],
                        wd.vocab, shi)
    for n in range(3):
        rcs |= stock_fn(wl.tp, wl.shard, big_addr[n], wl.rows, s_big_p[n], wl.vocab, shi)
    with Timer(torch, stream) as t_sb:
        for n in range(args.large_steps):
            rcs |= stock_fn(wl.tp, wl.shard, big_addr[n % 3], wl.rows, s_big_p[n % 3], wl.vocab, shi)
    if rcs:
        raise _lib.HgError(-abs(rcs), "stock gather loop")
    us_stock_m1 = t_sd.ms * 1000.0 / args.steps
    us_stock_big = t_sb.ms * 1000.0 / args.large_steps
    stock = {"workload": "stock path (hg_stock_gather: rank-order concatenation, no mailbox, no "
                         "rewrite) on the same inputs, back-to-back calls",
             "us_per_gather_m1": round(us_stock_m1, 3),
             "us_per_gather_m256_cold": round(us_stock_big, 3),
             "gbps_m256_cold": round(2 * wl.rows * wl.vocab * 2 / (us_stock_big * 1e-6) / 1e9, 1),
             "bytes_per_gather_m256": 2 * wl.rows * wl.vocab * 2}
    del s_big

    # ---------------- fused workload: lm_head producer + gather -------------
    producer = None
    if args.producer_steps > 0:
        log("producer: generating the M=256 x 7168 hidden states and the 163840 x 7168 head weight")
        x_bits = syn.hidden_states(wl)
        xd = syn.to_torch_bf16(x_bits, dev)
        w_dev = torch.empty((wl.tp, wl.shard, wl.hidden), dtype=torch.bfloat16, device=dev)
        w_r0 = None
        for r in range(wl.tp):
            wr = syn.head_weight_shard(wl, r)
            if r == 0:
                w_r0 = wr
            w_dev[r].copy_(syn.to_torch_bf16(wr, dev))
        prod_out = torch.empty((wl.rows, wl.vocab), dtype=torch.bfloat16, device=dev)
        prod_shards = torch.empty((wl.tp, wl.rows, wl.shard), dtype=torch.bfloat16, device=dev)
        xptr = ctypes.c_void_p(xd.data_ptr())
        wptrs = _lib.pointer_array([w_dev[r].data_ptr() for r in range(wl.tp)])
        sptrs = _lib.pointer_array([prod_shards[r].data_ptr() for r in range(wl.tp)])
        optr = ctypes.c_void_p(prod_out.data_ptr())
        gg, lm = lib.hg_gemm_gather, lib.hg_lmhead
        h = hg_big.handle
        for _ in range(2):
            rcs |= gg(h, xptr, wptrs, wl.hidden, wl.rows, optr, None, sh)
            rcs |= lm(wl.tp, wl.shard, xptr, wptrs, wl.hidden, wl.rows, sptrs, sh)
        # The two calls alternate, each between its own events, so that both
        # see the same clock: under sustained MFMA load the clock drops over
        # the first few milliseconds, and two loops run one after the other
        # would compare a cool chip with a throttled one.
        log(f"producer timed {args.producer_steps} x (GEMM + gather, GEMM alone), alternating")
        evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)]
               for _ in range(args.producer_steps)]
        torch.cuda.synchronize()
        for e in evs:
            e[0].record(stream)
            rcs |= gg(h, xptr, wptrs, wl.hidden, wl.rows, optr, None, sh)
            e[1].record(stream)
            rcs |= lm(wl.tp, wl.shard, xptr, wptrs, wl.hidden, wl.rows, sptrs, sh)
            e[2].record(stream)
        torch.cuda.synchronize()
        if rcs:
            raise _lib.HgError(-abs(rcs), "timed producer loop")
        flops = 2.0 * wl.rows * wl.hidden * wl.vocab
        w_bytes = wl.vocab * wl.hidden * 2
        pg = [e[0].elapsed_time(e[1]) * 1000.0 for e in evs]
        lmt = [e[1].elapsed_time(e[2]) * 1000.0 for e in evs]
        us_pg = statistics.median(pg)
        us_lm = statistics.median(lmt)
        # the same product for one decode row (M=1, rows 1..255 of X unused):
        # a weight stream; alternating again, medians
        evs1 = [[torch.cuda.Event(enable_timing=True) for _ in range(3)]
                for _ in range(args.producer_steps)]
        torch.cuda.synchronize()
        for e in evs1:
            e[0].record(stream)
            rcs |= gg(h, xptr, wptrs, wl.hidden, 1, optr, None, sh)
            e[1].record(stream)
            rcs |= lm(wl.tp, wl.shard, xptr, wptrs, wl.hidden, 1, sptrs, sh)
            e[2].record(stream)
        torch.cuda.synchronize()
        if rcs:
            raise _lib.HgError(-abs(rcs), "timed M=1 producer loop")
        us_pg1 = statistics.median(e[0].elapsed_time(e[1]) * 1000.0 for e in evs1)
        us_lm1 = statistics.median(e[1].elapsed_time(e[2]) * 1000.0 for e in evs1)
        producer = {"workload": "lm_head X[256,7168] @ W[163840,7168]^T (8 ranks x 20480) BF16, "
                                "fp32 accumulate, epilogue pushes into the mailbox, then collect",
                    "us_gemm_plus_gather": round(us_pg, 2),
                    "us_gemm_alone": round(us_lm, 2),
                    "timing": f"median of {args.producer_steps} alternating calls, each between HIP events",
                    "us_gemm_alone_min": round(min(lmt), 2),
                    "gemm_tflops": round(flops / (us_lm * 1e-6) / 1e12, 1),
                    "gemm_frac_of_mfma_bf16_peak": round(flops / (us_lm * 1e-6) / 2.5e15, 4),
                    "gemm_weight_gbps": round(w_bytes / (us_lm * 1e-6) / 1e9, 1),
                    "gemm_weight_frac_of_hbm_peak": round(w_bytes / (us_lm * 1e-6) / 8e12, 4),
                    "m1": {"us_gemm_plus_gather": round(us_pg1, 2), "us_gemm_alone": round(us_lm1, 2),
                           "gemm_weight_gbps": round(w_bytes / (us_lm1 * 1e-6) / 1e9, 1)}}
        # the gather of the producer path against the oracle applied to the product's own shards
        rcs |= lm(wl.tp, wl.shard, xptr, wptrs, wl.hidden, wl.rows, sptrs, sh)
        rcs |= gg(h, xptr, wptrs, wl.hidden, wl.rows, optr, None, sh)
        torch.cuda.synchronize()
        del w_dev

    # ---------------- mailbox state after the runs --------------------------
    armed = torch.full((wd.cap, wd.vocab // 2), -(1 << 31), dtype=torch.int32, device=dev)
    armed_big = torch.full((wl.cap, wl.vocab // 2), -(1 << 31), dtype=torch.int32, device=dev)
    for p in (0, 1):
        if not torch.equal(hg.mailbox(p).view(torch.int32), armed):
            log("FAIL: decode mailbox not all-sentinel after the run")
            return 1
        if not torch.equal(hg_big.mailbox(p).view(torch.int32), armed_big):
            log("FAIL: M=256 mailbox not all-sentinel after the run")
            return 1
    if us_graph is not None:
        for p in (0, 1):
            if not torch.equal(hg_g.mailbox(p).view(torch.int32), armed):
                log("FAIL: graph-replayed decode mailbox not all-sentinel")
                return 1
        if hg_g.parity != 0 or hg_g.poll_status() != _lib.HG_OK:  # 2 replays of K calls: even
            log("FAIL: device parity after the graph replays")
            return 1
    if us_split is not None:
        for p in (0, 1):
            if not torch.equal(hg_s.mailbox(p).view(torch.int32), armed):
                log("FAIL: split decode mailbox not all-sentinel")
                return 1
        if hg_s.poll_status() != _lib.HG_OK:
            log("FAIL: a bounded poll of the split variant gave up")
            return 1
    if hg.poll_status() != _lib.HG_OK or hg_big.poll_status() != _lib.HG_OK:
        log("FAIL: a bounded poll gave up")
        return 1

    # ---------------- cpu_baseline: the oracle, and the output check --------
    cpu = None
    if not args.no_cpu:
        from oracle import gather as og

        log("cpu baseline: oracle on the decode sets (M=1) and one M=256 set")
        samples = []
        want_dec = []
        t_end = time.perf_counter() + 10.0
        n = 0
        while n < 1000 and (n < wd.pool or time.perf_counter() < t_end):
            t0 = time.perf_counter()
            r = og.gather_definition(list(dec_sets[n % wd.pool]))
            samples.append(time.perf_counter() - t0)
            if n < wd.pool:
                want_dec.append(r)
            n += 1
        t0 = time.perf_counter()
        want_big = og.gather_definition(list(big_sets[0]))
        big_cpu_s = time.perf_counter() - t0
        us_cpu = statistics.median(samples) * 1e6
        cpu = {"value": round(us_cpu, 2), "unit": "us per gather (M=1)", "cores": 1,
               "kind": "oracle",
               "sample": f"oracle.gather.gather_definition (numpy, single thread) on the decode "
                         f"input sets: median of {len(samples)} calls; plus one M=256 call",
               "m256_gbps_algorithmic": round(big_bytes / big_cpu_s / 1e9, 3),
               "os_cpu_count": os.cpu_count(),
               "affinity": len(os.sched_getaffinity(0)),
               "torch_threads": torch.get_num_threads()}
        # the GPU outputs of the timed loop (call n used set n % pool) against the oracle
        got = outs[: wd.pool].cpu().contiguous().view(torch.int16).numpy().view(np.uint16)
        for k in range(min(wd.pool, args.steps)):
            if not np.array_equal(got[k], want_dec[k]):
                log(f"FAIL: decode output of call {k} differs from the oracle")
                return 1
        # each other workload: the last call on each pool set is that set's output
        for name, (sets, so, hw) in other_runs.items():
            got = so.cpu().contiguous().view(torch.int16).numpy().view(np.uint16)
            for k in range(len(sets)):
                if not np.array_equal(got[k], og.gather_definition(list(sets[k]))):
                    log(f"FAIL: {name} output of set {k} differs from the oracle")
                    return 1
            if hw.poll_status() != _lib.HG_OK:
                log(f"FAIL: {name}: a bounded poll gave up")
                return 1
        got = s_small.cpu().contiguous().view(torch.int16).numpy().view(np.uint16)
        for k in range(wd.pool):
            if not np.array_equal(got[k], og.stock_concat(list(dec_sets[k]))):
                log(f"FAIL: stock gather of set {k} differs from the oracle's concatenation")
                return 1
        if us_graph is not None:
            got = g_outs[: wd.pool].cpu().contiguous().view(torch.int16).numpy().view(np.uint16)
            for k in range(min(wd.pool, args.steps)):
                if not np.array_equal(got[k], want_dec[k]):
                    log(f"FAIL: graph-replayed decode output of call {k} differs from the oracle")
                    return 1
        if us_split is not None:
            got = s_outs[: wd.pool].cpu().contiguous().view(torch.int16).numpy().view(np.uint16)
            for k in range(min(wd.pool, args.steps)):
                if not np.array_equal(got[k], want_dec[k]):
                    log(f"FAIL: split decode output of call {k} differs from the oracle")
                    return 1
        if not np.array_equal(syn.from_torch_bf16(big_out[0]), want_big):
            log("FAIL: M=256 output differs from the oracle")
            return 1
        if producer is not None:
            from oracle import gemm as ogemm

            shards_bits = syn.from_torch_bf16(prod_shards)
            if not np.array_equal(syn.from_torch_bf16(prod_out), og.gather_definition(list(shards_bits))):
                log("FAIL: producer gather differs from the oracle on the product's shards")
                return 1
            # the GEMM oracle (float64, numpy's BLAS) on a bounded sample: rank
            # 0's whole shard product, X[256,7168] x W_0[20480,7168]^T (75.2
            # GFLOP of the 601.3), from the same seeded inputs as the GPU run
            import threadpoolctl

            t0 = time.perf_counter()
            ref = ogemm.lm_head_shard(x_bits, w_r0)
            t_ref = time.perf_counter() - t0
            err = ogemm.relative_frobenius_error(shards_bits[0], ref)
            if err > 1e-2:
                log(f"FAIL: GEMM relative error {err:.3e} on rank 0's shard")
                return 1
            blas = [p for p in threadpoolctl.threadpool_info() if p.get("user_api") == "blas"]
            sample_flops = 2.0 * wl.rows * wl.hidden * wl.shard
            cpu["gemm_oracle"] = {
                "value": round(sample_flops / t_ref / 1e9, 2), "unit": "GFLOP/s",
                "sample_gflop": round(sample_flops / 1e9, 2),
                "total_gflop": round(2.0 * wl.rows * wl.hidden * wl.vocab / 1e9, 2),
                "seconds": round(t_ref, 3),
                "sample": "oracle.gemm.lm_head_shard (numpy float64, the oracle as it stands) on "
                          "rank 0's whole shard: X[256,7168] x W_0[20480,7168]^T, the seeded inputs "
                          "of the GPU run; includes the BF16 -> float64 decode",
                "threads": blas[0]["num_threads"] if blas else 1,
                "blas": (blas[0].get("internal_api") if blas else "none"),
                "rel_frobenius_error_gpu_vs_oracle": err}

    # ---------------- counters (only if taken on this kernel source) --------
    # rocprof kernel times of the M=1 fused gather and the M=256 traffic, from
    # the committed summaries, while they were taken on the current sources
    m1_rocprof, traffic = current_profiles(M1_TRACES, COUNTERS, args.variant, kernel_source_hash())

    dec_bytes = 5 * wd.rows * wd.vocab * 2
    m1_kernel_us = m1_rocprof["eager"]["median_us"] if "eager" in m1_rocprof else None
    m1_basis_us = m1_kernel_us if m1_kernel_us is not None else us_m1
    line = {
        "metric": METRIC,
        "value": round(us_m1, 3),
        "unit": "us",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(t_dec.ms / args.steps, 6),
        "higher_is_better": False,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "u32",
        "data": "synthetic",
        "config": {"workload": "decode gather: TP=8 virtual ranks, V=163840 (shard 20480 BF16), "
                               "M=1, cap=8, back-to-back calls on one stream, inputs resident",
                   "variant": args.variant, "tp": wd.tp, "vocab": wd.vocab, "rows": wd.rows,
                   "cap": wd.cap},
        "decode_graph": None if us_graph is None else {
            "workload": "the same M=1 decode gathers captured into one HIP graph "
                        "(device-side parity) and replayed",
            "us_per_gather": round(us_graph, 3), "gathers_per_replay": args.steps},
        "decode_split": None if us_split is None else {
            "workload": "the same M=1 decode gathers through the split variant "
                        "(hg_push then hg_collect: two launches per gather)",
            "us_per_gather": round(us_split, 3)},
        "large_m": {"workload": "gather TP=8, V=163840, M=256, cap=256, 3 rotating buffer sets",
                    "us_per_gather_cold": round(us_cold, 3),
                    "gbps_algorithmic_cold": round(gbps_cold, 1),
                    "us_plain_stream_same_bytes_cold": round(us_ref, 3),
                    "plain_stream_over_gather": round(us_ref / us_cold, 4),
                    "plain_stream": "hgref_stream (libhgref.so): the same 5 x M x V x 2 bytes "
                                    "with 128-bit accesses and no compare or poll, 4 workgroups "
                                    "of 256 per CU, same rotating shard sets",
                    "us_per_gather_back_to_back": round(us_hot, 3),
                    "gbps_algorithmic_back_to_back": round(gbps_hot, 1),
                    "algorithmic_bytes_per_gather": big_bytes},
        "roofline": {"bound": "hbm", "achieved": round(gbps_cold, 1), "peak": HBM_PEAK_GBPS,
                     "unit": "GB/s", "frac": round(gbps_cold / HBM_PEAK_GBPS, 4),
                     "traffic": traffic,
                     "kernel": "k_fused (M=256 gather, cold)" if args.variant == "fused"
                               else "k_push + k_collect (M=256 gather, cold)"},
        "m1_kernel_time_rocprof": None if not m1_rocprof else {
            **{leg: {"median_us": t["median_us"], "calls": t["calls"], "kernel": t["kernel"],
                     "trace": os.path.relpath(M1_TRACES[leg], ROOT)} for leg, t in m1_rocprof.items()},
            **({"split_eager": {"push_median_us": m1_rocprof["eager"]["split"]["push"]["median_us"],
                                "collect_median_us": m1_rocprof["eager"]["split"]["collect"]["median_us"],
                                "sum_median_us": m1_rocprof["eager"]["split"]["sum_median_us"],
                                "trace": os.path.relpath(M1_TRACES["eager"], ROOT)}}
               if "split" in m1_rocprof.get("eager", {}) else {})},
        "roofline_m1": {"bound": "latency",
                        "achieved": round(dec_bytes / (m1_basis_us * 1e-6) / 1e9, 1),
                        "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                        "frac": round(dec_bytes / (m1_basis_us * 1e-6) / 1e9 / HBM_PEAK_GBPS, 4),
                        "basis": ("rocprof median kernel duration of the eager M=1 fused gather"
                                  if m1_kernel_us is not None else
                                  "HIP-event time per eager call (no kernel trace of the current "
                                  "sources committed)"),
                        "note": "M=1 moves 1.6 MB: the kernel's own chain of dependent memory "
                                "round trips (shard load, coherent push, poll of another "
                                "workgroup's push, stores), not bandwidth, sets its time"},
        "other_configs": others,
        "stock_ab": stock,
        "producer": producer,
        "cpu_baseline": cpu,
        "kernel_source_sha256_16": kernel_source_hash(),
    }
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
