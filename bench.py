#!/usr/bin/env python3
"""Throughput of the exact-attention hot path on one MI355X.

One step = one pass of the whole path over one batch of synthetic input:
fa_forward (O, lse) then fa_backward (dQ, dK, dV), on the long-context
causal problem B=1, H=32, N=16384, d=128, bf16 (fp32 accumulation).
Inputs are resident in HBM before timing starts.  For bf16, fa_backward
runs the query-parallel dQ kernel with the row statistics D = rowsum(dO o O)
and -lse folded in, then the key-parallel dK/dV kernel.  The per-kernel
table times each kernel alone, through the staged entry points
(preprocess, dK/dV, dQ), in a separate pass.

FLOP counting convention: forward 4*B*H*N^2*d, halved when causal; backward
2.5x forward.  The value is total (forward + backward) FLOPs per step over
the wall time of a step, in TFLOP/s.

Besides the step, "extra" carries the 4K shape, per-call timings (median,
p10, p90) of the five parity configurations, the block-sparse (forward and
backward), decoding,
dropout and FP8 paths, and the library GEMM's rate on N(0,1) operands in the
same run (the practical matrix-core ceiling for such data, with each kernel's
fraction of it).

Prints ONE JSON line.  Options: --gpus N (only 1: the path runs on one GPU),
--steps K, --warmup W, --no-cpu-baseline, --no-extra, --decode-only, --dropout-only,
--fp8-only, --sparse-only, --configs-only.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "attention fwd/bwd TFLOP/s and % of bf16 MFMA peak at N=4K/16K, d=128"
PEAK_BF16_TFLOPS = 2500.0     # MI355X published dense bf16 MFMA peak
PEAK_HBM_GBS = 8000.0         # MI355X published HBM3E bandwidth
KERNEL_SOURCES = ["fa_common.h", "fa_fwd.hip", "fa_bwd.hip"]


def kernel_source_digest() -> str:
    h = hashlib.sha256()
    for name in KERNEL_SOURCES:
        with open(os.path.join(ROOT, "io_aware_tiled_attention_amd", "csrc", name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def measured_traffic(kernel: str):
    """HBM bytes per launch from the committed rocprofv3 counter summary, or None.

    profiles/hbm_traffic.json holds FETCH_SIZE / WRITE_SIZE per dispatch,
    already scaled by the copy-kernel calibration, with the digest of the
    kernel sources they were taken on; stale counters (sources changed since)
    are not reported.
    """
    path = os.path.join(ROOT, "profiles", "hbm_traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        data = json.load(f)
    if data.get("source_digest") != kernel_source_digest():
        return None
    ent = data.get("kernels", {}).get(kernel)
    if not ent:
        return None
    return float(ent["fetch_bytes"]) + float(ent["write_bytes"])


class Step:
    """Pre-bound raw C-ABI calls of one step on torch's current stream."""

    def __init__(self, fa, torch, inputs, p, dev):
        self.torch = torch
        self.p = p
        self.q, self.k, self.v, self.do = (inputs[n].to(dev) for n in ("q", "k", "v", "do"))
        self.o = torch.empty_like(self.q)
        self.lse = torch.empty((p.B, p.H, p.N), dtype=torch.float32, device=dev)
        self.dq, self.dk, self.dv = (torch.empty_like(self.q) for _ in range(3))
        self.ws_bytes = fa.workspace_size(p.B, p.H, p.N, p.d)
        self.ws = torch.empty(self.ws_bytes, dtype=torch.uint8, device=dev)
        self.lib = fa.load_library()
        self.stream = torch.cuda.current_stream(dev).cuda_stream
        self.dt = fa.FA_BF16 if p.dtype == "bf16" else fa.FA_F32
        self.dev = dev

    def _ck(self, st, name):
        if st != 0:
            raise RuntimeError(f"{name} returned {st}: {self.lib.fa_strerror(st).decode()}")

    def forward(self):
        p = self
        self._ck(self.lib.fa_forward(p.q.data_ptr(), p.k.data_ptr(), p.v.data_ptr(), p.o.data_ptr(),
                                     p.lse.data_ptr(), self.p.B, self.p.H, self.p.N, self.p.d,
                                     int(self.p.causal), self.p.scale, self.dt, self.stream), "fa_forward")

    def bwd_pre(self):
        self._ck(self.lib.fa_backward_preprocess(self.o.data_ptr(), self.do.data_ptr(), self.lse.data_ptr(),
                                                 self.p.B, self.p.H, self.p.N, self.p.d, self.dt,
                                                 self.ws.data_ptr(), self.ws_bytes, self.stream),
                 "fa_backward_preprocess")

    def bwd_dkdv(self):
        p = self
        self._ck(self.lib.fa_backward_dkdv(p.q.data_ptr(), p.k.data_ptr(), p.v.data_ptr(), p.do.data_ptr(),
                                           p.dk.data_ptr(), p.dv.data_ptr(), self.p.B, self.p.H,
                                           self.p.N, self.p.d, int(self.p.causal), self.p.scale, self.dt,
                                           p.ws.data_ptr(), self.ws_bytes, self.stream), "fa_backward_dkdv")

    def bwd_dq(self):
        p = self
        self._ck(self.lib.fa_backward_dq(p.q.data_ptr(), p.k.data_ptr(), p.v.data_ptr(), p.do.data_ptr(),
                                         p.dq.data_ptr(), self.p.B, self.p.H, self.p.N, self.p.d,
                                         int(self.p.causal), self.p.scale, self.dt, p.ws.data_ptr(), self.ws_bytes,
                                         self.stream), "fa_backward_dq")

    def backward(self):
        p = self
        self._ck(self.lib.fa_backward(p.q.data_ptr(), p.k.data_ptr(), p.v.data_ptr(), p.o.data_ptr(), p.do.data_ptr(),
                                      p.lse.data_ptr(), p.dq.data_ptr(), p.dk.data_ptr(), p.dv.data_ptr(), self.p.B,
                                      self.p.H, self.p.N, self.p.d, int(self.p.causal), self.p.scale, self.dt,
                                      p.ws.data_ptr(), self.ws_bytes, self.stream), "fa_backward")

    # one step: the public calls, fa_forward then fa_backward (which, for bf16,
    # runs dQ with the row statistics folded in, then dK/dV)
    STEP = ("fwd", "bwd")
    # the per-kernel breakdown: the staged entry points, one kernel each
    STAGES = ("fwd", "bwd_pre", "bwd_dkdv", "bwd_dq")

    def run(self, events=None):
        fns = (self.forward, self.backward)
        if events is None:
            for fn in fns:
                fn()
            return
        events[0].record()
        for i, fn in enumerate(fns):
            fn()
            events[i + 1].record()

    def run_staged(self, events):
        events[0].record()
        for i, fn in enumerate((self.forward, self.bwd_pre, self.bwd_dkdv, self.bwd_dq)):
            fn()
            events[i + 1].record()


def time_steps(step, torch, steps, warmup):
    """Wall time per step (host clock around `steps` steps, bracketed by
    synchronisations) and the mean forward and backward times (HIP events)."""
    for _ in range(warmup):
        step.run()
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(len(Step.STEP) + 1)] for _ in range(steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        step.run(evs[i])
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    per = {name: [e[j].elapsed_time(e[j + 1]) for e in evs] for j, name in enumerate(Step.STEP)}
    return (t1 - t0) * 1e3 / steps, {name: sum(v) / len(v) for name, v in per.items()}


def time_kernels(step, torch, reps):
    """Mean time of each kernel of the step, one HIP-event pair per kernel,
    through the staged entry points (forward, preprocess, dK/dV, dQ)."""
    for _ in range(2):
        step.run_staged([torch.cuda.Event(enable_timing=True) for _ in range(5)])
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(5)] for _ in range(reps)]
    for i in range(reps):
        step.run_staged(evs[i])
    torch.cuda.synchronize()
    per = {name: [e[j].elapsed_time(e[j + 1]) for e in evs] for j, name in enumerate(Step.STAGES)}
    return {name: sum(v) / len(v) for name, v in per.items()}


def kernel_table(p, avg, step_avg):
    """Per-kernel time and throughput.  The convention counts the backward as
    2.5x the forward: five N x N x d products (S, dP, dV, dK, dQ; halved when
    causal).  dK/dV executes four of them (S, dP, dV, dK), all method work.
    dQ executes three (S, dP, dQ), but only dQ is method work: its S and dP
    recompute what dK/dV already formed, the price of a backward without
    atomics.  So each backward kernel reports its executed FLOPs and its
    share of the method's FLOPs, with a fraction of peak on each basis; the
    two kernels together execute 7/5 of the convention's backward FLOPs."""
    fwd_f, bwd_f = p.fwd_flops(), p.bwd_flops()
    unit = bwd_f / 5.0                       # one N x N x d product (halved when causal)
    elt = 2 if p.dtype == "bf16" else 4
    rows = p.B * p.H * p.N
    tens = rows * p.d * elt
    out = {}

    def mm(name, kernel, executed, method):
        ms = avg[name]
        out[name] = {"kernel": kernel, "ms": ms, "flops": method, "executed_flops": executed,
                     "method_flops": method,
                     "tflops": method / ms * 1e-9, "frac_peak": method / ms * 1e-9 / PEAK_BF16_TFLOPS,
                     "executed_tflops": executed / ms * 1e-9,
                     "frac_peak_executed": executed / ms * 1e-9 / PEAK_BF16_TFLOPS}

    sfx = "_bf16" if p.dtype == "bf16" else ""     # bf16 has its own backward kernels
    mm("fwd", "fa_fwd_kernel", fwd_f, fwd_f)
    mm("bwd_dkdv", f"fa_bwd_dkdv{sfx}_kernel", 4 * unit, 4 * unit)
    mm("bwd_dq", f"fa_bwd_dq{sfx}_kernel", 3 * unit, 1 * unit)
    pre_bytes = 2 * tens + 3 * rows * 4                        # read O, dO, lse; write D, -lse
    out["bwd_pre"] = {"kernel": "fa_bwd_pre_kernel", "ms": avg["bwd_pre"], "bytes": pre_bytes,
                      "gbs": pre_bytes / avg["bwd_pre"] * 1e-6}
    # the backward as fa_backward runs it (bf16: dQ with the row statistics
    # folded in, then dK/dV), timed in the step; the staged sum for reference
    out["bwd_total"] = {"ms": step_avg["bwd"], "staged_ms": avg["bwd_pre"] + avg["bwd_dkdv"] + avg["bwd_dq"]}
    out["bwd_total"]["tflops"] = bwd_f / out["bwd_total"]["ms"] * 1e-9
    out["bwd_total"]["frac_peak"] = out["bwd_total"]["tflops"] / PEAK_BF16_TFLOPS
    out["bwd_total"]["executed_tflops"] = 7 * unit / out["bwd_total"]["ms"] * 1e-9
    return out


PROBE_LIB = os.path.join(ROOT, "io_aware_tiled_attention_amd", "libfa_probe_gfx950.so")


def mfma_peak_measurement(torch, dev, iters=20000):
    """The attainable matrix-core rate of this GPU: v_mfma_f32_32x32x16_bf16
    with every operand in registers (libfa_probe_gfx950.so, include/fa_probe.h),
    on N(0,1) bf16 operands, at one and two waves per SIMD; the larger rate
    is the measured peak.  Under sustained matrix-core load the clock sits
    below the 2.4 GHz of the published 2.5 PFLOP/s."""
    import ctypes
    if not os.path.exists(PROBE_LIB):
        raise RuntimeError(f"{PROBE_LIB} is missing: build with `python -m io_aware_tiled_attention_amd.build`")
    lib = ctypes.CDLL(PROBE_LIB)
    vp, i = ctypes.c_void_p, ctypes.c_int
    lib.fa_probe_mfma_bf16.argtypes = [vp, vp, i, i, vp]
    lib.fa_probe_mfma_bf16.restype = i
    lib.fa_probe_mfma_bf16_flops.argtypes = [i, i]
    lib.fa_probe_mfma_bf16_flops.restype = ctypes.c_double
    g = torch.Generator().manual_seed(11)
    ops = torch.randn(8 * 64 * 8, generator=g).to(torch.bfloat16).to(dev)
    stream = torch.cuda.current_stream().cuda_stream
    out = {"what": "register-only v_mfma_f32_32x32x16_bf16, N(0,1) bf16 operands, 16 products per iteration "
                   f"cycling 4 A x 4 B fragments, {iters} iterations per wave"}
    best = 0.0
    for w in (1, 2):
        wgs = 256 * w
        sink = torch.empty(wgs * 256, dtype=torch.float32, device=dev)

        def run():
            st = lib.fa_probe_mfma_bf16(ops.data_ptr(), sink.data_ptr(), wgs, iters, stream)
            assert st == 0, st
        for _ in range(2):
            run()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record()
        for _ in range(5):
            run()
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / 5
        tf = lib.fa_probe_mfma_bf16_flops(wgs, iters) / ms * 1e-9
        out[f"tflops_{w}_wave_per_simd"] = tf
        best = max(best, tf)
    out["tflops"] = best
    out["frac_of_published_peak"] = best / PEAK_BF16_TFLOPS
    # the same instruction stream on all-zero operands: the matrix cores'
    # switching power, and with it the clock the power manager allows,
    # depends on the operand bits; with zeros the chip runs at its top clock
    zeros = torch.zeros_like(ops)
    wgs = 256
    sink = torch.empty(wgs * 256, dtype=torch.float32, device=dev)
    for _ in range(2):
        assert lib.fa_probe_mfma_bf16(zeros.data_ptr(), sink.data_ptr(), wgs, iters, stream) == 0
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record()
    for _ in range(5):
        assert lib.fa_probe_mfma_bf16(zeros.data_ptr(), sink.data_ptr(), wgs, iters, stream) == 0
    e1.record()
    torch.cuda.synchronize()
    out["tflops_zero_operands_1_wave_per_simd"] = lib.fa_probe_mfma_bf16_flops(wgs, iters) / (e0.elapsed_time(e1) / 5) * 1e-9
    return out


def kept_pairs(mask, n, bq, bk, causal):
    """Number of (query, key) pairs a block mask keeps, per mask head (exact count)."""
    import numpy as np
    m = mask.cpu().numpy() != 0
    rows = np.arange(n)
    cols = np.arange(n)
    out = []
    for h in range(m.shape[0]):
        keep = m[h][rows[:, None] // bq, cols[None, :] // bk]
        if causal:
            keep &= cols[None, :] <= rows[:, None]
        out.append(int(keep.sum()))
    return out


def sparse_measurement(fa, torch, dev, steps):
    """Block-sparse forward and backward on the 16K causal d=128 shape with a
    sliding-window plus global-column mask; FLOPs counted on the kept
    (query, key) pairs only (backward: 2.5x the forward's), and the dense
    causal forward and backward on the same inputs for comparison."""
    from workloads import PROBLEMS, block_mask, make_inputs
    p = PROBLEMS["causal_16k_d128_bwd"]
    bq = bk = 128
    window = 8                       # key blocks before the diagonal (1024 keys)
    mask = block_mask(1, p.N, bq, bk, "local_global", seed=0, window=window).to(dev)
    inputs = make_inputs(p, with_do=True)
    q, k, v, do = (inputs[n].to(dev) for n in ("q", "k", "v", "do"))
    o = torch.empty_like(q)
    lse = torch.empty((p.B, p.H, p.N), dtype=torch.float32, device=dev)
    dq, dk, dv = (torch.empty_like(q) for _ in range(3))
    stream = torch.cuda.current_stream().cuda_stream
    raw = fa.load_library()
    ws_n = raw.fa_backward_workspace_size(p.B, p.H, p.N, p.d)
    ws = torch.empty(ws_n, dtype=torch.uint8, device=dev)

    def run_sparse():
        st = raw.fa_forward_block_sparse(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(),
                                         mask.data_ptr(), 1, bq, bk, p.B, p.H, p.N, p.d, 1, p.scale, 1, stream)
        assert st == 0, st

    def run_dense():
        st = raw.fa_forward(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(),
                            p.B, p.H, p.N, p.d, 1, p.scale, 1, stream)
        assert st == 0, st

    def timed(fn):
        for _ in range(3):
            fn()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record()
        for _ in range(steps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / steps

    def run_sparse_bwd():
        st = raw.fa_backward_block_sparse(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), do.data_ptr(),
                                          lse.data_ptr(), dq.data_ptr(), dk.data_ptr(), dv.data_ptr(),
                                          mask.data_ptr(), 1, bq, bk, p.B, p.H, p.N, p.d, 1, p.scale, 1,
                                          ws.data_ptr(), ws_n, stream)
        assert st == 0, st

    def run_dense_bwd():
        st = raw.fa_backward(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), do.data_ptr(), lse.data_ptr(),
                             dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), p.B, p.H, p.N, p.d, 1, p.scale, 1,
                             ws.data_ptr(), ws_n, stream)
        assert st == 0, st

    ms_s, ms_d = timed(run_sparse), timed(run_dense)
    run_sparse()                    # O and lse of the masked problem for its backward
    ms_sb = timed(run_sparse_bwd)
    run_dense()
    ms_db = timed(run_dense_bwd)
    pairs = kept_pairs(mask, p.N, bq, bk, True)[0] * p.B * p.H
    dense_pairs = p.N * (p.N + 1) // 2 * p.B * p.H
    flops = 4.0 * p.d * pairs
    return {"workload": "causal_16k_d128 with a block mask: 128x128 blocks, sliding window of "
                        f"{window} key blocks plus the first key block column",
            "kept_fraction_of_causal_pairs": pairs / dense_pairs, "ms": ms_s, "dense_causal_ms": ms_d,
            "tflops_on_kept_pairs": flops / ms_s * 1e-9, "frac_peak": flops / ms_s * 1e-9 / PEAK_BF16_TFLOPS,
            "speedup_vs_dense_causal": ms_d / ms_s,
            "bwd_ms": ms_sb, "dense_causal_bwd_ms": ms_db, "bwd_tflops_on_kept_pairs": 2.5 * flops / ms_sb * 1e-9,
            "bwd_frac_peak": 2.5 * flops / ms_sb * 1e-9 / PEAK_BF16_TFLOPS, "bwd_speedup_vs_dense_causal": ms_db / ms_sb}


def dropout_measurement(fa, torch, dev, steps, p_drop=0.1):
    """Forward and backward with dropout (mask regenerated from Philox in
    every kernel) on the 16K causal d=128 shape, against the same calls
    without dropout.  FLOPs by the same convention (dropout adds none)."""
    from workloads import PROBLEMS, make_inputs
    p = PROBLEMS["causal_16k_d128_bwd"]
    inputs = make_inputs(p, with_do=True)
    q, k, v, do = (inputs[n].to(dev) for n in ("q", "k", "v", "do"))
    del inputs
    o = torch.empty_like(q)
    lse = torch.empty((p.B, p.H, p.N), dtype=torch.float32, device=dev)
    dq, dk, dv = (torch.empty_like(q) for _ in range(3))
    ws_bytes = fa.workspace_size(p.B, p.H, p.N, p.d)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
    raw = fa.load_library()
    stream = torch.cuda.current_stream().cuda_stream
    seed, offset = 0x5EED, 0

    def fwd(drop):
        if drop:
            st = raw.fa_forward_dropout(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(), p.B,
                                        p.H, p.N, p.d, 1, p.scale, 1, p_drop, seed, offset, stream)
        else:
            st = raw.fa_forward(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(), p.B, p.H,
                                p.N, p.d, 1, p.scale, 1, stream)
        assert st == 0, st

    def bwd(drop):
        args = (q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), do.data_ptr(), lse.data_ptr(),
                dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), p.B, p.H, p.N, p.d, 1, p.scale, 1)
        if drop:
            st = raw.fa_backward_dropout(*args, p_drop, seed, offset, ws.data_ptr(), ws_bytes, stream)
        else:
            st = raw.fa_backward(*args, ws.data_ptr(), ws_bytes, stream)
        assert st == 0, st

    def timed(fn):
        for _ in range(2):
            fn()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record()
        for _ in range(steps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / steps

    res = {"workload": f"{p.name} with dropout p={p_drop} (drop probability quantised to "
                       f"{int(p_drop * 256 + 0.5)}/256)", "p_drop": p_drop}
    for drop in (True, False):
        tag = "dropout" if drop else "plain"
        res[f"{tag}_fwd_ms"] = timed(lambda: fwd(drop))
        res[f"{tag}_bwd_ms"] = timed(lambda: bwd(drop))
    res["fwd_tflops"] = p.fwd_flops() / res["dropout_fwd_ms"] * 1e-9
    res["bwd_tflops"] = p.bwd_flops() / res["dropout_bwd_ms"] * 1e-9
    res["fwd_frac_peak"] = res["fwd_tflops"] / PEAK_BF16_TFLOPS
    res["bwd_frac_peak"] = res["bwd_tflops"] / PEAK_BF16_TFLOPS
    res["fwd_slowdown"] = res["dropout_fwd_ms"] / res["plain_fwd_ms"]
    res["bwd_slowdown"] = res["dropout_bwd_ms"] / res["plain_bwd_ms"]
    return res


PEAK_FP8_TFLOPS = 5000.0     # MI355X published dense fp8 MFMA peak


def fp8_measurement(fa, torch, dev, steps):
    """Forward with OCP E4M3 inputs on the 16K causal d=128 shape (the bench
    recipe rounded to E4M3), against the bf16 forward on the same values.
    FLOPs by the forward convention; peak = the published dense fp8 rate."""
    from workloads import PROBLEMS, make_inputs
    p = PROBLEMS["causal_16k_d128"]
    inputs = make_inputs(p)
    q16, k16, v16 = (inputs[n].to(dev) for n in ("q", "k", "v"))
    del inputs
    q8, k8, v8 = (t.float().to(torch.float8_e4m3fn) for t in (q16, k16, v16))
    o = torch.empty_like(q16)
    lse = torch.empty((p.B, p.H, p.N), dtype=torch.float32, device=dev)
    raw = fa.load_library()
    stream = torch.cuda.current_stream().cuda_stream

    def run8():
        st = raw.fa_forward_fp8(q8.data_ptr(), k8.data_ptr(), v8.data_ptr(), o.data_ptr(), lse.data_ptr(), p.B, p.H,
                                p.N, p.d, 1, p.scale, 1.0, 1.0, 1.0, stream)
        assert st == 0, st

    def run16():
        st = raw.fa_forward(q16.data_ptr(), k16.data_ptr(), v16.data_ptr(), o.data_ptr(), lse.data_ptr(), p.B, p.H,
                            p.N, p.d, 1, p.scale, 1, stream)
        assert st == 0, st

    def timed(fn):
        for _ in range(3):
            fn()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record()
        for _ in range(steps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / steps

    ms8, ms16 = timed(run8), timed(run16)
    flops = p.fwd_flops()
    return {"workload": f"{p.name} forward, Q/K/V rounded to OCP E4M3 (descale 1), bf16 output",
            "ms": ms8, "tflops": flops / ms8 * 1e-9, "frac_fp8_peak": flops / ms8 * 1e-9 / PEAK_FP8_TFLOPS,
            "bf16_forward_ms": ms16, "speedup_vs_bf16": ms16 / ms8}


def gemm_ceiling_measurement(torch, dev, steps, n=16384):
    """The practical matrix-core ceiling on this chip for data like the bench's:
    the vendor library's dense GEMM (torch.matmul -> hipBLASLt, bf16; and
    torch._scaled_mm, OCP E4M3 with bf16 output) on n x n x n operands drawn
    N(0,1).  The power manager lowers the clock with the data paths' switching
    activity, so random operands run well below the published peak; this is
    the rate the attention kernels' fractions are best read against.  Context
    only: the attention path does not call these routines."""
    g = torch.Generator(device="cpu")
    g.manual_seed(7)
    a = torch.randn((n, n), generator=g, dtype=torch.float32)
    b = torch.randn((n, n), generator=g, dtype=torch.float32)
    a16, b16 = a.to(torch.bfloat16).to(dev), b.to(torch.bfloat16).to(dev)
    del a, b

    def timed(fn):
        for _ in range(3):
            fn()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record()
        for _ in range(steps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / steps

    flops = 2.0 * n * n * n
    out = {"what": f"library GEMM {n}x{n}x{n} on N(0,1) operands (torch.matmul bf16; torch._scaled_mm E4M3 -> bf16)"}
    ms = timed(lambda: torch.matmul(a16, b16))
    out["bf16_tflops"] = flops / ms * 1e-9
    out["bf16_frac_peak"] = out["bf16_tflops"] / PEAK_BF16_TFLOPS
    try:
        one = torch.ones((), dtype=torch.float32, device=dev)
        a8 = a16.float().to(torch.float8_e4m3fn)
        b8 = b16.float().to(torch.float8_e4m3fn).t().contiguous().t()   # column-major right operand
        ms8 = timed(lambda: torch._scaled_mm(a8, b8, scale_a=one, scale_b=one, out_dtype=torch.bfloat16))
        out["fp8_tflops"] = flops / ms8 * 1e-9
        out["fp8_frac_peak"] = out["fp8_tflops"] / PEAK_FP8_TFLOPS
        del a8, b8
    except Exception as e:   # an FP8 GEMM this torch build lacks is reported, not fatal
        out["fp8_error"] = f"{type(e).__name__}: {e}"[:200]
    del a16, b16
    return out


CONFIG_NAMES = ["single_head_f32", "gpt2_small_bf16", "causal_4k_d128", "causal_16k_d128", "causal_bwd_4k_d64"]


def config_measurement(fa, torch, dev, warm=10, timed=50, names=None):
    """Per-call timing of each of the five parity configurations: `warm`
    untimed calls, then `timed` calls each bracketed by its own pair of HIP
    events on the launch stream; median, p10 and p90 in ms and TFLOP/s at the
    median (forward; the backward problem: its three-stage backward, with O and
    lse from the forward on the same inputs).  GPU only; the CPU oracle's
    per-head rate for the same passes is part of the cpu_baseline leg."""
    import numpy as np
    from workloads import PROBLEMS, make_inputs
    raw = fa.load_library()
    stream = torch.cuda.current_stream().cuda_stream
    out = {}
    for name in (names or CONFIG_NAMES):
        p = PROBLEMS[name]
        inputs = make_inputs(p)
        q, k, v = (inputs[n].to(dev) for n in ("q", "k", "v"))
        dt = 0 if p.dtype == "f32" else 1
        o = torch.empty_like(q)
        lse = torch.empty((p.B, p.H, p.N), dtype=torch.float32, device=dev)

        def fwd():
            st = raw.fa_forward(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(), p.B, p.H,
                                p.N, p.d, int(p.causal), p.scale, dt, stream)
            assert st == 0, st
        fn, flops, what = fwd, p.fwd_flops(), "forward"
        if p.backward:
            do = inputs["do"].to(dev)
            dq, dk, dv = (torch.empty_like(q) for _ in range(3))
            ws_n = raw.fa_backward_workspace_size(p.B, p.H, p.N, p.d)
            ws = torch.empty(ws_n, dtype=torch.uint8, device=dev)
            fwd()

            def bwd():
                st = raw.fa_backward(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), do.data_ptr(),
                                     lse.data_ptr(), dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), p.B, p.H, p.N, p.d,
                                     int(p.causal), p.scale, dt, ws.data_ptr(), ws_n, stream)
                assert st == 0, st
            fn, flops, what = bwd, p.bwd_flops(), "backward"
        for _ in range(warm):
            fn()
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(timed)]
        torch.cuda.synchronize()
        for e0, e1 in ev:
            e0.record()
            fn()
            e1.record()
        torch.cuda.synchronize()
        ms = np.array([e0.elapsed_time(e1) for e0, e1 in ev])
        med, p10, p90 = (float(np.percentile(ms, x)) for x in (50, 10, 90))
        out[name] = {"pass": what, "B": p.B, "H": p.H, "N": p.N, "d": p.d, "dtype": p.dtype, "causal": p.causal,
                     "calls": timed, "median_ms": med, "p10_ms": p10, "p90_ms": p90,
                     "tflops_at_median": flops / med * 1e-9, "frac_peak": flops / med * 1e-9 / PEAK_BF16_TFLOPS}
        del q, k, v, o, lse, inputs
        torch.cuda.empty_cache()
    return out


DECODE_SHAPES = [(1, 32, 1, 65536), (8, 32, 1, 8192)]    # (B, H, Nq, Nk), d = 128, bf16, causal


def decode_measurement(fa, torch, dev, steps, shapes=None):
    """Split-KV decoding (fa_decode, partial + merge kernels) on long caches.
    The work is bound by HBM: the algorithmic bytes are one read of K and V
    plus Q, and the writes of O and lse (the partial results in the workspace
    are the method's own overhead and not counted); GB/s against 8 TB/s."""
    from workloads import decode_inputs
    raw = fa.load_library()
    stream = torch.cuda.current_stream().cuda_stream
    out = []
    d = 128
    for B, H, Nq, Nk in (DECODE_SHAPES if shapes is None else shapes):
        inp = decode_inputs(B, H, Nq, Nk, d, "bf16", seed=B * 131 + Nk)
        q, k, v = (inp[n].to(dev) for n in ("q", "k", "v"))
        del inp
        o = torch.empty_like(q)
        lse = torch.empty((B, H, Nq), dtype=torch.float32, device=dev)
        splits = raw.fa_decode_num_splits(B, H, Nk, 0)
        ws_bytes = raw.fa_decode_workspace_size(B, H, Nq, Nk, d, 0)
        ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
        scale = d ** -0.5

        def run():
            st = raw.fa_decode(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(), B, H, Nq,
                               Nk, d, 1, scale, 1, 0, ws.data_ptr(), ws_bytes, stream)
            assert st == 0, st

        for _ in range(3):
            run()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record()
        for _ in range(steps):
            run()
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / steps
        kv_bytes = 2 * B * H * Nk * d * 2
        alg = kv_bytes + 2 * B * H * Nq * d * 2 + B * H * Nq * 4
        out.append({"B": B, "H": H, "Nq": Nq, "Nk": Nk, "d": d, "causal": True, "splits": splits, "ms": ms,
                    "algorithmic_bytes": alg, "gbs": alg / ms * 1e-6, "frac_hbm_peak": alg / ms * 1e-6 / PEAK_HBM_GBS})
        del q, k, v, o, lse, ws
        torch.cuda.empty_cache()
    return out


def cpu_baseline(inputs, p, heads):
    """The fp64 oracle on a bounded sample: `heads` whole heads of the workload.

    Each head's forward and backward (standard attention with materialised
    S and P, naive chain rule) is timed as the oracle stands.
    """
    from oracle import attention_ref as ref
    try:
        from threadpoolctl import threadpool_info
        threads = max((i.get("num_threads", 1) for i in threadpool_info()), default=1)
    except Exception:  # noqa: BLE001 - reporting only
        threads = 1
    import torch
    heads = max(1, min(heads, p.B * p.H))
    dt = 0.0
    for i in range(heads):
        b, h = divmod(i, p.H)
        q, k, v, do = (inputs[n][b, h].to(torch.float64).numpy() for n in ("q", "k", "v", "do"))
        t0 = time.perf_counter()
        ref.forward_head(q, k, v, causal=p.causal, scale=p.scale)
        ref.backward_head(q, k, v, do, causal=p.causal, scale=p.scale)
        dt += time.perf_counter() - t0
    flops = heads * 4.0 * p.N * p.N * p.d / (2 if p.causal else 1) * 3.5
    return {"value": flops / dt * 1e-12, "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
            "seconds": dt,
            "sample": f"{heads} of the {p.B * p.H} heads of {p.name} (N={p.N}, d={p.d}), forward + backward "
                      f"in fp64 numpy ({threads} BLAS threads, elementwise steps single-threaded; host has "
                      f"{os.cpu_count()} logical cpus); FLOPs counted with the same convention as the GPU"}


def cpu_config_heads():
    """The fp64 oracle on one head of each parity configuration (the same pass
    as config_measurement): seconds and the per-head rate."""
    import torch
    from oracle import attention_ref as ref
    from workloads import PROBLEMS, make_inputs
    out = {}
    for name in CONFIG_NAMES:
        p = PROBLEMS[name]
        inputs = make_inputs(p)
        qh, kh, vh = (inputs[n][0, 0].to(torch.float64).numpy() for n in ("q", "k", "v"))
        t0 = time.perf_counter()
        if p.backward:
            ref.backward_head(qh, kh, vh, inputs["do"][0, 0].to(torch.float64).numpy(), p.causal, p.scale)
            flops = p.bwd_flops()
        else:
            ref.forward_head(qh, kh, vh, p.causal, p.scale)
            flops = p.fwd_flops()
        sec = time.perf_counter() - t0
        out[name] = {"pass": "backward" if p.backward else "forward", "heads": 1, "seconds": sec,
                     "tflops": flops / (p.B * p.H) / sec * 1e-12}
    return out


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="causal_16k_d128_bwd")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-heads", type=int, default=4, help="whole heads timed on the CPU oracle")
    ap.add_argument("--no-extra", action="store_true",
                    help="skip the side measurements (N=4K d=128 fwd+bwd, block-sparse 16K forward, "
                         "split-KV decoding, dropout, FP8 forward)")
    ap.add_argument("--decode-only", action="store_true",
                    help="only the split-KV decoding measurement (one JSON line; for kernel traces)")
    ap.add_argument("--configs-only", action="store_true",
                    help="only the per-call timing of the five parity configurations (one JSON line)")
    ap.add_argument("--config", action="append", choices=CONFIG_NAMES, default=None,
                    help="with --configs-only: only this configuration (repeatable)")
    ap.add_argument("--sparse-only", action="store_true",
                    help="only the block-sparse forward and backward measurement (one JSON line)")
    ap.add_argument("--fp8-only", action="store_true",
                    help="only the FP8 forward measurement (one JSON line; for kernel traces)")
    ap.add_argument("--dropout-only", action="store_true",
                    help="only the dropout measurement (one JSON line; for kernel traces)")
    ap.add_argument("--decode-shape", type=int, default=None,
                    help="with --decode-only: only this entry of the decoding shapes")
    ap.add_argument("--mfma-peak-only", action="store_true",
                    help="only the register-only MFMA rate (one JSON line)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 1 GiB device copy three times (reference for HBM counters)")
    args = ap.parse_args(argv)

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py: this path runs on one GPU; --gpus {args.gpus} (WORLD_SIZE={world}) is not "
              "supported. Heads are independent, so several GPUs would each run this same kernel on "
              "their share of the heads.", file=sys.stderr)
        return 2

    import torch
    import io_aware_tiled_attention_amd as fa
    from workloads import PROBLEMS, make_inputs

    if not torch.cuda.is_available():
        print("bench.py needs a ROCm GPU", file=sys.stderr)
        return 1
    dev = torch.device("cuda", 0)
    if args.copy_calibration:
        n = 1 << 28                       # 2**28 fp32 = 1 GiB per tensor
        src = torch.ones(n, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration": {"bytes_read_per_copy": 4 * n, "bytes_written_per_copy": 4 * n,
                                               "copies": 3}}), flush=True)
        return 0
    if args.mfma_peak_only:
        print(json.dumps({"mfma_peak": mfma_peak_measurement(torch, dev)}), flush=True)
        return 0
    if args.configs_only:
        print(json.dumps({"configs": config_measurement(fa, torch, dev, names=args.config)}), flush=True)
        return 0
    if args.sparse_only:
        print(json.dumps({"block_sparse_16k_d128": sparse_measurement(fa, torch, dev, max(3, args.steps))}), flush=True)
        return 0
    if args.fp8_only:
        print(json.dumps({"fp8_16k_d128": fp8_measurement(fa, torch, dev, max(3, args.steps))}), flush=True)
        return 0
    if args.dropout_only:
        print(json.dumps({"dropout_16k_d128": dropout_measurement(fa, torch, dev, max(3, args.steps))}), flush=True)
        return 0
    if args.decode_only:
        shapes = None if args.decode_shape is None else [DECODE_SHAPES[args.decode_shape]]
        print(json.dumps({"decode_bf16_d128": decode_measurement(fa, torch, dev, max(10, args.steps), shapes)}),
              flush=True)
        return 0
    p = PROBLEMS[args.workload]
    inputs = make_inputs(p, with_do=True)
    step = Step(fa, torch, inputs, p, dev)
    ms_step, step_avg = time_steps(step, torch, args.steps, args.warmup)
    kt = kernel_table(p, time_kernels(step, torch, args.steps), step_avg)

    total_flops = p.fwd_flops() + p.bwd_flops()
    value = total_flops / ms_step * 1e-9
    dom = max(("fwd", "bwd_dkdv", "bwd_dq"), key=lambda k: kt[k]["ms"])
    traffic = measured_traffic(kt[dom]["kernel"])
    roofline = {"bound": "mfma", "kernel": kt[dom]["kernel"], "achieved": kt[dom]["tflops"],
                "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s", "frac": kt[dom]["tflops"] / PEAK_BF16_TFLOPS,
                "traffic": traffic, "flops_per_launch": kt[dom]["flops"], "avg_launch_ms": kt[dom]["ms"]}
    mp = mfma_peak_measurement(torch, dev)
    roofline["measured_peak"] = mp["tflops"]
    roofline["frac_of_measured_peak"] = kt[dom]["tflops"] / mp["tflops"]

    extra = {}
    if not args.no_extra:
        p4 = PROBLEMS["causal_4k_d128_bwd"]
        del step
        torch.cuda.empty_cache()
        s4 = Step(fa, torch, make_inputs(p4, with_do=True), p4, dev)
        ms4, step4 = time_steps(s4, torch, max(5, args.steps // 2), 3)
        k4 = kernel_table(p4, time_kernels(s4, torch, max(5, args.steps // 2)), step4)
        extra[p4.name] = {"B": p4.B, "H": p4.H, "N": p4.N, "d": p4.d, "causal": True, "ms_per_step": ms4,
                          "fwd_tflops": k4["fwd"]["tflops"], "fwd_frac_peak": k4["fwd"]["frac_peak"],
                          "bwd_tflops": k4["bwd_total"]["tflops"], "bwd_frac_peak": k4["bwd_total"]["frac_peak"]}
        del s4
        torch.cuda.empty_cache()
        extra["block_sparse_16k_d128"] = sparse_measurement(fa, torch, dev, max(5, args.steps // 2))
        torch.cuda.empty_cache()
        extra["decode_bf16_d128"] = decode_measurement(fa, torch, dev, max(10, args.steps))
        torch.cuda.empty_cache()
        extra["dropout_16k_d128"] = dropout_measurement(fa, torch, dev, max(5, args.steps // 2))
        torch.cuda.empty_cache()
        extra["fp8_16k_d128"] = fp8_measurement(fa, torch, dev, max(5, args.steps // 2))
        torch.cuda.empty_cache()
        extra["configs"] = config_measurement(fa, torch, dev)
        torch.cuda.empty_cache()
        ceil = gemm_ceiling_measurement(torch, dev, 5)
        g16 = ceil["bf16_tflops"]
        ceil["frac_of_bf16_gemm"] = {"fwd": kt["fwd"]["tflops"] / g16, "bwd_dkdv": kt["bwd_dkdv"]["executed_tflops"] / g16,
                                     "bwd_dq": kt["bwd_dq"]["executed_tflops"] / g16,
                                     "bwd_total_executed": kt["bwd_total"]["executed_tflops"] / g16}
        if "fp8_tflops" in ceil:
            ceil["fp8_fwd_frac_of_fp8_gemm"] = extra["fp8_16k_d128"]["tflops"] / ceil["fp8_tflops"]
        extra["gemm_ceiling"] = ceil

    out = {
        "metric": METRIC, "value": value, "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": ms_step, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": p.dtype, "data": "synthetic",
        "config": {"workload": f"{p.name}: causal attention forward + backward", "B": p.B, "H": p.H,
                   "N": p.N, "d": p.d, "causal": p.causal, "flops_per_step": total_flops,
                   "accumulation": "fp32"},
        "fwd": {"tflops": p.fwd_flops() / step_avg["fwd"] * 1e-9,
                "frac_peak": p.fwd_flops() / step_avg["fwd"] * 1e-9 / PEAK_BF16_TFLOPS, "ms": step_avg["fwd"],
                "frac_of_measured_peak": p.fwd_flops() / step_avg["fwd"] * 1e-9 / mp["tflops"]},
        "bwd": {"tflops": kt["bwd_total"]["tflops"], "frac_peak": kt["bwd_total"]["frac_peak"],
                "ms": kt["bwd_total"]["ms"], "frac_of_measured_peak": kt["bwd_total"]["tflops"] / mp["tflops"]},
        "mfma_peak": mp,
        "kernels": kt,
        "roofline": roofline,
        "extra": extra,
        "kernel_source_digest": kernel_source_digest(),
    }
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(inputs, p, args.cpu_heads)
        if not args.no_extra:
            out["cpu_baseline"]["per_config_one_head"] = cpu_config_heads()
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
