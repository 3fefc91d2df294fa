"""Shared helpers for the GPU parity tests: run the library, run the oracle, compare.

Tolerances (max-abs, against the fp64 oracle on the same rounded inputs):
  fp32 inputs: 1e-5 on O; on dQ, dK, dV 1e-5 * max(1, max|ref|): gradients
    reach |10| and more, and an fp32 exponent argument near 10 is only known
    to ~1e-6 (its ulp), which every probability inherits as relative error;
  bf16 inputs: 2e-2 on O, dQ, dK, dV (fp32 accumulation), except where one
    bf16 ulp of the reference value is larger (|x| >= 4): an output of
    magnitude 8 cannot be represented in bf16 to better than 0.031, so there
    the bar is one ulp of the reference value;
  lse: 1e-3 for every input type.
"""
from __future__ import annotations

import sys

import numpy as np
import torch

import io_aware_tiled_attention_amd as fa
from oracle import attention_ref as ref

TOL = {"f32": 1e-5, "bf16": 2e-2}
TOL_LSE = 1e-3


def require_gpu():
    if not torch.cuda.is_available():
        raise RuntimeError("GPU tests need a ROCm device (run them with -m gpu on an MI355X)")
    fa.load_library()  # raises if the HIP library is missing: no fallback


def dtype_name(t: torch.Tensor) -> str:
    return "f32" if t.dtype == torch.float32 else "bf16"


def to64(t: torch.Tensor) -> np.ndarray:
    return t.detach().to("cpu", torch.float64).numpy()


def announce(msg: str):
    print(f"[case] {msg}", flush=True)
    sys.stdout.flush()


def gpu_forward(inputs, causal, scale):
    dev = torch.device("cuda", 0)
    q, k, v = (inputs[n].to(dev) for n in ("q", "k", "v"))
    o, lse = fa.forward(q, k, v, causal=causal, scale=scale)
    torch.cuda.synchronize()
    return o.cpu(), lse.cpu()


def gpu_backward(inputs, causal, scale, o=None, lse=None):
    """Forward on the GPU for O and lse (unless given), then the backward."""
    dev = torch.device("cuda", 0)
    q, k, v, do = (inputs[n].to(dev) for n in ("q", "k", "v", "do"))
    if o is None:
        o, lse = fa.forward(q, k, v, causal=causal, scale=scale)
    else:
        o, lse = o.to(dev), lse.to(dev)
    dq, dk, dv = fa.backward(q, k, v, o, do, lse, causal=causal, scale=scale)
    torch.cuda.synchronize()
    return o.cpu(), lse.cpu(), dq.cpu(), dk.cpu(), dv.cpu()


def bf16_ulp(x: np.ndarray) -> np.ndarray:
    """Spacing of bf16 numbers at |x| (8 significand bits): 2**(floor(log2|x|) - 7)."""
    ax = np.maximum(np.abs(x), np.finfo(np.float32).tiny)
    return np.exp2(np.floor(np.log2(ax)) - 7)


def max_err(got: torch.Tensor, want: np.ndarray) -> float:
    g = to64(got)
    assert np.all(np.isfinite(g)), "non-finite values in GPU output"
    return float(np.max(np.abs(g - want))) if g.size else 0.0


def assert_close(name, got, want, tol, bf16_output=False):
    """max |got - want| <= tol, per element; bf16 outputs: <= max(tol, ulp(want))."""
    g = to64(got)
    assert np.all(np.isfinite(g)), f"{name}: non-finite values in GPU output"
    want = np.asarray(want, dtype=np.float64)
    if g.size == 0:
        return
    err = np.abs(g - want)
    bar = np.maximum(tol, bf16_ulp(want)) if bf16_output else np.full_like(err, tol)
    worst = int(np.argmax(err / bar))
    ratio = float(err.flat[worst] / bar.flat[worst])
    mag = float(np.max(np.abs(want)))
    print(f"    {name}: max|err| = {float(err.max()):.3e} (tol {tol:.0e}{'/ulp' if bf16_output else ''}, "
          f"worst err/bar = {ratio:.2f}, max|ref| = {mag:.3f})", flush=True)
    assert ratio <= 1.0, (f"{name}: error {float(err.flat[worst]):.3e} > bar {float(bar.flat[worst]):.3e} "
                          f"at ref {float(want.flat[worst]):.4f}")


def check_forward_full(inputs, causal, scale, heads=None):
    """Compare O and lse of every row of the listed (b, h) heads (all if None)."""
    o, lse = gpu_forward(inputs, causal, scale)
    q, k, v = (to64(inputs[n]) for n in ("q", "k", "v"))
    tol = TOL[dtype_name(inputs["q"])]
    B, H = q.shape[:2]
    heads = heads if heads is not None else [(b, h) for b in range(B) for h in range(H)]
    for b, h in heads:
        o_ref, lse_ref = ref.forward_head(q[b, h], k[b, h], v[b, h], causal=causal, scale=scale)
        assert_close(f"O[{b},{h}]", o[b, h], o_ref, tol, bf16_output=o.dtype == torch.bfloat16)
        assert_close(f"lse[{b},{h}]", lse[b, h], lse_ref, TOL_LSE)
    return o, lse


def check_forward_rows(inputs, causal, scale, rows_per_head, seed=0, o=None, lse=None):
    """Compare sampled rows of every head (first, last, tile edges, random)."""
    if o is None:
        o, lse = gpu_forward(inputs, causal, scale)
    q, k, v = (inputs[n] for n in ("q", "k", "v"))
    B, H, N, _ = q.shape
    tol = TOL[dtype_name(q)]
    rng = np.random.default_rng(seed)
    fixed = [0, 1, 31, 32, 63, 64, 127, 128, N // 2, N - 2, N - 1]
    o_got, o_want, l_got, l_want = [], [], [], []
    for b in range(B):
        for h in range(H):
            rows = sorted(set([r for r in fixed if 0 <= r < N] +
                              rng.integers(0, N, size=rows_per_head).tolist()))
            o_ref, lse_ref = ref.forward_rows(to64(q[b, h]), to64(k[b, h]), to64(v[b, h]), rows,
                                              causal=causal, scale=scale)
            o_got.append(o[b, h, rows])
            o_want.append(o_ref)
            l_got.append(lse[b, h, rows])
            l_want.append(lse_ref)
    assert_close("sampled O rows", torch.cat(o_got), np.concatenate(o_want), tol,
                 bf16_output=o.dtype == torch.bfloat16)
    assert_close("sampled lse rows", torch.cat(l_got), np.concatenate(l_want), TOL_LSE)
    return o, lse


def grad_tol(dtype: str, want: np.ndarray) -> float:
    base = TOL[dtype]
    if dtype == "f32":
        return base * max(1.0, float(np.max(np.abs(want))) if np.size(want) else 1.0)
    return base


def check_backward_heads(inputs, causal, scale, heads=None, o=None, lse=None):
    o, lse, dq, dk, dv = gpu_backward(inputs, causal, scale, o, lse)
    q, k, v, do = (to64(inputs[n]) for n in ("q", "k", "v", "do"))
    dt = dtype_name(inputs["q"])
    B, H = q.shape[:2]
    heads = heads if heads is not None else [(b, h) for b in range(B) for h in range(H)]
    for b, h in heads:
        dq_r, dk_r, dv_r = ref.backward_head(q[b, h], k[b, h], v[b, h], do[b, h], causal=causal, scale=scale)
        bf = dt == "bf16"
        assert_close(f"dQ[{b},{h}]", dq[b, h], dq_r, grad_tol(dt, dq_r), bf16_output=bf)
        assert_close(f"dK[{b},{h}]", dk[b, h], dk_r, grad_tol(dt, dk_r), bf16_output=bf)
        assert_close(f"dV[{b},{h}]", dv[b, h], dv_r, grad_tol(dt, dv_r), bf16_output=bf)
    return dq, dk, dv
