"""Shared helpers for the GPU parity tests: run the library, run the oracle, compare.

Tolerances (max-abs, against the fp64 oracle on the same rounded inputs):
  fp32 inputs: 1e-5 on O; on dQ, dK, dV 1e-5 * max(1, max|ref|): gradients
    reach |10| and more, and an fp32 exponent argument near 10 is only known
    to ~1e-6 (its ulp), which every probability inherits as relative error;
  bf16 inputs: max-abs 2e-2 on O, dQ, dK, dV (fp32 accumulation) wherever
    the reference value has |x| < 8.  Half a bf16 ulp there is at most
    2^-6 = 0.0156 (the rounding of the output itself), which leaves
    0.0044 of the bar for the error before that rounding.  At |x| >= 8 half
    an ulp alone is 0.031 or more, so no bf16 output can meet 2e-2; there the
    bar is half an ulp of the reference (the representational floor) plus
    2^-10 |x| for the error before the rounding (the same allowance, relative
    to |x|, that 2e-2 leaves just below 8);
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


BF16_ABS_LIMIT = 8.0


def bf16_bar(want: np.ndarray, tol: float) -> np.ndarray:
    """Per-element bar for a bf16 output: ``tol`` where |ref| < 8, else half an
    ulp of the reference plus 2^-10 |ref| (see the module docstring)."""
    a = np.abs(want)
    return np.where(a < BF16_ABS_LIMIT, tol, 0.5 * bf16_ulp(want) + 2.0 ** -10 * a)


def max_err(got: torch.Tensor, want: np.ndarray) -> float:
    g = to64(got)
    assert np.all(np.isfinite(g)), "non-finite values in GPU output"
    return float(np.max(np.abs(g - want))) if g.size else 0.0


def assert_close(name, got, want, tol, bf16_output=False):
    """max |got - want| <= tol per element; bf16 outputs: <= bf16_bar(want, tol).

    Prints the largest error, the worst error/bar ratio, the largest
    reference magnitude, and for bf16 outputs how many reference values lie
    at |x| >= 8 (where the bar is half an ulp plus 2^-10 |x|) and the largest
    error among the others (held to ``tol`` exactly)."""
    g = to64(got)
    assert np.all(np.isfinite(g)), f"{name}: non-finite values in GPU output"
    want = np.asarray(want, dtype=np.float64)
    if g.size == 0:
        return
    err = np.abs(g - want)
    bar = bf16_bar(want, tol) if bf16_output else np.full_like(err, tol)
    worst = int(np.argmax(err / bar))
    ratio = float(err.flat[worst] / bar.flat[worst])
    mag = float(np.max(np.abs(want)))
    extra = ""
    if bf16_output:
        big = np.abs(want) >= BF16_ABS_LIMIT
        small_err = float(err[~big].max()) if np.any(~big) else 0.0
        extra = f", {int(big.sum())} with |ref| >= 8, max|err| where |ref| < 8 = {small_err:.3e}"
    print(f"    {name}: max|err| = {float(err.max()):.3e} (tol {tol:.0e}{'/bf16 bar' if bf16_output else ''}, "
          f"worst err/bar = {ratio:.2f}, max|ref| = {mag:.3f}{extra})", flush=True)
    assert ratio <= 1.0, (f"{name}: error {float(err.flat[worst]):.3e} > bar {float(bar.flat[worst]):.3e} "
                          f"at ref {float(want.flat[worst]):.4f}")
    return float(err.max()), ratio


def check_forward_full(inputs, causal, scale, heads=None, o=None, lse=None):
    """Compare O and lse of every row of the listed (b, h) heads (all if None);
    O and lse from the GPU forward unless given."""
    if o is None:
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


def operand_rounding_terms(q, k, v, do, causal, scale):
    """Sizes of the terms that the backward's bf16-rounded operands multiply
    (fp64, one head of standard attention):
      M_dV = P^T |dO|                (P is rounded to bf16 before dV = P^T dO)
      M_dQ = scale W |K|,  M_dK = scale W^T |Q|,  W = P o (|dP - D| + A)
    (dS = P o (dP - D) is rounded to bf16 before dQ and dK; A_r = sum_c
    |dO_rc O_rc| bounds the error that the bf16 rounding of the stored O
    puts into D_r).  Rounding an operand to bf16 moves it by at most 2^-8 of
    itself, so 2^-8 M bounds, to first order, what that rounding does to
    each gradient element."""
    s = scale * (q @ k.T)
    if causal:
        s[np.triu_indices(s.shape[0], 1)] = -np.inf
    m = np.max(s, axis=1, keepdims=True)
    p = np.exp(s - m)
    del s
    p /= np.sum(p, axis=1, keepdims=True)
    o = p @ v
    m_dv = p.T @ np.abs(do)
    dp = do @ v.T
    dsum = np.sum(do * o, axis=1)
    a = np.sum(np.abs(do * o), axis=1)
    w = p * (np.abs(dp - dsum[:, None]) + a[:, None])
    del p, dp
    return scale * (w @ np.abs(k)), scale * (w.T @ np.abs(q)), m_dv


def assert_close_or_operand_bound(name, got, want, m_terms):
    """bf16 gradient against max(bf16_bar, half an ulp + 2^-8 M): the strict
    bar, or where the bf16 rounding of the products' operands can exceed it,
    that rounding's first-order bound (M from operand_rounding_terms).  Also
    prints how many elements exceed the strict bar alone."""
    g = to64(got)
    assert np.all(np.isfinite(g)), f"{name}: non-finite values in GPU output"
    err = np.abs(g - want)
    strict = bf16_bar(want, TOL["bf16"])
    bar = np.maximum(strict, 0.5 * bf16_ulp(want) + 2.0 ** -8 * m_terms)
    worst = int(np.argmax(err / bar))
    ratio = float(err.flat[worst] / bar.flat[worst])
    over = err > strict
    print(f"    {name}: max|err| = {float(err.max()):.3e}, worst err/strict bar = {float(np.max(err / strict)):.2f}, "
          f"{int(over.sum())} of {err.size} above the strict bar, worst err/operand bound = {ratio:.2f}, "
          f"max|ref| = {float(np.abs(want).max()):.3f}", flush=True)
    assert ratio <= 1.0, (f"{name}: error {float(err.flat[worst]):.3e} > bar {float(bar.flat[worst]):.3e} "
                          f"at ref {float(want.flat[worst]):.4f}")


def check_backward_heads(inputs, causal, scale, heads=None, o=None, lse=None, operand_bound=False):
    """dQ, dK, dV of the listed heads (all if None) against the oracle.  With
    ``operand_bound`` (bf16 only) the gradients are held to
    assert_close_or_operand_bound instead of the strict bar."""
    o, lse, dq, dk, dv = gpu_backward(inputs, causal, scale, o, lse)
    q, k, v, do = (to64(inputs[n]) for n in ("q", "k", "v", "do"))
    dt = dtype_name(inputs["q"])
    B, H = q.shape[:2]
    heads = heads if heads is not None else [(b, h) for b in range(B) for h in range(H)]
    for b, h in heads:
        dq_r, dk_r, dv_r = ref.backward_head(q[b, h], k[b, h], v[b, h], do[b, h], causal=causal, scale=scale)
        bf = dt == "bf16"
        if operand_bound and bf:
            m_dq, m_dk, m_dv = operand_rounding_terms(q[b, h], k[b, h], v[b, h], do[b, h], causal, scale)
            assert_close_or_operand_bound(f"dQ[{b},{h}]", dq[b, h], dq_r, m_dq)
            assert_close_or_operand_bound(f"dK[{b},{h}]", dk[b, h], dk_r, m_dk)
            assert_close_or_operand_bound(f"dV[{b},{h}]", dv[b, h], dv_r, m_dv)
            continue
        assert_close(f"dQ[{b},{h}]", dq[b, h], dq_r, grad_tol(dt, dq_r), bf16_output=bf)
        assert_close(f"dK[{b},{h}]", dk[b, h], dk_r, grad_tol(dt, dk_r), bf16_output=bf)
        assert_close(f"dV[{b},{h}]", dv[b, h], dv_r, grad_tol(dt, dv_r), bf16_output=bf)
    return dq, dk, dv
