"""Seeded synthetic inputs for the attention problems (no attention arithmetic).

Shared by the oracle-side tests, the GPU parity tests and bench.py.  This
module only draws and rounds random numbers; it computes nothing of the
method.  Tensors are CPU torch tensors of shape [B, H, N, d] in the problem's
dtype, drawn in fp32 from one ``torch.Generator`` per problem in the order
Q, K, V, dO and rounded once to the dtype (round to nearest even).

Problems (named by what they are):

* ``single_head_f32``      B=1  H=1  N=256   d=64  fp32, non-causal, forward
* ``gpt2_small_bf16``      B=8  H=12 N=1024  d=64  bf16, non-causal, forward
* ``causal_4k_d128``       B=4  H=32 N=4096  d=128 bf16, causal, forward
* ``causal_16k_d128``      B=1  H=32 N=16384 d=128 bf16, causal; Q, K, V
  drawn N(0,1)*0.5, then in every (b, h) a random 1% of K rows (164 of
  16384) multiplied by 8 to make later key blocks raise the running max
* ``causal_bwd_4k_d64``    B=4  H=16 N=4096  d=64  bf16, causal, backward
  (dO ~ N(0,1))
* ``causal_16k_d128_bwd``  the 16K problem above plus dO ~ N(0,1)
* ``causal_4k_d128_bwd``   the 4K d=128 problem plus dO ~ N(0,1)
"""
from __future__ import annotations

import dataclasses
import math
from typing import Dict, Optional

import torch


@dataclasses.dataclass(frozen=True)
class Problem:
    name: str
    B: int
    H: int
    N: int
    d: int
    dtype: str          # "f32" or "bf16"
    causal: bool
    seed: int
    backward: bool = False
    qkv_mult: float = 1.0
    stress_frac: float = 0.0
    stress_mult: float = 1.0

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.d)

    @property
    def torch_dtype(self):
        return torch.float32 if self.dtype == "f32" else torch.bfloat16

    def fwd_flops(self) -> float:
        """4*B*H*N^2*d, halved when causal (the stated counting convention)."""
        f = 4.0 * self.B * self.H * self.N * self.N * self.d
        return f / 2 if self.causal else f

    def bwd_flops(self) -> float:
        """2.5 x the forward count (the stated counting convention)."""
        return 2.5 * self.fwd_flops()


PROBLEMS: Dict[str, Problem] = {p.name: p for p in [
    Problem("single_head_f32", 1, 1, 256, 64, "f32", False, 1001),
    Problem("gpt2_small_bf16", 8, 12, 1024, 64, "bf16", False, 1002),
    Problem("causal_4k_d128", 4, 32, 4096, 128, "bf16", True, 1003),
    Problem("causal_16k_d128", 1, 32, 16384, 128, "bf16", True, 1004,
            qkv_mult=0.5, stress_frac=0.01, stress_mult=8.0),
    Problem("causal_bwd_4k_d64", 4, 16, 4096, 64, "bf16", True, 1005, backward=True),
    Problem("causal_16k_d128_bwd", 1, 32, 16384, 128, "bf16", True, 1006,
            backward=True, qkv_mult=0.5, stress_frac=0.01, stress_mult=8.0),
    Problem("causal_4k_d128_bwd", 4, 32, 4096, 128, "bf16", True, 1007, backward=True),
]}


def make_inputs(p: Problem, *, with_do: Optional[bool] = None):
    """Draw q, k, v (and do) for problem ``p``; returns a dict of CPU tensors."""
    if with_do is None:
        with_do = p.backward
    g = torch.Generator(device="cpu")
    g.manual_seed(p.seed)
    shape = (p.B, p.H, p.N, p.d)
    q = torch.randn(shape, generator=g, dtype=torch.float32)
    k = torch.randn(shape, generator=g, dtype=torch.float32)
    v = torch.randn(shape, generator=g, dtype=torch.float32)
    if p.qkv_mult != 1.0:
        q.mul_(p.qkv_mult)
        k.mul_(p.qkv_mult)
        v.mul_(p.qkv_mult)
    if p.stress_frac > 0.0:
        count = int(round(p.stress_frac * p.N))
        for b in range(p.B):
            for h in range(p.H):
                rows = torch.randperm(p.N, generator=g)[:count]
                k[b, h, rows] *= p.stress_mult
    out = {"q": q, "k": k, "v": v}
    if with_do:
        out["do"] = torch.randn(shape, generator=g, dtype=torch.float32)
    return {name: t.to(p.torch_dtype).contiguous() for name, t in out.items()}


def random_inputs(B: int, H: int, N: int, d: int, dtype: str, seed: int,
                  with_do: bool = False, mult: float = 1.0):
    """Ad-hoc seeded N(0,1)*mult inputs for edge-case shapes (ragged N etc.)."""
    p = Problem("adhoc", B, H, N, d, dtype, False, seed, backward=with_do, qkv_mult=mult)
    return make_inputs(p)


def block_mask(heads: int, n: int, block_q: int, block_k: int, kind: str, seed: int,
               density: float = 0.5, window: int = 2):
    """Seeded uint8 block masks [heads, ceil(n/block_q), ceil(n/block_k)] (an input, no attention arithmetic).

    kind: "random" (each block kept with probability `density`), "ones",
    "local" (key blocks whose start lies within `window` query-block widths of
    the row block, sliding-window attention) or "local_global" (local plus the
    first key block column, as in long-document patterns).
    """
    tq, tk = -(-n // block_q), -(-n // block_k)
    g = torch.Generator().manual_seed(seed)
    if kind == "random":
        return (torch.rand((heads, tq, tk), generator=g) < density).to(torch.uint8)
    if kind == "ones":
        return torch.ones((heads, tq, tk), dtype=torch.uint8)
    rows = torch.arange(tq)[:, None] * block_q
    cols = torch.arange(tk)[None, :] * block_k
    m = (cols <= rows + block_q - 1) & (cols + block_k - 1 >= rows - window * block_q)
    if kind == "local_global":
        m[:, 0] = True
    elif kind != "local":
        raise ValueError(kind)
    return m.to(torch.uint8)[None].repeat(heads, 1, 1)


def decode_inputs(B: int, H: int, Nq: int, Nk: int, d: int, dtype: str, seed: int, mult: float = 1.0):
    """Seeded N(0,1)*mult decoding inputs: q [B, H, Nq, d] (the newest Nq
    positions) and a cache k, v [B, H, Nk, d]; a dict of CPU tensors."""
    g = torch.Generator(device="cpu")
    g.manual_seed(seed)
    q = torch.randn((B, H, Nq, d), generator=g, dtype=torch.float32) * mult
    k = torch.randn((B, H, Nk, d), generator=g, dtype=torch.float32) * mult
    v = torch.randn((B, H, Nk, d), generator=g, dtype=torch.float32) * mult
    td = torch.float32 if dtype == "f32" else torch.bfloat16
    return {name: t.to(td).contiguous() for name, t in (("q", q), ("k", k), ("v", v))}


def fp8_inputs(B: int, H: int, N: int, d: int, seed: int, mult: float = 1.0):
    """Seeded N(0,1)*mult q, k, v rounded once to OCP E4M3 (torch.float8_e4m3fn),
    returned as uint8 codes [B, H, N, d] (CPU tensors)."""
    g = torch.Generator(device="cpu")
    g.manual_seed(seed)
    out = {}
    for name in ("q", "k", "v"):
        x = torch.randn((B, H, N, d), generator=g, dtype=torch.float32) * mult
        out[name] = x.to(torch.float8_e4m3fn).view(torch.uint8).contiguous()
    return out


def device_inputs(B: int, H: int, N: int, d: int, dtype: str, seed: int, device, names=("q", "k", "v")):
    """Seeded N(0,1) inputs drawn directly on `device` (for sequences too long
    to draw and copy from the host in reasonable time): one device generator,
    the tensors in the order of `names`, each drawn in fp32 in slices of at
    most 2^26 elements and rounded once to the dtype.  A dict of device tensors."""
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    td = torch.float32 if dtype == "f32" else torch.bfloat16
    out = {}
    for name in names:
        t = torch.empty((B, H, N, d), dtype=td, device=device)
        flat = t.view(-1)
        step = 1 << 26
        for i in range(0, flat.numel(), step):
            n = min(step, flat.numel() - i)
            flat[i:i + n] = torch.randn(n, generator=g, dtype=torch.float32, device=device).to(td)
        out[name] = t
    return out
