"""Launch order of the (head, tile) workgroups (needs an MI355X).

When B*H is a multiple of 8 the kernels deal the heads out to the XCDs and
walk each XCD's heads in groups; otherwise the heads are interleaved over the
grid.  The order changes nothing that a workgroup computes, so every head of
a batched call must be bit-identical to the same head computed alone (B*H = 1,
which takes the interleaved order).  A tile skipped or computed twice, or a
head written to another's output, shows up as a difference.

Shapes: B*H = 40 (5 heads per XCD) and 72 (9 per XCD).  At N = 2100 (17
query or key tiles of 128, the last ragged) the forward, dK/dV and dQ groups
hold 4 heads, so the XCDs' heads split into full groups and a short last one
(5 = 4 + 1, 9 = 4 + 4 + 1), and the FP8 forward's groups hold 6 (5 = one
short group, 9 = 6 + 3).  At N = 640 (5 tiles) every group is short.
"""
import pytest
import torch

import io_aware_tiled_attention_amd as fa
from workloads import fp8_inputs, random_inputs

from gpu_helpers import announce, require_gpu

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


def _per_head(fn, tensors):
    """fn applied to each head alone ([1, 1, N, d] contiguous copies); results re-stacked."""
    B, H = tensors[0].shape[:2]
    outs = []
    for b in range(B):
        for h in range(H):
            outs.append(fn(*(t[b:b + 1, h:h + 1].contiguous() for t in tensors)))
    return [torch.cat([o[i] for o in outs], dim=1).reshape(B, H, *outs[0][i].shape[2:]) for i in range(len(outs[0]))]


def _same(name, got, want):
    assert got.shape == want.shape, name
    eq = (got == want) | (torch.isnan(got) & torch.isnan(want))
    assert bool(eq.all()), f"{name}: {int((~eq).sum())} elements differ between the batched and per-head calls"


CASES = [(5, 8, 2100, 128, True), (1, 72, 2100, 128, True), (1, 40, 640, 64, False), (9, 8, 640, 128, True)]


@pytest.mark.parametrize("B,H,N,d,causal", CASES)
def test_forward_and_backward_batched_equal_per_head(B, H, N, d, causal):
    announce(f"launch order bf16 B={B} H={H} N={N} d={d} causal={causal}")
    dev = torch.device("cuda", 0)
    inp = random_inputs(B, H, N, d, "bf16", seed=4242 + N + H, with_do=True)
    q, k, v, do = (inp[n].to(dev) for n in ("q", "k", "v", "do"))
    o, lse = fa.forward(q, k, v, causal=causal)
    dq, dk, dv = fa.backward(q, k, v, o, do, lse, causal=causal)
    torch.cuda.synchronize()

    def one(q1, k1, v1, do1):
        o1, lse1 = fa.forward(q1, k1, v1, causal=causal)
        dq1, dk1, dv1 = fa.backward(q1, k1, v1, o1, do1, lse1, causal=causal)
        return [o1, lse1, dq1, dk1, dv1]

    ref = _per_head(one, [q, k, v, do])
    torch.cuda.synchronize()
    for name, got, want in zip(("o", "lse", "dq", "dk", "dv"), (o, lse, dq, dk, dv), ref):
        _same(name, got, want)


@pytest.mark.parametrize("B,H,N,d,causal", [(1, 72, 2100, 128, True), (5, 8, 2100, 64, False)])
def test_fp8_batched_equal_per_head(B, H, N, d, causal):
    announce(f"launch order fp8 B={B} H={H} N={N} d={d} causal={causal}")
    dev = torch.device("cuda", 0)
    inp = fp8_inputs(B, H, N, d, seed=777 + H)
    q, k, v = (inp[n].to(dev).view(torch.float8_e4m3fn) for n in ("q", "k", "v"))
    o, lse = fa.forward_fp8(q, k, v, causal=causal)
    torch.cuda.synchronize()
    ref = _per_head(lambda a, b, c: list(fa.forward_fp8(a, b, c, causal=causal)), [q, k, v])
    torch.cuda.synchronize()
    _same("o", o, ref[0])
    _same("lse", lse, ref[1])
