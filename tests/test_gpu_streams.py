"""Calls on two streams at once (needs an MI355X).

The library keeps no state between calls: every buffer is the caller's, the
workspace included, and each call only enqueues kernels on the stream it is
given.  Two independent problems run concurrently on two streams (default
priority) must therefore give exactly what each gives alone.
"""
import pytest
import torch

import io_aware_tiled_attention_amd as fa
from workloads import block_mask, decode_inputs, random_inputs

from gpu_helpers import announce, require_gpu

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


def _problem(seed, N, d, causal):
    dev = torch.device("cuda", 0)
    inp = random_inputs(2, 8, N, d, "bf16", seed=seed, with_do=True)
    return {n: inp[n].to(dev) for n in ("q", "k", "v", "do")}, causal


def _run(p, causal, ws):
    o, lse = fa.forward(p["q"], p["k"], p["v"], causal=causal)
    dq, dk, dv = fa.backward(p["q"], p["k"], p["v"], o, p["do"], lse, causal=causal, workspace=ws)
    return [o, lse, dq, dk, dv]


def test_two_streams_concurrently_equal_each_alone():
    announce("two streams: forward + backward of two problems at once")
    dev = torch.device("cuda", 0)
    p1, c1 = _problem(7001, 2048, 128, True)
    p2, c2 = _problem(7002, 1500, 64, False)
    ws1 = torch.empty(fa.workspace_size(2, 8, 2048, 128), dtype=torch.uint8, device=dev)
    ws2 = torch.empty(fa.workspace_size(2, 8, 1500, 64), dtype=torch.uint8, device=dev)
    alone1 = _run(p1, c1, ws1)
    alone2 = _run(p2, c2, ws2)
    torch.cuda.synchronize()
    alone1 = [t.clone() for t in alone1]
    alone2 = [t.clone() for t in alone2]

    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    for rep in range(3):
        torch.cuda.synchronize()
        with torch.cuda.stream(s1):
            got1 = _run(p1, c1, ws1)
        with torch.cuda.stream(s2):
            got2 = _run(p2, c2, ws2)
        torch.cuda.synchronize()
        for name, a, b in zip(("o", "lse", "dq", "dk", "dv"), got1, alone1):
            assert torch.equal(a, b), f"rep {rep}: problem 1 {name} differs when run beside problem 2"
        for name, a, b in zip(("o", "lse", "dq", "dk", "dv"), got2, alone2):
            assert torch.equal(a, b), f"rep {rep}: problem 2 {name} differs when run beside problem 1"


def test_two_streams_block_sparse_and_decode():
    announce("two streams: block-sparse forward beside split-KV decoding")
    dev = torch.device("cuda", 0)
    inp = random_inputs(1, 4, 1024, 128, "bf16", seed=7003)
    q, k, v = (inp[n].to(dev) for n in ("q", "k", "v"))
    mask = block_mask(4, 1024, 128, 64, "random", seed=9, density=0.5).to(dev)
    dinp = decode_inputs(2, 8, 4, 6000, 128, "bf16", seed=7004)
    dq_, dk_, dv_ = (dinp[n].to(dev) for n in ("q", "k", "v"))
    o_s, lse_s = fa.forward_block_sparse(q, k, v, mask, 128, 64, causal=True)
    o_d, lse_d = fa.decode(dq_, dk_, dv_, causal=True)
    torch.cuda.synchronize()
    want = [o_s.clone(), lse_s.clone(), o_d.clone(), lse_d.clone()]
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    for rep in range(3):
        torch.cuda.synchronize()
        with torch.cuda.stream(s1):
            a = fa.forward_block_sparse(q, k, v, mask, 128, 64, causal=True)
        with torch.cuda.stream(s2):
            b = fa.decode(dq_, dk_, dv_, causal=True)
        torch.cuda.synchronize()
        for name, x, y in zip(("o_sparse", "lse_sparse", "o_decode", "lse_decode"), [*a, *b], want):
            assert torch.equal(x, y), f"rep {rep}: {name} differs under concurrency"
