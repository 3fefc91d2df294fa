"""GPU parity of fa_decode (split-KV decoding) against the fp64 oracle (needs an MI355X).

Decoding: "Как работает FlashAttention математически", section 9
(FlashDecoding): the new query rows are the last Nq positions and attend to
the cached keys; the per-chunk partial results are merged with the rule for
concatenated key blocks ("Overview of Flash Attention series", Tiling).  The
result does not depend on the number of chunks beyond rounding.
"""
import numpy as np
import pytest
import torch

import io_aware_tiled_attention_amd as fa
from workloads import decode_inputs, random_inputs

from gpu_helpers import TOL, TOL_LSE, announce, assert_close, require_gpu, to64
from oracle import attention_ref as ref

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


def run_decode(inputs, causal, scale, splits=0, workspace=None):
    """fa_decode on the GPU; O and lse start as NaN so that a row the kernel
    never writes fails the comparison."""
    dev = torch.device("cuda", 0)
    q, k, v = (inputs[n].to(dev) for n in ("q", "k", "v"))
    o = torch.full_like(q, float("nan"))
    lse = torch.full(q.shape[:3], float("nan"), dtype=torch.float32, device=dev)
    fa.decode(q, k, v, causal=causal, scale=scale, num_splits=splits, out=o, lse=lse, workspace=workspace)
    torch.cuda.synchronize()
    return o.cpu(), lse.cpu()


def check(inputs, o, lse, causal, scale, heads=None):
    q, k, v = (to64(inputs[n]) for n in ("q", "k", "v"))
    B, H = q.shape[:2]
    tol = TOL["f32" if inputs["q"].dtype == torch.float32 else "bf16"]
    heads = heads if heads is not None else [(b, h) for b in range(B) for h in range(H)]
    for b, h in heads:
        o_r, lse_r = ref.decode_head(q[b, h], k[b, h], v[b, h], causal, scale)
        assert_close(f"O[{b},{h}]", o[b, h], o_r, tol, bf16_output=o.dtype == torch.bfloat16)
        assert_close(f"lse[{b},{h}]", lse[b, h], lse_r, TOL_LSE)


@pytest.mark.parametrize("dtype,B,H,Nq,Nk,d,causal,splits", [
    ("bf16", 1, 4, 1, 4096, 128, True, 0),
    ("bf16", 2, 3, 1, 1000, 64, False, 0),
    ("bf16", 1, 2, 7, 777, 128, True, 5),
    ("bf16", 1, 2, 32, 33, 128, True, 0),
    ("bf16", 1, 2, 32, 32, 64, True, 1),
    ("bf16", 1, 2, 4, 100, 64, True, 50),      # more chunks requested than tiles
    ("bf16", 1, 3, 1, 1, 128, True, 0),        # a one-entry cache
    ("bf16", 2, 2, 3, 31, 64, False, 0),       # less than one tile of keys
    ("bf16", 1, 2, 20, 10, 128, False, 0),     # non-causal: more queries than keys
    ("f32", 1, 2, 1, 513, 128, True, 0),
    ("f32", 2, 2, 5, 300, 64, False, 3),
    ("f32", 1, 1, 16, 16, 128, True, 0),
    ("f32", 1, 2, 32, 2049, 64, True, 9),
    ("bf16", 1, 2, 3, 8192, 64, True, 100),    # more than 64 chunks: the merge takes two rounds
    ("f32", 1, 1, 2, 4200, 128, False, 130),   # three merge rounds, chunks of one or two tiles
])
def test_decode_matches_oracle(dtype, B, H, Nq, Nk, d, causal, splits):
    S = fa.fa_decode_num_splits(B, H, Nk, splits)
    announce(f"decode {dtype} B={B} H={H} Nq={Nq} Nk={Nk} d={d} causal={causal} splits={splits}->{S}")
    inputs = decode_inputs(B, H, Nq, Nk, d, dtype, seed=1200 + Nq * 7 + Nk + d)
    scale = 1.0 / np.sqrt(d)
    o, lse = run_decode(inputs, causal, scale, splits)
    check(inputs, o, lse, causal, scale)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_decode_result_independent_of_chunk_count(dtype):
    announce(f"decode {dtype} chunk counts 1, 2, 7, 64, auto")
    B, H, Nq, Nk, d = 1, 2, 3, 2048, 128
    inputs = decode_inputs(B, H, Nq, Nk, d, dtype, seed=1301)
    scale = 1.0 / np.sqrt(d)
    outs = []
    for s in (1, 2, 7, 64, 0):
        o, lse = run_decode(inputs, True, scale, s)
        check(inputs, o, lse, True, scale)
        outs.append((o.double(), lse.double()))
    tol = TOL[dtype]
    for o, lse in outs[1:]:
        assert float((o - outs[0][0]).abs().max()) <= 2 * tol
        assert float((lse - outs[0][1]).abs().max()) <= TOL_LSE


def test_decode_workspace_contents_do_not_matter():
    """The workspace is scratch: one buffer filled with garbage (0xff bytes,
    then whatever the previous call left) serves calls with different chunk
    counts, each exact."""
    announce("decode workspace reuse: chunk counts 16, 5, 64, 16 on one garbage-filled workspace")
    dev = torch.device("cuda", 0)
    B, H, Nq, Nk, d = 2, 3, 4, 4096, 128
    inputs = decode_inputs(B, H, Nq, Nk, d, "bf16", seed=1303)
    need = max(fa.fa_decode_workspace_size(B, H, Nq, Nk, d, s) for s in (16, 5, 64))
    ws = torch.full((need,), 255, dtype=torch.uint8, device=dev)
    scale = 1.0 / np.sqrt(d)
    for s in (16, 5, 64, 16):
        o, lse = run_decode(inputs, True, scale, s, workspace=ws)
        check(inputs, o, lse, True, scale)


def test_decode_equals_last_rows_of_causal_forward():
    announce("decode == last 32 rows of causal forward, bf16 N=1500 d=128")
    B, H, N, d, nq = 1, 2, 1500, 128, 32
    inputs = random_inputs(B, H, N, d, "bf16", seed=1302)
    dev = torch.device("cuda", 0)
    q, k, v = (inputs[n].to(dev) for n in ("q", "k", "v"))
    o_f, lse_f = fa.forward(q, k, v, causal=True)
    o_d, lse_d = fa.decode(q[:, :, N - nq:].contiguous(), k, v, causal=True)
    torch.cuda.synchronize()
    dec = {"q": inputs["q"][:, :, N - nq:].contiguous(), "k": inputs["k"], "v": inputs["v"]}
    check(dec, o_d.cpu(), lse_d.cpu(), True, 1.0 / np.sqrt(d))
    diff = (o_d.float() - o_f[:, :, N - nq:].float()).abs().max().item()
    assert diff <= 2 * TOL["bf16"], diff
    assert (lse_d - lse_f[:, :, N - nq:]).abs().max().item() <= TOL_LSE


@pytest.mark.parametrize("B,H,Nq,Nk", [(1, 32, 1, 65536), (8, 32, 4, 8192)])
def test_decode_full_size_sampled_heads(B, H, Nq, Nk):
    announce(f"decode bf16 B={B} H={H} Nq={Nq} Nk={Nk} d=128 causal, sampled heads")
    d = 128
    inputs = decode_inputs(B, H, Nq, Nk, d, "bf16", seed=1400 + B)
    scale = 1.0 / np.sqrt(d)
    o, lse = run_decode(inputs, True, scale)
    rng = np.random.default_rng(7)
    heads = {(0, 0), (B - 1, H - 1)} | {(int(rng.integers(B)), int(rng.integers(H))) for _ in range(4)}
    check(inputs, o, lse, True, scale, heads=sorted(heads))
    assert torch.isfinite(o.float()).all() and torch.isfinite(lse).all()


def test_decode_empty_problem_leaves_outputs_alone():
    announce("decode Nq=0")
    dev = torch.device("cuda", 0)
    q = torch.empty((1, 2, 0, 64), dtype=torch.bfloat16, device=dev)
    k = torch.randn((1, 2, 16, 64), device=dev).to(torch.bfloat16)
    o, lse = fa.decode(q, k, k, causal=True)
    torch.cuda.synchronize()
    assert o.shape == (1, 2, 0, 64) and lse.shape == (1, 2, 0)
