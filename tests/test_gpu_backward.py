"""GPU parity of fa_backward against the fp64 chain-rule oracle (needs an MI355X)."""
import math

import numpy as np
import pytest
import torch

import io_aware_tiled_attention_amd as fa
from oracle import attention_ref as ref
from workloads import PROBLEMS, make_inputs, random_inputs

from gpu_helpers import TOL, announce, assert_close, check_backward_heads, gpu_backward, require_gpu, to64

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


def test_causal_bwd_4k_d64_all_heads():
    """C5: all 4 x 16 heads compared whole; O and lse come from fa_forward on
    the same inputs."""
    p = PROBLEMS["causal_bwd_4k_d64"]
    announce(p.name + " (all 64 heads whole)")
    check_backward_heads(make_inputs(p), p.causal, p.scale)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("n", [1, 2, 63, 65, 129, 257])
def test_ragged_lengths(n, causal, d, dtype):
    announce(f"bwd ragged N={n} d={d} causal={causal} {dtype}")
    inputs = random_inputs(2, 2, n, d, dtype, seed=9000 + n + d, with_do=True)
    check_backward_heads(inputs, causal, 1.0 / math.sqrt(d))


@pytest.mark.parametrize("dtype,d", [("f32", 64), ("f32", 128), ("bf16", 64), ("bf16", 128)])
def test_multi_block(dtype, d):
    announce(f"bwd N=640 d={d} {dtype}")
    inputs = random_inputs(1, 3, 640, d, dtype, seed=123 + d, with_do=True)
    check_backward_heads(inputs, False, 1.0 / math.sqrt(d))
    # A sharper softmax (scale 0.3 at d=64 gives |dQ| up to 8) only in fp32:
    # in bf16, D_i = do_i . o_i is formed from the stored bf16 O, whose
    # rounding alone moves dQ by ~0.03 there (reproduced exactly by a CPU
    # emulation of the rounding steps), beyond the 2e-2 bar.
    check_backward_heads(inputs, True, 0.3 if dtype == "f32" else 1.0 / math.sqrt(d))


def test_causal_4k_d128_backward_eight_heads():
    """The 4K d=128 backward shape: heads 0-7 of batch 0 (one per XCD) and
    the last head, whole."""
    p = PROBLEMS["causal_4k_d128_bwd"]
    announce(p.name + " (heads (0,0)-(0,7) and (3,31) whole)")
    inputs = make_inputs(p)
    check_backward_heads(inputs, True, p.scale, heads=[(0, h) for h in range(8)] + [(3, 31)])


@pytest.mark.slow
def test_causal_16k_d128_backward_eight_heads():
    """The 16K d=128 backward (the bench workload, not one of the five parity
    configurations): heads 0-7 whole, one per XCD.  Its stressed keys (1% of
    K scaled by 8) put probabilities near 1 on thousands of queries, so dV_j
    sums thousands of sizeable terms P_ij dO_i, each with P_ij rounded to bf16
    (the matrix cores' operand type).  A CPU emulation of that rounding alone
    (fp64 otherwise) puts one element of head 4 at 0.0219 from the fp64 value
    (reference 6.39693, emulated 6.375, exactly the GPU's result), past the
    strict 2e-2.  So the gradients here are held to the strict bar or, where
    the bf16 rounding of the operands can exceed it, to that rounding's
    first-order bound; the count of elements above the strict bar is printed."""
    p = PROBLEMS["causal_16k_d128_bwd"]
    announce(p.name + " (heads 0-7 whole)")
    inputs = make_inputs(p)
    check_backward_heads(inputs, True, p.scale, heads=[(0, h) for h in range(8)], operand_bound=True)


def test_backward_matches_finite_differences_of_gpu_forward_sign():
    """dV from the GPU against the GPU forward's own response to a V step."""
    announce("bwd vs forward difference")
    dev = torch.device("cuda", 0)
    inputs = random_inputs(1, 1, 96, 64, "f32", seed=77, with_do=True)
    q, k, v, do = (inputs[n].to(dev) for n in ("q", "k", "v", "do"))
    o, lse = fa.forward(q, k, v, causal=True)
    dq, dk, dv = fa.backward(q, k, v, o, do, lse, causal=True)
    h = 1e-2
    dirv = torch.randn(v.shape, generator=torch.Generator().manual_seed(3)).to(dev)
    o_p, _ = fa.forward(q, k, v + h * dirv, causal=True)
    o_m, _ = fa.forward(q, k, v - h * dirv, causal=True)
    fd = float(((o_p - o_m) * do).sum() / (2 * h))
    an = float((dv * dirv).sum())
    assert abs(fd - an) <= 1e-3 * max(1.0, abs(an))


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_staged_entry_points_equal_fused(dtype):
    """preprocess, dq, dkdv entry points == fa_backward, bit for bit."""
    announce(f"staged backward {dtype}")
    dev = torch.device("cuda", 0)
    inputs = random_inputs(2, 3, 300, 128, dtype, seed=31, with_do=True)
    q, k, v, do = (inputs[n].to(dev) for n in ("q", "k", "v", "do"))
    o, lse = fa.forward(q, k, v, causal=True)
    dq1, dk1, dv1 = fa.backward(q, k, v, o, do, lse, causal=True)
    dq2, dk2, dv2 = fa.backward_stages(q, k, v, o, do, lse, causal=True)
    torch.cuda.synchronize()
    assert torch.equal(dk1, dk2) and torch.equal(dv1, dv2) and torch.equal(dq1, dq2)


def test_workspace_reuse_and_garbage_contents():
    """A reused workspace full of garbage gives the same gradients."""
    announce("workspace reuse")
    dev = torch.device("cuda", 0)
    inputs = random_inputs(1, 2, 500, 64, "bf16", seed=41, with_do=True)
    q, k, v, do = (inputs[n].to(dev) for n in ("q", "k", "v", "do"))
    o, lse = fa.forward(q, k, v, causal=False)
    ws = torch.full((fa.workspace_size(1, 2, 500, 64),), 0x7F, dtype=torch.uint8, device=dev)
    dq1, dk1, dv1 = fa.backward(q, k, v, o, do, lse, workspace=ws)
    dq2, dk2, dv2 = fa.backward(q, k, v, o, do, lse, workspace=ws)
    torch.cuda.synchronize()
    assert torch.equal(dk1, dk2) and torch.equal(dv1, dv2) and torch.equal(dq1, dq2)


@pytest.mark.parametrize("dtype,B,H,N,d", [("f32", 2, 3, 100003, 128), ("bf16", 1, 9, 250001, 64)])
def test_preprocess_strides_over_more_rows_than_its_grid(dtype, B, H, N, d):
    """The row statistics D_i = dO_i . O_i and -lse_i (in the exponent domain:
    base 2 for bf16, base e for fp32) for more rows than one pass of the
    preprocess grid covers (65536 blocks of 8 rows at fp32 d=128, of 32 rows at
    bf16 d=64), with a ragged last block.  White box: the workspace holds D for
    every row, then -lse, each region padded to 256 bytes; it starts as NaN so
    that a row left unwritten shows."""
    rows = B * H * N
    announce(f"backward preprocess {dtype} rows={rows} d={d}")
    dev = torch.device("cuda", 0)
    tdt = torch.float32 if dtype == "f32" else torch.bfloat16
    g = torch.Generator(device=dev).manual_seed(77)
    o = torch.randn((B, H, N, d), generator=g, device=dev).to(tdt)
    do = torch.randn((B, H, N, d), generator=g, device=dev).to(tdt)
    lse = torch.randn((B, H, N), generator=g, device=dev) * 3.0
    need = fa.workspace_size(B, H, N, d)
    ws = torch.full((need // 4,), float("nan"), dtype=torch.float32, device=dev)
    code = fa._lib.FA_F32 if dtype == "f32" else fa._lib.FA_BF16
    st = fa.fa_backward_preprocess(o.data_ptr(), do.data_ptr(), lse.data_ptr(), B, H, N, d, code, ws.data_ptr(),
                                   need, torch.cuda.current_stream().cuda_stream)
    assert st == 0
    torch.cuda.synchronize()
    region = (rows * 4 + 255) // 256 * 256 // 4
    dsum, nlse = ws[:rows], ws[region:region + rows]
    prod = o.reshape(rows, d).double() * do.reshape(rows, d).double()
    want = prod.sum(-1)
    bound = 1e-5 * prod.abs().sum(-1) + 1e-30
    err = (dsum.double() - want).abs()
    assert bool(torch.isfinite(dsum).all()), "a row's D was not written"
    assert bool((err <= bound).all()), f"D: worst err/bound {float((err / bound).max()):.3g}"
    factor = 1.0 / math.log(2.0) if dtype == "bf16" else 1.0
    want_n = -lse.reshape(rows).double() * factor
    assert bool(torch.isfinite(nlse).all()), "a row's -lse was not written"
    assert float((nlse.double() - want_n).abs().max()) <= 1e-6 * float(want_n.abs().max())
