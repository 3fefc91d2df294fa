"""GPU parity of fa_backward_block_sparse against the fp64 oracle (needs an MI355X).

The gradients of block-sparse attention ("Overview of Flash Attention series",
section Block-sparse Flashattention; backward steps from its Backward Pass):
blocks the mask removes pass no gradient, rows that keep no key get dQ = 0,
and keys no kept block reaches get dK = dV = 0.  O and lse come from the GPU's
block-sparse forward on the same inputs; the oracle computes its gradients
from Q, K, V, dO alone.
"""
import numpy as np
import pytest
import torch

import io_aware_tiled_attention_amd as fa
from workloads import block_mask, random_inputs

from gpu_helpers import announce, assert_close, dtype_name, grad_tol, require_gpu, to64
from oracle import attention_ref as ref

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


def run(inputs, mask, bq, bk, causal, scale):
    dev = torch.device("cuda", 0)
    q, k, v, do = (inputs[n].to(dev) for n in ("q", "k", "v", "do"))
    m = mask.to(dev)
    o, lse = fa.forward_block_sparse(q, k, v, m, bq, bk, causal=causal, scale=scale)
    dq, dk, dv = fa.backward_block_sparse(q, k, v, o, do, lse, m, bq, bk, causal=causal, scale=scale)
    torch.cuda.synchronize()
    return dq.cpu(), dk.cpu(), dv.cpu()


def check(inputs, mask, bq, bk, causal, scale, heads=None):
    dq, dk, dv = run(inputs, mask, bq, bk, causal, scale)
    q, k, v, do = (to64(inputs[n]) for n in ("q", "k", "v", "do"))
    dt = dtype_name(inputs["q"])
    bf = dt == "bf16"
    m = mask.numpy()
    B, H = q.shape[:2]
    heads = heads if heads is not None else [(b, h) for b in range(B) for h in range(H)]
    for b, h in heads:
        mh = m[h if m.shape[0] > 1 else 0]
        dq_r, dk_r, dv_r = ref.backward_block_sparse_head(q[b, h], k[b, h], v[b, h], do[b, h], mh, bq, bk,
                                                          causal, scale)
        assert_close(f"dQ[{b},{h}]", dq[b, h], dq_r, grad_tol(dt, dq_r), bf16_output=bf)
        assert_close(f"dK[{b},{h}]", dk[b, h], dk_r, grad_tol(dt, dk_r), bf16_output=bf)
        assert_close(f"dV[{b},{h}]", dv[b, h], dv_r, grad_tol(dt, dv_r), bf16_output=bf)
    return dq, dk, dv


@pytest.mark.parametrize("dtype,N,d,bq,bk,causal,kind,mheads", [
    ("bf16", 1024, 128, 128, 64, False, "random", 4),
    ("bf16", 1000, 64, 64, 64, True, "random", 1),
    ("bf16", 1024, 128, 256, 128, True, "local_global", 1),
    ("bf16", 777, 128, 32, 64, False, "random", 4),
    ("bf16", 600, 128, 96, 192, True, "random", 4),
    ("f32", 257, 64, 32, 128, True, "random", 1),
    ("f32", 320, 128, 64, 64, False, "local", 4),
    ("f32", 300, 128, 32, 64, True, "random", 4),
])
def test_block_sparse_backward_matches_oracle(dtype, N, d, bq, bk, causal, kind, mheads):
    announce(f"block-sparse backward {dtype} N={N} d={d} blocks {bq}x{bk} causal={causal} {kind} "
             f"mask_heads={mheads}")
    inputs = random_inputs(2, 4, N, d, dtype, seed=1900 + N + d + bq, with_do=True)
    mask = block_mask(mheads, N, bq, bk, kind, seed=N + bk + 1, density=0.45)
    check(inputs, mask, bq, bk, causal, 1.0 / np.sqrt(d))


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_block_sparse_backward_empty_rows_and_unreached_keys(dtype):
    announce(f"block-sparse backward {dtype}: rows with no key, keys no block reaches")
    N, d, bq, bk = 512, 64, 64, 64
    inputs = random_inputs(1, 2, N, d, dtype, seed=1931, with_do=True)
    mask = block_mask(2, N, bq, bk, "random", seed=15, density=0.5)
    mask[0, 3, :] = 0          # head 0: query block 3 keeps nothing
    mask[0, :, 6] = 0          # head 0: key block 6 is kept by no query block
    mask[1, :, :] = 0
    mask[1, 5, 2] = 1          # head 1: one block kept at all
    dq, dk, dv = check(inputs, mask, bq, bk, False, 0.125)
    assert torch.all(dq[0, 0, 192:256] == 0), "rows that keep no key must get dQ = 0"
    assert torch.all(dk[0, 0, 384:448] == 0) and torch.all(dv[0, 0, 384:448] == 0), "unreached keys: dK = dV = 0"
    keep_rows = torch.zeros(N, dtype=torch.bool)
    keep_rows[320:384] = True
    assert torch.all(dq[0, 1, ~keep_rows] == 0)
    keep_keys = torch.zeros(N, dtype=torch.bool)
    keep_keys[128:192] = True
    assert torch.all(dk[0, 1, ~keep_keys] == 0) and torch.all(dv[0, 1, ~keep_keys] == 0)


@pytest.mark.parametrize("causal", [False, True])
def test_block_sparse_backward_all_ones_equals_dense_bitwise(causal):
    announce(f"block-sparse backward all-ones mask vs dense, causal={causal}")
    dev = torch.device("cuda", 0)
    inputs = random_inputs(2, 3, 1000, 128, "bf16", seed=1940 + causal, with_do=True)
    q, k, v, do = (inputs[n].to(dev) for n in ("q", "k", "v", "do"))
    mask = block_mask(1, 1000, 128, 64, "ones", seed=0).to(dev)
    o, lse = fa.forward(q, k, v, causal=causal)
    g_s = fa.backward_block_sparse(q, k, v, o, do, lse, mask, 128, 64, causal=causal)
    g_d = fa.backward(q, k, v, o, do, lse, causal=causal)
    torch.cuda.synchronize()
    for name, a, b in zip(("dq", "dk", "dv"), g_s, g_d):
        assert torch.equal(a, b), name


def test_block_sparse_backward_long_local_global_sampled_heads():
    announce("block-sparse backward N=8192 d=128 local+global causal, 1 head checked")
    N, d, bq, bk = 8192, 128, 128, 128
    inputs = random_inputs(1, 2, N, d, "bf16", seed=1950, with_do=True)
    mask = block_mask(1, N, bq, bk, "local_global", seed=0, window=3)
    check(inputs, mask, bq, bk, True, 1.0 / np.sqrt(d), heads=[(0, 1)])


def test_block_sparse_backward_rejects_bad_geometry_before_launch():
    dev = torch.device("cuda", 0)
    inputs = random_inputs(1, 1, 256, 64, "bf16", seed=1960, with_do=True)
    q, k, v, do = (inputs[n].to(dev) for n in ("q", "k", "v", "do"))
    lse = torch.zeros((1, 1, 256), device=dev)
    for bq, bk, shape in ((32, 32, (1, 8, 8)), (16, 64, (1, 16, 4))):
        mask = torch.ones(shape, dtype=torch.uint8, device=dev)
        with pytest.raises(fa.FaError, match="FA_ERR_MASK"):
            fa.backward_block_sparse(q, k, v, q, do, lse, mask, bq, bk)


@pytest.mark.parametrize("dtype,d,bq,bk", [("bf16", 128, 64, 64), ("f32", 64, 32, 64)])
def test_block_sparse_full_tile_lists_at_max_n(dtype, d, bq, bk):
    """N = 65536, the largest block-sparse N: every query block keeps key block
    0, and query block r keeps every key block.  Key tile 0's dK/dV workgroup
    then lists every query block (1024 blocks of 64 rows in bf16, 2048 of 32 in
    fp32) and query block r's forward and dQ workgroups list all 1024 key
    tiles -- full lists.  The reference splits exactly by query rows: rows
    outside block r attend keys 0..bk-1 only, rows of block r attend all keys;
    gradients of K and V add over the two groups.

    dO is drawn N(0, 0.2^2): here all 65536 rows send gradient to the same 64
    keys, and with N(0, 1) their dK and dV reach 27 in magnitude, past the
    range (|x| <~ 5) the bf16 bar was set for; there the bar is one output ulp
    while the rounding of dS to bf16, summed over 65536 rows, alone reaches
    about two (a reference that rounds dS likewise leaves only the output's
    own rounding).  At 0.2 the gradients stay within that range."""
    N, r = 65536, 300
    announce(f"block-sparse full lists: {dtype} N={N} d={d} blocks {bq}x{bk}")
    dev = torch.device("cuda", 0)
    inputs = random_inputs(1, 1, N, d, dtype, seed=1970 + d, with_do=True)
    inputs["do"] = (inputs["do"].float() * 0.2).to(inputs["do"].dtype)
    mask = torch.zeros((1, N // bq, N // bk), dtype=torch.uint8)
    mask[0, :, 0] = 1
    mask[0, r, :] = 1
    q, k, v, do = (inputs[n].to(dev) for n in ("q", "k", "v", "do"))
    m = mask.to(dev)
    scale = 1.0 / np.sqrt(d)
    o, lse = fa.forward_block_sparse(q, k, v, m, bq, bk, scale=scale)
    dq, dk, dv = fa.backward_block_sparse(q, k, v, o, do, lse, m, bq, bk, scale=scale)
    torch.cuda.synchronize()
    o, lse, dq, dk, dv = (t[0, 0].cpu() for t in (o, lse, dq, dk, dv))

    q64, k64, v64, do64 = (to64(inputs[n][0, 0]) for n in ("q", "k", "v", "do"))
    rows_r = np.arange(r * bq, (r + 1) * bq)
    rest = np.setdiff1d(np.arange(N), rows_r)
    o_ref, lse_ref, dq_ref = np.zeros((N, d)), np.zeros(N), np.zeros((N, d))
    dk_ref, dv_ref = np.zeros((N, d)), np.zeros((N, d))
    # rows outside block r: dense attention over keys 0 .. bk-1
    o_ref[rest], lse_ref[rest] = ref.forward_head(q64[rest], k64[:bk], v64[:bk], False, scale)
    gq, gk, gv = ref.backward_head(q64[rest], k64[:bk], v64[:bk], do64[rest], False, scale)
    dq_ref[rest] = gq
    dk_ref[:bk] += gk
    dv_ref[:bk] += gv
    # rows of block r: dense attention over all keys
    o_ref[rows_r], lse_ref[rows_r] = ref.forward_head(q64[rows_r], k64, v64, False, scale)
    gq, gk, gv = ref.backward_head(q64[rows_r], k64, v64, do64[rows_r], False, scale)
    dq_ref[rows_r] = gq
    dk_ref += gk
    dv_ref += gv

    from gpu_helpers import TOL, TOL_LSE
    bf = dtype == "bf16"
    assert_close("O", o, o_ref, TOL[dtype], bf16_output=bf)
    assert_close("lse", lse, lse_ref, TOL_LSE)
    assert_close("dQ", dq, dq_ref, grad_tol(dtype, dq_ref), bf16_output=bf)
    assert_close("dK", dk, dk_ref, grad_tol(dtype, dk_ref), bf16_output=bf)
    assert_close("dV", dv, dv_ref, grad_tol(dtype, dv_ref), bf16_output=bf)
