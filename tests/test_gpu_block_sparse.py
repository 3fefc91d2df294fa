"""GPU parity of fa_forward_block_sparse against the fp64 oracle (needs an MI355X).

Block-sparse attention: "Overview of Flash Attention series", section
Block-sparse Flashattention (masked blocks carry no weight; a row that keeps
no key has O = 0 and lse = -inf).
"""
import numpy as np
import pytest
import torch

import io_aware_tiled_attention_amd as fa
from workloads import block_mask, random_inputs

from gpu_helpers import TOL, TOL_LSE, announce, assert_close, require_gpu, to64
from oracle import attention_ref as ref

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


def run_sparse(inputs, mask, bq, bk, causal, scale):
    dev = torch.device("cuda", 0)
    q, k, v = (inputs[n].to(dev) for n in ("q", "k", "v"))
    o, lse = fa.forward_block_sparse(q, k, v, mask.to(dev), bq, bk, causal=causal, scale=scale)
    torch.cuda.synchronize()
    return o.cpu(), lse.cpu()


def check(inputs, mask, bq, bk, causal, scale, heads=None):
    o, lse = run_sparse(inputs, mask, bq, bk, causal, scale)
    q, k, v = (to64(inputs[n]) for n in ("q", "k", "v"))
    B, H = q.shape[:2]
    tol = TOL["f32" if inputs["q"].dtype == torch.float32 else "bf16"]
    m = mask.numpy()
    heads = heads if heads is not None else [(b, h) for b in range(B) for h in range(H)]
    n_empty = 0
    for b, h in heads:
        o_r, lse_r = ref.forward_block_sparse_head(q[b, h], k[b, h], v[b, h], m[h if m.shape[0] > 1 else 0],
                                                   bq, bk, causal, scale)
        empty = np.isneginf(lse_r)
        n_empty += int(empty.sum())
        og, lg = o[b, h], lse[b, h]
        assert torch.all(og[torch.from_numpy(empty)] == 0), "rows with no key must be 0"
        assert torch.all(torch.isneginf(lg[torch.from_numpy(empty)])), "rows with no key must have lse = -inf"
        keep = torch.from_numpy(~empty)
        assert_close(f"O[{b},{h}]", og[keep], o_r[~empty], tol, bf16_output=og.dtype == torch.bfloat16)
        assert_close(f"lse[{b},{h}]", lg[keep], lse_r[~empty], TOL_LSE)
    return o, lse, n_empty


@pytest.mark.parametrize("dtype,N,d,bq,bk,causal,kind,mheads", [
    ("bf16", 1024, 128, 128, 64, False, "random", 4),
    ("bf16", 1000, 64, 64, 64, True, "random", 1),
    ("bf16", 1024, 128, 256, 128, True, "local_global", 1),
    ("bf16", 777, 128, 32, 64, False, "random", 4),
    ("f32", 257, 64, 32, 128, True, "random", 1),
    ("f32", 320, 128, 64, 64, False, "local", 4),
])
def test_block_sparse_matches_oracle(dtype, N, d, bq, bk, causal, kind, mheads):
    announce(f"block-sparse {dtype} N={N} d={d} blocks {bq}x{bk} causal={causal} {kind} mask_heads={mheads}")
    inputs = random_inputs(2, 4, N, d, dtype, seed=900 + N + d + bq)
    mask = block_mask(mheads, N, bq, bk, kind, seed=N + bk, density=0.45)
    check(inputs, mask, bq, bk, causal, 1.0 / np.sqrt(d))


def test_block_sparse_rows_with_no_key():
    announce("block-sparse empty mask rows")
    N, d, bq, bk = 512, 64, 64, 64
    inputs = random_inputs(1, 2, N, d, "bf16", seed=931)
    mask = block_mask(2, N, bq, bk, "random", seed=5, density=0.5)
    mask[0, 3, :] = 0          # head 0: query block 3 keeps nothing
    mask[1, :, :] = 0
    mask[1, 5, 2] = 1          # head 1: only one block kept at all
    _, _, n_empty = check(inputs, mask, bq, bk, False, 0.125)
    assert n_empty >= 64 + 7 * 64


def test_block_sparse_all_ones_equals_dense_bitwise():
    announce("block-sparse all-ones mask vs dense forward")
    dev = torch.device("cuda", 0)
    for causal in (False, True):
        inputs = random_inputs(2, 3, 1000, 128, "bf16", seed=940 + causal)
        q, k, v = (inputs[n].to(dev) for n in ("q", "k", "v"))
        mask = block_mask(1, 1000, 128, 64, "ones", seed=0).to(dev)
        o_s, lse_s = fa.forward_block_sparse(q, k, v, mask, 128, 64, causal=causal)
        o_d, lse_d = fa.forward(q, k, v, causal=causal)
        torch.cuda.synchronize()
        assert torch.equal(o_s, o_d) and torch.equal(lse_s, lse_d)


def test_block_sparse_long_local_global_sampled_heads():
    announce("block-sparse N=8192 d=128 local+global, 2 heads checked")
    N, d, bq, bk = 8192, 128, 128, 128
    inputs = random_inputs(1, 4, N, d, "bf16", seed=950)
    mask = block_mask(1, N, bq, bk, "local_global", seed=0, window=3)
    check(inputs, mask, bq, bk, True, 1.0 / np.sqrt(d), heads=[(0, 0), (0, 3)])


def test_block_sparse_rejects_bad_geometry_before_launch():
    dev = torch.device("cuda", 0)
    inputs = random_inputs(1, 1, 256, 64, "bf16", seed=960)
    q, k, v = (inputs[n].to(dev) for n in ("q", "k", "v"))
    mask = torch.ones((1, 8, 8), dtype=torch.uint8, device=dev)
    with pytest.raises(fa.FaError, match="FA_ERR_MASK"):
        fa.forward_block_sparse(q, k, v, mask, 32, 32)   # block_k not a multiple of 64
