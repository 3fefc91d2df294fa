"""fa_backward_noalloc against fa_backward, through the C ABI (needs an MI355X).

fa_backward_noalloc runs the same kernels as fa_backward with the workspace
in the library's own per-GPU device array, so its gradients must equal
fa_backward's bit for bit.  Consecutive calls reuse the array, which keeps
the previous call's contents: the second call of each pair is smaller, so a
statistic left over from the larger call would show.  The outputs start as
NaN so that an element left unwritten shows too.
"""
import math

import pytest
import torch

import io_aware_tiled_attention_amd as fa
from io_aware_tiled_attention_amd import _lib
from oracle import attention_ref as ref
from workloads import random_inputs

from gpu_helpers import TOL, announce, assert_close, grad_tol, require_gpu, to64

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


def _case(B, H, N, d, dtype, causal, seed):
    dev = torch.device("cuda", 0)
    inp = random_inputs(B, H, N, d, dtype, seed=seed, with_do=True)
    q, k, v, do = (inp[n].to(dev) for n in ("q", "k", "v", "do"))
    scale = 1.0 / math.sqrt(d)
    o, lse = fa.forward(q, k, v, causal=causal, scale=scale)
    want = fa.backward(q, k, v, o, do, lse, causal=causal, scale=scale)
    got = [torch.full_like(q, float("nan")) for _ in range(3)]
    st = _lib.fa_backward_noalloc(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), do.data_ptr(),
                                  lse.data_ptr(), got[0].data_ptr(), got[1].data_ptr(), got[2].data_ptr(),
                                  B, H, N, d, causal, scale, fa.FA_BF16 if dtype == "bf16" else fa.FA_F32,
                                  torch.cuda.current_stream().cuda_stream)
    assert st == 0, _lib.fa_strerror(st)
    torch.cuda.synchronize()
    return inp, scale, [w.cpu() for w in want], [g.cpu() for g in got]


@pytest.mark.parametrize("first,second", [
    ((4, 16, 4096, 64, "bf16", True), (1, 2, 300, 128, "bf16", False)),
    ((2, 3, 1000, 128, "f32", True), (1, 1, 65, 64, "f32", True)),
])
def test_noalloc_equals_backward_on_two_calls_second_smaller(first, second):
    for shape, seed in ((first, 61), (second, 62)):
        B, H, N, d, dtype, causal = shape
        announce(f"fa_backward_noalloc B={B} H={H} N={N} d={d} {dtype} causal={causal}")
        inp, scale, want, got = _case(B, H, N, d, dtype, causal, seed)
        for name, w, g in zip(("dQ", "dK", "dV"), want, got):
            assert torch.equal(w, g), f"{name}: fa_backward_noalloc differs from fa_backward"
        # and one head against the oracle, at the usual bars
        q, k, v, do = (to64(inp[n][0, 0]) for n in ("q", "k", "v", "do"))
        dq_r, dk_r, dv_r = ref.backward_head(q, k, v, do, causal=causal, scale=scale)
        for name, g, r in (("dQ", got[0], dq_r), ("dK", got[1], dk_r), ("dV", got[2], dv_r)):
            assert_close(f"{name}[0,0]", g[0, 0], r, grad_tol(dtype, r), bf16_output=dtype == "bf16")


def test_noalloc_at_the_largest_accepted_size():
    """2^21 rows: a workspace of exactly FA_NOALLOC_SCRATCH_BYTES."""
    B, H, N, d = 1, 32, 65536, 64
    assert fa.workspace_size(B, H, N, d) == _lib.NOALLOC_SCRATCH_BYTES
    announce(f"fa_backward_noalloc at the scratch limit B={B} H={H} N={N} d={d} bf16 causal")
    _, _, want, got = _case(B, H, N, d, "bf16", True, 63)
    for name, w, g in zip(("dQ", "dK", "dV"), want, got):
        assert torch.equal(w, g), f"{name}: fa_backward_noalloc differs from fa_backward"
    announce("fa_backward_noalloc one row past the limit")
    dev = torch.device("cuda", 0)
    t = torch.zeros(1, 1, (1 << 21) + 1, 64, dtype=torch.bfloat16, device=dev)
    lse = torch.zeros(1, 1, (1 << 21) + 1, dtype=torch.float32, device=dev)
    with pytest.raises(fa.FaError, match="FA_ERR_SCRATCH"):
        fa.backward_noalloc(t, t, t, t, t, lse, causal=True)
