"""GPU parity of fa_forward_fp8 against the fp64 oracle (needs an MI355X).

Inputs are OCP E4M3 codes with per-tensor descale factors; the oracle is
exact attention of the decoded values.  Two kinds of checks:
  * inputs whose probabilities are exactly representable in E4M3 (all equal,
    or powers of two), where the only rounding left is fp32 accumulation and
    the bf16 output -- compared at the bf16 bar;
  * random inputs, compared elementwise against the oracle's bound for
    probabilities rounded to E4M3 (``fp8_p_rounding_bound``) plus one bf16
    ulp of the output; lse, which does not see that rounding, at 1e-3.
"""
import math

import numpy as np
import pytest
import torch

import io_aware_tiled_attention_amd as fa
from oracle import attention_ref as ref
from workloads import fp8_inputs

from gpu_helpers import TOL, TOL_LSE, announce, assert_close, bf16_ulp, require_gpu, to64

pytestmark = pytest.mark.gpu
F8 = torch.float8_e4m3fn


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


def run_fp8(inputs, causal, scale, ds=(1.0, 1.0, 1.0)):
    dev = torch.device("cuda", 0)
    q, k, v = (inputs[n].to(dev).view(F8) for n in ("q", "k", "v"))
    o = torch.full(q.shape, float("nan"), dtype=torch.bfloat16, device=dev)
    lse = torch.full(q.shape[:3], float("nan"), dtype=torch.float32, device=dev)
    fa.forward_fp8(q, k, v, causal=causal, scale=scale, q_descale=ds[0], k_descale=ds[1], v_descale=ds[2],
                   out=o, lse=lse)
    torch.cuda.synchronize()
    return o.cpu(), lse.cpu()


def codes(x):
    return torch.as_tensor(x, dtype=torch.float32).to(F8).view(torch.uint8).contiguous()


@pytest.mark.parametrize("d,n,causal", [(128, 256, False), (128, 200, True), (64, 333, False), (64, 64, True)])
def test_fp8_uniform_probabilities_exact(d, n, causal):
    """Q = 0: every visible key has probability exactly 1 / count (p = 1 before
    normalising, exact in E4M3): O is the mean of the visible V rows."""
    announce(f"fp8 uniform P d={d} N={n} causal={causal}")
    B, H = 1, 2
    g = torch.Generator().manual_seed(n + d)
    v = torch.randn(B, H, n, d, generator=g)
    inputs = {"q": codes(torch.zeros(B, H, n, d)), "k": codes(torch.randn(B, H, n, d, generator=g)), "v": codes(v)}
    o, lse = run_fp8(inputs, causal, 0.5, ds=(1.0, 1.0, 0.75))
    for h in range(H):
        o_r, lse_r = ref.forward_fp8_head(inputs["q"][0, h].numpy(), inputs["k"][0, h].numpy(),
                                          inputs["v"][0, h].numpy(), 1.0, 1.0, 0.75, causal, 0.5)
        assert_close(f"O[0,{h}]", o[0, h], o_r, TOL["bf16"], bf16_output=True)
        assert_close(f"lse[0,{h}]", lse[0, h], lse_r, TOL_LSE)


@pytest.mark.parametrize("d,n,causal", [(128, 192, False), (128, 257, True), (64, 300, False)])
def test_fp8_power_of_two_probabilities_exact(d, n, causal):
    """Integer scores with scale ln 2: every unnormalised probability is a power
    of two (exact in E4M3), different per key, so the packing of P and the V^T
    reads are checked at the bf16 bar."""
    announce(f"fp8 power-of-two P d={d} N={n} causal={causal}")
    B, H = 1, 2
    rng = np.random.default_rng(n)
    q = np.zeros((B, H, n, d))
    q[..., 0] = 1.0
    k = np.zeros((B, H, n, d))
    k[..., 0] = -rng.integers(0, 7, size=(B, H, n))        # scores 0 .. -6
    k[:, :, 0, 0] = 0.0
    v = rng.standard_normal((B, H, n, d))
    inputs = {"q": codes(q), "k": codes(k), "v": codes(v)}
    scale = math.log(2.0)
    o, lse = run_fp8(inputs, causal, scale)
    for h in range(H):
        o_r, lse_r = ref.forward_fp8_head(inputs["q"][0, h].numpy(), inputs["k"][0, h].numpy(),
                                          inputs["v"][0, h].numpy(), 1.0, 1.0, 1.0, causal, scale)
        assert_close(f"O[0,{h}]", o[0, h], o_r, TOL["bf16"], bf16_output=True)
        assert_close(f"lse[0,{h}]", lse[0, h], lse_r, TOL_LSE)


def check_bound(inputs, causal, scale, ds, heads=None):
    o, lse = run_fp8(inputs, causal, scale, ds)
    B, H = inputs["q"].shape[:2]
    heads = heads if heads is not None else [(b, h) for b in range(B) for h in range(H)]
    worst = 0.0
    for b, h in heads:
        args = (inputs["q"][b, h].numpy(), inputs["k"][b, h].numpy(), inputs["v"][b, h].numpy(), *ds)
        o_r, lse_r = ref.forward_fp8_head(*args, causal, scale)
        bound = ref.fp8_p_rounding_bound(*args, causal, scale)
        got = to64(o[b, h])
        assert np.all(np.isfinite(got)), "non-finite output"
        # P rounding (derived bound) + output rounding to bf16 (half an ulp) + fp32 slack
        bar = bound + 0.5 * bf16_ulp(o_r) + 1e-4 * np.maximum(1.0, np.abs(o_r))
        err = np.abs(got - o_r)
        ratio = float(np.max(err / bar))
        worst = max(worst, ratio)
        print(f"    O[{b},{h}]: max|err| {err.max():.3e}, max bound {bound.max():.3e}, "
              f"rms err {np.sqrt(np.mean(err ** 2)):.3e}, worst err/bar {ratio:.3f}", flush=True)
        assert ratio <= 1.0
        assert_close(f"lse[{b},{h}]", lse[b, h], lse_r, TOL_LSE)
    return worst


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("n", [1, 65, 130, 448])
def test_fp8_random_inputs_within_rounding_bound(n, causal, d):
    announce(f"fp8 random N={n} d={d} causal={causal}")
    inputs = fp8_inputs(2, 2, n, d, seed=3000 + n + d)
    check_bound(inputs, causal, 1.0 / math.sqrt(d), (0.8, 1.25, 0.5))


def test_fp8_4k_d128_sampled_heads():
    announce("fp8 B=1 H=8 N=4096 d=128 causal, two heads")
    inputs = fp8_inputs(1, 8, 4096, 128, seed=3100)
    check_bound(inputs, True, 1.0 / math.sqrt(128), (1.0, 1.0, 1.0), heads=[(0, 0), (0, 7)])


@pytest.mark.slow
def test_fp8_16k_bench_configuration_sampled_heads():
    """The launch configuration the bench times: B=1, H=32, N=16384, d=128,
    causal, the 16K problem's inputs (N(0,1)*0.5 with 1% of K rows x8) rounded
    once to E4M3, descale 1.  Two whole heads against the oracle's bound."""
    from workloads import PROBLEMS, make_inputs
    p = PROBLEMS["causal_16k_d128"]
    announce("fp8 bench configuration B=1 H=32 N=16384 d=128 causal, heads 5 and 31")
    inp = make_inputs(p)
    inputs = {n: inp[n].float().to(F8).view(torch.uint8).contiguous() for n in ("q", "k", "v")}
    del inp
    check_bound(inputs, True, p.scale, (1.0, 1.0, 1.0), heads=[(0, 5), (0, 31)])
