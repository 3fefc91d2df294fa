"""GPU parity of the dropout forward and backward against the fp64 oracle (needs an MI355X).

Dropout on the attention probabilities with a regenerated mask
("Как работает FlashAttention математически", section 5; "Overview of Flash
Attention series", Backward Pass).  The keep mask is a pure function of
(seed, offset, head, query, key) through Philox4x32-10, so the GPU's mask is
compared bit for bit with the oracle's: recovered from outputs whose inputs
make every kept entry visible (Q = K = 0, V or dO one-hot).  Then O, lse,
dQ, dK and dV are compared with the oracle at the usual tolerances.
"""
import math

import numpy as np
import pytest
import torch

import io_aware_tiled_attention_amd as fa
from oracle import attention_ref as ref
from workloads import random_inputs

from gpu_helpers import TOL, TOL_LSE, announce, assert_close, grad_tol, require_gpu, to64

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


def onehot_planes(n, d, dtype):
    """[n, d] with row j = 2^(j // d) e_(j % d): a sum over rows decodes which rows took part."""
    x = torch.zeros(n, d, dtype=torch.float64)
    j = torch.arange(n)
    x[j, j % d] = torch.pow(2.0, (j // d).double())
    return x.to(dtype)


def decode_bits(vals, n, d):
    """vals[r, c] = sum_m bit(r, c + m d) 2^m (integers) -> bits [rows, n]."""
    rows = vals.shape[0]
    v = np.rint(vals).astype(np.int64)
    bits = np.zeros((rows, n), dtype=bool)
    for m in range(-(-n // d)):
        cols = np.arange(m * d, min(n, (m + 1) * d))
        bits[:, cols] = (v[:, cols - m * d] >> m) & 1 == 1
    return bits


@pytest.mark.parametrize("dtype,n,causal,p", [("f32", 512, False, 0.1), ("f32", 333, True, 0.5),
                                              ("bf16", 256, False, 0.25), ("bf16", 200, True, 0.1)])
def test_forward_mask_is_bit_exact(dtype, n, causal, p):
    """Q = K = 0 gives P = 1 / (number of visible keys); with V one-hot planes
    O_ic * count_i * (1 - t/256) = sum of kept keys' bit planes."""
    announce(f"dropout forward mask bits {dtype} N={n} causal={causal} p={p}")
    dev = torch.device("cuda", 0)
    d, B, H = 128, 1, 3
    td = torch.float32 if dtype == "f32" else torch.bfloat16
    z = torch.zeros(B, H, n, d, dtype=td, device=dev)
    v = onehot_planes(n, d, td).to(dev).expand(B, H, n, d).contiguous()
    seed, offset = 0xDEADBEEF12345, 9
    o, _ = fa.forward(z, z, v, causal=causal, dropout_p=p, seed=seed, offset=offset)
    torch.cuda.synchronize()
    t = ref.dropout_threshold(p)
    count = (np.arange(n) + 1) if causal else np.full(n, n)
    for h in range(H):
        vals = to64(o[0, h]) * count[:, None] * (1.0 - t / 256.0)
        got = decode_bits(vals, n, d)
        want = ref.dropout_keep_mask(h, n, n, seed, offset, t)
        if causal:
            want &= np.tril(np.ones((n, n), dtype=bool))
        assert np.array_equal(got, want), f"head {h}: {int((got != want).sum())} mask bits differ"


@pytest.mark.parametrize("dtype,n,causal", [("f32", 384, False), ("bf16", 256, True), ("f32", 190, True)])
def test_backward_dv_mask_is_bit_exact(dtype, n, causal):
    """dV = (P o Z)^T dO / (1 - t/256) with Q = K = 0 and dO one-hot planes
    recovers the mask column by column through the dK/dV kernel."""
    announce(f"dropout dV mask bits {dtype} N={n} causal={causal}")
    dev = torch.device("cuda", 0)
    d, B, H, p = 128, 2, 2, 0.3
    td = torch.float32 if dtype == "f32" else torch.bfloat16
    z = torch.zeros(B, H, n, d, dtype=td, device=dev)
    v = torch.randn(B, H, n, d, device=dev).to(td)
    do = onehot_planes(n, d, td).to(dev).expand(B, H, n, d).contiguous()
    seed, offset = 77, 0x1000
    o, lse = fa.forward(z, z, v, causal=causal, dropout_p=p, seed=seed, offset=offset)
    _, _, dv = fa.backward(z, z, v, o, do, lse, causal=causal, dropout_p=p, seed=seed, offset=offset)
    torch.cuda.synchronize()
    t = ref.dropout_threshold(p)
    count = (np.arange(n) + 1) if causal else np.full(n, n)
    for b in range(B):
        for h in range(H):
            # dV[j, c] = sum_i Z_ij / count_i * 2^(i // d) [i % d == c] / (1 - t/256); causal counts differ per i,
            # so decode with the oracle's own P (1 / count_i) folded in: compare against the exact dV of the mask
            want_z = ref.dropout_keep_mask(b * H + h, n, n, seed, offset, t)
            if causal:
                want_z &= np.tril(np.ones((n, n), dtype=bool))
            pz = want_z / count[:, None] / (1.0 - t / 256.0)
            want = pz.T @ to64(do[b, h])
            got = to64(dv[b, h])
            if dtype == "f32":
                np.testing.assert_allclose(got, want, rtol=1e-5, atol=1e-6)
            else:
                assert_close(f"dV[{b},{h}]", dv[b, h], want, 2e-2, bf16_output=True)
            if not causal:
                bits = decode_bits(got * n * (1.0 - t / 256.0), n, d)   # rows = keys j
                assert np.array_equal(bits, want_z.T)


def run_dropout(inputs, causal, scale, p, seed, offset):
    dev = torch.device("cuda", 0)
    q, k, v, do = (inputs[n].to(dev) for n in ("q", "k", "v", "do"))
    o, lse = fa.forward(q, k, v, causal=causal, scale=scale, dropout_p=p, seed=seed, offset=offset)
    dq, dk, dv = fa.backward(q, k, v, o, do, lse, causal=causal, scale=scale, dropout_p=p, seed=seed,
                             offset=offset)
    torch.cuda.synchronize()
    return o.cpu(), lse.cpu(), dq.cpu(), dk.cpu(), dv.cpu()


def check_dropout(inputs, causal, scale, p, seed, offset, heads=None):
    o, lse, dq, dk, dv = run_dropout(inputs, causal, scale, p, seed, offset)
    q, k, v, do = (to64(inputs[n]) for n in ("q", "k", "v", "do"))
    dt = "f32" if inputs["q"].dtype == torch.float32 else "bf16"
    bf = dt == "bf16"
    B, H, N, _ = q.shape
    t = ref.dropout_threshold(p)
    heads = heads if heads is not None else [(b, h) for b in range(B) for h in range(H)]
    for b, h in heads:
        keep = ref.dropout_keep_mask(b * H + h, N, N, seed, offset, t)
        o_r, lse_r = ref.forward_dropout_head(q[b, h], k[b, h], v[b, h], keep, t, causal, scale)
        assert_close(f"O[{b},{h}]", o[b, h], o_r, TOL[dt], bf16_output=bf)
        assert_close(f"lse[{b},{h}]", lse[b, h], lse_r, TOL_LSE)
        dq_r, dk_r, dv_r = ref.backward_dropout_head(q[b, h], k[b, h], v[b, h], do[b, h], keep, t, causal, scale)
        # dS = P (dP o Z / (1 - t/256) - D) is rounded to the input type before the dQ and dK
        # products, so its absolute rounding error -- and the gradients' -- grows by 1 / (1 - t/256)
        rs = 256.0 / (256.0 - t)
        assert_close(f"dQ[{b},{h}]", dq[b, h], dq_r, grad_tol(dt, dq_r) * rs, bf16_output=bf)
        assert_close(f"dK[{b},{h}]", dk[b, h], dk_r, grad_tol(dt, dk_r) * rs, bf16_output=bf)
        assert_close(f"dV[{b},{h}]", dv[b, h], dv_r, grad_tol(dt, dv_r) * rs, bf16_output=bf)
    return o, lse, dq, dk, dv


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("n,p", [(1, 0.1), (65, 0.5), (200, 0.1), (257, 0.25)])
def test_dropout_matches_oracle(n, p, causal, d, dtype):
    announce(f"dropout N={n} d={d} causal={causal} {dtype} p={p}")
    inputs = random_inputs(2, 3, n, d, dtype, seed=7000 + n + d, with_do=True)
    check_dropout(inputs, causal, 1.0 / math.sqrt(d), p, seed=1234 + n, offset=d)


@pytest.mark.parametrize("dtype,d", [("bf16", 128), ("f32", 64)])
def test_dropout_multi_block(dtype, d):
    announce(f"dropout N=640 d={d} {dtype} causal")
    inputs = random_inputs(1, 2, 640, d, dtype, seed=77 + d, with_do=True)
    check_dropout(inputs, True, 1.0 / math.sqrt(d), 0.2, seed=(1 << 40) + 5, offset=3)


def test_dropout_is_deterministic_and_keyed():
    announce("dropout determinism: same (seed, offset) bit-identical, other offset different")
    inputs = random_inputs(1, 2, 300, 128, "bf16", seed=31, with_do=True)
    a = run_dropout(inputs, True, 1 / math.sqrt(128), 0.3, 5, 0)
    b = run_dropout(inputs, True, 1 / math.sqrt(128), 0.3, 5, 0)
    c = run_dropout(inputs, True, 1 / math.sqrt(128), 0.3, 5, 1)
    for x, y in zip(a, b):
        assert torch.equal(x, y)
    assert not torch.equal(a[0], c[0])
    assert torch.equal(a[1], c[1])      # lse is that of the undropped scores


def test_dropout_p0_is_the_plain_path():
    announce("dropout p=0 == plain attention")
    inputs = random_inputs(1, 2, 200, 64, "bf16", seed=32, with_do=True)
    dev = torch.device("cuda", 0)
    q, k, v, do = (inputs[n].to(dev) for n in ("q", "k", "v", "do"))
    o1, l1 = fa.forward(q, k, v, causal=True, dropout_p=0.0, seed=9)
    o2, l2 = fa.forward(q, k, v, causal=True)
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    g1 = fa.backward(q, k, v, o1, do, l1, causal=True, dropout_p=0.0, seed=9)
    g2 = fa.backward(q, k, v, o2, do, l2, causal=True)
    for x, y in zip(g1, g2):
        assert torch.equal(x, y)


def test_dropout_2k_d128_sampled_heads():
    announce("dropout bf16 B=1 H=4 N=2048 d=128 causal p=0.1, two heads")
    inputs = random_inputs(1, 4, 2048, 128, "bf16", seed=33, with_do=True)
    check_dropout(inputs, True, 1 / math.sqrt(128), 0.1, seed=2024, offset=17, heads=[(0, 0), (0, 3)])


@pytest.mark.slow
def test_dropout_16k_bench_configuration_sampled_rows():
    """The launch configuration the bench times: the 16K problem (B=1, H=32,
    N=16384, d=128, causal, stressed K) with p = 0.1, seed 0x5EED, offset 0.
    Sampled query rows of two heads, each against all of its keys, with the
    keep mask regenerated for those rows by the oracle."""
    from workloads import PROBLEMS, make_inputs
    p = PROBLEMS["causal_16k_d128_bwd"]
    announce("dropout bench configuration B=1 H=32 N=16384 d=128 causal p=0.1, sampled rows of heads 0 and 31")
    inputs = make_inputs(p, with_do=True)
    dev = torch.device("cuda", 0)
    q, k, v = (inputs[n].to(dev) for n in ("q", "k", "v"))
    o, lse = fa.forward(q, k, v, causal=True, scale=p.scale, dropout_p=0.1, seed=0x5EED, offset=0)
    torch.cuda.synchronize()
    o, lse = o.cpu(), lse.cpu()
    t = ref.dropout_threshold(0.1)
    rows = np.array([0, 1, 3, 777, 4096, 9999, 16380, 16383])
    for h in (0, 31):
        keep = ref.dropout_keep_rows(h, rows, p.N, 0x5EED, 0, t)
        qh, kh, vh = (to64(inputs[n][0, h]) for n in ("q", "k", "v"))
        o_r, lse_r = ref.forward_dropout_rows(qh[rows], kh, vh, rows, keep, t, True, p.scale, q_selected=True)
        assert_close(f"O[0,{h}] rows", o[0, h][torch.as_tensor(rows)], o_r, TOL["bf16"], bf16_output=True)
        assert_close(f"lse[0,{h}] rows", lse[0, h][torch.as_tensor(rows)], lse_r, TOL_LSE)
