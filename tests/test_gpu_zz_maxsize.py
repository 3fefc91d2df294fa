"""The longest sequence the boundary accepts (needs an MI355X; about two minutes).

The kernels address one head with 32-bit byte offsets, and fa_forward /
fa_backward accept a head while (N + 256) * d * element size <= 2^31 - 1
(a ragged last tile addresses up to 256 rows past N).  At bf16, d = 128 that
is N = 8388351: every per-head offset is then as large as it can be, and the
last tile is ragged.  One head, causal, inputs drawn on the device from a
seed (workloads.device_inputs).

* Forward, N(0,1) inputs, scale 1: sampled query rows at both ends and in the
  middle, each against all of its keys, compared with the oracle's definition
  (forward_rows) at the bf16 and lse bars.
* Backward with K = 0: every allowed key then gets the weight 1/(i+1), and the
  definition reduces to prefix and suffix sums, written out here in fp64:
    lse_i = ln(i+1),   O_i = (1/(i+1)) sum_{j<=i} v_j,
    dV_j = sum_{i>=j} dO_i / (i+1),
    dK_j = scale * sum_{i>=j} (dO_i . v_j - D_i) q_i / (i+1),  D_i = dO_i . O_i,
    dQ = scale * dS K = 0.
  dQ is checked whole; O, lse, dK, dV on sampled rows.
* Split-KV decoding of 32 new queries against a cache of that length, with the
  library's chunking and with one chunk, against the oracle's decode_head.
* The largest grid the boundary accepts: B*H*ceil(N/128) = 2^23 - 1 one-row
  heads, so every launch has its most workgroups (the backward's dK/dV grid
  then holds 2^32 - 512 work items).  With one key per row P = 1 exactly, so
  O = V and dV = dO bit for bit, lse = scale * q . k, and dS = 0 up to the
  rounding of D, so dQ and dK vanish.
* The largest decoding merge grid: B*H*Nq = 2^26 - 32 rows of 64 threads (2^32
  - 2048 work items), 32 queries over 64 zero keys in two chunks: every weight
  is 1/64, so O is the mean of V and lse = ln 64.

Named to run last: together these take about two minutes.
"""
import math

import numpy as np
import pytest
import torch

import io_aware_tiled_attention_amd as fa
from oracle import attention_ref as ref
from workloads import device_inputs

from gpu_helpers import TOL, TOL_LSE, announce, assert_close, require_gpu, to64

pytestmark = [pytest.mark.gpu, pytest.mark.slow]

D = 128
N_MAX = (2**31 - 1) // (D * 2) - 256      # bf16: the largest N the boundary accepts
SCALE = 1.0 / math.sqrt(D)
# Forward and decoding use scale 1: scores ~ N(0, d), so each row's softmax is
# dominated by its few largest scores and O is of order one.  At 1/sqrt(d) a
# softmax over millions of keys is nearly uniform and O ~ mean(V) ~ 1e-3, which
# the absolute bar could not tell from zero.
SHARP = 1.0


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


def test_boundary_accepts_n_max_and_rejects_one_more():
    z = torch.zeros(1, dtype=torch.bfloat16, device="cuda")
    st = fa.fa_forward(z.data_ptr(), z.data_ptr(), z.data_ptr(), z.data_ptr(), z.data_ptr(), 1, 1, N_MAX + 1, D, 1,
                       SCALE, 1, None)
    assert st == 2   # FA_ERR_SHAPE, before any pointer is used


def test_forward_at_n_max_sampled_rows():
    announce(f"max-size forward: B=1 H=1 N={N_MAX} d={D} bf16 causal")
    dev = torch.device("cuda", 0)
    inp = device_inputs(1, 1, N_MAX, D, "bf16", seed=8388, device=dev)
    q, k, v = inp["q"], inp["k"], inp["v"]
    o, lse = fa.forward(q, k, v, causal=True, scale=SHARP)
    torch.cuda.synchronize()
    rows = np.array([0, 1, 4097, N_MAX // 2 + 3, N_MAX - 129, N_MAX - 2, N_MAX - 1])
    ridx = torch.as_tensor(rows, device=dev)
    q_rows = to64(q[0, 0].index_select(0, ridx))
    o_rows, lse_rows = o[0, 0].index_select(0, ridx).cpu(), lse[0, 0].index_select(0, ridx).cpu()
    del o, lse, q
    announce("max-size forward: oracle rows")
    k64, v64 = to64(k[0, 0]), to64(v[0, 0])
    del k, v, inp
    torch.cuda.empty_cache()
    o_ref, lse_ref = ref.forward_rows(q_rows, k64, v64, rows, causal=True, scale=SHARP, q_selected=True)
    assert_close("O rows", o_rows, o_ref, TOL["bf16"], bf16_output=True)
    assert_close("lse rows", lse_rows, lse_ref, TOL_LSE)


def test_backward_at_n_max_zero_keys_closed_form():
    announce(f"max-size backward (K = 0): B=1 H=1 N={N_MAX} d={D} bf16 causal")
    dev = torch.device("cuda", 0)
    inp = device_inputs(1, 1, N_MAX, D, "bf16", seed=8389, device=dev, names=("q", "v", "do"))
    q, v, do = inp["q"], inp["v"], inp["do"]
    k = torch.zeros_like(q)
    o, lse = fa.forward(q, k, v, causal=True, scale=SCALE)
    dq, dk, dv = fa.backward(q, k, v, o, do, lse, causal=True, scale=SCALE)
    torch.cuda.synchronize()
    assert int(torch.count_nonzero(dq)) == 0, "dQ = scale * dS K must vanish for K = 0"
    rows = np.array([0, 1, 777, N_MAX // 3, N_MAX - 200, N_MAX - 1])
    ridx = torch.as_tensor(rows, device=dev)
    got = {n: t[0, 0].index_select(0, ridx).cpu() for n, t in (("o", o), ("lse", lse), ("dk", dk), ("dv", dv))}
    del o, lse, dq, dk, dv, k
    announce("max-size backward: closed forms")
    q64, v64, do64 = to64(q[0, 0]), to64(v[0, 0]), to64(do[0, 0])
    del q, v, do, inp
    torch.cuda.empty_cache()
    w = 1.0 / np.arange(1, N_MAX + 1, dtype=np.float64)          # P_ij = 1/(i+1) for j <= i
    o_all = np.cumsum(v64, axis=0)
    o_all *= w[:, None]                                         # O_i: mean of v_0 .. v_i
    dsum = np.einsum("nd,nd->n", do64, o_all)                   # D_i = dO_i . O_i
    assert_close("lse rows", got["lse"], np.log(rows + 1.0), TOL_LSE)
    assert_close("O rows", got["o"], o_all[rows], TOL["bf16"], bf16_output=True)
    del o_all
    dv_ref = np.stack([do64[j:].T @ w[j:] for j in rows])
    dk_ref = np.stack([SCALE * (q64[j:].T @ ((do64[j:] @ v64[j] - dsum[j:]) * w[j:])) for j in rows])
    assert_close("dV rows", got["dv"], dv_ref, TOL["bf16"], bf16_output=True)
    assert_close("dK rows", got["dk"], dk_ref, TOL["bf16"], bf16_output=True)


@pytest.mark.parametrize("splits", [0, 1])
def test_decode_at_n_max(splits):
    # the longest cache the boundary accepts, 32 new queries (the most per call), causal;
    # splits 0: the library's chunking (hundreds of chunks), 1: one chunk per head
    announce(f"max-size decode: B=1 H=1 Nq=32 Nk={N_MAX} d={D} bf16 causal splits={splits}")
    dev = torch.device("cuda", 0)
    cache = device_inputs(1, 1, N_MAX, D, "bf16", seed=8390, device=dev, names=("k", "v"))
    qn = device_inputs(1, 1, 32, D, "bf16", seed=8391, device=dev, names=("q",))["q"]
    o, lse = fa.decode(qn, cache["k"], cache["v"], causal=True, scale=SHARP, num_splits=splits)
    torch.cuda.synchronize()
    o, lse = o.cpu(), lse.cpu()
    k64, v64 = to64(cache["k"][0, 0]), to64(cache["v"][0, 0])
    del cache
    torch.cuda.empty_cache()
    o_ref, lse_ref = ref.decode_head(to64(qn[0, 0]), k64, v64, causal=True, scale=SHARP)
    assert_close("O", o[0, 0], o_ref, TOL["bf16"], bf16_output=True)
    assert_close("lse", lse[0, 0], lse_ref, TOL_LSE)


def test_largest_grid_one_row_heads():
    heads = 2**23 - 1                     # one 128-row tile per head: the most workgroups accepted
    d = 64
    announce(f"largest grid: B=1 H={heads} N=1 d={d} bf16 forward + backward")
    dev = torch.device("cuda", 0)
    inp = device_inputs(1, heads, 1, d, "bf16", seed=8392, device=dev, names=("q", "k", "v", "do"))
    q, k, v, do = inp["q"], inp["k"], inp["v"], inp["do"]
    scale = 1.0 / math.sqrt(d)
    o, lse = fa.forward(q, k, v, causal=True, scale=scale)
    dq, dk, dv = fa.backward(q, k, v, o, do, lse, causal=True, scale=scale)
    torch.cuda.synchronize()
    assert torch.equal(o, v), "one key per row: O must equal V"
    assert torch.equal(dv, do), "one key per row: dV must equal dO"
    assert float(dq.abs().max()) <= 1e-3 and float(dk.abs().max()) <= 1e-3
    # lse at sampled heads against the oracle (one row each)
    hs = torch.as_tensor(np.random.default_rng(0).choice(heads, 512, replace=False), device=dev)
    q64, k64, v64 = (to64(t[0].index_select(0, hs)) for t in (q, k, v))
    lse_s = lse[0].index_select(0, hs).cpu()
    ref_lse = np.array([ref.forward_head(q64[i], k64[i], v64[i], True, scale)[1] for i in range(len(hs))])
    assert_close("lse", lse_s, ref_lse, TOL_LSE)
    # the FP8 forward's grid at the same size: O = V again (P = 1 is exact in E4M3)
    del dq, dk, dv, do, o
    q8, k8, v8 = (t.to(torch.float8_e4m3fn) for t in (q, k, v))
    del q, k, v, inp
    o8, lse8 = fa.forward_fp8(q8, k8, v8, causal=True, scale=scale)
    torch.cuda.synchronize()
    assert torch.equal(o8, v8.to(torch.bfloat16)), "FP8, one key per row: O must equal V"
    assert bool(torch.isfinite(lse8).all())


def test_largest_decode_merge_grid():
    heads, nq, nk, d = 2**21 - 1, 32, 64, 64
    announce(f"largest decode merge grid: B=1 H={heads} Nq={nq} Nk={nk} d={d} bf16, 2 chunks")
    dev = torch.device("cuda", 0)
    q = device_inputs(1, heads, nq, d, "bf16", seed=8393, device=dev, names=("q",))["q"]
    v = device_inputs(1, heads, nk, d, "bf16", seed=8394, device=dev, names=("v",))["v"]
    k = torch.zeros_like(v)
    assert fa.fa_decode_num_splits(1, heads, nk, 2) == 2
    o, lse = fa.decode(q, k, v, causal=False, scale=1.0 / math.sqrt(d), num_splits=2)
    torch.cuda.synchronize()
    assert float((lse.double() - math.log(nk)).abs().max()) <= TOL_LSE
    err = 0.0
    for h0 in range(0, heads, 1 << 16):                       # fp64 in slices of heads
        sl = slice(h0, min(heads, h0 + (1 << 16)))
        want = v[0, sl].double().mean(dim=1, keepdim=True)  # [h, 1, d], broadcast over the queries
        err = max(err, float((o[0, sl].double() - want).abs().max()))
    assert err <= TOL["bf16"], f"O: max|err| {err:.3g}"
