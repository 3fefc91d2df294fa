"""The entry points under HIP graph capture (needs an MI355X).

Callers in tight loops (serving, training steps) capture launches into a
graph and replay it.  The library allocates nothing, clears nothing with
memset and never synchronises, so its calls capture as plain kernel nodes.
Each graph here is replayed several times with eager work and
synchronisations between the replays, and every replay must reproduce the
eager result bit for bit (the kernels are deterministic).
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


def _replay_and_compare(g, outs, eager, inputs_refill):
    """Replay g three times; between replays run unrelated eager work and
    refill the static inputs with the same values; compare every replay."""
    for rep in range(3):
        junk = torch.randn(1 << 20, device="cuda").mul_(2.0).sum()   # eager work on the same device
        inputs_refill()
        torch.cuda.synchronize()
        for o in outs:
            o.fill_(float("nan"))                                     # replay must overwrite every element
        g.replay()
        torch.cuda.synchronize()
        for name, a, b in zip(("out%d" % i for i in range(len(outs))), outs, eager):
            assert torch.equal(a, b), f"replay {rep}: {name} differs from the eager result"
        del junk


@pytest.mark.parametrize("causal", [False, True])
def test_forward_and_backward_capture(causal):
    announce(f"graph capture: forward + backward bf16 B=2 H=4 N=1000 d=128 causal={causal}")
    dev = torch.device("cuda", 0)
    inp = random_inputs(2, 4, 1000, 128, "bf16", seed=2100 + causal, with_do=True)
    src = {n: inp[n].to(dev) for n in ("q", "k", "v", "do")}
    q, k, v, do = (src[n].clone() for n in ("q", "k", "v", "do"))
    o_e, lse_e = fa.forward(q, k, v, causal=causal)
    g_e = fa.backward(q, k, v, o_e, do, lse_e, causal=causal)
    torch.cuda.synchronize()

    o, lse = torch.empty_like(q), torch.empty_like(lse_e)
    dq, dk, dv = (torch.empty_like(q) for _ in range(3))
    ws = torch.empty(fa.workspace_size(2, 4, 1000, 128), dtype=torch.uint8, device=dev)
    fa.forward(q, k, v, causal=causal, out=o, lse=lse)      # first call outside capture (one-time setup)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fa.forward(q, k, v, causal=causal, out=o, lse=lse)
        fa.backward(q, k, v, o, do, lse, causal=causal, dq=dq, dk=dk, dv=dv, workspace=ws)

    def refill():
        for n, t in (("q", q), ("k", k), ("v", v), ("do", do)):
            t.copy_(src[n])
    _replay_and_compare(g, [o, lse, dq, dk, dv], [o_e, lse_e, *g_e], refill)


def test_block_sparse_and_dropout_capture():
    announce("graph capture: block-sparse forward+backward and dropout forward+backward")
    dev = torch.device("cuda", 0)
    N, bq, bk = 640, 64, 64
    inp = random_inputs(1, 4, N, 64, "bf16", seed=2110, with_do=True)
    q, k, v, do = (inp[n].to(dev) for n in ("q", "k", "v", "do"))
    mask = block_mask(4, N, bq, bk, "random", seed=3, density=0.5).to(dev)
    o_s, lse_s = fa.forward_block_sparse(q, k, v, mask, bq, bk, causal=True)
    gs_e = fa.backward_block_sparse(q, k, v, o_s, do, lse_s, mask, bq, bk, causal=True)
    o_d, lse_d = fa.forward(q, k, v, causal=True, dropout_p=0.2, seed=77, offset=5)
    gd_e = fa.backward(q, k, v, o_d, do, lse_d, causal=True, dropout_p=0.2, seed=77, offset=5)
    torch.cuda.synchronize()

    outs = [torch.empty_like(t) for t in (o_s, lse_s, *gs_e, o_d, lse_d, *gd_e)]
    os_, ls_, dqs, dks, dvs, od_, ld_, dqd, dkd, dvd = outs
    ws = torch.empty(fa.workspace_size(1, 4, N, 64), dtype=torch.uint8, device=dev)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fa.forward_block_sparse(q, k, v, mask, bq, bk, causal=True, out=os_, lse=ls_)
        fa.backward_block_sparse(q, k, v, os_, do, ls_, mask, bq, bk, causal=True, dq=dqs, dk=dks, dv=dvs,
                                 workspace=ws)
        fa.forward(q, k, v, causal=True, dropout_p=0.2, seed=77, offset=5, out=od_, lse=ld_)
        fa.backward(q, k, v, od_, do, ld_, causal=True, dropout_p=0.2, seed=77, offset=5, dq=dqd, dk=dkd, dv=dvd,
                    workspace=ws)
    _replay_and_compare(g, outs, [o_s, lse_s, *gs_e, o_d, lse_d, *gd_e], lambda: None)


@pytest.mark.parametrize("splits", [0, 1])
def test_decode_capture(splits):
    announce(f"graph capture: split-KV decoding Nq=4 Nk=5000 splits={splits}")
    dev = torch.device("cuda", 0)
    inp = decode_inputs(2, 8, 4, 5000, 128, "bf16", seed=2120)
    q, k, v = (inp[n].to(dev) for n in ("q", "k", "v"))
    o_e, lse_e = fa.decode(q, k, v, causal=True, num_splits=splits)
    torch.cuda.synchronize()
    o, lse = torch.empty_like(o_e), torch.empty_like(lse_e)
    need = fa.fa_decode_workspace_size(2, 8, 4, 5000, 128, splits)
    ws = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fa.decode(q, k, v, causal=True, num_splits=splits, out=o, lse=lse, workspace=ws)
    _replay_and_compare(g, [o, lse], [o_e, lse_e], lambda: None)
