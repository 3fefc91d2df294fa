"""The C-ABI library loads, exports every declared symbol and rejects bad calls.

CPU-only: every call here returns from argument validation before the first
HIP call, so no device is touched.
"""
import ctypes
import os
import re

import pytest

import io_aware_tiled_attention_amd as fa
from io_aware_tiled_attention_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fa.h")
FAKE = 0x1000  # 16-byte aligned, never dereferenced: validation fails first


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(fa_[a-z0-9_]+)\s*\(", text)))


def test_library_exports_every_declared_symbol():
    lib = fa.load_library()
    names = declared_functions()
    assert set(names) == set(_lib.EXPORTED)
    for name in names:
        assert hasattr(lib, name), name
        assert ctypes.cast(getattr(lib, name), ctypes.c_void_p).value


def test_enums_match_header():
    text = open(HEADER).read()
    for name, value in re.findall(r"(FA_[A-Z0-9_]+)\s*=\s*(\d+)", text):
        if name in ("FA_F32", "FA_BF16"):
            assert getattr(_lib, name) == int(value)
        else:
            assert _lib.STATUS[int(value)] == name


def test_strerror_covers_every_status():
    for code in list(_lib.STATUS) + [99, -1]:
        msg = fa.fa_strerror(code)
        assert isinstance(msg, str) and msg
    assert fa.fa_strerror(99) == "unknown fa_status"


def fwd(**kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, o=FAKE, lse=FAKE, B=1, H=2, N=64, d=64, causal=0,
             scale=0.125, dtype=_lib.FA_BF16, stream=None)
    a.update(kw)
    return fa.fa_forward(a["q"], a["k"], a["v"], a["o"], a["lse"], a["B"], a["H"], a["N"], a["d"],
                         a["causal"], a["scale"], a["dtype"], a["stream"])


def bwd(**kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, o=FAKE, do=FAKE, lse=FAKE, dq=FAKE, dk=FAKE, dv=FAKE, B=1, H=2,
             N=64, d=64, causal=1, scale=0.125, dtype=_lib.FA_BF16, ws=0x100000, ws_bytes=1 << 30,
             stream=None)
    a.update(kw)
    return fa.fa_backward(a["q"], a["k"], a["v"], a["o"], a["do"], a["lse"], a["dq"], a["dk"], a["dv"],
                          a["B"], a["H"], a["N"], a["d"], a["causal"], a["scale"], a["dtype"], a["ws"],
                          a["ws_bytes"], a["stream"])


@pytest.mark.parametrize("kw,status", [
    (dict(q=0), 1), (dict(k=0), 1), (dict(v=0), 1), (dict(o=0), 1), (dict(lse=0), 1),
    (dict(B=-1), 2), (dict(H=-3), 2), (dict(N=-1), 2), (dict(B=1 << 20, H=1 << 12), 2),
    (dict(N=1 << 30, d=128), 2),
    (dict(d=32), 3), (dict(d=96), 3), (dict(d=0), 3), (dict(d=256), 3),
    (dict(dtype=2), 4), (dict(dtype=-1), 4),
    (dict(scale=float("nan")), 5), (dict(scale=float("inf")), 5), (dict(scale=-0.5), 5),
    # finite, but scale * log2(e) overflows float (the kernels' exponent factor)
    (dict(scale=3e38), 5), (dict(scale=3e38, dtype=_lib.FA_F32), 5),
    (dict(q=FAKE + 2), 8), (dict(lse=FAKE + 4), 8), (dict(o=FAKE + 8), 8),
])
def test_forward_rejects_invalid_arguments(kw, status):
    assert fwd(**kw) == status


@pytest.mark.parametrize("kw", [dict(B=0), dict(H=0), dict(N=0), dict(N=0, q=0, k=0, v=0, o=0, lse=0)])
def test_forward_empty_problem_is_a_noop(kw):
    assert fwd(**kw) == 0


@pytest.mark.parametrize("kw,status", [
    (dict(q=0), 1), (dict(do=0), 1), (dict(lse=0), 1), (dict(dq=0), 1), (dict(dk=0), 1), (dict(dv=0), 1),
    (dict(o=0), 1),
    (dict(N=-5), 2), (dict(d=80), 3), (dict(dtype=7), 4), (dict(scale=float("-inf")), 5),
    (dict(ws=0), 6), (dict(ws_bytes=100), 6), (dict(ws=0x100010), 8), (dict(dv=FAKE + 6), 8),
])
def test_backward_rejects_invalid_arguments(kw, status):
    assert bwd(**kw) == status


def test_backward_workspace_exact_size_is_accepted_by_validation():
    need = fa.workspace_size(1, 2, 64, 64)
    assert bwd(ws_bytes=need - 1) == 6
    # with the exact size validation passes; a NULL tensor then fails next
    assert bwd(ws_bytes=need, dq=0) == 1


def bwd_noalloc(**kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, o=FAKE, do=FAKE, lse=FAKE, dq=FAKE, dk=FAKE, dv=FAKE, B=1, H=2,
             N=64, d=64, causal=1, scale=0.125, dtype=_lib.FA_BF16, stream=None)
    a.update(kw)
    return fa.fa_backward_noalloc(a["q"], a["k"], a["v"], a["o"], a["do"], a["lse"], a["dq"], a["dk"], a["dv"],
                                  a["B"], a["H"], a["N"], a["d"], a["causal"], a["scale"], a["dtype"], a["stream"])


@pytest.mark.parametrize("kw,status", [
    (dict(q=0), 1), (dict(do=0), 1), (dict(lse=0), 1), (dict(dq=0), 1), (dict(dk=0), 1), (dict(dv=0), 1),
    (dict(o=0), 1),
    (dict(N=-5), 2), (dict(d=80), 3), (dict(dtype=7), 4), (dict(scale=float("-inf")), 5),
    (dict(dv=FAKE + 6), 8),
    # past the built-in scratch: more than 2^21 rows (16 MiB of workspace)
    (dict(B=1, H=1, N=(1 << 21) + 1), 11), (dict(B=2, H=32, N=65536, d=128), 11),
    # an invalid argument is reported before the scratch limit
    (dict(B=2, H=32, N=65536, q=0), 1),
])
def test_backward_noalloc_rejects_invalid_arguments_before_any_hip_call(kw, status):
    """fa_backward_noalloc validates exactly as fa_backward (no workspace
    argument), then checks its built-in scratch size, all before touching
    the device."""
    assert bwd_noalloc(**kw) == status


def test_backward_noalloc_empty_problem_is_ok():
    assert bwd_noalloc(N=0) == 0
    assert bwd_noalloc(B=0, q=0) == 0


def test_backward_noalloc_scratch_limit_matches_the_workspace_size():
    """2^21 rows fit exactly: the workspace is two 4-byte statistics per row."""
    assert _lib.NOALLOC_SCRATCH_BYTES == 16 << 20
    assert fa.workspace_size(1, 1, 1 << 21, 64) == _lib.NOALLOC_SCRATCH_BYTES
    assert fa.workspace_size(1, 1, (1 << 21) + 1, 64) > _lib.NOALLOC_SCRATCH_BYTES
    text = open(HEADER).read()
    assert "#define FA_NOALLOC_SCRATCH_BYTES ((size_t)16 << 20)" in text


def test_workspace_size_is_linear_in_n_and_aligned():
    for d in (64, 128):
        for n in (1, 17, 4096, 16384):
            rows = 3 * 5 * n
            want = 2 * (((rows * 4 + 255) // 256) * 256)
            assert fa.workspace_size(3, 5, n, d) == want
    assert fa.workspace_size(1, 1, 0, 64) == 0
    assert fa.workspace_size(1, 1, 16, 48) == 0
    assert fa.workspace_size(-1, 1, 16, 64) == 0


def test_python_binding_rejects_bad_tensors_on_cpu():
    import torch
    q = torch.zeros(1, 1, 8, 64)
    with pytest.raises(ValueError):
        fa.forward(q, q, q)
    with pytest.raises(ValueError):
        fa.forward(q[0], q[0], q[0])


def test_staged_backward_validation():
    B, H, N, d = 1, 2, 64, 64
    ws, need = 0x100000, fa.workspace_size(1, 2, 64, 64)
    bf = _lib.FA_BF16
    assert fa.fa_backward_preprocess(0, FAKE, FAKE, B, H, N, d, bf, ws, need, None) == 1
    assert fa.fa_backward_preprocess(FAKE, FAKE, 0, B, H, N, d, bf, ws, need, None) == 1
    assert fa.fa_backward_preprocess(FAKE, FAKE, FAKE, B, H, N, d, bf, ws, need - 1, None) == 6
    assert fa.fa_backward_preprocess(FAKE, FAKE, FAKE, B, H, N, 32, bf, ws, need, None) == 3
    assert fa.fa_backward_preprocess(FAKE, FAKE, FAKE, B, H, 0, d, bf, 0, 0, None) == 0
    kv_args = [FAKE] * 6          # q, k, v, dout, dk, dv
    assert fa.fa_backward_dkdv(*kv_args, B, H, N, d, 1, 0.1, bf, 0, need, None) == 6
    bad = list(kv_args)
    bad[3] = 0  # dout
    assert fa.fa_backward_dkdv(*bad, B, H, N, d, 1, 0.1, bf, ws, need, None) == 1
    bad = list(kv_args)
    bad[5] = FAKE + 8  # dv misaligned
    assert fa.fa_backward_dkdv(*bad, B, H, N, d, 1, 0.1, bf, ws, need, None) == 8
    assert fa.fa_backward_dkdv(*kv_args, B, H, N, d, 1, float("nan"), bf, ws, need, None) == 5
    dq_args = [FAKE] * 5          # q, k, v, dout, dq
    bad = list(dq_args)
    bad[4] = 0
    assert fa.fa_backward_dq(*bad, B, H, N, d, 1, 0.1, bf, ws, need, None) == 1
    assert fa.fa_backward_dq(*dq_args, B, H, N, d, 1, 0.1, 3, ws, need, None) == 4
    assert fa.fa_backward_dq(*dq_args, -1, H, N, d, 1, 0.1, bf, ws, need, None) == 2


def fwd_sparse(**kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, o=FAKE, lse=FAKE, mask=FAKE, mask_heads=1, block_q=128, block_k=64, B=1, H=2,
             N=1024, d=128, causal=1, scale=0.125, dtype=_lib.FA_BF16, stream=None)
    a.update(kw)
    return fa.fa_forward_block_sparse(a["q"], a["k"], a["v"], a["o"], a["lse"], a["mask"], a["mask_heads"],
                                      a["block_q"], a["block_k"], a["B"], a["H"], a["N"], a["d"], a["causal"],
                                      a["scale"], a["dtype"], a["stream"])


@pytest.mark.parametrize("kw,status", [
    (dict(mask=0), 1), (dict(q=0), 1), (dict(lse=0), 1),
    (dict(N=-1), 2), (dict(d=96), 3), (dict(dtype=3), 4), (dict(scale=float("nan")), 5),
    (dict(block_q=0), 9), (dict(block_q=48), 9), (dict(block_q=-32), 9), (dict(block_k=32), 9),
    (dict(block_k=96), 9), (dict(block_k=0), 9), (dict(mask_heads=0), 9), (dict(mask_heads=3), 9),
    (dict(N=65536 + 64), 9),
    (dict(o=FAKE + 4), 8),
])
def test_block_sparse_forward_rejects_invalid_arguments(kw, status):
    assert fwd_sparse(**kw) == status


@pytest.mark.parametrize("kw", [dict(B=0), dict(N=0, mask=0, q=0), dict(H=0, mask_heads=1)])
def test_block_sparse_forward_empty_problem_is_a_noop(kw):
    assert fwd_sparse(**kw) == 0


def bwd_sparse(**kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, o=FAKE, do=FAKE, lse=FAKE, dq=FAKE, dk=FAKE, dv=FAKE, mask=FAKE, mask_heads=1,
             block_q=128, block_k=64, B=1, H=2, N=1024, d=128, causal=1, scale=0.125, dtype=_lib.FA_BF16,
             ws=0x100000, ws_bytes=1 << 30, stream=None)
    a.update(kw)
    return fa.fa_backward_block_sparse(a["q"], a["k"], a["v"], a["o"], a["do"], a["lse"], a["dq"], a["dk"], a["dv"],
                                       a["mask"], a["mask_heads"], a["block_q"], a["block_k"], a["B"], a["H"],
                                       a["N"], a["d"], a["causal"], a["scale"], a["dtype"], a["ws"], a["ws_bytes"],
                                       a["stream"])


@pytest.mark.parametrize("kw,status", [
    (dict(mask=0), 1), (dict(q=0), 1), (dict(do=0), 1), (dict(lse=0), 1), (dict(dk=0), 1), (dict(dq=0), 1),
    (dict(N=-1), 2), (dict(d=96), 3), (dict(dtype=3), 4), (dict(scale=float("inf")), 5),
    (dict(block_q=0), 9), (dict(block_q=48), 9), (dict(block_k=32), 9), (dict(block_k=96), 9),
    (dict(mask_heads=0), 9), (dict(mask_heads=3), 9), (dict(N=65536 + 64), 9),
    (dict(ws=0), 6), (dict(ws_bytes=16), 6), (dict(ws=0x100000 + 64), 8), (dict(dv=FAKE + 4), 8),
])
def test_block_sparse_backward_rejects_invalid_arguments(kw, status):
    assert bwd_sparse(**kw) == status


@pytest.mark.parametrize("kw", [dict(B=0), dict(N=0, mask=0, q=0, ws=0), dict(H=0, mask_heads=1)])
def test_block_sparse_backward_empty_problem_is_a_noop(kw):
    assert bwd_sparse(**kw) == 0


def test_block_sparse_accepts_per_head_masks_and_large_blocks_in_validation():
    # mask_heads = H and block sizes that are multiples (validation only; the call then fails at the
    # NULL pointer check that follows geometry)
    assert fwd_sparse(mask_heads=2, block_q=256, block_k=128, q=0) == 1
    assert fwd_sparse(N=65536, block_q=32, block_k=64, k=0) == 1


def test_per_head_byte_size_limit():
    # one head of fp32 d=128 at N = 2^22 spans 2^31 bytes: past the 32-bit offsets
    assert fwd(N=1 << 22, d=128, dtype=_lib.FA_F32) == 2
    # the same N in bf16 spans 2^30 bytes: validation passes, the NULL check fails next
    assert fwd(N=1 << 22, d=128, dtype=_lib.FA_BF16, q=0) == 1


@pytest.mark.parametrize("d,dtype,elt", [(128, _lib.FA_BF16, 2), (64, _lib.FA_BF16, 2), (128, _lib.FA_F32, 4),
                                         (64, _lib.FA_F32, 4)])
def test_per_head_limit_boundary_includes_the_ragged_tile_slack(d, dtype, elt):
    # largest accepted N: (N + 256) rows of d elements within 2^31 - 1 bytes (a ragged last
    # tile addresses up to 256 rows past N with 32-bit offsets)
    n_max = (2**31 - 1) // (d * elt) - 256
    assert fwd(N=n_max, d=d, dtype=dtype, q=0) == 1         # accepted: fails at the NULL check next
    assert fwd(N=n_max + 1, d=d, dtype=dtype, q=0) == 2     # rejected as a shape error first
    assert bwd(N=n_max + 1, d=d, dtype=dtype) == 2


@pytest.mark.parametrize("N", [1, 128, 200, 4096])
def test_launch_work_item_limit(N):
    # A launch's work items (workgroups x threads) must fit in 32 bits; the
    # largest per-tile grid is one 512-thread workgroup per 128 rows of a head,
    # so B * H * ceil(N / 128) must stay below 2^23.  At N = 1 that is reachable
    # with small tensors (2^23 heads of one row), so it is checked, not assumed.
    tiles_per_head = -(-N // 128)
    heads_max = (2**23 - 1) // tiles_per_head
    assert fwd(B=1, H=heads_max, N=N, d=64, q=0) == 1        # accepted: fails at the NULL check next
    assert fwd(B=1, H=heads_max + 1, N=N, d=64, q=0) == 2    # rejected as a shape error first
    assert bwd(B=1, H=heads_max + 1, N=N, d=64) == 2
    assert fa.fa_backward_workspace_size(1, heads_max + 1, N, 64) == 0
    assert fa.fa_backward_workspace_size(1, heads_max, N, 64) > 0


def dec(**kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, o=FAKE, lse=FAKE, B=2, H=4, Nq=1, Nk=4096, d=128, causal=1, scale=0.125,
             dtype=_lib.FA_BF16, splits=0, ws=0x100000, ws_bytes=1 << 30, stream=None)
    a.update(kw)
    return fa.fa_decode(a["q"], a["k"], a["v"], a["o"], a["lse"], a["B"], a["H"], a["Nq"], a["Nk"], a["d"],
                        a["causal"], a["scale"], a["dtype"], a["splits"], a["ws"], a["ws_bytes"], a["stream"])


@pytest.mark.parametrize("kw,status", [
    (dict(q=0), 1), (dict(k=0), 1), (dict(v=0), 1), (dict(o=0), 1), (dict(lse=0), 1),
    (dict(Nq=33), 2), (dict(Nq=-1), 2), (dict(Nk=0), 2), (dict(Nk=-4), 2), (dict(Nq=8, Nk=7), 2),
    (dict(splits=-1), 2), (dict(B=-1), 2),
    (dict(d=96), 3), (dict(dtype=5), 4), (dict(scale=float("inf")), 5),
    (dict(ws=0), 6), (dict(ws_bytes=64), 6),
    (dict(ws=0x100080), 8), (dict(k=FAKE + 2), 8), (dict(lse=FAKE + 4), 8),
])
def test_decode_rejects_invalid_arguments(kw, status):
    assert dec(**kw) == status


@pytest.mark.parametrize("kw", [
    dict(Nq=8, Nk=7, causal=0, q=0),     # non-causal: Nq > Nk is a valid shape
    dict(Nq=32, Nk=32, q=0),
])
def test_decode_valid_shapes_pass_validation(kw):
    assert dec(**kw) == 1


@pytest.mark.parametrize("kw", [dict(Nq=0), dict(B=0), dict(H=0), dict(Nq=0, Nk=0, q=0, k=0, ws=0)])
def test_decode_empty_problem_is_a_noop(kw):
    assert dec(**kw) == 0


def test_decode_grid_work_item_limit():
    # both decoding grids (B*H*chunks and B*H*Nq workgroups of 64 threads) must
    # stay below 2^32 work items, i.e. B * H * max(chunks, Nq) below 2^26
    heads = 2**26 // 32                                  # Nq = 32: exactly 2^26 rows of the merge grid
    assert dec(B=1, H=heads, Nq=32, Nk=64, splits=2, q=0) == 2
    assert fa.fa_decode_workspace_size(1, heads, 32, 64, 128, 2) == 0
    assert dec(B=1, H=heads - 1, Nq=32, Nk=64, splits=2, q=0) == 1     # accepted: NULL check next
    assert fa.fa_decode_workspace_size(1, heads - 1, 32, 64, 128, 2) > 0
    # the chunk grid cannot reach it first: chunks <= ceil(Nk / 32), and the
    # cache's own shape check keeps B * H * ceil(Nk / 128) below 2^23


def test_decode_split_count_and_workspace_size():
    # automatic: about 512 (head, chunk) workgroups, >= 8 tiles of 32 keys per chunk
    assert fa.fa_decode_num_splits(1, 32, 65536, 0) == 16
    assert fa.fa_decode_num_splits(8, 32, 8192, 0) == 2
    assert fa.fa_decode_num_splits(64, 32, 8192, 0) == 1
    assert fa.fa_decode_num_splits(1, 1, 300, 0) == 1
    assert fa.fa_decode_num_splits(1, 1, 4096, 0) == 16
    assert fa.fa_decode_num_splits(1, 1, 1 << 20, 0) == 512
    # requested: kept, but never more chunks than 32-key tiles
    assert fa.fa_decode_num_splits(1, 1, 4096, 7) == 7
    assert fa.fa_decode_num_splits(1, 1, 65, 100) == 3
    assert fa.fa_decode_num_splits(1, 1, 65, -1) == 0
    for B, H, nq, nk, d, s in [(1, 32, 1, 65536, 128, 0), (2, 3, 5, 1000, 64, 4), (1, 1, 32, 1, 128, 0),
                               (64, 32, 1, 8192, 128, 0)]:
        S = fa.fa_decode_num_splits(B, H, nk, s)
        rows = B * H * S * nq
        # partial O and partial lse; nothing with one chunk per head
        want = 0 if S == 1 else -(-rows * d * 4 // 256) * 256 + -(-rows * 4 // 256) * 256
        assert fa.fa_decode_workspace_size(B, H, nq, nk, d, s) == want
    assert dec(Nq=5, Nk=1000, d=64, B=2, H=3, splits=4, ws_bytes=fa.fa_decode_workspace_size(2, 3, 5, 1000, 64, 4) - 1) == 6
    assert dec(Nq=5, Nk=1000, d=64, B=2, H=3, splits=4, ws_bytes=fa.fa_decode_workspace_size(2, 3, 5, 1000, 64, 4),
               q=0) == 1
    # one chunk per head needs no workspace: NULL passes validation (then the NULL q fails)
    assert dec(Nk=64, splits=1, ws=0, ws_bytes=0, q=0) == 1
    assert fa.fa_decode_workspace_size(1, 1, 33, 64, 128, 0) == 0
    assert fa.fa_decode_workspace_size(1, 1, 0, 64, 128, 0) == 0


def fwd_drop(**kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, o=FAKE, lse=FAKE, B=1, H=2, N=64, d=64, causal=0, scale=0.125,
             dtype=_lib.FA_BF16, p=0.1, seed=1, offset=0, stream=None)
    a.update(kw)
    return fa.fa_forward_dropout(a["q"], a["k"], a["v"], a["o"], a["lse"], a["B"], a["H"], a["N"], a["d"],
                                 a["causal"], a["scale"], a["dtype"], a["p"], a["seed"], a["offset"], a["stream"])


def bwd_drop(**kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, o=FAKE, do=FAKE, lse=FAKE, dq=FAKE, dk=FAKE, dv=FAKE, B=1, H=2,
             N=64, d=64, causal=1, scale=0.125, dtype=_lib.FA_BF16, p=0.1, seed=1, offset=0, ws=0x100000,
             ws_bytes=1 << 30, stream=None)
    a.update(kw)
    return fa.fa_backward_dropout(a["q"], a["k"], a["v"], a["o"], a["do"], a["lse"], a["dq"], a["dk"], a["dv"],
                                  a["B"], a["H"], a["N"], a["d"], a["causal"], a["scale"], a["dtype"], a["p"],
                                  a["seed"], a["offset"], a["ws"], a["ws_bytes"], a["stream"])


@pytest.mark.parametrize("kw,status", [
    (dict(q=0), 1), (dict(lse=0), 1), (dict(N=-1), 2), (dict(d=32), 3), (dict(dtype=9), 4),
    (dict(scale=float("nan")), 5), (dict(o=FAKE + 4), 8),
    (dict(p=1.0), 10), (dict(p=-0.01), 10), (dict(p=float("nan")), 10), (dict(p=float("inf")), 10),
    (dict(p=0.999), 10),
    (dict(p=255.4 / 256, q=0), 1),     # rounds to t = 255: accepted, then the NULL q fails
])
def test_forward_dropout_rejects_invalid_arguments(kw, status):
    assert fwd_drop(**kw) == status


@pytest.mark.parametrize("kw,status", [
    (dict(dq=0), 1), (dict(ws=0), 6), (dict(N=-2), 2), (dict(p=1.5), 10), (dict(p=-1.0), 10),
    (dict(p=1.5, N=-2), 2),     # shape errors come first
    (dict(ws=0x100008), 8),
])
def test_backward_dropout_rejects_invalid_arguments(kw, status):
    assert bwd_drop(**kw) == status


def test_dropout_empty_problem_is_a_noop_but_checks_p():
    assert fwd_drop(N=0, q=0) == 0
    assert bwd_drop(B=0, q=0) == 0
    assert fwd_drop(N=0, p=2.0) == 10


def fwd_fp8(**kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, o=FAKE, lse=FAKE, B=1, H=2, N=64, d=128, causal=1, scale=0.1,
             qs=1.0, ks=0.5, vs=2.0, stream=None)
    a.update(kw)
    return fa.fa_forward_fp8(a["q"], a["k"], a["v"], a["o"], a["lse"], a["B"], a["H"], a["N"], a["d"], a["causal"],
                             a["scale"], a["qs"], a["ks"], a["vs"], a["stream"])


@pytest.mark.parametrize("kw,status", [
    (dict(q=0), 1), (dict(o=0), 1), (dict(N=-1), 2), (dict(N=1 << 23, q=0), 2), (dict(d=96), 3),
    (dict(scale=float("nan")), 5), (dict(qs=0.0), 5), (dict(ks=-1.0), 5), (dict(vs=float("inf")), 5),
    (dict(v=FAKE + 8), 8), (dict(N=1 << 22, q=0), 1),
    # finite descale factors whose product with scale and log2(e) overflows float
    (dict(scale=1.0, qs=1e30, ks=1e30), 5), (dict(scale=3e38, qs=1.0, ks=1.0), 5),
    (dict(scale=1e30, qs=1e5, ks=1e4), 5),
])
def test_forward_fp8_rejects_invalid_arguments(kw, status):
    assert fwd_fp8(**kw) == status


def test_scale_just_below_the_exponent_factor_overflow_passes_validation():
    """2e38 * log2(e) is still a finite float: validation passes it and then
    stops at the next check (a NULL tensor)."""
    assert fwd(scale=2e38, o=0) == 1
    assert fwd_fp8(scale=1e30, qs=1e5, ks=1e2, o=0) == 1


def test_forward_fp8_empty_problem_is_a_noop():
    assert fwd_fp8(N=0, q=0) == 0
    assert fwd_fp8(N=0, qs=0.0) == 5
