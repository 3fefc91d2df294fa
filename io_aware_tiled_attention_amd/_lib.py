"""ctypes loader for libfa_gfx950.so and the raw C-ABI entry points.

Argument marshalling only: the signatures mirror include/fa.h one to one.
Loading fails loudly when the library has not been built; there is no
fallback path.
"""
from __future__ import annotations

import ctypes
import os
import threading

LIB_NAME = "libfa_gfx950.so"
LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), LIB_NAME)

# enum fa_dtype / enum fa_status (include/fa.h)
FA_F32 = 0
FA_BF16 = 1
STATUS = {
    0: "FA_OK", 1: "FA_ERR_NULL", 2: "FA_ERR_SHAPE", 3: "FA_ERR_HEADDIM", 4: "FA_ERR_DTYPE",
    5: "FA_ERR_SCALE", 6: "FA_ERR_WORKSPACE", 7: "FA_ERR_HIP", 8: "FA_ERR_ALIGN", 9: "FA_ERR_MASK", 10: "FA_ERR_DROPOUT",
    11: "FA_ERR_SCRATCH",
}
# FA_NOALLOC_SCRATCH_BYTES (include/fa.h): the workspace fa_backward_noalloc holds per GPU
NOALLOC_SCRATCH_BYTES = 16 << 20
EXPORTED = ("fa_forward", "fa_forward_block_sparse", "fa_backward", "fa_backward_block_sparse",
            "fa_backward_workspace_size",
            "fa_backward_preprocess", "fa_backward_dkdv", "fa_backward_dq", "fa_forward_dropout",
            "fa_backward_dropout", "fa_forward_fp8", "fa_decode",
            "fa_decode_workspace_size", "fa_decode_num_splits", "fa_backward_noalloc", "fa_strerror")

_lock = threading.Lock()
_lib = None


class FaError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        name = STATUS.get(status, str(status))
        msg = load().fa_strerror(status).decode()
        super().__init__(f"{where} failed with {name}: {msg}")


def load() -> ctypes.CDLL:
    """Load (once) and return the HIP attention library."""
    global _lib
    with _lock:
        if _lib is not None:
            return _lib
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is missing: build it first with "
                "`python -m io_aware_tiled_attention_amd.build` (there is no fallback path)")
        lib = ctypes.CDLL(LIB_PATH)
        vp, i, f, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
        lib.fa_forward.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, f, i, vp]
        lib.fa_forward.restype = i
        lib.fa_forward_block_sparse.argtypes = [vp, vp, vp, vp, vp, vp, i, i, i, i, i, i, i, i, f, i, vp]
        lib.fa_forward_block_sparse.restype = i
        lib.fa_backward.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, i, i, i, i, i, f, i, vp, sz, vp]
        lib.fa_backward.restype = i
        lib.fa_backward_block_sparse.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, i, i, i, i, i, i, i, i,
                                                 f, i, vp, sz, vp]
        lib.fa_backward_block_sparse.restype = i
        lib.fa_backward_workspace_size.argtypes = [i, i, i, i]
        lib.fa_backward_workspace_size.restype = sz
        lib.fa_backward_preprocess.argtypes = [vp, vp, vp, i, i, i, i, i, vp, sz, vp]
        lib.fa_backward_preprocess.restype = i
        lib.fa_backward_dkdv.argtypes = [vp, vp, vp, vp, vp, vp, i, i, i, i, i, f, i, vp, sz, vp]
        lib.fa_backward_dkdv.restype = i
        lib.fa_backward_dq.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, f, i, vp, sz, vp]
        lib.fa_backward_dq.restype = i
        u64, u32 = ctypes.c_uint64, ctypes.c_uint32
        lib.fa_forward_dropout.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, f, i, f, u64, u32, vp]
        lib.fa_forward_dropout.restype = i
        lib.fa_backward_dropout.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, i, i, i, i, i, f, i, f, u64, u32,
                                            vp, sz, vp]
        lib.fa_backward_dropout.restype = i
        lib.fa_forward_fp8.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, f, f, f, f, vp]
        lib.fa_forward_fp8.restype = i
        lib.fa_decode.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, i, f, i, i, vp, sz, vp]
        lib.fa_decode.restype = i
        lib.fa_decode_workspace_size.argtypes = [i, i, i, i, i, i]
        lib.fa_decode_workspace_size.restype = sz
        lib.fa_decode_num_splits.argtypes = [i, i, i, i]
        lib.fa_decode_num_splits.restype = i
        lib.fa_backward_noalloc.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, i, i, i, i, i, f, i, vp]
        lib.fa_backward_noalloc.restype = i
        lib.fa_strerror.argtypes = [i]
        lib.fa_strerror.restype = ctypes.c_char_p
        _lib = lib
        return lib


def fa_forward(q, k, v, o, lse, B, H, N, d, causal, scale, dtype, stream) -> int:
    return load().fa_forward(q, k, v, o, lse, B, H, N, d, int(causal), float(scale), dtype, stream)


def fa_forward_block_sparse(q, k, v, o, lse, block_mask, mask_heads, block_q, block_k, B, H, N, d, causal,
                            scale, dtype, stream) -> int:
    return load().fa_forward_block_sparse(q, k, v, o, lse, block_mask, mask_heads, block_q, block_k, B, H, N, d,
                                          int(causal), float(scale), dtype, stream)


def fa_backward(q, k, v, o, dout, lse, dq, dk, dv, B, H, N, d, causal, scale, dtype,
                workspace, workspace_bytes, stream) -> int:
    return load().fa_backward(q, k, v, o, dout, lse, dq, dk, dv, B, H, N, d, int(causal),
                              float(scale), dtype, workspace, workspace_bytes, stream)


def fa_backward_block_sparse(q, k, v, o, dout, lse, dq, dk, dv, block_mask, mask_heads, block_q, block_k, B, H, N,
                             d, causal, scale, dtype, workspace, workspace_bytes, stream) -> int:
    return load().fa_backward_block_sparse(q, k, v, o, dout, lse, dq, dk, dv, block_mask, mask_heads, block_q,
                                           block_k, B, H, N, d, int(bool(causal)), scale, dtype, workspace,
                                           workspace_bytes, stream)


def fa_backward_preprocess(o, dout, lse, B, H, N, d, dtype, workspace, workspace_bytes, stream) -> int:
    return load().fa_backward_preprocess(o, dout, lse, B, H, N, d, dtype, workspace, workspace_bytes, stream)


def fa_backward_dkdv(q, k, v, dout, dk, dv, B, H, N, d, causal, scale, dtype,
                     workspace, workspace_bytes, stream) -> int:
    return load().fa_backward_dkdv(q, k, v, dout, dk, dv, B, H, N, d, int(causal),
                                   float(scale), dtype, workspace, workspace_bytes, stream)


def fa_backward_dq(q, k, v, dout, dq, B, H, N, d, causal, scale, dtype,
                   workspace, workspace_bytes, stream) -> int:
    return load().fa_backward_dq(q, k, v, dout, dq, B, H, N, d, int(causal), float(scale),
                                 dtype, workspace, workspace_bytes, stream)


def fa_backward_workspace_size(B, H, N, d) -> int:
    return load().fa_backward_workspace_size(B, H, N, d)


def fa_forward_dropout(q, k, v, o, lse, B, H, N, d, causal, scale, dtype, p_drop, seed, offset, stream) -> int:
    return load().fa_forward_dropout(q, k, v, o, lse, B, H, N, d, int(causal), float(scale), dtype, float(p_drop),
                                     int(seed), int(offset), stream)


def fa_backward_dropout(q, k, v, o, dout, lse, dq, dk, dv, B, H, N, d, causal, scale, dtype, p_drop, seed, offset,
                        workspace, workspace_bytes, stream) -> int:
    return load().fa_backward_dropout(q, k, v, o, dout, lse, dq, dk, dv, B, H, N, d, int(causal), float(scale),
                                      dtype, float(p_drop), int(seed), int(offset), workspace, workspace_bytes,
                                      stream)


def fa_forward_fp8(q, k, v, o, lse, B, H, N, d, causal, scale, q_descale, k_descale, v_descale, stream) -> int:
    return load().fa_forward_fp8(q, k, v, o, lse, B, H, N, d, int(causal), float(scale), float(q_descale),
                                 float(k_descale), float(v_descale), stream)


def fa_decode(q, k, v, o, lse, B, H, Nq, Nk, d, causal, scale, dtype, num_splits,
              workspace, workspace_bytes, stream) -> int:
    return load().fa_decode(q, k, v, o, lse, B, H, Nq, Nk, d, int(causal), float(scale), dtype,
                            num_splits, workspace, workspace_bytes, stream)


def fa_decode_workspace_size(B, H, Nq, Nk, d, num_splits) -> int:
    return load().fa_decode_workspace_size(B, H, Nq, Nk, d, num_splits)


def fa_decode_num_splits(B, H, Nk, num_splits) -> int:
    return load().fa_decode_num_splits(B, H, Nk, num_splits)


def fa_backward_noalloc(q, k, v, o, dout, lse, dq, dk, dv, B, H, N, d, causal, scale, dtype, stream) -> int:
    return load().fa_backward_noalloc(q, k, v, o, dout, lse, dq, dk, dv, B, H, N, d, int(causal), float(scale),
                                      dtype, stream)


def fa_strerror(status: int) -> str:
    return load().fa_strerror(status).decode()
