"""Python binding of the layer operations in ``libtlgemm.so`` (C ABI in ``include/tlglayer.h``).

Argument marshalling only: the layer normalisation and the attention run in
the library's HIP kernels.  ``tlg_layernorm`` and ``tlg_attention`` keep the C
names and take raw device pointers; ``layernorm`` and ``attention`` are torch
conveniences that allocate the outputs and run on torch's current stream.
"""

from __future__ import annotations

import ctypes

from . import tlgemm

# Every symbol include/tlglayer.h declares.
EXPORTS = ("tlg_layernorm", "tlg_attention")

_lib = tlgemm.lib()
_i64, _vp, _ci = ctypes.c_int64, ctypes.c_void_p, ctypes.c_int
_lib.tlg_layernorm.argtypes = [_vp, _vp, _vp, _vp, _vp, _vp, _i64, _i64, ctypes.c_float, _ci, _vp]
_lib.tlg_layernorm.restype = _ci
_lib.tlg_attention.argtypes = [_vp, _vp, _vp, _i64, _i64, _i64, _i64, _ci, _ci, _vp]
_lib.tlg_attention.restype = _ci


def tlg_layernorm(X, gamma, beta, Y, mean, rstd, rows, C, eps, dtype, stream=0) -> None:
    """Raw-pointer call; mean and rstd may be 0 (not written)."""
    tlgemm._check(_lib.tlg_layernorm(X, gamma, beta, Y, mean or None, rstd or None, rows, C, float(eps),
                                     tlgemm._code(dtype, tlgemm.DTYPE_CODES), stream or None))


def tlg_attention(qkv, out, lse, B, T, n_head, head_size, dtype, causal=True, stream=0) -> None:
    """Raw-pointer call; lse may be 0 (not written)."""
    tlgemm._check(_lib.tlg_attention(qkv, out, lse or None, B, T, n_head, head_size,
                                     tlgemm._code(dtype, tlgemm.DTYPE_CODES), int(bool(causal)), stream or None))


def _contig(name, t):
    if not (t.is_cuda and t.is_contiguous()):
        raise ValueError(f"{name} must be a contiguous device tensor")


def layernorm(X, gamma, beta, eps: float = 1e-5, stats: bool = False):
    """Y = LayerNorm(X) over the last dimension of a [rows][C] tensor; with ``stats`` also (mean, rstd)."""
    import torch

    for n, t in (("X", X), ("gamma", gamma), ("beta", beta)):
        _contig(n, t)
    rows, C = X.shape
    Y = torch.empty_like(X)
    mean = torch.empty(rows, dtype=torch.float32, device=X.device) if stats else None
    rstd = torch.empty(rows, dtype=torch.float32, device=X.device) if stats else None
    tlg_layernorm(X.data_ptr(), gamma.data_ptr(), beta.data_ptr(), Y.data_ptr(),
                  mean.data_ptr() if stats else 0, rstd.data_ptr() if stats else 0, rows, C, eps,
                  tlgemm._torch_dtype_name(X), torch.cuda.current_stream(X.device).cuda_stream)
    return (Y, mean, rstd) if stats else Y


def attention(qkv, n_head: int, causal: bool = True, with_lse: bool = False):
    """out [B][T][C] of causal attention over qkv [B][T][3C]; with ``with_lse`` also lse [B][n_head][T]."""
    import torch

    _contig("qkv", qkv)
    B, T, C3 = qkv.shape
    C = C3 // 3
    out = torch.empty((B, T, C), dtype=qkv.dtype, device=qkv.device)
    lse = torch.empty((B, n_head, T), dtype=torch.float32, device=qkv.device) if with_lse else None
    tlg_attention(qkv.data_ptr(), out.data_ptr(), lse.data_ptr() if with_lse else 0, B, T, n_head, C // n_head,
                  tlgemm._torch_dtype_name(qkv), causal, torch.cuda.current_stream(qkv.device).cuda_stream)
    return (out, lse) if with_lse else out
