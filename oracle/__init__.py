"""CPU oracle for Y = X·Wᵀ (+ b, optional tanh-GELU) and the layer around it.  TEST INFRASTRUCTURE.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The product library never does, and
this package imports nothing from it: the two share only the seeded inputs.

The arithmetic lives in ``oracle.c`` (plain C, double accumulation in
ascending k, OpenMP over output rows, every element computed independently),
built with gcc into ``liboracle.so`` beside it.  This module is marshalling
only: it hands numpy storage arrays to the C functions and returns float64.

Pins (checked by ``tests/test_oracle.py`` without a GPU): exact rational brute
force on tiny shapes, the hand-worked examples in ``tests/golden``, identity,
permutation and all-ones closed forms, numpy float64 matmul, linearity,
layout equivalence, and the GELU identities plus its distance to the erf form.

The two operations around the GEMMs in a GPT-2 layer are written out in C
the same way: ``layernorm`` (biased variance over the row, eps inside the
square root) and ``attention`` (softmax of q·k/sqrt(HS) over the keys up to
the query's position, applied to v, with the log-sum-exp).  Pins
(``tests/test_oracle_layer.py``): torch's float64 layer_norm and
scaled_dot_product_attention on the CPU, a hand-worked normalisation, a
constant row, shift/scale invariance and the unit moments of the output; one
position returns its value row, identical keys average the values, later
positions do not touch earlier outputs, and the probabilities sum to one.

Two steps are done here rather than in C, each a plain one: the transposed
first operand of the ``AT_*`` layouts ("Writing a CUDA matmul that catches
cuBLAS", sections "Putting it in the model, where it behaves differently" and
"Then: a language model on top of it": x(m,k) = A[k][m]) is transposed back
to ``[M][K]`` with numpy before the C loop, and the residual of that page's
section "The residual and GELU go the same way, and cost three detours" is
added to the float64 result after bias and GELU, widened exactly from its
stored type.  Pins: the ``AT_*`` result equals the plain layout on the
transposed input and numpy's matmul; a zero weight with a residual returns
the residual exactly; the residual adds linearly.
"""

from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

_DT = {"f32": 0, "f16": 1, "bf16": 2}
_LAYOUT = {"NK": 0, "KN": 1}  # the C loop's weight layouts; "AT_*" transpose X first
_STORAGE = {"f32": np.float32, "f16": np.float16, "bf16": np.uint16}

_lib = None


def build(force: bool = False) -> str:
    """Compile ``oracle.c`` with gcc (no fast-math, no FMA contraction)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp", "-ffp-contract=off",
               "-fno-fast-math", "-Wall", "-Wextra", "-o", tmp, _SRC, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build()
        lib = ctypes.CDLL(_LIB)
        i64, vp, dp = ctypes.c_int64, ctypes.c_void_p, ctypes.POINTER(ctypes.c_double)
        ci = ctypes.c_int
        lib.oracle_linear_rows.argtypes = [i64, i64, i64, ci, ci, vp, vp, vp, ci, i64, i64, dp, ci]
        lib.oracle_linear_rows.restype = ci
        lib.oracle_linear_points.argtypes = [i64, i64, i64, ci, ci, vp, vp, vp, ci, i64,
                                             ctypes.POINTER(i64), ctypes.POINTER(i64), dp, ci]
        lib.oracle_linear_points.restype = ci
        lib.oracle_gelu_tanh.argtypes = [ctypes.c_double]
        lib.oracle_gelu_tanh.restype = ctypes.c_double
        lib.oracle_decode.argtypes = [vp, i64, ci]
        lib.oracle_decode.restype = ctypes.c_double
        lib.oracle_max_threads.restype = ci
        lib.oracle_layernorm.argtypes = [i64, i64, ci, vp, vp, vp, ctypes.c_double, dp, dp, dp, ci]
        lib.oracle_layernorm.restype = ci
        lib.oracle_attention.argtypes = [i64, i64, i64, i64, ci, vp, ci, dp, dp, ci]
        lib.oracle_attention.restype = ci
        _lib = lib
    return _lib


def _dims(X, W, layout):
    """(M, N, K) from the stored shapes: X [M][K] or [K][M] (AT_*), W [N][K] or [K][N]."""
    if layout not in ("NK", "KN", "AT_NK", "AT_KN"):
        raise ValueError(f"unknown layout {layout!r}")
    K, M = np.shape(X) if layout.startswith("AT_") else np.shape(X)[::-1]
    N = np.shape(W)[1] if layout.endswith("KN") else np.shape(W)[0]
    return M, N, K


def _widen(a, dtype):
    a = np.ascontiguousarray(a, dtype=_STORAGE[dtype])
    if dtype == "bf16":
        return (a.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return a.astype(np.float64)


def _prep(X, W, b, dtype, layout, M, N, K):
    st = _STORAGE[dtype]
    X = np.ascontiguousarray(X, dtype=st)
    W = np.ascontiguousarray(W, dtype=st)
    if layout.startswith("AT_"):
        if X.shape != (K, M):
            raise ValueError(f"X shape {X.shape} != {(K, M)} for layout {layout}")
        X = np.ascontiguousarray(X.T)
        layout = layout[3:]
    if X.shape != (M, K):
        raise ValueError(f"X shape {X.shape} != {(M, K)}")
    want = (N, K) if layout == "NK" else (K, N)
    if W.shape != want:
        raise ValueError(f"W shape {W.shape} != {want} for layout {layout}")
    if b is not None:
        b = np.ascontiguousarray(b, dtype=st)
        if b.shape != (N,):
            raise ValueError(f"bias shape {b.shape} != {(N,)}")
    return X, W, b, layout


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def linear_rows(X, W, b=None, *, dtype="f32", layout="NK", gelu=False, rows=None,
                threads: int = 0, residual=None, out_dtype=None) -> np.ndarray:
    """Float64 reference for rows ``rows = (m0, m1)`` of the output (all by default)."""
    M, N, K = _dims(X, W, layout)
    X, W, b, layout = _prep(X, W, b, dtype, layout, M, N, K)
    m0, m1 = (0, M) if rows is None else rows
    out = np.empty((m1 - m0, N), dtype=np.float64)
    flags = (1 if b is not None else 0) | (2 if gelu else 0)
    rc = _load().oracle_linear_rows(M, N, K, _DT[dtype], _LAYOUT[layout], _ptr(X), _ptr(W), _ptr(b),
                                    flags, m0, m1,
                                    out.ctypes.data_as(ctypes.POINTER(ctypes.c_double)), threads)
    if rc != 0:
        raise ValueError("oracle rejected its arguments")
    if residual is not None:
        if np.shape(residual) != (M, N):
            raise ValueError(f"residual shape {np.shape(residual)} != {(M, N)}")
        out += _widen(np.asarray(residual)[m0:m1], out_dtype or dtype)
    return out


def linear(X, W, b=None, *, dtype="f32", layout="NK", gelu=False, threads: int = 0, residual=None,
           out_dtype=None) -> np.ndarray:
    """Float64 reference of the whole output ``[M][N]``."""
    return linear_rows(X, W, b, dtype=dtype, layout=layout, gelu=gelu, threads=threads, residual=residual,
                       out_dtype=out_dtype)


def linear_points(X, W, b=None, *, dtype="f32", layout="NK", gelu=False, mi, ni,
                  threads: int = 0, residual=None, out_dtype=None) -> np.ndarray:
    """Float64 reference of the elements ``(mi[i], ni[i])``."""
    M, N, K = _dims(X, W, layout)
    X, W, b, layout = _prep(X, W, b, dtype, layout, M, N, K)
    mi = np.ascontiguousarray(mi, dtype=np.int64)
    ni = np.ascontiguousarray(ni, dtype=np.int64)
    out = np.empty(mi.shape[0], dtype=np.float64)
    flags = (1 if b is not None else 0) | (2 if gelu else 0)
    i64p = ctypes.POINTER(ctypes.c_int64)
    rc = _load().oracle_linear_points(M, N, K, _DT[dtype], _LAYOUT[layout], _ptr(X), _ptr(W),
                                      _ptr(b), flags, mi.shape[0], mi.ctypes.data_as(i64p),
                                      ni.ctypes.data_as(i64p),
                                      out.ctypes.data_as(ctypes.POINTER(ctypes.c_double)), threads)
    if rc != 0:
        raise ValueError("oracle rejected its arguments")
    if residual is not None:
        if np.shape(residual) != (M, N):
            raise ValueError(f"residual shape {np.shape(residual)} != {(M, N)}")
        out += _widen(np.asarray(residual)[mi, ni], out_dtype or dtype)
    return out


def linear_case(case, threads: int = 0, rows=None) -> np.ndarray:
    """Reference for an ``inputs.LinearCase`` (with its residual, if it has one)."""
    return linear_rows(case.X, case.W, case.b, dtype=case.in_dtype, layout=case.layout,
                       gelu=case.gelu, rows=rows, threads=threads, residual=getattr(case, "R", None),
                       out_dtype=case.out_dtype)


def layernorm(X, gamma, beta, *, dtype="f32", eps: float = 1e-5, threads: int = 0):
    """Float64 (Y [rows][C], mean [rows], rstd [rows]) of the row-wise layer normalisation of X."""
    st = _STORAGE[dtype]
    X = np.ascontiguousarray(X, dtype=st)
    gamma = np.ascontiguousarray(gamma, dtype=st)
    beta = np.ascontiguousarray(beta, dtype=st)
    rows, C = X.shape
    if gamma.shape != (C,) or beta.shape != (C,):
        raise ValueError("gamma and beta must have C elements")
    Y = np.empty((rows, C), dtype=np.float64)
    mean = np.empty(rows, dtype=np.float64)
    rstd = np.empty(rows, dtype=np.float64)
    dp = ctypes.POINTER(ctypes.c_double)
    rc = _load().oracle_layernorm(rows, C, _DT[dtype], _ptr(X), _ptr(gamma), _ptr(beta), float(eps),
                                  Y.ctypes.data_as(dp), mean.ctypes.data_as(dp), rstd.ctypes.data_as(dp), threads)
    if rc != 0:
        raise ValueError("oracle rejected its arguments")
    return Y, mean, rstd


def attention(qkv, n_head: int, *, dtype="f32", causal: bool = True, threads: int = 0):
    """Float64 (out [B][T][C], lse [B][NH][T]) of scaled dot-product attention over qkv [B][T][3C]."""
    qkv = np.ascontiguousarray(qkv, dtype=_STORAGE[dtype])
    B, T, C3 = qkv.shape
    if C3 % (3 * n_head):
        raise ValueError("3C must split into three blocks of n_head heads")
    C = C3 // 3
    HS = C // n_head
    out = np.empty((B, T, C), dtype=np.float64)
    lse = np.empty((B, n_head, T), dtype=np.float64)
    dp = ctypes.POINTER(ctypes.c_double)
    rc = _load().oracle_attention(B, T, n_head, HS, _DT[dtype], _ptr(qkv), int(bool(causal)),
                                  out.ctypes.data_as(dp), lse.ctypes.data_as(dp), threads)
    if rc != 0:
        raise ValueError("oracle rejected its arguments")
    return out, lse


def gelu_tanh(y: float) -> float:
    return _load().oracle_gelu_tanh(float(y))


def decode(stored: np.ndarray, dtype: str) -> np.ndarray:
    """The oracle's own widening of stored elements to float64."""
    a = np.ascontiguousarray(stored, dtype=_STORAGE[dtype]).ravel()
    lib = _load()
    p = a.ctypes.data_as(ctypes.c_void_p)
    return np.array([lib.oracle_decode(p, i, _DT[dtype]) for i in range(a.size)])


def max_threads() -> int:
    return _load().oracle_max_threads()


def normalized_error(y, ref) -> float:
    """max|y - ref| / max|ref|, the matmul error measure of "Writing a CUDA
    matmul that catches cuBLAS", section "The measurement was nearly wrong".

    Both maxima run over the whole output; the denominator is the reference's
    largest magnitude, never the result's.  Shapes must match exactly (no
    broadcasting).  A NaN anywhere in ``y`` yields NaN, which passes no
    tolerance; a zero reference gives 0 for a zero result and inf otherwise.
    """
    y = np.asarray(y, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    if y.shape != ref.shape:
        raise ValueError(f"result shape {y.shape} != reference shape {ref.shape}")
    if ref.size == 0:
        return 0.0
    denom = np.max(np.abs(ref))
    num = np.max(np.abs(y - ref))
    if np.isnan(num):
        return float("nan")
    if denom == 0.0:
        return 0.0 if num == 0.0 else float("inf")
    return float(num / denom)
