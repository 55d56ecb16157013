"""Python binding of ``libtlgemm.so`` (C ABI in ``include/tlgemm.h``).

Argument marshalling only: every step of the multiply runs in the library's
HIP kernels.  The functions keep the C names (``gemm_plan``, ``gemm_run``,
``gemm_destroy``, ...); ``linear`` is a convenience that plans, allocates the
output with torch and runs on torch's current stream.

Importing this module loads the library and raises ``ImportError`` if it has
not been built: there is no fallback path.

torch is imported before the library is opened.  The library's dependency
``libamdhip64.so.7`` then binds to the HIP runtime torch already loaded, so
torch's allocations, streams and the library's launches share one runtime
(a second runtime in the same process does not see the GPU).
"""

from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libtlgemm.so")

F32, F16, BF16 = 0, 1, 2
NK, KN, AT_NK, AT_KN = 0, 1, 2, 3
EPI_BIAS, EPI_GELU_TANH, EPI_RESIDUAL = 1, 2, 4
VARIANT_AUTO, VARIANT_GENERIC, VARIANT_STREAM, VARIANT_TILED = -1, 0, 1, 2
VARIANT_NAMES = {VARIANT_GENERIC: "generic", VARIANT_STREAM: "stream", VARIANT_TILED: "tiled"}

OK = 0
ERR_INVALID_ARG, ERR_UNSUPPORTED, ERR_MISALIGNED, ERR_WORKSPACE, ERR_NOMEM, ERR_LAUNCH = -1, -2, -3, -4, -5, -6

DTYPE_CODES = {"f32": F32, "f16": F16, "bf16": BF16}
LAYOUT_CODES = {"NK": NK, "KN": KN, "AT_NK": AT_NK, "AT_KN": AT_KN}

# Every symbol include/tlgemm.h declares.
EXPORTS = ("gemm_plan", "gemm_plan_ex", "gemm_workspace_size", "gemm_plan_info", "gemm_run", "gemm_run_no_alloc",
           "gemm_destroy", "gemm_plan_describe", "gemm_status_string", "gemm_last_error")


class TlgError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{message} (status {status})")
        self.status = status


class PlanOpts(ctypes.Structure):
    _fields_ = [("variant", ctypes.c_int), ("split_k", ctypes.c_int), ("tile", ctypes.c_int)]


class PlanInfo(ctypes.Structure):
    _fields_ = [("variant", ctypes.c_int), ("tile_m", ctypes.c_int), ("tile_n", ctypes.c_int),
                ("tile_k", ctypes.c_int), ("split_k", ctypes.c_int), ("threads", ctypes.c_int),
                ("workgroups", ctypes.c_int64), ("launches", ctypes.c_int),
                ("workspace_bytes", ctypes.c_size_t)]


def _load() -> ctypes.CDLL:
    import torch  # noqa: F401  (load the process's HIP runtime first)

    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is not built; run `python -m dense_gemm_transformer_amd.build` "
                          "(there is no non-HIP fallback)")
    lib = ctypes.CDLL(LIB_PATH)
    i64, vp, sz, u32, ci = ctypes.c_int64, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_uint32, ctypes.c_int
    lib.gemm_plan.argtypes = [ctypes.POINTER(vp), i64, i64, i64, ci, ci, ci, u32]
    lib.gemm_plan.restype = ci
    lib.gemm_plan_ex.argtypes = [ctypes.POINTER(vp), i64, i64, i64, ci, ci, ci, u32, ctypes.POINTER(PlanOpts)]
    lib.gemm_plan_ex.restype = ci
    lib.gemm_workspace_size.argtypes = [vp]
    lib.gemm_workspace_size.restype = sz
    lib.gemm_plan_info.argtypes = [vp, ctypes.POINTER(PlanInfo)]
    lib.gemm_plan_info.restype = ci
    lib.gemm_run.argtypes = [vp, vp, vp, vp, vp, vp, sz, vp]
    lib.gemm_run.restype = ci
    lib.gemm_run_no_alloc.argtypes = [vp, vp, vp, vp, vp, vp]
    lib.gemm_run_no_alloc.restype = ci
    lib.gemm_destroy.argtypes = [vp]
    lib.gemm_destroy.restype = ci
    lib.gemm_plan_describe.argtypes = [vp, ctypes.c_char_p, sz]
    lib.gemm_plan_describe.restype = ci
    lib.gemm_status_string.argtypes = [ci]
    lib.gemm_status_string.restype = ctypes.c_char_p
    lib.gemm_last_error.argtypes = []
    lib.gemm_last_error.restype = ctypes.c_char_p
    return lib


_lib = _load()


def lib() -> ctypes.CDLL:
    return _lib


def gemm_status_string(status: int) -> str:
    return _lib.gemm_status_string(status).decode()


def gemm_last_error() -> str:
    return _lib.gemm_last_error().decode()


def _check(status: int) -> None:
    if status != OK:
        raise TlgError(status, f"{gemm_status_string(status)}: {gemm_last_error()}")


def _code(v, table):
    return table[v] if isinstance(v, str) else int(v)


def gemm_plan_ex(M, N, K, in_dtype="f32", out_dtype=None, layout="NK", epi_flags=0,
                 variant=VARIANT_AUTO, split_k=0, tile=0):
    """Returns a raw plan handle (int); free it with ``gemm_destroy``."""
    out_dtype = in_dtype if out_dtype is None else out_dtype
    h = ctypes.c_void_p()
    opts = PlanOpts(variant, split_k, tile)
    _check(_lib.gemm_plan_ex(ctypes.byref(h), M, N, K, _code(in_dtype, DTYPE_CODES),
                             _code(out_dtype, DTYPE_CODES), _code(layout, LAYOUT_CODES), epi_flags,
                             ctypes.byref(opts)))
    return h.value


def gemm_plan(M, N, K, in_dtype="f32", out_dtype=None, layout="NK", epi_flags=0):
    out_dtype = in_dtype if out_dtype is None else out_dtype
    h = ctypes.c_void_p()
    _check(_lib.gemm_plan(ctypes.byref(h), M, N, K, _code(in_dtype, DTYPE_CODES), _code(out_dtype, DTYPE_CODES),
                          _code(layout, LAYOUT_CODES), epi_flags))
    return h.value


def gemm_workspace_size(handle) -> int:
    return _lib.gemm_workspace_size(handle)


def gemm_plan_info(handle) -> PlanInfo:
    info = PlanInfo()
    _check(_lib.gemm_plan_info(handle, ctypes.byref(info)))
    return info


def gemm_plan_describe(handle) -> str:
    need = _lib.gemm_plan_describe(handle, None, 0)
    if need < 0:
        _check(need)
    buf = ctypes.create_string_buffer(need + 1)
    _lib.gemm_plan_describe(handle, buf, need + 1)
    return buf.value.decode()


def gemm_run_no_alloc(handle, X, W, bias, Y, stream=0) -> None:
    """gemm_run with the library's own per-device scratch in place of a workspace."""
    _check(_lib.gemm_run_no_alloc(handle, X, W, bias or None, Y, stream or None))


def gemm_run(handle, X, W, bias, Y, workspace=0, ws_bytes=0, stream=0) -> None:
    """All pointer arguments are integers (device addresses); stream is a hipStream_t value."""
    _check(_lib.gemm_run(handle, X, W, bias or None, Y, workspace or None, ws_bytes, stream or None))


def gemm_destroy(handle) -> None:
    _check(_lib.gemm_destroy(handle))


@dataclass
class Plan:
    """Owning wrapper of a plan handle."""

    handle: int
    M: int
    N: int
    K: int
    in_dtype: str
    out_dtype: str
    layout: str
    epi_flags: int

    @classmethod
    def create(cls, M, N, K, in_dtype="f32", out_dtype=None, layout="NK", bias=False, gelu=False,
               variant=VARIANT_AUTO, split_k=0, tile=0, residual=False) -> "Plan":
        out_dtype = in_dtype if out_dtype is None else out_dtype
        epi = (EPI_BIAS if bias else 0) | (EPI_GELU_TANH if gelu else 0) | (EPI_RESIDUAL if residual else 0)
        h = gemm_plan_ex(M, N, K, in_dtype, out_dtype, layout, epi, variant, split_k, tile)
        return cls(h, M, N, K, in_dtype, out_dtype, layout, epi)

    @property
    def info(self) -> PlanInfo:
        return gemm_plan_info(self.handle)

    @property
    def workspace_size(self) -> int:
        return gemm_workspace_size(self.handle)

    def describe(self) -> str:
        return gemm_plan_describe(self.handle)

    def run_ptrs(self, X, W, bias, Y, workspace=0, ws_bytes=0, stream=0) -> None:
        gemm_run(self.handle, X, W, bias, Y, workspace, ws_bytes, stream)

    def close(self) -> None:
        if self.handle:
            gemm_destroy(self.handle)
            self.handle = 0

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


# ---- torch convenience (torch supplies device memory and the stream) -------------------

def _torch_dtype_name(t) -> str:
    import torch

    return {torch.float32: "f32", torch.float16: "f16", torch.bfloat16: "bf16"}[t.dtype]


def torch_dtype(name: str):
    import torch

    return {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}[name]


def run(plan: Plan, X, W, bias=None, Y=None, workspace=None, stream=None):
    """Run ``plan`` on torch device tensors; allocates Y (and workspace) if not given.

    With a residual plan Y is required: it holds the residual and receives the result.
    """
    import torch

    if plan.epi_flags & EPI_RESIDUAL and Y is None:
        raise ValueError("a residual plan reads Y: pass the residual tensor as Y")
    if Y is None:
        Y = torch.empty((plan.M, plan.N), dtype=torch_dtype(plan.out_dtype), device=X.device)
    need = plan.workspace_size
    if need and (workspace is None or workspace.numel() * workspace.element_size() < need):
        workspace = torch.zeros(need, dtype=torch.uint8, device=X.device)  # zero before first use
    cur = torch.cuda.current_stream(X.device)
    s = stream if stream is not None else cur
    if s != cur:  # Y and the workspace were allocated (and the workspace zeroed) on the current stream
        s.wait_stream(cur)
    for name, t in (("X", X), ("W", W), ("Y", Y), ("bias", bias)):
        if t is not None and not (t.is_cuda and t.is_contiguous()):
            raise ValueError(f"{name} must be a contiguous device tensor")
    plan.run_ptrs(X.data_ptr(), W.data_ptr(), 0 if bias is None else bias.data_ptr(), Y.data_ptr(),
                  0 if not need else workspace.data_ptr(), need, s.cuda_stream)
    return Y


def linear(X, W, bias=None, *, gelu=False, layout="NK", out_dtype=None, variant=VARIANT_AUTO, split_k=0,
           tile=0, residual=None):
    """Y = act(X·Wᵀ + bias) (+ residual) for torch device tensors.

    W is out×in for ``layout="NK"``; the ``AT_*`` layouts take X stored [K][M].
    ``residual`` ([M][N], the output dtype) is updated in place and returned.
    """
    M, K = (X.shape[1], X.shape[0]) if layout.startswith("AT_") else (X.shape[0], X.shape[1])
    N = W.shape[1] if layout.endswith("KN") else W.shape[0]
    in_dt = _torch_dtype_name(X)
    plan = Plan.create(M, N, K, in_dt, out_dtype or in_dt, layout, bias is not None, gelu, variant, split_k, tile,
                       residual is not None)
    try:
        return run(plan, X, W, bias, Y=residual)
    finally:
        plan.close()
