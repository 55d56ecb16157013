"""Helpers for the GPU tests: move seeded storage arrays to the device and
read results back as float64.  Marshalling only."""

from __future__ import annotations

import numpy as np
import torch

from dense_gemm_transformer_amd import inputs, tlgemm
from oracle import normalized_error  # noqa: F401  (the one pinned measure)

TOL = {"f32": 1e-5, "f16": 1e-2, "bf16": 1e-2}  # max|err| / max|ref|, keyed by the input type


def to_device(a: np.ndarray, dtype: str, device="cuda:0") -> torch.Tensor:
    if dtype == "bf16":
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(device)
    return torch.from_numpy(np.ascontiguousarray(a)).to(device)


def to_f64(t: torch.Tensor) -> np.ndarray:
    t = t.detach().cpu()
    if t.dtype == torch.bfloat16:
        return inputs.widen(t.view(torch.int16).numpy().view(np.uint16), "bf16")
    return t.numpy().astype(np.float64)


def device_case(case: inputs.LinearCase, device="cuda:0"):
    X = to_device(case.X, case.in_dtype, device)
    W = to_device(case.W, case.in_dtype, device)
    b = None if case.b is None else to_device(case.b, case.in_dtype, device)
    return X, W, b


def run_case(case: inputs.LinearCase, variant=tlgemm.VARIANT_AUTO, split_k=0, tile=0, dev=None, plan=None):
    """Run one case through the C ABI; returns (Y tensor, plan description)."""
    X, W, b = dev if dev is not None else device_case(case)
    own = plan is None
    R = getattr(case, "R", None)
    if own:
        plan = tlgemm.Plan.create(case.M, case.N, case.K, case.in_dtype, case.out_dtype, case.layout,
                                  case.b is not None, case.gelu, variant, split_k, tile, R is not None)
    try:
        # with a residual, Y starts as the residual and is updated in place
        Y = None if R is None else to_device(R, case.out_dtype, X.device)
        Y = tlgemm.run(plan, X, W, b, Y=Y)
        torch.cuda.synchronize()
        return Y, plan.describe()
    finally:
        if own:
            plan.close()
