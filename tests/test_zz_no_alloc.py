"""gemm_run_no_alloc: gemm_run with the library's own per-device scratch in place of a caller workspace,
for callers that cannot allocate (graph capture, serving loops, harnesses that forbid hipMalloc).

Each call is checked against gemm_run with its own zeroed workspace on the same plan and inputs (bitwise:
the same kernels sum in the same order) and against the oracle (max|err|/max|ref| <= 1e-5 for fp32 inputs,
1e-2 for 16-bit).  Calls come in pairs, the second on a smaller input, and plans of both split kinds
(arrival counters, fp32 partials) share the one scratch in turn.
"""

import numpy as np
import pytest

from dense_gemm_transformer_amd import inputs, tlgemm
import oracle

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():  # pragma: no cover - CPU container
    pytest.skip("needs a GPU", allow_module_level=True)

from gpu_helpers import TOL, device_case, normalized_error, to_device, to_f64  # noqa: E402

# (M, N, K, in, out, bias, gelu, residual, variant, tile option, split)
RUNS = [
    ((16, 768, 3072, "f16", "f16", True, True, False), (tlgemm.VARIANT_STREAM, 3, 6)),     # counters + partials
    ((16, 264, 2048, "f16", "f16", True, True, False), (tlgemm.VARIANT_STREAM, 3, 4)),     # smaller
    ((128, 768, 3072, "f32", "f32", True, False, False), (tlgemm.VARIANT_TILED, 2, 8)),   # fp32 partials
    ((64, 256, 1024, "f32", "f32", True, False, True), (tlgemm.VARIANT_TILED, 2, 4)),     # smaller, residual
    ((33, 520, 2048, "bf16", "f32", False, True, False), (tlgemm.VARIANT_STREAM, 3, 4)),  # counters again
    ((16, 4096, 4096, "f16", "f16", False, False, False), (tlgemm.VARIANT_AUTO, 0, 0)),   # no scratch needed
    ((16, 256, 512, "f16", "f16", True, False, False), (tlgemm.VARIANT_AUTO, 0, 0)),
]


def _one(seed, shape, force):
    M, N, K, i, o, bias, gelu, res = shape
    c = inputs.random_case(seed, M, N, K, i, o, "NK", bias=bias, gelu=gelu, residual=res)
    plan = tlgemm.Plan.create(M, N, K, i, o, "NK", bias, gelu, force[0], force[2], force[1], res)
    try:
        X, W, b = device_case(c)
        s = torch.cuda.current_stream()
        R = to_device(c.R, o) if res else None
        y_ref = R.clone() if res else torch.empty((M, N), dtype=tlgemm.torch_dtype(o), device="cuda:0")
        y_ref = tlgemm.run(plan, X, W, b, Y=y_ref)
        y = R.clone() if res else torch.full((M, N), float("nan"), dtype=tlgemm.torch_dtype(o), device="cuda:0")
        tlgemm.gemm_run_no_alloc(plan.handle, X.data_ptr(), W.data_ptr(), 0 if b is None else b.data_ptr(),
                                 y.data_ptr(), s.cuda_stream)
        torch.cuda.synchronize()
        assert torch.equal(y, y_ref), plan.describe()
        err = normalized_error(to_f64(y), oracle.linear_case(c))
        assert err <= TOL[i], f"{plan.describe()}: err {err:.3e}"
        return plan.workspace_size
    finally:
        plan.close()


def test_no_alloc_matches_gemm_run():
    sizes = [_one(90 + n, shape, force) for n, (shape, force) in enumerate(RUNS)]
    assert sizes[0] > sizes[1] > 0 and sizes[2] > sizes[3] > 0 and sizes[5] == 0


def test_no_alloc_twice_in_a_row_same_plan_kind():
    """Two calls back to back without a synchronisation in between, the second smaller."""
    outs = []
    for seed, (M, N, K) in ((95, (16, 768, 3072)), (96, (16, 264, 1536))):
        c = inputs.random_case(seed, M, N, K, "f16", "f16", "NK", bias=True)
        plan = tlgemm.Plan.create(M, N, K, "f16", "f16", "NK", True, False, tlgemm.VARIANT_STREAM, 3, 3)
        X, W, b = device_case(c)
        y = torch.empty((M, N), dtype=torch.float16, device="cuda:0")
        tlgemm.gemm_run_no_alloc(plan.handle, X.data_ptr(), W.data_ptr(), b.data_ptr(), y.data_ptr(),
                                 torch.cuda.current_stream().cuda_stream)
        outs.append((c, plan, X, W, b, y))
    torch.cuda.synchronize()
    for c, plan, X, W, b, y in outs:
        assert torch.equal(y, tlgemm.run(plan, X, W, b)), plan.describe()
        assert normalized_error(to_f64(y), oracle.linear_case(c)) <= TOL["f16"]
        plan.close()


def test_no_alloc_refuses_plans_beyond_the_scratch():
    plan = tlgemm.Plan.create(4096, 4096, 4096, "f32", variant=tlgemm.VARIANT_TILED, split_k=8, tile=1)
    try:
        assert plan.workspace_size > 32 << 20
        X = torch.zeros((4096, 4096), dtype=torch.float32, device="cuda:0")
        Y = torch.zeros_like(X)
        with pytest.raises(tlgemm.TlgError) as e:
            tlgemm.gemm_run_no_alloc(plan.handle, X.data_ptr(), X.data_ptr(), 0, Y.data_ptr(), 0)
        assert e.value.status == tlgemm.ERR_WORKSPACE and "scratch" in str(e.value)
        torch.cuda.synchronize()
        assert not torch.any(Y)  # nothing ran
    finally:
        plan.close()
