"""Captured launch sequences: the path recorded in a HIP graph and replayed.

"Optimizing a GPT-2-class transformer on a GPU" (Act III, the launch tax)
records a layer's launches once and replays them.  The library launches only
kernels on the caller's stream (no memsets; split-K tickets are reset by the
kernels themselves), so a captured sequence replays unchanged.  Each replay
here is checked bitwise against the eager run, with eager work and a
synchronisation between replays, and the eager result against the oracle.
"""

import numpy as np
import pytest

from dense_gemm_transformer_amd import inputs, tlgemm
import oracle

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():  # pragma: no cover - CPU container
    pytest.skip("needs a GPU", allow_module_level=True)

from gpu_helpers import TOL, device_case, normalized_error, to_f64  # noqa: E402


def _setup(case, **force):
    X, W, b = device_case(case)
    plan = tlgemm.Plan.create(case.M, case.N, case.K, case.in_dtype, case.out_dtype, case.layout,
                              case.b is not None, case.gelu, **force)
    Y = torch.empty((case.M, case.N), dtype=tlgemm.torch_dtype(case.out_dtype), device="cuda:0")
    ws = torch.zeros(max(plan.workspace_size, 1), dtype=torch.uint8, device="cuda:0")
    return {"case": case, "X": X, "W": W, "b": b, "Y": Y, "plan": plan, "ws": ws}


def _launch(g, stream):
    p = g["plan"]
    p.run_ptrs(g["X"].data_ptr(), g["W"].data_ptr(), 0 if g["b"] is None else g["b"].data_ptr(),
               g["Y"].data_ptr(), g["ws"].data_ptr() if p.workspace_size else 0, p.workspace_size,
               stream.cuda_stream)


def test_captured_sequence_replays_bitwise():
    gemms = [
        _setup(inputs.random_case(40, 128, 2304, 768, "f32", bias=True)),              # pipelined stream chunks
        _setup(inputs.random_case(41, 16, 520, 3000, "f16", bias=True, gelu=True),
               variant=tlgemm.VARIANT_STREAM, tile=3, split_k=4),                     # stream, ticketed split
        _setup(inputs.random_case(42, 128, 768, 768, "f32", bias=True),
               variant=tlgemm.VARIANT_TILED, tile=2, split_k=4),                      # tiled split + reducer
        _setup(inputs.random_case(43, 256, 384, 512, "bf16", bias=True, gelu=True)),  # planner's choice
        _setup(inputs.workload_fp16_narrow()),                                         # the narrow layer
        _setup(inputs.random_case(44, 512, 512, 1536, "bf16", bias=True),
               variant=tlgemm.VARIANT_TILED, tile=7, split_k=2),                      # direct LDS loads, split
        _setup(inputs.random_case(45, 512, 256, 768, "f16", gelu=True),
               variant=tlgemm.VARIANT_TILED, tile=9),                                 # four direct-load stages
        _setup(inputs.random_case(46, 1024, 512, 256, "bf16", bias=True),
               variant=tlgemm.VARIANT_TILED, tile=10),                                # persistent workgroups
    ]
    assert all("load=direct" in g["plan"].describe() for g in gemms[-3:-1])
    assert "persistent" in gemms[-1]["plan"].describe()
    assert gemms[0]["plan"].describe().endswith(" pipelined")
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())  # inputs, outputs and zeroed workspaces come from the default stream
    with torch.cuda.stream(s):
        for g in gemms:
            _launch(g, s)
    s.synchronize()
    eager = [g["Y"].clone() for g in gemms]
    for g in gemms:
        c = g["case"]
        assert normalized_error(to_f64(g["Y"]), oracle.linear_case(c)) <= TOL[c.in_dtype], g["plan"].describe()

    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=s):
        for g in gemms:
            _launch(g, s)
    for rep in range(4):
        for g in gemms:
            g["Y"].fill_(float("nan"))
        # eager work between replays on the same buffers and workspaces
        with torch.cuda.stream(s):
            _launch(gemms[rep % len(gemms)], s)
        s.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for g, want in zip(gemms, eager):
            assert torch.equal(g["Y"], want), f"replay {rep}: {g['plan'].describe()}"
