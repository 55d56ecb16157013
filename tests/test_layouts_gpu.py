"""Parity of the transposed-first-operand layouts and the residual epilogue.

The transposed layouts complete the four transpose cases of "Writing a CUDA
matmul that catches cuBLAS" (sections "Putting it in the model, where it
behaves differently" and "Then: a language model on top of it"): the first
operand stored [K][M], as dYᵀ is in the weight gradient dW = dYᵀ·X.  The
residual adds the result onto what Y holds (section "The residual and GELU go
the same way, and cost three detours").  Same bar as the other parity tests:
max|Y - ref| / max|ref| <= 1e-5 (fp32 inputs) or 1e-2 (fp16/bf16 inputs)
against the CPU oracle, bitwise for the exact cases.
"""

import numpy as np
import pytest

from dense_gemm_transformer_amd import inputs, tlgemm
import oracle

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():  # pragma: no cover - CPU container
    pytest.skip("needs a GPU", allow_module_level=True)

from gpu_helpers import TOL, normalized_error, run_case, to_f64  # noqa: E402

PAIRS = [("f32", "f32"), ("f16", "f16"), ("f16", "f32"), ("bf16", "bf16"), ("bf16", "f32")]
EPIS = [(False, False), (True, False), (False, True), (True, True)]


def _check(case, **force):
    Y, desc = run_case(case, **force)
    err = normalized_error(to_f64(Y), oracle.linear_case(case))
    assert err <= TOL[case.in_dtype], f"{desc}: err {err:.3e}"
    return Y, desc


@pytest.mark.parametrize("pair", PAIRS, ids=lambda p: f"{p[0]}->{p[1]}")
@pytest.mark.parametrize("layout", ["AT_NK", "AT_KN"])
@pytest.mark.parametrize("residual", [False, True], ids=["plain", "residual"])
def test_transposed_first_operand(pair, layout, residual):
    """Generic (any alignment) and every tiled tile, with and without split-K, ragged and exact-fit."""
    shapes = [(37, 70, 29), (130, 65, 100)]  # M not a multiple of 8: the generic kernel
    for M, N, K in shapes:
        c = inputs.random_case(61, M, N, K, pair[0], pair[1], layout, residual=residual)
        _, desc = _check(c)
        assert "variant=generic" in desc
    for tile in (1, 2, 3, 4, 5, 6):
        for (M, N, K), split in [((136, 136, 72), 1), ((256, 256, 256), 1), ((64, 64, 64), 1),
                                 ((200, 264, 400), 3), ((512, 512, 1024), 4)]:
            c = inputs.random_case(62, M, N, K, pair[0], pair[1], layout, residual=residual)
            _, desc = _check(c, variant=tlgemm.VARIANT_TILED, tile=tile, split_k=split)
            assert f"layout={layout} " in desc


@pytest.mark.parametrize("pair", PAIRS, ids=lambda p: f"{p[0]}->{p[1]}")
@pytest.mark.parametrize("epi", EPIS, ids=["none", "bias", "gelu", "bias+gelu"])
def test_residual_every_variant(pair, epi):
    """act(X·Wᵀ + b) + Y through generic, stream (one launch and ticketed split) and tiled (staged and
    per-element epilogues, with and without split-K)."""
    runs = [
        ((37, 70, 29), dict(variant=tlgemm.VARIANT_GENERIC)),
        ((16, 136, 520), dict(variant=tlgemm.VARIANT_STREAM, tile=1)),
        ((33, 520, 2048), dict(variant=tlgemm.VARIANT_STREAM, tile=3, split_k=4)),
        ((130, 136, 72), dict(variant=tlgemm.VARIANT_TILED, tile=2)),           # ragged: per element
        ((256, 256, 256), dict(variant=tlgemm.VARIANT_TILED, tile=1)),          # exact fit: staged
        ((256, 256, 512), dict(variant=tlgemm.VARIANT_TILED, tile=2, split_k=4)),
        ((200, 264, 400), dict(variant=tlgemm.VARIANT_TILED, tile=2, split_k=3)),
    ]
    for (M, N, K), force in runs:
        c = inputs.random_case(63, M, N, K, pair[0], pair[1], "NK", bias=epi[0], gelu=epi[1], residual=True)
        _check(c, **force)


@pytest.mark.parametrize("variant,tile,split", [(tlgemm.VARIANT_GENERIC, 0, 0), (tlgemm.VARIANT_TILED, 1, 1),
                                                 (tlgemm.VARIANT_TILED, 2, 4)])
def test_zero_weight_residual_and_transposed_identity_bitwise(variant, tile, split):
    """W = 0: Y keeps the residual exactly; W = I with the transposed layout: Y is Aᵀ exactly."""
    M, N, K = 64, 128, 256
    R = inputs.normal(71, (M, N), 1.0, "f32")
    c = inputs.LinearCase("zero", M, N, K, "f32", "f32", "NK", False, False,
                          inputs.normal(72, (M, K), 1.0, "f32"), np.zeros((N, K), np.float32), None, R)
    Y, _ = run_case(c, variant=variant, tile=tile, split_k=split)
    assert np.array_equal(Y.cpu().numpy(), R)
    A = inputs.normal(73, (K, M), 1.0, "f32")
    eye = np.eye(K, dtype=np.float32)
    c = inputs.LinearCase("eye", M, K, K, "f32", "f32", "AT_NK", False, False, A, eye, None)
    Y, _ = run_case(c, variant=variant, tile=tile, split_k=split)
    assert np.array_equal(Y.cpu().numpy(), A.T)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_weight_gradient_fc_shape(dtype):
    """dW = dYᵀ·X for the GPT-2 fc layer at 8192 tokens ([3072][8192]ᵀ·[8192][768]), accumulated onto
    a previous gradient; every output against the oracle."""
    M, N, K = 3072, 768, 8192
    dY = inputs.normal(81, (K, M), 1.0, dtype)   # stored [tokens][out]
    X = inputs.normal(82, (K, N), 1.0, dtype)    # stored [tokens][in]
    G = inputs.normal(83, (M, N), 1.0, dtype)    # previous gradient (residual)
    c = inputs.LinearCase("dW_fc", M, N, K, dtype, dtype, "AT_KN", False, False, dY, X, None, G)
    _, desc = _check(c)
    assert "variant=tiled" in desc
