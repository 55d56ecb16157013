"""Maximum sizes: operands past the 2 GiB reach of one buffer descriptor, and outputs of more
than 2^31 elements, against the oracle at sampled outputs (the whole product would take the
oracle hours).  Inputs are seeded periodic blocks with prime sides (``inputs.periodic_normal``),
so an address that overflows 32 bits still reads a different value than the right one."""

import numpy as np
import pytest

from dense_gemm_transformer_amd import inputs, tlgemm
import oracle

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():  # pragma: no cover - CPU container
    pytest.skip("needs a GPU", allow_module_level=True)

from gpu_helpers import TOL, device_case, normalized_error, to_f64  # noqa: E402


def _sample_check(case, Y, npts=1500, seed=3):
    """max|err|/max|ref| over sampled outputs, the four corners and the last row's tail; the samples
    are gathered on the device so that a multi-GiB output never crosses to the host."""
    rng = np.random.default_rng(seed)
    mi = np.concatenate([rng.integers(0, case.M, npts), [0, 0, case.M - 1, case.M - 1],
                         np.full(64, case.M - 1)])
    ni = np.concatenate([rng.integers(0, case.N, npts), [0, case.N - 1, 0, case.N - 1],
                         np.arange(case.N - 64, case.N)])
    idx = torch.from_numpy(mi * case.N + ni).to(Y.device)
    got = to_f64(Y.reshape(-1)[idx])
    ref = oracle.linear_points(case.X, case.W, case.b, dtype=case.in_dtype, layout=case.layout, gelu=case.gelu,
                               mi=mi, ni=ni)
    return normalized_error(got, ref)


def _run(case, **force):
    X, W, b = device_case(case)
    plan = tlgemm.Plan.create(case.M, case.N, case.K, case.in_dtype, case.out_dtype, case.layout, False, False,
                              **force)
    try:
        Y = tlgemm.run(plan, X, W, b)
        torch.cuda.synchronize()
        return Y, plan.describe()
    finally:
        plan.close()
        del X, W


def test_weight_past_2gib_takes_64bit_addresses():
    """A [K][N] bf16 weight of exactly 2 GiB (32768 × 32768): past one buffer descriptor's reach, so the tiled
    kernel's guarded path with 64-bit addresses runs it (128 rows: one 128×128 tile row over 256 tiles)."""
    case = inputs.large_case(40, 128, 32768, 32768, "bf16", "f32", "KN")
    assert case.W.nbytes == 2 ** 31
    Y, desc = _run(case)
    assert "variant=tiled" in desc, desc
    err = _sample_check(case, Y)
    assert err <= TOL["bf16"], f"{desc}: err {err:.3e}"


@pytest.mark.parametrize("out_dtype", ["f32", "bf16"])
def test_output_past_2g_elements(out_dtype):
    """65536 × 65536 outputs (2^32 elements: 16 GiB fp32, 8 GiB bf16) from K = 64: every output offset past
    2^31 elements, through the 256×256 tiles and their staged epilogue."""
    case = inputs.large_case(41, 65536, 65536, 64, "bf16" if out_dtype == "bf16" else "f32", out_dtype, "NK")
    Y, desc = _run(case)
    assert "tile=256x256" in desc, desc
    err = _sample_check(case, Y)
    del Y
    torch.cuda.empty_cache()
    assert err <= TOL[case.in_dtype], f"{desc}: err {err:.3e}"


def test_stream_weight_rows_past_2gib():
    """16 rows against a 4 GiB fp16 weight (256 rows of 2^23): the stream kernel's row addresses pass 2^31
    bytes and its split-K runs over 16 workgroups; sampled outputs against the oracle."""
    case = inputs.large_case(42, 16, 256, 2 ** 23, "f16", "f16", "NK")
    assert case.W.nbytes == 2 ** 32
    Y, desc = _run(case)
    assert "variant=stream" in desc, desc
    err = _sample_check(case, Y, npts=120)
    assert err <= TOL["f16"], f"{desc}: err {err:.3e}"
