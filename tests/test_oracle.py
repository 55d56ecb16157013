"""Pins for the CPU oracle, independent of the oracle's own code (no GPU).

Each test fixes the oracle against something other than itself: hand-worked
values, exact rational arithmetic, closed forms, numpy's float64 matmul, the
format definitions, and mathematical identities of the tanh-GELU.
"""

import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest

from dense_gemm_transformer_amd import inputs

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
DTYPES = ("f32", "f16", "bf16")


def _store(values, dtype):
    return inputs.store(np.asarray(values, dtype=np.float64), dtype)


def _exact(stored, dtype):
    """Exact value of each stored element via numpy's own widening."""
    return inputs.widen(stored, dtype)


# --- hand-worked examples -------------------------------------------------------------

def _hand_cases():
    with open(os.path.join(GOLDEN, "linear_hand_examples.json")) as f:
        return json.load(f)["cases"]


@pytest.mark.parametrize("case", _hand_cases(), ids=lambda c: c["name"])
@pytest.mark.parametrize("dtype", DTYPES)
def test_hand_examples(oracle_lib, case, dtype):
    X = _store(case["X"], dtype)
    W = _store(case["W"], dtype)
    b = None if case["b"] is None else _store(case["b"], dtype)
    ref = oracle_lib.linear(X, W, b, dtype=dtype, layout=case["layout"])
    assert np.array_equal(ref, np.asarray(case["Y"], dtype=np.float64))


def test_number_formats(oracle_lib):
    with open(os.path.join(GOLDEN, "number_formats.json")) as f:
        fmt = json.load(f)
    for dtype, storage in (("f16", np.uint16), ("bf16", np.uint16)):
        bits = np.array([int(h, 16) for h, _ in fmt[dtype]], dtype=storage)
        want = np.array([v for _, v in fmt[dtype]], dtype=np.float64)
        stored = bits.view(np.float16) if dtype == "f16" else bits
        got = oracle_lib.decode(stored, dtype)
        assert np.array_equal(got, want), dtype
        assert np.array_equal(np.signbit(got), np.signbit(want)), dtype


# --- exact rational brute force -------------------------------------------------------

def _special_values(dtype):
    v = [0.0, -0.0, 1.0, -1.0, 0.5, 3.0, -7.25, 1e-3, 250.0]
    if dtype == "f16":
        v += [6.0e-8, 6.1e-5, -65504.0]  # subnormal, near the smallest normal, largest finite
    elif dtype == "bf16":
        v += [1e-39, 3.0e38 / 1e6]
    else:
        v += [1e-40, 1.5e-30, 3.0e30]
    return np.array(v)


LAYOUTS = ["NK", "KN", "AT_NK", "AT_KN"]


@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("layout", LAYOUTS)
def test_rational_bruteforce(oracle_lib, dtype, layout):
    """Oracle vs exact Fraction sums for every M, N, K in 1..6 (plus bias and a residual).

    Products of two stored values are exact in double, so the oracle's only
    rounding is K additions plus the residual's: |oracle - exact| <=
    (K+2) * 2^-53 * (sum|terms| + |r|) (a rigorous bound for recursive
    summation).  A dropped term, a wrong index or a transposed operand is off
    by far more.  x(m,k) is X[m][k], or X[k][m] for the transposed layouts.
    """
    rng = np.random.default_rng(7)
    specials = _special_values(dtype)
    u = 2.0 ** -53
    for M in range(1, 7):
        for N in range(1, 7):
            for K in range(1, 7):
                pool = np.concatenate([rng.standard_normal(8) * 3, specials])
                at, kn = layout.startswith("AT_"), layout.endswith("KN")
                xv = rng.choice(pool, size=(K, M) if at else (M, K))
                wv = rng.choice(pool, size=(K, N) if kn else (N, K))
                bv = rng.choice(pool, size=(N,))
                rv = rng.choice(pool, size=(M, N))
                X, W, b, R = _store(xv, dtype), _store(wv, dtype), _store(bv, dtype), _store(rv, dtype)
                ref = oracle_lib.linear(X, W, b, dtype=dtype, layout=layout, residual=R)
                Xe, We, be, Re = _exact(X, dtype), _exact(W, dtype), _exact(b, dtype), _exact(R, dtype)
                for m in range(M):
                    for n in range(N):
                        terms = [Fraction(Xe[k, m] if at else Xe[m, k]) * Fraction(We[k, n] if kn else We[n, k])
                                 for k in range(K)] + [Fraction(be[n]), Fraction(Re[m, n])]
                        exact = sum(terms, Fraction(0))
                        bound = (K + 2) * u * float(sum(abs(t) for t in terms))
                        assert abs(Fraction(ref[m, n]) - exact) <= Fraction(bound), (M, N, K, m, n)


# --- closed forms -------------------------------------------------------------------

@pytest.mark.parametrize("dtype", DTYPES)
def test_identity_and_permutation(oracle_lib, dtype):
    K = 37
    X = inputs.normal(11, (5, K), 1.0, dtype)
    eye = _store(np.eye(K), dtype)
    assert np.array_equal(oracle_lib.linear(X, eye, dtype=dtype), _exact(X, dtype))
    perm = np.random.default_rng(3).permutation(K)
    P = _store(np.eye(K)[perm], dtype)  # row n of W selects input perm[n]
    assert np.array_equal(oracle_lib.linear(X, P, dtype=dtype), _exact(X, dtype)[:, perm])
    # KN: B = P^T gives the same selection
    assert np.array_equal(oracle_lib.linear(X, np.ascontiguousarray(P.T), dtype=dtype, layout="KN"),
                          _exact(X, dtype)[:, perm])


@pytest.mark.parametrize("dtype", DTYPES)
def test_ones_and_zero_weights(oracle_lib, dtype):
    M, N, K = 3, 4, 4096
    ones_x = _store(np.ones((M, K)), dtype)
    ones_w = _store(np.ones((N, K)), dtype)
    assert np.all(oracle_lib.linear(ones_x, ones_w, dtype=dtype) == K)
    b = inputs.normal(5, (N,), 0.02, dtype)
    zero_w = _store(np.zeros((N, K)), dtype)
    out = oracle_lib.linear(ones_x, zero_w, b, dtype=dtype)
    assert np.array_equal(out, np.broadcast_to(_exact(b, dtype), (M, N)))


# --- library special case and invariants ----------------------------------------------

@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("layout", LAYOUTS)
def test_matches_numpy_float64(oracle_lib, dtype, layout):
    case = inputs.random_case(21, 33, 47, 129, dtype, layout=layout, bias=True, residual=True)
    ref = oracle_lib.linear_case(case)
    Xe, We, be = _exact(case.X, dtype), _exact(case.W, dtype), _exact(case.b, dtype)
    Re = _exact(case.R, dtype)
    lib = (Xe.T if layout.startswith("AT_") else Xe) @ (We if layout.endswith("KN") else We.T) + be + Re
    assert np.max(np.abs(ref - lib)) <= 1e-13 * np.max(np.abs(lib))


@pytest.mark.parametrize("dtype", DTYPES)
def test_zero_weight_returns_residual(oracle_lib, dtype):
    """W = 0 and no bias: every product is zero, GELU(0) = 0, so Y is the residual exactly."""
    M, N, K = 7, 9, 33
    X = inputs.normal(31, (M, K), 1.0, dtype)
    R = inputs.normal(32, (M, N), 1.0, dtype)
    W = _store(np.zeros((N, K)), dtype)
    for gelu in (False, True):
        out = oracle_lib.linear(X, W, dtype=dtype, gelu=gelu, residual=R)
        assert np.array_equal(out, _exact(R, dtype))


@pytest.mark.parametrize("dtype", DTYPES)
def test_transposed_first_operand_identity(oracle_lib, dtype):
    """AT_NK with W = I returns the stored [K][M] operand transposed, bitwise."""
    K, M = 37, 5
    A = inputs.normal(12, (K, M), 1.0, dtype)
    eye = _store(np.eye(K), dtype)
    assert np.array_equal(oracle_lib.linear(A, eye, dtype=dtype, layout="AT_NK"), _exact(A, dtype).T)
    assert np.array_equal(oracle_lib.linear(A, eye, dtype=dtype, layout="AT_KN"), _exact(A, dtype).T)


def test_linearity(oracle_lib):
    rng = np.random.default_rng(9)
    X1 = _store(rng.integers(-8, 8, (6, 50)), "f32")
    X2 = _store(rng.integers(-8, 8, (6, 50)), "f32")
    W = _store(rng.integers(-8, 8, (9, 50)), "f32")
    a, c = 3.0, -2.0
    lhs = oracle_lib.linear((a * X1 + c * X2).astype(np.float32), W)
    rhs = a * oracle_lib.linear(X1, W) + c * oracle_lib.linear(X2, W)
    assert np.array_equal(lhs, rhs)  # small integers: every step is exact


@pytest.mark.parametrize("dtype", DTYPES)
def test_layout_equivalence(oracle_lib, dtype):
    case = inputs.random_case(4, 7, 13, 65, dtype, bias=True, gelu=True)
    a = oracle_lib.linear(case.X, case.W, case.b, dtype=dtype, gelu=True)
    b = oracle_lib.linear(case.X, np.ascontiguousarray(case.W.T), case.b, dtype=dtype, layout="KN",
                          gelu=True)
    assert np.array_equal(a, b)


def test_row_independence(oracle_lib):
    K = 300
    row = inputs.normal(1, (1, K), 1.0, "f32")
    X = np.repeat(row, 5, axis=0)
    W = inputs.normal(2, (11, K), 0.02, "f32")
    out = oracle_lib.linear(X, W)
    assert all(np.array_equal(out[0], out[i]) for i in range(5))


def test_rows_and_points_match_full(oracle_lib):
    case = inputs.random_case(8, 19, 23, 71, "bf16", bias=True, gelu=True)
    full = oracle_lib.linear_case(case)
    assert np.array_equal(oracle_lib.linear_case(case, rows=(5, 12)), full[5:12])
    mi = np.array([0, 18, 7, 7])
    ni = np.array([22, 0, 3, 4])
    pts = oracle_lib.linear_points(case.X, case.W, case.b, dtype="bf16", gelu=True, mi=mi, ni=ni)
    assert np.array_equal(pts, full[mi, ni])


def test_empty_shapes(oracle_lib):
    assert oracle_lib.linear(np.zeros((0, 4), np.float32), np.zeros((3, 4), np.float32)).shape == (0, 3)
    out = oracle_lib.linear(np.zeros((2, 0), np.float32), np.zeros((3, 0), np.float32),
                            np.array([1, 2, 3], np.float32))
    assert np.array_equal(out, np.array([[1, 2, 3], [1, 2, 3]], dtype=np.float64))


def test_rejects_bad_arguments(oracle_lib):
    with pytest.raises(ValueError):
        oracle_lib.linear(np.zeros((2, 3), np.float32), np.zeros((4, 5), np.float32))


# --- GELU ---------------------------------------------------------------------------

def test_gelu_identities(oracle_lib):
    g = oracle_lib.gelu_tanh
    assert g(0.0) == 0.0
    for x in np.linspace(-8, 8, 161):
        # 0.5*x*(1+tanh(u)) - 0.5*(-x)*(1+tanh(-u)) = x for the odd u(x)
        assert abs(g(x) - g(-x) - x) <= 4e-16 * max(1.0, abs(x))
    assert abs((g(1e-6) - g(-1e-6)) / 2e-6 - 0.5) < 1e-9  # slope 1/2 at zero
    assert abs(g(12.0) - 12.0) < 1e-12 and abs(g(-12.0)) < 1e-12
    xs = np.linspace(-0.5, 6, 400)
    assert np.all(np.diff([g(x) for x in xs]) > 0)  # increasing right of its minimum


def test_gelu_close_to_erf_form(oracle_lib):
    """The tanh form approximates x*Phi(x); over the real line the two differ
    by at most 4.73e-4 (at |x| ~ 2.7).  A wrong constant or a dropped cubic
    term moves the maximum well past that (0.045 instead of 0.044715 already
    gives 5.6e-4)."""
    worst = 0.0
    for x in np.linspace(-10, 10, 20001):
        exact = 0.5 * x * (1.0 + math.erf(x / math.sqrt(2.0)))
        worst = max(worst, abs(oracle_lib.gelu_tanh(x) - exact))
    assert 4.6e-4 < worst < 4.8e-4


def test_gelu_applied_after_bias(oracle_lib):
    X = _store([[1.0, 2.0]], "f32")
    W = _store([[0.5, -0.25]], "f32")  # dot = 0
    b = _store([1.5], "f32")
    out = oracle_lib.linear(X, W, b, gelu=True)
    assert out[0, 0] == oracle_lib.gelu_tanh(1.5)


# --- the pass/fail measure: max|y - ref| / max|ref| ----------------------------------------
# "Writing a CUDA matmul that catches cuBLAS", section "The measurement was nearly
# wrong": the error is the largest absolute deviation over the output, divided by the
# largest magnitude of the reference.  Hand-worked values, each chosen so that one
# plausible slip (a dropped abs, a denominator over the result, a signed maximum,
# broadcasting) gives a different number.

def test_error_measure_exact_match_is_zero(oracle_lib):
    ref = np.array([[1.0, -4.0], [2.0, 3.0]])
    assert oracle_lib.normalized_error(ref.copy(), ref) == 0.0


def test_error_measure_hand_values(oracle_lib):
    ref = np.array([[1.0, -4.0], [2.0, 3.0]])
    # one element 0.5 too low: |err| = 0.5, max|ref| = 4 (from the negative entry) -> 0.125;
    # a signed max of ref would give 0.5 / 3, a signed max of (y - ref) would give 0.
    y = ref.copy()
    y[1, 0] -= 0.5
    assert oracle_lib.normalized_error(y, ref) == 0.125
    # the worst of several deviations counts: 0.25 and -1.0 -> 1.0 / 4
    y = ref.copy()
    y[0, 0] += 0.25
    y[1, 1] -= 1.0
    assert oracle_lib.normalized_error(y, ref) == 0.25
    # the denominator is the reference's, not the result's: a result entry of 10 where
    # the reference holds 2 gives 8 / 4 = 2 (over the result it would be 8 / 10)
    y = ref.copy()
    y[1, 0] = 10.0
    assert oracle_lib.normalized_error(y, ref) == 2.0


def test_error_measure_is_relative_to_the_whole_output(oracle_lib):
    # a deviation of 1e-3 on an entry of size 1e-3 is small against max|ref| = 1000
    ref = np.array([1e-3, 1000.0])
    y = np.array([2e-3, 1000.0])
    assert oracle_lib.normalized_error(y, ref) == pytest.approx(1e-6, rel=1e-12)


def test_error_measure_zero_reference_and_empty(oracle_lib):
    z = np.zeros((3, 3))
    assert oracle_lib.normalized_error(z, z) == 0.0
    y = z.copy()
    y[2, 1] = -1e-30
    assert oracle_lib.normalized_error(y, z) == float("inf")
    assert oracle_lib.normalized_error(np.zeros((0, 4)), np.zeros((0, 4))) == 0.0


def test_error_measure_nan_fails_every_tolerance(oracle_lib):
    ref = np.array([1.0, 2.0, 3.0])
    y = ref.copy()
    y[1] = np.nan
    err = oracle_lib.normalized_error(y, ref)
    assert not err <= 1e-2 and not err <= 1e30


def test_error_measure_rejects_shape_mismatch(oracle_lib):
    ref = np.ones((4, 3))
    with pytest.raises(ValueError):
        oracle_lib.normalized_error(np.ones(3), ref)  # would broadcast over the rows
    with pytest.raises(ValueError):
        oracle_lib.normalized_error(np.ones((3, 4)), ref)


def test_error_measure_is_the_one_the_gpu_tests_use():
    """The GPU test helpers take the measure from the oracle package instead of keeping a copy."""
    import ast

    src = open(os.path.join(os.path.dirname(__file__), "gpu_helpers.py")).read()
    tree = ast.parse(src)
    assert not any(isinstance(n, ast.FunctionDef) and n.name == "normalized_error" for n in ast.walk(tree))
    assert any(isinstance(n, ast.ImportFrom) and n.module == "oracle" and
               any(a.name == "normalized_error" for a in n.names) for n in ast.walk(tree))
