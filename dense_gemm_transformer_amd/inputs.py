"""Seeded synthetic inputs for the transformer linear layer Y = X·Wᵀ (+ b).

This module only draws numbers and stores them in the element formats the
kernels read. It holds none of the multiply's arithmetic, so both the HIP path
and the CPU oracle can be fed from it without sharing any of the computation.

Recipe (one source of truth for tests and the benchmark):

* Generator: numpy ``PCG64`` seeded per tensor. The pages fix their weights with
  a seeded generator but never say which one ("Optimizing a GPT-2-class
  transformer on a GPU", Results), so the draws differ from theirs.
* Seeds: ``1000 * workload + 10 * layer + tensor`` with tensor X = 1, W = 2,
  b = 3 (backward: dY = 5, accumulated weight gradient = 6; LayerNorm: X, gamma,
  beta = 1, 2, 3 of workload 7; attention: qkv = 1 of workload 8), plus ``100000 * g`` for the g-th linear of a GPT-2 layer (qkv 0,
  attn-out 1, fc 2, proj 3), so that no two tensors of a stack share a seed.
* Values are drawn in float64, rounded to float32 with round-to-nearest-even,
  then (for half formats) rounded again to float16 / bfloat16 with
  round-to-nearest-even. The stored values are exactly what the kernels read;
  the oracle widens those same stored values.
* "N(0, 0.02)" means standard deviation 0.02 (the GPT-2 initialisation).

Storage arrays: float32 -> ``np.float32``, float16 -> ``np.float16``,
bfloat16 -> ``np.uint16`` holding the raw bit patterns.
"""

from __future__ import annotations

from dataclasses import dataclass

import numpy as np

DTYPES = ("f32", "f16", "bf16")
TENSOR_X, TENSOR_W, TENSOR_B = 1, 2, 3


def seed_for(workload: int, layer: int, tensor: int, gemm: int = 0) -> int:
    return 1000 * workload + 10 * layer + tensor + 100_000 * gemm


def _rng(seed: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(seed))


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round float32 to bfloat16 (round to nearest, ties to even); raw bits.

    NaN inputs map to a quiet NaN. This is the storage conversion of the
    generator, applied once when inputs are made.
    """
    a = np.ascontiguousarray(a, dtype=np.float32)
    u = a.view(np.uint32).astype(np.uint64)
    lsb = (u >> 16) & 1
    rounded = ((u + 0x7FFF + lsb) >> 16).astype(np.uint16)
    nan = np.isnan(a)
    if nan.any():
        rounded = rounded.copy()
        rounded[nan] = ((u[nan] >> 16).astype(np.uint16) | np.uint16(0x0040))
    return rounded


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """Widen raw bfloat16 bits to float32 (exact)."""
    b = np.ascontiguousarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32)


def store(values_f64: np.ndarray, dtype: str) -> np.ndarray:
    """Round float64 draws into the storage format ``dtype``."""
    f32 = np.asarray(values_f64, dtype=np.float64).astype(np.float32)
    if dtype == "f32":
        return f32
    if dtype == "f16":
        return f32.astype(np.float16)
    if dtype == "bf16":
        return f32_to_bf16_bits(f32)
    raise ValueError(f"unknown dtype {dtype!r}")


def widen(stored: np.ndarray, dtype: str) -> np.ndarray:
    """Stored values as float64 (exact widening; for checks and plots)."""
    if dtype == "bf16":
        return bf16_bits_to_f32(stored).astype(np.float64)
    return np.asarray(stored).astype(np.float64)


def normal(seed: int, shape, std: float, dtype: str) -> np.ndarray:
    return store(_rng(seed).standard_normal(size=shape) * std, dtype)


def uniform(seed: int, shape, lo: float, hi: float, dtype: str) -> np.ndarray:
    return store(_rng(seed).uniform(lo, hi, size=shape), dtype)


@dataclass
class LinearCase:
    """One linear layer's inputs in storage form.

    ``X`` is ``[M][K]``, or ``[K][M]`` for the ``"AT_*"`` layouts.  ``W`` is
    out×in ``[N][K]`` for ``"NK"``/``"AT_NK"`` and ``[K][N]`` for
    ``"KN"``/``"AT_KN"``.  ``b`` is ``None`` when the layer has no bias; ``R``,
    when given, is the residual ``[M][N]`` (output type) the result is added to.
    """

    name: str
    M: int
    N: int
    K: int
    in_dtype: str
    out_dtype: str
    layout: str
    bias: bool
    gelu: bool
    X: np.ndarray
    W: np.ndarray
    b: np.ndarray | None
    R: np.ndarray | None = None

    @property
    def flops(self) -> int:
        return 2 * self.M * self.N * self.K


# GPT-2-small linear shapes: (name, N, K, gelu) with d_model 768, d_ff 3072.
GPT2_LINEARS = (
    ("qkv", 2304, 768, False),
    ("attn_out", 768, 768, False),
    ("fc", 3072, 768, True),
    ("proj", 768, 3072, False),
)


def gpt2_weights(workload: int, layer: int, gemm: int, dtype: str):
    """Weight ``[N][K]`` and bias ``[N]`` of linear ``gemm`` of a GPT-2 layer, both ~ N(0, 0.02)."""
    _, N, K, _ = GPT2_LINEARS[gemm]
    W = normal(seed_for(workload, layer, TENSOR_W, gemm), (N, K), 0.02, dtype)
    b = normal(seed_for(workload, layer, TENSOR_B, gemm), (N,), 0.02, dtype)
    return W, b


def gpt2_activation(workload: int, layer: int, gemm: int, M: int, dtype: str):
    """Input ``[M][K]`` ~ N(0, 1) of linear ``gemm`` of a GPT-2 layer."""
    K = GPT2_LINEARS[gemm][2]
    return normal(seed_for(workload, layer, TENSOR_X, gemm), (M, K), 1.0, dtype)


def workload_fp32_linear_128x768(workload: int = 1) -> LinearCase:
    """fp32 linear, M=128, K=768, N=768, bias, no activation."""
    M, N, K = 128, 768, 768
    X = normal(seed_for(workload, 0, TENSOR_X), (M, K), 1.0, "f32")
    W = normal(seed_for(workload, 0, TENSOR_W), (N, K), 0.02, "f32")
    b = normal(seed_for(workload, 0, TENSOR_B), (N,), 0.02, "f32")
    return LinearCase("linear_128x768x768_f32", M, N, K, "f32", "f32", "NK", True, False, X, W, b)


def workload_fp16_narrow(workload: int = 2, copy: int = 0, M: int = 16, N: int = 4096,
                         K: int = 4096, dtype: str = "f16") -> LinearCase:
    """Narrow linear 16×4096×4096, X, W ~ U(-1,1)·0.05, fp16 in, fp16 out."""
    X = uniform(seed_for(workload, 0, TENSOR_X), (M, K), -0.05, 0.05, dtype)
    W = uniform(seed_for(workload, copy, TENSOR_W), (N, K), -0.05, 0.05, dtype)
    return LinearCase(f"narrow_{M}x{N}x{K}_{dtype}", M, N, K, dtype, dtype, "NK", False, False,
                      X, W, None)


def workload_gpt2_layer(workload: int = 3, M: int = 128, dtype: str = "f32", layer: int = 0):
    """The four GPT-2-small linears of one layer at M rows (bias on all, GELU on fc)."""
    cases = []
    for g, (name, N, K, gelu) in enumerate(GPT2_LINEARS):
        W, b = gpt2_weights(workload, layer, g, dtype)
        X = gpt2_activation(workload, layer, g, M, dtype)
        cases.append(LinearCase(f"{name}_{M}x{N}x{K}_{dtype}", M, N, K, dtype, dtype, "NK", True, gelu, X, W, b))
    return cases


def workload_square(workload: int = 4, n: int = 4096, dtype: str = "f32") -> LinearCase:
    """Square GEMM C = A·B, row-major A [M][K] and B [K][N], U(-1,1), no bias.

    With bfloat16 inputs the output stays float32.
    """
    A = uniform(seed_for(workload, 0, TENSOR_X), (n, n), -1.0, 1.0, dtype)
    B = uniform(seed_for(workload, 0, TENSOR_W), (n, n), -1.0, 1.0, dtype)
    return LinearCase(f"square_{n}_{dtype}", n, n, n, dtype, "f32", "KN", False, False, A, B, None)


def workload_gpt2_stack(workload: int = 5, batch: int = 64, seq: int = 128, layers: int = 12,
                        dtype: str = "f32"):
    """Batched GPT-2-small stack: ``layers`` × four linears at M = batch·seq.

    Activations are drawn independently for every GEMM (the stack is not
    chained: there is no attention or layernorm between the linears).
    """
    M = batch * seq
    out = []
    for layer in range(layers):
        out.extend(workload_gpt2_layer(workload, M, dtype, layer))
    return out


def normal_around(seed: int, shape, mean: float, std: float, dtype: str) -> np.ndarray:
    """``mean + N(0, std)`` drawn in float64 and stored like ``normal``."""
    return store(mean + _rng(seed).standard_normal(shape) * std, dtype)


def workload_gpt2_layernorm(workload: int = 7, rows: int = 8192, C: int = 768, dtype: str = "f32"):
    """LayerNorm input of the GPT-2-small stack: X [rows][C] ~ N(0, 1), gamma ~ 1 + N(0, 0.1), beta ~ N(0, 0.1)."""
    X = normal(seed_for(workload, 0, TENSOR_X), (rows, C), 1.0, dtype)
    gamma = normal_around(seed_for(workload, 0, TENSOR_W), (C,), 1.0, 0.1, dtype)
    beta = normal(seed_for(workload, 0, TENSOR_B), (C,), 0.1, dtype)
    return X, gamma, beta


def workload_gpt2_attention(workload: int = 8, B: int = 64, T: int = 128, n_head: int = 12, head_size: int = 64,
                            dtype: str = "f32"):
    """The qkv projection output [B][T][3C] ~ N(0, 1) that GPT-2-small attention reads (C = n_head * head_size)."""
    return normal(seed_for(workload, 0, TENSOR_X), (B, T, 3 * n_head * head_size), 1.0, dtype)


def gpt2_block_params(workload: int, layer: int, C: int, dtype: str) -> dict:
    """One GPT-2 block's parameters (storage arrays): weights and biases ~ N(0, 0.02) as in the linear
    workloads, layer-norm gains ~ 1 + N(0, 0.1) and shifts ~ N(0, 0.1).  Seed of parameter i (in the order
    of ``block.PARAM_NAMES``): ``seed_for(workload, layer, 10 + i)``."""
    shapes = {"ln1_g": (C,), "ln1_b": (C,), "w_qkv": (3 * C, C), "b_qkv": (3 * C,), "w_attn": (C, C),
              "b_attn": (C,), "ln2_g": (C,), "ln2_b": (C,), "w_fc": (4 * C, C), "b_fc": (4 * C,),
              "w_proj": (C, 4 * C), "b_proj": (C,)}
    out = {}
    for i, (name, shape) in enumerate(shapes.items()):
        seed = seed_for(workload, layer, 10 + i)
        if name.endswith("_g"):
            out[name] = normal_around(seed, shape, 1.0, 0.1, dtype)
        elif name.startswith("ln"):
            out[name] = normal(seed, shape, 0.1, dtype)
        else:
            out[name] = normal(seed, shape, 0.02, dtype)
    return out


TENSOR_DY, TENSOR_G = 5, 6  # output gradient and the weight gradient accumulated so far


def workload_gpt2_backward(workload: int = 6, T: int = 8192, dtype: str = "f32", layer: int = 0):
    """Backward GEMMs of the four GPT-2-small linears of one layer over T tokens.

    For each linear Y = X·Wᵀ (X [T][K], W [N][K]) and an output gradient dY
    [T][N] ~ N(0, 1): the input gradient dX = dY·W, layout ``"KN"`` with the
    weight read as stored, and the weight gradient dW = dYᵀ·X added onto the
    gradient G [N][K] ~ N(0, 0.02) accumulated so far, layout ``"AT_KN"`` with
    dY as the transposed first operand and residual G.  Returns the dX cases,
    then the dW cases, in the order of the linears.
    """
    dx, dw = [], []
    for g, (name, N, K, _) in enumerate(GPT2_LINEARS):
        W, _b = gpt2_weights(workload, layer, g, dtype)
        X = gpt2_activation(workload, layer, g, T, dtype)
        dY = normal(seed_for(workload, layer, TENSOR_DY, g), (T, N), 1.0, dtype)
        G = normal(seed_for(workload, layer, TENSOR_G, g), (N, K), 0.02, dtype)
        dx.append(LinearCase(f"{name}_dX_{T}x{K}x{N}_{dtype}", T, K, N, dtype, dtype, "KN", False, False,
                             dY, W, None))
        dw.append(LinearCase(f"{name}_dW_{N}x{K}x{T}_{dtype}", N, K, T, dtype, dtype, "AT_KN", False, False,
                             dY, X, None, G))
    return dx + dw


TENSOR_R = 4  # residual, in random_case


def random_case(seed: int, M: int, N: int, K: int, in_dtype: str = "f32", out_dtype: str | None = None,
                layout: str = "NK", bias: bool = False, gelu: bool = False,
                x_scale: float = 1.0, w_scale: float = 0.05, residual: bool = False) -> LinearCase:
    """A generic seeded case for parity tests of arbitrary shapes and all four layouts."""
    out_dtype = out_dtype or in_dtype
    xshape = (K, M) if layout.startswith("AT_") else (M, K)
    X = normal(seed * 16 + TENSOR_X, xshape, x_scale, in_dtype)
    wshape = (K, N) if layout.endswith("KN") else (N, K)
    W = normal(seed * 16 + TENSOR_W, wshape, w_scale, in_dtype)
    b = normal(seed * 16 + TENSOR_B, (N,), w_scale, in_dtype) if bias else None
    R = normal(seed * 16 + TENSOR_R, (M, N), 1.0, out_dtype) if residual else None
    return LinearCase(f"rand_{M}x{N}x{K}_{in_dtype}_{layout}{'_res' if residual else ''}", M, N, K, in_dtype,
                      out_dtype, layout, bias, gelu, X, W, b, R)


def periodic_normal(seed: int, shape, std: float, dtype: str, block=(1021, 1031)) -> np.ndarray:
    """``N(0, std)`` values of one ``block`` (prime sides) repeated over ``shape``: element (i, j) is
    block[i % 1021][j % 1031].  Operands of several GiB are drawn in seconds this way, and an address off
    by a multiple of 2^30 or 2^31 bytes still lands on a different value (the strides share no factor with
    the primes)."""
    rows, cols = shape
    b = normal(seed, (min(rows, block[0]), min(cols, block[1])), std, dtype)
    reps = (-(-rows // b.shape[0]), -(-cols // b.shape[1]))
    return np.ascontiguousarray(np.tile(b, reps)[:rows, :cols])


def large_case(seed: int, M: int, N: int, K: int, in_dtype: str, out_dtype: str | None = None,
               layout: str = "NK") -> LinearCase:
    """``random_case`` for operands of several GiB: X ~ N(0, 1) and W ~ N(0, 0.05) as periodic blocks."""
    out_dtype = out_dtype or in_dtype
    xshape = (K, M) if layout.startswith("AT_") else (M, K)
    wshape = (K, N) if layout.endswith("KN") else (N, K)
    X = periodic_normal(seed * 16 + TENSOR_X, xshape, 1.0, in_dtype)
    W = periodic_normal(seed * 16 + TENSOR_W, wshape, 0.05, in_dtype)
    return LinearCase(f"large_{M}x{N}x{K}_{in_dtype}_{layout}", M, N, K, in_dtype, out_dtype, layout, False, False,
                      X, W, None, None)
