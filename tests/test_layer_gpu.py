"""Layer normalisation and fused attention through the C ABI against the oracle, element by element."""

import numpy as np
import pytest
import torch

import oracle
from dense_gemm_transformer_amd import inputs, layer
from gpu_helpers import TOL, to_device, to_f64

pytestmark = pytest.mark.gpu
normalized_error = oracle.normalized_error


def _ln_check(rows, C, dtype, seed=0, eps=1e-5):
    X = inputs.normal(seed * 8 + 1, (rows, C), 1.0, dtype)
    g = inputs.normal_around(seed * 8 + 2, (C,), 1.0, 0.1, dtype)
    b = inputs.normal(seed * 8 + 3, (C,), 0.1, dtype)
    Y, mean, rstd = layer.layernorm(*(to_device(a, dtype) for a in (X, g, b)), eps=eps, stats=True)
    torch.cuda.synchronize()
    ref, rmean, rrstd = oracle.layernorm(X, g, b, dtype=dtype, eps=eps)
    err = normalized_error(to_f64(Y), ref)
    assert err <= TOL[dtype], (rows, C, dtype, err)
    assert np.max(np.abs(mean.cpu().numpy() - rmean)) <= 1e-5 * max(1.0, np.max(np.abs(rmean)))
    assert np.max(np.abs(rstd.cpu().numpy() / rrstd - 1.0)) <= 1e-5
    return err


@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
def test_layernorm_shapes(dtype):
    # odd rows (a half-empty last workgroup), odd C (unequal halves, scalar path), vector paths, the limit
    for rows, C in [(1, 1), (3, 7), (5, 768), (17, 1000), (2, 2), (4, 6), (3, 4096), (33, 1600), (9, 4000)]:
        _ln_check(rows, C, dtype, seed=rows + C)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_layernorm_gpt2_stack_input(dtype):
    X, g, b = inputs.workload_gpt2_layernorm(dtype=dtype)
    Y = layer.layernorm(*(to_device(a, dtype) for a in (X, g, b)))
    torch.cuda.synchronize()
    ref, _, _ = oracle.layernorm(X, g, b, dtype=dtype)
    assert normalized_error(to_f64(Y), ref) <= TOL[dtype]


def test_layernorm_constant_row_gives_beta():
    X = np.full((4, 768), 0.5, dtype=np.float32)
    g = inputs.normal(5, (768,), 1.0, "f32")
    b = inputs.normal(6, (768,), 1.0, "f32")
    Y = layer.layernorm(*(to_device(a, "f32") for a in (X, g, b)))
    assert torch.equal(Y.cpu(), torch.from_numpy(np.broadcast_to(b, (4, 768)).copy()))


def _att_check(B, T, NH, dtype, causal=True, seed=0):
    qkv = inputs.normal(seed * 8 + 4, (B, T, 3 * NH * 64), 1.0, dtype)
    out, lse = layer.attention(to_device(qkv, dtype), NH, causal=causal, with_lse=True)
    torch.cuda.synchronize()
    ref, rlse = oracle.attention(qkv, NH, dtype=dtype, causal=causal)
    err = normalized_error(to_f64(out), ref)
    assert err <= TOL[dtype], (B, T, NH, dtype, causal, err)
    assert np.max(np.abs(lse.cpu().numpy() - rlse)) <= 1e-4 * max(1.0, np.max(np.abs(rlse)))
    return err


@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
@pytest.mark.parametrize("causal", [True, False], ids=["causal", "full"])
def test_attention_shapes(dtype, causal):
    # one position; ragged key blocks; one and several query blocks; the 256 limit
    for B, T, NH in [(1, 1, 1), (2, 7, 3), (2, 33, 2), (1, 128, 12), (1, 129, 2), (2, 256, 2)]:
        _att_check(B, T, NH, dtype, causal, seed=B * 1000 + T + NH)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_attention_gpt2_stack_input(dtype):
    qkv = inputs.workload_gpt2_attention(dtype=dtype)
    out = layer.attention(to_device(qkv, dtype), 12)
    torch.cuda.synchronize()
    ref, _ = oracle.attention(qkv, 12, dtype=dtype)
    assert normalized_error(to_f64(out), ref) <= TOL[dtype]


def test_attention_is_causal_on_the_gpu():
    qkv = inputs.normal(91, (2, 64, 3 * 2 * 64), 1.0, "f32")
    a = layer.attention(to_device(qkv, "f32"), 2).cpu()
    later = qkv.copy()
    later[:, 40:] = inputs.normal(92, (2, 24, 3 * 2 * 64), 1.0, "f32")
    b = layer.attention(to_device(later, "f32"), 2).cpu()
    assert torch.equal(a[:, :40], b[:, :40]) and not torch.equal(a[:, 40:], b[:, 40:])
