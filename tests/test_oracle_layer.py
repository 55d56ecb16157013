"""Pins of the oracle's layer normalisation and attention (no GPU): hand-worked values, torch's float64
library routines on the CPU, closed forms and invariants that a dropped term, a wrong index or a missing
mask would break."""

import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
from dense_gemm_transformer_amd import inputs

GOLDEN = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "layer_hand_examples.json")))


def _ln_torch(X, g, b, eps):
    return torch.nn.functional.layer_norm(torch.from_numpy(X), (X.shape[1],), torch.from_numpy(g),
                                          torch.from_numpy(b), eps).numpy()


@pytest.mark.parametrize("ex", range(len(GOLDEN["layernorm"])))
def test_layernorm_hand_examples(ex):
    e = GOLDEN["layernorm"][ex]
    f = lambda k: np.array(e[k], dtype=np.float32)
    Y, mean, rstd = oracle.layernorm(f("x")[None], f("gamma"), f("beta"), eps=e["eps"])
    assert np.allclose(Y[0], e["y"], rtol=0, atol=1e-15)
    assert mean[0] == e["mean"] and abs(rstd[0] - e["rstd"]) <= 1e-15


@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
@pytest.mark.parametrize("rows,C", [(1, 1), (3, 7), (17, 768), (5, 1000)])
def test_layernorm_matches_torch_float64(dtype, rows, C):
    X = inputs.normal(11, (rows, C), 1.0, dtype) if dtype == "f32" else inputs.normal(11, (rows, C), 1.0, dtype)
    g = inputs.normal(12, (C,), 0.2, dtype)
    b = inputs.normal(13, (C,), 0.2, dtype)
    Y, mean, rstd = oracle.layernorm(X, g, b, dtype=dtype, eps=1e-5)
    Xw, gw, bw = (inputs.widen(a, dtype) for a in (X, g, b))
    ref = _ln_torch(Xw, gw, bw, 1e-5)
    assert np.max(np.abs(Y - ref)) <= 1e-12 * max(1.0, np.max(np.abs(ref)))
    assert np.allclose(mean, Xw.mean(axis=1), rtol=0, atol=1e-13)
    assert np.allclose(rstd, 1.0 / np.sqrt(Xw.var(axis=1) + 1e-5), rtol=1e-12, atol=0)


def test_layernorm_constant_row_gives_beta_exactly():
    X = np.full((4, 768), 0.5, dtype=np.float32)
    g = inputs.normal(21, (768,), 1.0, "f32")
    b = inputs.normal(22, (768,), 1.0, "f32")
    Y, mean, rstd = oracle.layernorm(X, g, b, eps=1e-5)
    assert np.array_equal(Y, np.broadcast_to(b.astype(np.float64), Y.shape)) and np.all(mean == 0.5)


def test_layernorm_shift_and_scale_invariance_and_unit_moments():
    # multiples of 1/1024 in [-4, 4): 4x + 8 is exact in fp32
    X = (np.random.default_rng(31).integers(-4096, 4096, (9, 300)) / 1024.0).astype(np.float32)
    ones, zeros = np.ones(300, np.float32), np.zeros(300, np.float32)
    Y, _, _ = oracle.layernorm(X, ones, zeros, eps=0.0)
    Y2, _, _ = oracle.layernorm((X * 4.0 + 8.0).astype(np.float32), ones, zeros, eps=0.0)  # exact in fp32
    assert np.max(np.abs(Y - Y2)) <= 1e-12
    assert np.max(np.abs(Y.mean(axis=1))) <= 1e-13 and np.max(np.abs((Y ** 2).mean(axis=1) - 1.0)) <= 1e-12


def _split(qkv_w, n_head):
    B, T, C3 = qkv_w.shape
    C = C3 // 3
    hs = C // n_head
    f = lambda blk: torch.from_numpy(np.ascontiguousarray(
        qkv_w[:, :, blk * C:(blk + 1) * C].reshape(B, T, n_head, hs).transpose(0, 2, 1, 3)))
    return f(0), f(1), f(2)


def test_attention_hand_example():
    e = GOLDEN["attention"][0]
    out, lse = oracle.attention(np.array(e["qkv"], dtype=np.float32), e["n_head"])
    assert np.allclose(out, e["out"], rtol=0, atol=1e-15) and np.allclose(lse, e["lse"], rtol=0, atol=1e-15)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("B,T,NH,HS", [(1, 1, 1, 4), (2, 7, 3, 8), (1, 33, 2, 64)])
def test_attention_matches_torch_float64(dtype, causal, B, T, NH, HS):
    qkv = inputs.normal(41, (B, T, 3 * NH * HS), 0.7, dtype)
    out, lse = oracle.attention(qkv, NH, dtype=dtype, causal=causal)
    q, k, v = _split(inputs.widen(qkv, dtype), NH)
    ref = torch.nn.functional.scaled_dot_product_attention(q, k, v, is_causal=causal)
    ref = ref.transpose(1, 2).reshape(B, T, NH * HS).numpy()
    assert np.max(np.abs(out - ref)) <= 1e-12
    s = (q @ k.transpose(-1, -2)) / math.sqrt(HS)
    if causal:
        s = s.masked_fill(torch.triu(torch.ones(T, T, dtype=torch.bool), 1), float("-inf"))
    assert np.max(np.abs(lse - torch.logsumexp(s, dim=-1).numpy())) <= 1e-12


def test_attention_single_position_returns_its_value_row():
    qkv = inputs.normal(51, (3, 1, 3 * 2 * 16), 1.0, "f32")
    out, lse = oracle.attention(qkv, 2)
    C = 32
    assert np.array_equal(out, qkv[:, :, 2 * C:].astype(np.float64))
    q, k = qkv[:, 0, :C].astype(np.float64), qkv[:, 0, C:2 * C].astype(np.float64)
    s = (q.reshape(3, 2, 16) * k.reshape(3, 2, 16)).sum(-1) / 4.0
    assert np.allclose(lse[:, :, 0], s, rtol=0, atol=1e-14)


def test_attention_identical_keys_average_the_values():
    T, NH, HS = 9, 2, 8
    C = NH * HS
    qkv = inputs.normal(61, (2, T, 3 * C), 1.0, "f32")
    qkv[:, :, C:2 * C] = qkv[:, :1, C:2 * C]  # every key equals the first
    out, lse = oracle.attention(qkv, NH)
    v = qkv[:, :, 2 * C:].astype(np.float64)
    want = np.cumsum(v, axis=1) / np.arange(1, T + 1)[None, :, None]
    assert np.max(np.abs(out - want)) <= 1e-13
    q = qkv[:, :, :C].astype(np.float64).reshape(2, T, NH, HS)
    k0 = qkv[:, 0, C:2 * C].astype(np.float64).reshape(2, 1, NH, HS)
    s = ((q * k0).sum(-1) / math.sqrt(HS)).transpose(0, 2, 1)  # [B][NH][T]: every key scores the same
    assert np.allclose(lse - s, np.log(np.arange(1, T + 1))[None, None, :], rtol=0, atol=1e-13)


def test_attention_is_causal_and_rows_sum_to_one():
    T, NH, HS = 12, 3, 4
    C = NH * HS
    qkv = inputs.normal(71, (2, T, 3 * C), 1.0, "f32")
    out, lse = oracle.attention(qkv, NH)
    later = qkv.copy()
    later[:, 6:, :] = inputs.normal(72, (2, T - 6, 3 * C), 1.0, "f32")
    out2, lse2 = oracle.attention(later, NH)
    assert np.array_equal(out[:, :6], out2[:, :6]) and np.array_equal(lse[:, :, :6], lse2[:, :, :6])
    assert not np.array_equal(out[:, 6:], out2[:, 6:])
    q, k, _ = _split(qkv.astype(np.float64), NH)
    s = ((q @ k.transpose(-1, -2)) / 2.0).numpy()
    for i in range(T):
        assert np.allclose(np.exp(s[:, :, i, :i + 1] - lse[:, :, i, None]).sum(-1), 1.0, rtol=0, atol=1e-13)


def test_attention_head_offsets():
    """Swapping two heads' query, key and value columns swaps their outputs exactly."""
    T, NH, HS = 5, 3, 4
    C = NH * HS
    qkv = inputs.normal(81, (1, T, 3 * C), 1.0, "f32")
    out, lse = oracle.attention(qkv, NH)
    sw = qkv.copy()
    for blk in range(3):
        a, b = blk * C, blk * C + 2 * HS  # heads 0 and 2
        sw[:, :, a:a + HS], sw[:, :, b:b + HS] = qkv[:, :, b:b + HS], qkv[:, :, a:a + HS]
    out2, lse2 = oracle.attention(sw, NH)
    assert np.array_equal(out2[:, :, :HS], out[:, :, 2 * HS:]) and np.array_equal(out2[:, :, 2 * HS:], out[:, :, :HS])
    assert np.array_equal(lse2[:, 0], lse[:, 2]) and np.array_equal(lse2[:, 1], lse[:, 1])
