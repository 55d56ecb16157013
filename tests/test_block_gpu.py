"""A GPT-2 block composed from the library's entry points against the same composition of oracle stages.

Each oracle stage is fed the previous stage's result rounded to the storage type the GPU keeps between
kernels (fp32 or bf16), so the comparison measures the kernels, not the rounding the pipeline itself
prescribes."""

import numpy as np
import pytest
import torch

import oracle
from dense_gemm_transformer_amd import block, inputs
from gpu_helpers import TOL, to_device, to_f64

pytestmark = pytest.mark.gpu


def _oracle_block(x, P, B, T, n_head, dtype):
    st = lambda a: inputs.store(a, dtype)  # the storage the GPU keeps between kernels
    h, _, _ = oracle.layernorm(x, P["ln1_g"], P["ln1_b"], dtype=dtype)
    qkv = oracle.linear(st(h), P["w_qkv"], P["b_qkv"], dtype=dtype)
    att, _ = oracle.attention(st(qkv).reshape(B, T, -1), n_head, dtype=dtype)
    x1 = oracle.linear(st(att.reshape(B * T, -1)), P["w_attn"], P["b_attn"], dtype=dtype, residual=x)
    h2, _, _ = oracle.layernorm(st(x1), P["ln2_g"], P["ln2_b"], dtype=dtype)
    f = oracle.linear(st(h2), P["w_fc"], P["b_fc"], dtype=dtype, gelu=True)
    return oracle.linear(st(f), P["w_proj"], P["b_proj"], dtype=dtype, residual=st(x1))


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("B,T", [(2, 64), (1, 128)])
def test_block_forward_matches_the_oracle_composition(dtype, B, T):
    C, NH = 768, 12
    P = inputs.gpt2_block_params(9, 0, C, dtype)
    x = inputs.normal(inputs.seed_for(9, 0, 1), (B * T, C), 1.0, dtype)
    blk = block.GPT2Block(block.BlockShape(B, T, C, NH, dtype), {k: to_device(v, dtype) for k, v in P.items()})
    xd = to_device(x, dtype)
    blk.forward(xd, torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    ref = _oracle_block(x, P, B, T, NH, dtype)
    err = oracle.normalized_error(to_f64(xd), ref)
    assert err <= TOL[dtype], err


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_block_forward_replays_bitwise_from_a_graph(dtype):
    """Two blocks captured once (after a device copy of the input into place) replay bitwise equal to the
    eager forward, with eager work on the same buffers between replays."""
    B, T, C, NH = 2, 64, 768, 12
    blocks = [block.GPT2Block(block.BlockShape(B, T, C, NH, dtype),
                              {k: to_device(v, dtype) for k, v in inputs.gpt2_block_params(9, li, C, dtype).items()})
              for li in range(2)]
    x0 = to_device(inputs.normal(inputs.seed_for(9, 0, 1), (B * T, C), 1.0, dtype), dtype)
    x = x0.clone()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        for blk in blocks:
            blk.forward(x, s.cuda_stream)
    s.synchronize()
    want = x.clone()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        x.copy_(x0)
        for blk in blocks:
            blk.forward(x, s.cuda_stream)
    for rep in range(3):
        x.fill_(float("nan"))
        with torch.cuda.stream(s):  # eager work on the same buffers between replays
            blocks[rep % 2].forward(x0.clone(), s.cuda_stream)
        s.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(x, want), f"replay {rep}"
