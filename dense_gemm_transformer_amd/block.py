"""A GPT-2 transformer block forward pass composed from the library's entry points.

    x <- x + attn_out(attention(qkv(ln1(x))))
    x <- x + proj(gelu(fc(ln2(x))))

Seven launches per block on one stream: two layer normalisations, the qkv
projection (bias), fused causal attention, the attention output projection
with the residual accumulated into x (the fused residual epilogue), fc with
bias and tanh-GELU, and proj with the residual accumulated into x.  This is
the layer that "Optimizing a GPT-2-class transformer on a GPU" optimises (its
"layer forward"), without embeddings, final normalisation or logits.

Marshalling only: torch supplies device memory and the stream, every step is
a kernel of ``libtlgemm.so``.  Buffers and plans are made once per block and
reused by every forward call, so a forward allocates nothing.
"""

from __future__ import annotations

from dataclasses import dataclass

from . import layer, tlgemm

PARAM_NAMES = ("ln1_g", "ln1_b", "w_qkv", "b_qkv", "w_attn", "b_attn", "ln2_g", "ln2_b", "w_fc", "b_fc", "w_proj",
               "b_proj")


def param_shapes(C: int) -> dict:
    """Shapes of one block's parameters; weights are stored out x in, as PyTorch stores them."""
    return {"ln1_g": (C,), "ln1_b": (C,), "w_qkv": (3 * C, C), "b_qkv": (3 * C,), "w_attn": (C, C), "b_attn": (C,),
            "ln2_g": (C,), "ln2_b": (C,), "w_fc": (4 * C, C), "b_fc": (4 * C,), "w_proj": (C, 4 * C),
            "b_proj": (C,)}


@dataclass
class BlockShape:
    B: int
    T: int
    C: int
    n_head: int
    dtype: str

    @property
    def M(self) -> int:
        return self.B * self.T

    def flops(self) -> int:
        """GEMM flops plus the two attention products (causal: T(T+1)/2 key-query pairs per head)."""
        M, C = self.M, self.C
        gemm = 2 * M * C * (3 * C + C + 4 * C + 4 * C)
        att = 2 * 2 * self.B * self.n_head * (C // self.n_head) * self.T * (self.T + 1) // 2
        return gemm + att


class GPT2Block:
    """One block with its parameters (device tensors), plans and work buffers."""

    def __init__(self, shape: BlockShape, params: dict, eps: float = 1e-5):
        import torch

        self.s = shape
        self.p = params
        self.eps = eps
        M, C, dt = shape.M, shape.C, shape.dtype
        dev = params["w_qkv"].device
        tdt = tlgemm.torch_dtype(dt)
        mk = lambda N, K, **kw: tlgemm.Plan.create(M, N, K, dt, dt, "NK", bias=True, **kw)
        self.plans = {"qkv": mk(3 * C, C), "attn": mk(C, C, residual=True), "fc": mk(4 * C, C, gelu=True),
                      "proj": mk(C, 4 * C, residual=True)}
        self.ws = {k: torch.zeros(max(p.workspace_size, 1), dtype=torch.uint8, device=dev)
                   for k, p in self.plans.items()}
        self.h = torch.empty((M, C), dtype=tdt, device=dev)
        self.qkv = torch.empty((M, 3 * C), dtype=tdt, device=dev)
        self.att = torch.empty((M, C), dtype=tdt, device=dev)
        self.fc = torch.empty((M, 4 * C), dtype=tdt, device=dev)
        # the workspaces were zero-filled on the current stream; forward may run on another one
        torch.cuda.synchronize(dev)

    def _gemm(self, name, X, W, b, Y, stream):
        p = self.plans[name]
        ws = self.ws[name]
        p.run_ptrs(X.data_ptr(), W.data_ptr(), b.data_ptr(), Y.data_ptr(),
                   ws.data_ptr() if p.workspace_size else 0, p.workspace_size, stream)

    def forward(self, x, stream: int) -> None:
        """x [B*T][C] (device, the block's dtype) is updated in place on ``stream`` (a raw hipStream_t)."""
        s, p, dt = self.s, self.p, self.s.dtype
        M, C = s.M, s.C
        layer.tlg_layernorm(x.data_ptr(), p["ln1_g"].data_ptr(), p["ln1_b"].data_ptr(), self.h.data_ptr(), 0, 0,
                            M, C, self.eps, dt, stream)
        self._gemm("qkv", self.h, p["w_qkv"], p["b_qkv"], self.qkv, stream)
        layer.tlg_attention(self.qkv.data_ptr(), self.att.data_ptr(), 0, s.B, s.T, s.n_head, C // s.n_head, dt,
                            True, stream)
        self._gemm("attn", self.att, p["w_attn"], p["b_attn"], x, stream)  # x += attn_out(att)
        layer.tlg_layernorm(x.data_ptr(), p["ln2_g"].data_ptr(), p["ln2_b"].data_ptr(), self.h.data_ptr(), 0, 0,
                            M, C, self.eps, dt, stream)
        self._gemm("fc", self.h, p["w_fc"], p["b_fc"], self.fc, stream)
        self._gemm("proj", self.fc, p["w_proj"], p["b_proj"], x, stream)  # x += proj(gelu(fc))
