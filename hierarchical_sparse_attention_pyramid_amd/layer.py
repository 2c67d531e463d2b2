"""Autograd wrapper and projected attention block around the Lighthouse layer.

The layer replaces causal scaled-dot-product attention inside an ordinary
attention block (gist.science technical summary, §2.C: the attention on the
gathered subsequence is the stock kernel; the layer drops into existing
training flows).  Gradients flow from the block output back through the
scatter, the attention and the gather into the projected queries, keys and
values, and from there into the projection weights; the selection receives
none (§2.B).

Every step of the layer runs in liblighthouse.so (lh_forward / lh_backward);
the projections are plain dense GEMMs (torch, i.e. hipBLASLt / rocBLAS).
Projections are bias-free and head-major: columns h*d .. h*d+d-1 of the
projected queries belong to head h (likewise keys, values, and the rows of
the output projection's input).
"""
from __future__ import annotations

import torch

from . import binding


class LighthouseFunction(torch.autograd.Function):
    """out = Lighthouse(q, k, v) on [B, H, N, d] tensors; backward via lh_backward."""

    @staticmethod
    def forward(ctx, q, k, v, p: int, L: int, S: int):
        q, k, v = (t.contiguous() for t in (q, k, v))
        out, bufs, shape = binding.forward(q, k, v, p, L, S)
        ctx.lh = (bufs, shape)
        return out

    @staticmethod
    def backward(ctx, dout):
        bufs, shape = ctx.lh
        dq, dk, dv = binding.backward(shape, dout.contiguous(), bufs)
        return dq, dk, dv, None, None, None


def lighthouse(q, k, v, p: int, L: int, S: int):
    """Differentiable Lighthouse attention on [B, H, N, d] (fp32 or bf16)."""
    return LighthouseFunction.apply(q, k, v, p, L, S)


class LighthouseAttention(torch.nn.Module):
    """y = (Lighthouse(x Wq^T, x Wk^T, x Wv^T) merged over heads) Wo^T.

    x: [B, N, D]; Wq, Wk, Wv: [H*d, D]; Wo: [D, H*d]."""

    def __init__(self, d_model: int, heads: int, head_dim: int, p: int, L: int, S: int,
                 dtype=torch.bfloat16, device="cuda"):
        super().__init__()
        self.H, self.d, self.p, self.L, self.S = heads, head_dim, p, L, S
        kw = dict(dtype=dtype, device=device)
        inner = heads * head_dim
        self.wq = torch.nn.Parameter(torch.empty(inner, d_model, **kw))
        self.wk = torch.nn.Parameter(torch.empty(inner, d_model, **kw))
        self.wv = torch.nn.Parameter(torch.empty(inner, d_model, **kw))
        self.wo = torch.nn.Parameter(torch.empty(d_model, inner, **kw))
        for w in (self.wq, self.wk, self.wv, self.wo):
            torch.nn.init.normal_(w, std=d_model ** -0.5)

    def _heads(self, x2, w, B, N):
        # [B*N, D] @ [D, H*d] -> [B, H, N, d] (2-D GEMM; heads made contiguous)
        y = torch.nn.functional.linear(x2, w)
        return y.view(B, N, self.H, self.d).transpose(1, 2).contiguous()

    def forward(self, x):
        B, N, D = x.shape
        x2 = x.reshape(B * N, D)
        q, k, v = (self._heads(x2, w, B, N) for w in (self.wq, self.wk, self.wv))
        o = lighthouse(q, k, v, self.p, self.L, self.S)
        o2 = o.transpose(1, 2).reshape(B * N, self.H * self.d)
        return torch.nn.functional.linear(o2, self.wo).view(B, N, D)
