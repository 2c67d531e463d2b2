"""Autograd wrapper and projected attention block around the Lighthouse layer.

The layer replaces causal scaled-dot-product attention inside an ordinary
attention block (gist.science technical summary, §2.C: the attention on the
gathered subsequence is the stock kernel; the layer drops into existing
training flows).  Gradients flow from the block output back through the
scatter, the attention and the gather into the projected queries, keys and
values, and from there into the projection weights; the selection receives
none (§2.B).

Scatter reading.  `scatter="causal"` (the default here) sends each entry's
output to the tokens from its end token on, so no output depends on a later
token once the selection is fixed (bitsgeniais phase 4: the scatter keeps
causality).  `scatter="span"` broadcasts an entry's output over its whole
span: every token except the last of its coarsest span then reads later
tokens (up to p^(L-1) - 1 of them), which a language model in training
would use to see the tokens it predicts.  The joint top-K looks at the whole
sequence in either reading (a discrete dependence with no gradient).

Every step of the layer runs in liblighthouse.so (lh_forward / lh_backward);
the projections are plain dense GEMMs (torch, i.e. hipBLASLt / rocBLAS).
Projections are bias-free and head-major: columns h*d .. h*d+d-1 of the
projected queries belong to head h (likewise keys, values, and the rows of
the output projection's input).

The block keeps activations token-major: one GEMM projects x to a packed
[B*N, 3*H*d] buffer, the layer reads q, k, v as strided [B,H,N,d] views of
it and writes its output token-major, and its backward writes dq, dk, dv
into one packed gradient buffer.  No layout copies run on either side of
the layer, the gradient of x is one GEMM over the packed gradient, and the
weight gradients of the three input projections are one GEMM.
"""
from __future__ import annotations

import torch

from . import binding


class LighthouseFunction(torch.autograd.Function):
    """out = Lighthouse(q, k, v) on [B, H, N, d] tensors (strided views with a
    contiguous last dimension and one common layout are used in place);
    backward via lh_backward."""

    @staticmethod
    def forward(ctx, q, k, v, p: int, L: int, S: int, scatter: str):
        out, bufs, shape = binding.forward(q, k, v, p, L, S, scatter=scatter)
        ctx.lh = (bufs, shape)
        return out

    @staticmethod
    def backward(ctx, dout):
        bufs, shape = ctx.lh
        dq, dk, dv = binding.backward(shape, dout, bufs)
        return dq, dk, dv, None, None, None, None


def lighthouse(q, k, v, p: int, L: int, S: int, scatter: str = "causal"):
    """Differentiable Lighthouse attention on [B, H, N, d] (fp32 or bf16);
    scatter: "causal" or "span" (see the module docstring)."""
    return LighthouseFunction.apply(q, k, v, p, L, S, scatter)


def _heads(t2, B: int, N: int, H: int, d: int, part: int, parts: int):
    """[B,H,N,d] view of columns part*H*d .. (part+1)*H*d of a [B*N, parts*H*d]
    token-major buffer."""
    return t2.view(B, N, parts, H, d)[:, :, part].permute(0, 2, 1, 3)


class LighthousePackedFunction(torch.autograd.Function):
    """o2 [B*N, H*d] = Lighthouse on the q, k, v column blocks of a packed
    qkv2 [B*N, 3*H*d], both token-major; the gradient is one packed buffer."""

    @staticmethod
    def forward(ctx, qkv2, B: int, N: int, H: int, d: int, p: int, L: int, S: int, scatter: str):
        qkv2 = qkv2.contiguous()
        q, k, v = (_heads(qkv2, B, N, H, d, i, 3) for i in range(3))
        o2 = torch.empty(B * N, H * d, dtype=qkv2.dtype, device=qkv2.device)
        _, bufs, shape = binding.forward(q, k, v, p, L, S, out=_heads(o2, B, N, H, d, 0, 1),
                                         scatter=scatter)
        ctx.lh = (bufs, shape, B, N, H, d)
        return o2

    @staticmethod
    def backward(ctx, do2):
        bufs, shape, B, N, H, d = ctx.lh
        do2 = do2.contiguous()
        dqkv2 = torch.empty(B * N, 3 * H * d, dtype=do2.dtype, device=do2.device)
        binding.backward(shape, _heads(do2, B, N, H, d, 0, 1), bufs,
                         *(_heads(dqkv2, B, N, H, d, i, 3) for i in range(3)))
        return dqkv2, None, None, None, None, None, None, None, None


class LighthouseAttention(torch.nn.Module):
    """y = (Lighthouse(x Wq^T, x Wk^T, x Wv^T) merged over heads) Wo^T.

    x: [B, N, D]; Wq, Wk, Wv: [H*d, D]; Wo: [D, H*d].  scatter: "causal"
    (default; the drop-in for causal attention) or "span"."""

    def __init__(self, d_model: int, heads: int, head_dim: int, p: int, L: int, S: int,
                 dtype=torch.bfloat16, device="cuda", scatter: str = "causal"):
        super().__init__()
        self.H, self.d, self.p, self.L, self.S = heads, head_dim, p, L, S
        self.scatter = scatter
        kw = dict(dtype=dtype, device=device)
        inner = heads * head_dim
        self.wq = torch.nn.Parameter(torch.empty(inner, d_model, **kw))
        self.wk = torch.nn.Parameter(torch.empty(inner, d_model, **kw))
        self.wv = torch.nn.Parameter(torch.empty(inner, d_model, **kw))
        self.wo = torch.nn.Parameter(torch.empty(d_model, inner, **kw))
        for w in (self.wq, self.wk, self.wv, self.wo):
            torch.nn.init.normal_(w, std=d_model ** -0.5)

    def forward(self, x):
        B, N, D = x.shape
        x2 = x.reshape(B * N, D)
        # one GEMM for the three input projections: [B*N, 3*H*d], token-major
        qkv2 = torch.nn.functional.linear(x2, torch.cat((self.wq, self.wk, self.wv)))
        o2 = LighthousePackedFunction.apply(qkv2, B, N, self.H, self.d, self.p, self.L, self.S,
                                            self.scatter)
        return torch.nn.functional.linear(o2, self.wo).view(B, N, D)
