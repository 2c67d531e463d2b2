"""Plain CPU oracle of the Lighthouse layer inside an attention block with
input and output projections (forward and backward).

TEST INFRASTRUCTURE ONLY.  Only the tests may import this module.  It shares
no code with the HIP library and is never called on the product path.

Source: gist.science technical summary, §2.B and §2.C (and the bitsgeniais
post, phase 3): the layer is a drop-in replacement for causal attention in
an attention block, and its gradient flows through the scatter, the
attention and the gather into the projected queries, keys and values (hence
into the projection weights); the selection receives no gradient.

Reading R13 (the pages do not spell the block out): bias-free linear
projections, head-major -- columns h*d .. h*d+d-1 of X Wq^T are head h's
queries (likewise keys and values) -- and Y = concat_h(out_h) Wo^T.

Precision follows the layer oracle: each step is computed in float64 from
its stored inputs and rounded once to the storage type at the points where
the block stores a tensor (the projected q, k, v; the layer output; the
gradient handed to the layer; the layer's dq, dk, dv; the block output and
every gradient the block returns).
"""
from __future__ import annotations

import numpy as np

from . import lighthouse as O


def _heads(a: np.ndarray, H: int) -> list:
    N, HD = a.shape
    d = HD // H
    return [a[:, h * d:(h + 1) * d] for h in range(H)]


def projected_forward(x, wq, wk, wv, wo, H: int, p: int, L: int, S: int, dtype: str,
                      mode: str = "span"):
    """One batch element: x [N, D], wq/wk/wv [H*d, D], wo [D, H*d], all stored
    in `dtype`; `mode` is the layer's scatter reading ("span" or "causal").
    Returns (y stored, cache for the backward)."""
    x64, wq64, wk64, wv64, wo64 = (O.to_f64(a, dtype) for a in (x, wq, wk, wv, wo))
    q, k, v = (O.round_to(x64 @ w.T, dtype) for w in (wq64, wk64, wv64))
    fwds = [O.forward_head(qh, kh, vh, p, L, S, dtype, mode)
            for qh, kh, vh in zip(_heads(q, H), _heads(k, H), _heads(v, H))]
    o = np.concatenate([O.to_f64(f["out"], dtype) for f in fwds], axis=1)
    y = O.round_to(o @ wo64.T, dtype)
    cache = dict(x64=x64, w64=(wq64, wk64, wv64, wo64), o=o, fwds=fwds, H=H, p=p, L=L, mode=mode)
    return y, cache


def projected_backward(dy, cache: dict, dtype: str):
    """Gradients (dx, dwq, dwk, dwv, dwo) of sum(y * dy), each rounded once to
    the storage type."""
    x64, (wq64, wk64, wv64, wo64), o = cache["x64"], cache["w64"], cache["o"]
    H, p, L = cache["H"], cache["p"], cache["L"]
    dy64 = O.to_f64(dy, dtype)
    dwo = dy64.T @ o
    do = O.round_to(dy64 @ wo64, dtype)                 # the gradient handed to the layer
    parts = [O.backward_head(dh, f, p, L, dtype) for dh, f in zip(_heads(do, H), cache["fwds"])]
    dq, dk, dv = (np.concatenate([O.to_f64(O.round_to(g[i], dtype), dtype) for g in parts], axis=1)
                  for i in range(3))
    dwq, dwk, dwv = (g.T @ x64 for g in (dq, dk, dv))
    dx = dq @ wq64 + dk @ wk64 + dv @ wv64
    return tuple(O.round_to(a, dtype) for a in (dx, dwq, dwk, dwv, dwo))


def projected_forward_fixed(x, wq, wk, wv, wo, fwds, H: int, p: int, L: int, mode: str = "span"):
    """float64 block output with every head's selection held fixed (the
    selections of `fwds`), for gradient checks."""
    q, k, v = (x @ w.T for w in (wq, wk, wv))
    o = np.concatenate([O.forward_fixed(qh, kh, vh, f["sub_idx"], f["pos"], p, L, mode)
                        for qh, kh, vh, f in zip(_heads(q, H), _heads(k, H), _heads(v, H), fwds)],
                       axis=1)
    return o @ wo.T
