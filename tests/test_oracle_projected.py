"""Pins of the attention-block oracle (oracle/projected.py): the layer with
its input and output projections."""
from __future__ import annotations

import numpy as np
import pytest
import torch

from oracle import lighthouse as O
from oracle import projected as P


def rng(seed):
    return np.random.default_rng(seed)


@pytest.mark.parametrize("mode", O.SCATTER_MODES)
def test_block_backward_matches_finite_differences(mode):
    """Every head's selection held fixed: central differences of sum(y * dy)
    with respect to the block input and all four projection weights."""
    r = rng(31)
    N, D, H, d, p, L, S = 16, 6, 2, 4, 2, 3, 9
    x = r.standard_normal((N, D))
    wq, wk, wv = (r.standard_normal((H * d, D)) / np.sqrt(D) for _ in range(3))
    wo = r.standard_normal((D, H * d)) / np.sqrt(H * d)
    dy = r.standard_normal((N, D))
    y, cache = P.projected_forward(x, wq, wk, wv, wo, H, p, L, S, "f64", mode)
    grads = P.projected_backward(dy, cache, "f64")
    np.testing.assert_allclose(
        P.projected_forward_fixed(x, wq, wk, wv, wo, cache["fwds"], H, p, L, mode), y, atol=1e-12)
    args = [x, wq, wk, wv, wo]
    h = 1e-6
    for which, g in enumerate(grads):
        for idx in np.ndindex(*args[which].shape):
            a = [t.copy() for t in args]
            a[which][idx] += h
            fp = (P.projected_forward_fixed(*a, cache["fwds"], H, p, L, mode) * dy).sum()
            a[which][idx] -= 2 * h
            fm = (P.projected_forward_fixed(*a, cache["fwds"], H, p, L, mode) * dy).sum()
            assert abs((fp - fm) / (2 * h) - g[idx]) < 1e-6 * (1 + abs(g[idx])), (which, idx)


def test_block_degenerate_matches_torch_autograd():
    """L = 1 (every token is its own entry, S = N): the block is dense causal
    attention between the projections."""
    r = rng(32)
    N, D, H, d = 24, 10, 2, 4
    x = r.standard_normal((N, D))
    wq, wk, wv = (r.standard_normal((H * d, D)) for _ in range(3))
    wo = r.standard_normal((D, H * d))
    dy = r.standard_normal((N, D))
    y, cache = P.projected_forward(x, wq, wk, wv, wo, H, 2, 1, N, "f64")
    mine = P.projected_backward(dy, cache, "f64")
    t = [torch.tensor(a, requires_grad=True) for a in (x, wq, wk, wv, wo)]
    xt, wqt, wkt, wvt, wot = t
    heads = lambda w: (xt @ w.T).view(N, H, d).transpose(0, 1)[None]
    o = torch.nn.functional.scaled_dot_product_attention(heads(wqt), heads(wkt), heads(wvt),
                                                         is_causal=True)
    yt = o[0].transpose(0, 1).reshape(N, H * d) @ wot.T
    np.testing.assert_allclose(y, yt.detach().numpy(), rtol=1e-10, atol=1e-10)
    yt.backward(torch.from_numpy(dy))
    for g, tt in zip(mine, t):
        np.testing.assert_allclose(g, tt.grad.numpy(), rtol=1e-10, atol=1e-10)
