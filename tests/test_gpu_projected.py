"""GPU parity of the attention block (Lighthouse layer between Q/K/V and
output projections, autograd through lh_forward / lh_backward) against the
block oracle on the same seeded storage values."""
from __future__ import annotations

import numpy as np
import pytest
import torch

from oracle import lighthouse as O
from oracle import projected as P
from synth import inputs as synth
from tests.helpers import check_close, to_f64

pytestmark = pytest.mark.gpu

CASES = [
    # name, N, D, H, d, p, L, S, dtype
    ("block_bf16", 2048, 256, 4, 64, 4, 3, 300, "bf16"),
    ("block_d128_bf16", 1024, 256, 2, 128, 4, 4, 200, "bf16"),
    ("block_fp32", 256, 128, 2, 64, 4, 3, 48, "fp32"),
]


def dev(a, dtype):
    if dtype == "bf16":
        return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(a).cuda()


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_block_matches_oracle(case, gpu_lib):
    from hierarchical_sparse_attention_pyramid_amd.layer import LighthouseAttention
    name, N, D, H, d, p, L, S, dt = case
    print(f"[gpu-block] {name}: N={N} D={D} H={H} d={d} p={p} L={L} S={S} {dt}", flush=True)
    seed = 500 + 10 * [c[0] for c in CASES].index(name)
    x = synth.block_tensor(seed, (N, D), dt)
    ws = [synth.block_tensor(seed + 1 + i, (H * d, D), dt, D ** -0.5) for i in range(3)]
    wo = synth.block_tensor(seed + 4, (D, H * d), dt, (H * d) ** -0.5)
    dy = synth.block_tensor(seed + 5, (N, D), dt)

    tdt = torch.bfloat16 if dt == "bf16" else torch.float32
    m = LighthouseAttention(D, H, d, p, L, S, dtype=tdt)
    with torch.no_grad():
        for prm, a in zip((m.wq, m.wk, m.wv, m.wo), (*ws, wo)):
            prm.copy_(dev(a, dt))
    xt = dev(x, dt)[None].requires_grad_(True)
    y = m(xt)
    y.backward(dev(dy, dt)[None])
    torch.cuda.synchronize()

    yr, cache = P.projected_forward(x, *ws, wo, H, p, L, S, dt)
    gr = P.projected_backward(dy, cache, dt)
    check_close(to_f64(y[0]), O.to_f64(yr, dt), dt, "block output")
    for got, ref, what in zip((xt.grad[0], m.wq.grad, m.wk.grad, m.wv.grad, m.wo.grad), gr,
                              ("dx", "dWq", "dWk", "dWv", "dWo")):
        check_close(to_f64(got), O.to_f64(ref, dt), dt, what)
