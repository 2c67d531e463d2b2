"""lh_score on the hand-derived rows of tests/golden/score_order.json: the
kernel's float32 bit patterns follow the halving-tree order of the scorer
(squares, y[i] += y[i + w/2] for w = d..2, correctly rounded square root),
which a sequential or adjacent-pair summation would not reproduce."""
from __future__ import annotations

import json
import os

import numpy as np
import pytest
import torch

from synth import inputs as synth
from tests.helpers import to_device

pytestmark = pytest.mark.gpu

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "score_order.json")


@pytest.mark.parametrize("dt", ["fp32", "bf16"])
@pytest.mark.parametrize("d", [64, 128])
def test_score_order_golden(gpu_lib, d, dt):
    lb = gpu_lib
    g = json.load(open(GOLDEN))
    names = list(g["rows"])
    N, p, L = 16, 2, 2
    x = np.zeros((N, d), np.float32)
    for t in range(N):  # token t carries row t % 2 of the golden
        row = g["rows"][names[t % 2]]
        for m, ex in enumerate(row["x_pow2_exponents"]):
            if ex is not None:
                x[t, m * (d // 8)] = np.float32(2.0 ** ex)
    host = synth.bf16_bits_from_f32(x) if dt == "bf16" else x  # powers of two: exact in bf16
    q = to_device(host[None, None], dt)
    print(f"[gpu-score-order] d={d} {dt}", flush=True)
    shape = lb.make_shape(1, 1, N, d, p, L, N // 2, q.dtype)
    z = lb.lh_query_sizes(shape)
    score = torch.empty(1, 1, z.M, dtype=torch.float32, device="cuda")
    lb.lh_score(shape, q, q, score, lb.workspace(z.ws_score))  # k = q: score = 2 * norm
    torch.cuda.synchronize()
    bits = score[0, 0].cpu().numpy().view(np.uint32)
    for t in range(N):
        want = int(g["rows"][names[t % 2]]["score_q_eq_k_bits"], 16)
        assert bits[t] == want, (t, hex(bits[t]), hex(want))
    assert np.all(bits[N:] == bits[0])  # both rows score the same: level 1 inherits it
