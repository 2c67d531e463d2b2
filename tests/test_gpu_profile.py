"""lh_profile_step: it runs the same launches as lh_forward + lh_backward
(outputs equal bit for bit), and it reports one non-negative time per stage,
mapped to the stage's name also where the stages do not run in index order
(bf16 storage: the dQ pass forms rowsum(dO*O) and runs before the dK/dV pass,
so the rowsum stage is empty)."""
from __future__ import annotations

import numpy as np
import pytest
import torch

from synth import inputs as synth
from tests.helpers import to_device

pytestmark = pytest.mark.gpu

CASES = [("bf16", 1, 16, 8192, 64, 4, 4, 4000), ("fp32", 1, 2, 2048, 64, 4, 3, 400)]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_profile_step(case, gpu_lib):
    lb = gpu_lib
    dt, B, H, N, d, p, L, S = case
    print(f"[profile] {dt}", flush=True)
    host = {}
    for t in ("q", "k", "v", "dout"):
        a = np.stack([np.stack([synth.head_tensor(77, t, b, h, N, d) for h in range(H)])
                      for b in range(B)])
        host[t] = synth.bf16_bits_from_f32(a) if dt == "bf16" else a
    x = {t: to_device(a, dt) for t, a in host.items()}
    out, bufs, shape = lb.forward(x["q"], x["k"], x["v"], p, L, S)
    dq, dk, dv = lb.backward(shape, x["dout"], bufs)
    torch.cuda.synchronize()
    ref = [t.clone() for t in (out, dq, dk, dv, bufs.sel, bufs.pos)]
    for t in (out, dq, dk, dv):
        t.zero_()
    z = bufs.sizes
    ws = lb.workspace(max(z.ws_forward, z.ws_backward))
    ms = lb.lh_profile_step(shape, x["q"], x["k"], x["v"], out, bufs, x["dout"], dq, dk, dv, ws)
    for a, b in zip((out, dq, dk, dv, bufs.sel, bufs.pos), ref):
        assert torch.equal(a, b)
    assert list(ms) == lb.PROFILE_STAGES
    assert all(v >= 0.0 for v in ms.values()), ms
    for k in ("pyramid_score", "topk", "gather", "attention_fwd", "scatter", "scatter_bwd",
              "attention_dkdv", "attention_dq", "gather_bwd"):
        assert ms[k] > 0.0, (k, ms)
    if dt == "bf16":  # two event records with no kernel between them
        assert ms["attention_delta"] < 0.25 * ms["attention_dq"], ms
    else:
        assert ms["attention_delta"] > 0.0, ms
