"""Non-finite inputs: NaN and infinity rows in q, k, v.

The values that come out are unspecified for such inputs (the header says
so), but the maps must stay valid, since every later stage indexes memory
through them: `sel` strictly ascending inside the candidate range,
`sub_idx` a permutation of the chosen entries, `pos` its inverse and -1
elsewhere.  The run must finish without a launch error.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

from oracle import lighthouse as O
from synth import inputs as synth

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("kind", ["nan", "inf", "neg_inf", "mixed"])
@pytest.mark.parametrize("dt", ["bf16", "fp32"])
def test_non_finite_rows_keep_the_maps_valid(kind, dt, gpu_lib):
    lb = gpu_lib
    B, H, N, d, p, L, S = 1, 2, 1024, 64, 4, 4, 200
    print(f"[robust] {kind} {dt}", flush=True)
    rng = np.random.default_rng(17)
    host = {t: np.stack([synth.head_tensor(31, t, 0, h, N, d) for h in range(H)])[None]
            for t in ("q", "k", "v", "dout")}
    rows = rng.choice(N, size=24, replace=False)
    bad = {"nan": np.nan, "inf": np.inf, "neg_inf": -np.inf}
    for i, r in enumerate(rows):
        val = bad[kind] if kind in bad else list(bad.values())[i % 3]
        t = ("q", "k", "v")[i % 3]
        host[t][0, i % H, r, i % d] = val
    tdt = torch.bfloat16 if dt == "bf16" else torch.float32
    dev = {t: torch.from_numpy(a).cuda().to(tdt) for t, a in host.items()}
    out, bufs, shape = lb.forward(dev["q"], dev["k"], dev["v"], p, L, S)
    dq, dk, dv = lb.backward(shape, dev["dout"], bufs)
    torch.cuda.synchronize()
    sizes = O.level_sizes(N, p, L)
    M, nc = sum(sizes), sizes[-1]
    C, K = M - nc, S - nc
    for h in range(H):
        sel = bufs.sel[0, h].cpu().numpy()
        sub_idx = bufs.sub_idx[0, h].cpu().numpy()
        pos = bufs.pos[0, h].cpu().numpy()
        assert len(sel) == K and np.all(np.diff(sel) > 0) and sel.min() >= 0 and sel.max() < C
        chosen = np.concatenate([sel, np.arange(C, M)])
        assert np.array_equal(np.sort(sub_idx), chosen)
        assert np.array_equal(pos[sub_idx], np.arange(S))
        mask = np.ones(M, bool)
        mask[sub_idx] = False
        assert np.all(pos[mask] == -1)
