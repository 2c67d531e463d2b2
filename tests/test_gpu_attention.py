"""GPU parity of the attention entry points (lh_attention,
lh_attention_backward) at shapes that pick each workgroup width of the d = 64
key-block (dK, dV) pass: grids of at least 256 workgroups of 256 keys use the
wide (eight-wave) workgroups, smaller ones four waves of 128 keys.  Both with
a sequence length that is not a multiple of the key block (a partial last
block), plus a d = 128 case.

Two heads of each case are compared in full with the oracle's float64
attention and gradients, at the layer's bar (bf16 storage: max|g - r| /
max|r| <= 2e-2).  Inputs are seeded standard normals rounded once to bf16.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

from oracle import lighthouse as O
from synth import inputs as synth
from tests.helpers import check_close, to_device, to_f64

pytestmark = pytest.mark.gpu

# name, B, H, S, d
CASES = [
    ("wide_ragged_d64", 1, 16, 4000, 64),    # 16 key blocks of 256 x 16 heads = 256: wide
    ("narrow_ragged_d64", 2, 2, 3000, 64),   # 12 x 4 = 48: four-wave workgroups
    ("ragged_d128", 1, 8, 2500, 128),
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_attention_entry_points(case, gpu_lib):
    lb = gpu_lib
    name, B, H, S, d = case
    print(f"[attention] {name}: B={B} H={H} S={S} d={d}", flush=True)
    rng = np.random.default_rng(300 + CASES.index(case))
    host = {t: synth.bf16_bits_from_f32(rng.standard_normal((B, H, S, d), dtype=np.float32))
            for t in ("q", "k", "v", "do")}
    dev = {t: to_device(a, "bf16") for t, a in host.items()}
    shape = lb.make_shape(B, H, S, d, 2, 1, S, torch.bfloat16)
    z = lb.lh_query_sizes(shape)
    os_ = torch.empty(B, H, S, d, dtype=torch.float32, device="cuda")
    lse = torch.empty(B, H, S, dtype=torch.float32, device="cuda")
    lb.lh_attention(shape, dev["q"], dev["k"], dev["v"], os_, lse)
    dq, dk, dv = (torch.empty(B, H, S, d, dtype=torch.float32, device="cuda") for _ in range(3))
    lb.lh_attention_backward(shape, dev["q"], dev["k"], dev["v"], os_, lse, dev["do"], dq, dk, dv,
                             lb.workspace(z.ws_attention_backward))
    torch.cuda.synchronize()
    for i in rng.choice(B * H, size=2, replace=False):
        b, h = divmod(int(i), H)
        qs, ks, vs, dos = (O.to_f64(host[t][b, h], "bf16") for t in ("q", "k", "v", "do"))
        ref, ref_lse = O.attention(qs, ks, vs)
        check_close(to_f64(os_[b, h]), ref, "bf16", f"os[{b},{h}]")
        check_close(to_f64(lse[b, h]), ref_lse, "bf16", f"lse[{b},{h}]")
        for nm, got, r in zip(("dq", "dk", "dv"), (dq, dk, dv), O.attention_backward(qs, ks, vs, dos)):
            check_close(to_f64(got[b, h]), r, "bf16", f"{nm}[{b},{h}]")
