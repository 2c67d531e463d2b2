"""GPU parity of the token-side broadcast kernels (the forward scatter and the
gather backward) at each number of tokens a row group walks.  A launch takes
64 tokens per row group unless that leaves fewer than 1,024 workgroups, then
32, then 16; the head count picks the size here: at N = 4,096 and d = 64 the
single-tensor scatter gets 16 tokens with 8 heads, 32 with 128 and 64 with
256 (the backward's launches over one or two gradients pick theirs the same
way).  Both scatter readings.  Three heads of each case are compared with the
oracle's forward and backward chain at the layer's bar (bf16: max|g - r| /
max|r| <= 2e-2), and the maps bit for bit.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

from oracle import lighthouse as O
from synth import inputs as synth
from tests.helpers import check_close, to_device, to_f64

pytestmark = pytest.mark.gpu

N, D, P, L, S = 4096, 64, 4, 3, 512
CASES = [(8, "span"), (128, "span"), (256, "span"), (8, "causal"), (128, "causal"), (256, "causal")]


@pytest.mark.parametrize("H,mode", CASES, ids=[f"H{h}_{m}" for h, m in CASES])
def test_broadcast_row_group_sizes(H, mode, gpu_lib):
    lb = gpu_lib
    print(f"[bcast] H={H} {mode}", flush=True)
    rng = np.random.default_rng(7000 + H)
    host = {t: synth.bf16_bits_from_f32(rng.standard_normal((1, H, N, D), dtype=np.float32))
            for t in ("q", "k", "v", "dout")}
    dev = {t: to_device(a, "bf16") for t, a in host.items()}
    out, bufs, shape = lb.forward(dev["q"], dev["k"], dev["v"], P, L, S, scatter=mode)
    dq, dk, dv = lb.backward(shape, dev["dout"], bufs)
    torch.cuda.synchronize()
    for h in sorted({0, H // 2, H - 1}):
        f = O.forward_head(host["q"][0, h], host["k"][0, h], host["v"][0, h], P, L, S, "bf16", mode)
        np.testing.assert_array_equal(bufs.sel[0, h].cpu().numpy(), f["sel"])
        np.testing.assert_array_equal(bufs.pos[0, h].cpu().numpy(), f["pos"])
        check_close(to_f64(out[0, h]), O.to_f64(f["out"], "bf16"), "bf16", f"out[0,{h}]")
        grads = O.backward_head(host["dout"][0, h], f, P, L, "bf16")
        for name, got, ref in zip(("dq", "dk", "dv"), (dq, dk, dv), grads):
            check_close(to_f64(got[0, h]), ref, "bf16", f"{name}[0,{h}]")
