"""GPU parity of the attention entry points (lh_attention,
lh_attention_backward) at shapes that pick each workgroup width of the d = 64
key-block (dK, dV) pass: grids of at least 256 workgroups of 256 keys use the
wide (eight-wave) workgroups, smaller ones four waves of 128 keys.  Both with
a sequence length that is not a multiple of the key block (a partial last
block), plus a d = 128 case.  The float32 cases run the float32 path on
sequences of 2,000 rows (31 full 64-row tiles and a partial one, each row's
work split over 16 lane groups) with 8 to 32 heads.

Two heads of each case are compared in full with the oracle's float64
attention and gradients, at the layer's bar (bf16 storage: max|g - r| /
max|r| <= 2e-2; float32: max|g - r| <= 1e-4).  Inputs are seeded standard
normals, rounded once to bf16 for bf16 storage.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

from oracle import lighthouse as O
from synth import inputs as synth
from tests.helpers import check_close, to_device, to_f64

pytestmark = pytest.mark.gpu

# name, B, H, S, d, storage
CASES = [
    ("wide_ragged_d64", 1, 16, 4000, 64, "bf16"),    # 16 key blocks of 256 x 16 heads = 256: wide
    ("narrow_ragged_d64", 2, 2, 3000, 64, "bf16"),   # 12 x 4 = 48: four-wave workgroups
    ("ragged_d128", 1, 8, 2500, 128, "bf16"),
    ("f32_ragged_h8_d64", 1, 8, 2000, 64, "fp32"),
    ("f32_ragged_h32_d64", 2, 16, 2000, 64, "fp32"),
    ("f32_ragged_h8_d128", 2, 4, 2000, 128, "fp32"),
    ("f32_ragged_h32_d128", 1, 32, 2000, 128, "fp32"),
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_attention_entry_points(case, gpu_lib):
    lb = gpu_lib
    name, B, H, S, d, dt = case
    print(f"[attention] {name}: B={B} H={H} S={S} d={d} {dt}", flush=True)
    rng = np.random.default_rng(300 + CASES.index(case))
    host = {t: rng.standard_normal((B, H, S, d), dtype=np.float32) for t in ("q", "k", "v", "do")}
    if dt == "bf16":
        host = {t: synth.bf16_bits_from_f32(a) for t, a in host.items()}
    dev = {t: to_device(a, dt) for t, a in host.items()}
    shape = lb.make_shape(B, H, S, d, 2, 1, S, torch.bfloat16 if dt == "bf16" else torch.float32)
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
        qs, ks, vs, dos = (O.to_f64(host[t][b, h], dt) for t in ("q", "k", "v", "do"))
        ref, ref_lse = O.attention(qs, ks, vs)
        check_close(to_f64(os_[b, h]), ref, dt, f"os[{b},{h}]")
        check_close(to_f64(lse[b, h]), ref_lse, dt, f"lse[{b},{h}]")
        for nm, got, r in zip(("dq", "dk", "dv"), (dq, dk, dv), O.attention_backward(qs, ks, vs, dos)):
            check_close(to_f64(got[b, h]), r, dt, f"{nm}[{b},{h}]")


# The forward's key-range split (lh_forward on causal grids too small to
# balance: the query blocks with more key tiles than the mean load of a
# resident workgroup slot run as two chunks, merged by a second kernel).
# Dense layers (L = 1, so the subsequence is the token sequence itself) are
# compared with the oracle's float64 causal attention and with the unsplit
# kernel of lh_attention on the same subsequence.  The small cases split every
# block of two or more tiles, with lengths that put a block's diagonal in
# either chunk and leave waves of a chunk with no visible keys; the 16-head
# cases split only the heavier blocks (both kinds of item in one grid).
SPLIT_CASES = [(64, 1, 3), (64, 63, 3), (64, 64, 3), (64, 65, 3), (64, 127, 3), (64, 129, 3),
               (64, 300, 3), (64, 1000, 3), (64, 4000, 3), (128, 1, 3), (128, 130, 3),
               (128, 257, 3), (128, 513, 3), (128, 900, 3), (128, 2500, 16), (64, 4000, 16)]


@pytest.mark.parametrize("d,S,H", SPLIT_CASES, ids=[f"d{d}_S{s}_H{h}" for d, s, h in SPLIT_CASES])
def test_forward_key_split(d, S, H, gpu_lib):
    lb = gpu_lib
    B = 1
    print(f"[attention split] S={S} d={d} H={H}", flush=True)
    rng = np.random.default_rng(1000 * d + S + H)
    host = {t: synth.bf16_bits_from_f32(rng.standard_normal((B, H, S, d), dtype=np.float32))
            for t in ("q", "k", "v")}
    dev = {t: to_device(a, "bf16") for t, a in host.items()}
    out, bufs, shape = lb.forward(dev["q"], dev["k"], dev["v"], 2, 1, S)
    os2 = torch.empty(B, H, S, d, dtype=torch.float32, device="cuda")
    lse2 = torch.empty(B, H, S, dtype=torch.float32, device="cuda")
    lb.lh_attention(shape, bufs.qs, bufs.ks, bufs.vs, os2, lse2)
    torch.cuda.synchronize()
    for h in sorted({0, H // 2, H - 1}):
        ref, ref_lse = O.attention(*(O.to_f64(host[t][0, h], "bf16") for t in ("q", "k", "v")))
        check_close(to_f64(bufs.os[0, h]), ref, "bf16", f"os[0,{h}]")
        check_close(to_f64(bufs.lse[0, h]), ref_lse, "bf16", f"lse[0,{h}]")
        # split and unsplit differ only in where each chunk's weights are rounded
        dos = float(np.max(np.abs(to_f64(bufs.os[0, h]) - to_f64(os2[0, h]))))
        assert dos <= 4e-3 * float(np.max(np.abs(ref))), f"os split vs unsplit: {dos}"
        dl = float(np.max(np.abs(to_f64(bufs.lse[0, h]) - to_f64(lse2[0, h]))))
        assert dl <= 4e-3, f"lse split vs unsplit: {dl}"
