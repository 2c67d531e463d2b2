"""Seeded sweep of random configurations through the whole layer
(lh_forward + lh_backward) against the oracle.

The hand-picked parity cases pin specific edge cases; this sweep draws
shapes the library accepts at random (fixed seeds, so the list is the same
on every run): p from 2 to 9 (powers of two and not), L from 1 to 5, S
anywhere in [N/p^(L-1), M], d in {64, 128}, fp32 and bf16, B and H in 1..3,
packed or strided token layouts; plus eight larger shapes (N up to 16K, S up
to 4K).  Every configuration is compared at the layer's bar: selection and
maps bit-exact; out and dq, dk, dv within the float tolerances.  Inputs come
from the shared seeded generator.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

from oracle import lighthouse as O
from synth import inputs as synth
from tests.helpers import check_close, to_device, to_f64

pytestmark = pytest.mark.gpu


def draw_configs(n: int, seed: int = 20261203):
    rng = np.random.default_rng(seed)
    out = []
    while len(out) < n:
        p = int(rng.integers(2, 10))
        L = int(rng.integers(1, 6))
        if p ** (L - 1) > 512:
            continue
        base = p ** (L - 1)
        N = base * int(rng.integers(max(1, 48 // base), max(2, 1200 // base) + 1))
        if N > 1500 or N < 16:
            continue
        sizes = O.level_sizes(N, p, L)
        M, nc = sum(sizes), sizes[-1]
        S = int(rng.integers(nc, M + 1))
        d = int(rng.choice([64, 128]))
        dt = str(rng.choice(["fp32", "bf16"]))
        B, H = int(rng.integers(1, 3)), int(rng.integers(1, 4))
        strided = bool(rng.integers(0, 2))
        out.append((f"s{len(out):02d}_p{p}_L{L}_N{N}_S{S}_d{d}_{dt}_B{B}H{H}{'_str' if strided else ''}",
                    B, H, N, d, p, L, S, dt, strided))
    return out


def draw_large_configs(n: int, seed: int = 20261204):
    """Larger shapes (several top-K slices and gather blocks per head, many
    attention tiles): N in [2048, 16384], B = H = 1, S up to 4096."""
    rng = np.random.default_rng(seed)
    out = []
    while len(out) < n:
        p = int(rng.integers(2, 9))
        L = int(rng.integers(2, 7))
        if p ** (L - 1) > 4096:
            continue
        base = p ** (L - 1)
        N = base * int(rng.integers(max(1, 2048 // base), 16384 // base + 1))
        if N < 2048 or N > 16384:
            continue
        sizes = O.level_sizes(N, p, L)
        M, nc = sum(sizes), sizes[-1]
        if nc > 4096:
            continue
        S = int(rng.integers(nc, min(M, 4096) + 1))
        d = int(rng.choice([64, 128]))
        dt = str(rng.choice(["fp32", "bf16"]))
        strided = bool(rng.integers(0, 2))
        out.append((f"big{len(out):02d}_p{p}_L{L}_N{N}_S{S}_d{d}_{dt}{'_str' if strided else ''}",
                    1, 1, N, d, p, L, S, dt, strided))
    return out


CONFIGS = draw_configs(24) + draw_large_configs(8)


@pytest.mark.parametrize("cfg", CONFIGS, ids=[c[0] for c in CONFIGS])
def test_random_config_matches_oracle(cfg, gpu_lib):
    lb = gpu_lib
    name, B, H, N, d, p, L, S, dt, strided = cfg
    print(f"[sweep] {name}", flush=True)
    seed = 5000 + CONFIGS.index(cfg)
    host = {}
    for t in ("q", "k", "v", "dout"):
        a = np.stack([np.stack([synth.head_tensor(seed, t, b, h, N, d) for h in range(H)])
                      for b in range(B)])
        host[t] = synth.bf16_bits_from_f32(a) if dt == "bf16" else a
    dev = {t: to_device(a, dt) for t, a in host.items()}
    tdt = dev["q"].dtype
    if strided:  # q, k, v inside one token-major [B, N, 3, H, d] buffer; out/dout token-major
        qkv = torch.empty(B, N, 3, H, d, dtype=tdt, device="cuda")
        q, k, v = (qkv[:, :, i].permute(0, 2, 1, 3) for i in range(3))
        for dst, t in zip((q, k, v), ("q", "k", "v")):
            dst.copy_(dev[t])
        ob = torch.empty(B, N, H, d, dtype=tdt, device="cuda")
        out = ob.permute(0, 2, 1, 3)
        dob = torch.empty(B, N, H, d, dtype=tdt, device="cuda")
        dout = dob.permute(0, 2, 1, 3)
        dout.copy_(dev["dout"])
        gb = torch.empty(B, N, 3, H, d, dtype=tdt, device="cuda")
        grads = [gb[:, :, i].permute(0, 2, 1, 3) for i in range(3)]
    else:
        q, k, v, dout = dev["q"], dev["k"], dev["v"], dev["dout"]
        out, grads = None, [None, None, None]
    out, bufs, shape = lb.forward(q, k, v, p, L, S, out=out)
    dq, dk, dv = lb.backward(shape, dout, bufs, *grads)
    torch.cuda.synchronize()
    for b in range(B):
        for h in range(H):
            f = O.forward_head(host["q"][b, h], host["k"][b, h], host["v"][b, h], p, L, S, dt)
            where = f"{name}[{b},{h}]"
            np.testing.assert_array_equal(bufs.sel[b, h].cpu().numpy(), f["sel"], err_msg=where)
            np.testing.assert_array_equal(bufs.sub_idx[b, h].cpu().numpy(), f["sub_idx"], err_msg=where)
            np.testing.assert_array_equal(bufs.pos[b, h].cpu().numpy(), f["pos"], err_msg=where)
            check_close(to_f64(out[b, h]), O.to_f64(f["out"], dt), dt, f"out {where}")
            g = O.backward_head(host["dout"][b, h], f, p, L, dt)
            for nm, got, ref in zip(("dq", "dk", "dv"), (dq, dk, dv), g):
                check_close(to_f64(got[b, h]), ref, dt, f"{nm} {where}")


# Layer shapes with many heads and long subsequences, so that the d = 64
# dK/dV pass takes its wide workgroups, with factors whose scatter and
# gather backward take the generic (not power-of-two) ancestor walk; two
# sampled heads each, compared in full.
LARGE_GRID = [
    # name, B, H, N, d, p, L, S, dtype
    ("grid_p3_d64", 1, 16, 27 * 1024, 64, 3, 4, 4500, "bf16"),
    ("grid_p5_d64", 2, 8, 25 * 1200, 64, 5, 3, 4100, "bf16"),
    ("grid_p3_d128", 1, 16, 27 * 512, 128, 3, 4, 3000, "bf16"),
]


@pytest.mark.parametrize("cfg", LARGE_GRID, ids=[c[0] for c in LARGE_GRID])
def test_large_grid_layer_matches_oracle(cfg, gpu_lib):
    lb = gpu_lib
    name, B, H, N, d, p, L, S, dt = cfg
    print(f"[sweep] {name}", flush=True)
    seed = 8000 + LARGE_GRID.index(cfg)
    host = {}
    for t in ("q", "k", "v", "dout"):
        a = np.stack([np.stack([synth.head_tensor(seed, t, b, h, N, d) for h in range(H)])
                      for b in range(B)])
        host[t] = synth.bf16_bits_from_f32(a)
    dev = {t: to_device(a, dt) for t, a in host.items()}
    out, bufs, shape = lb.forward(dev["q"], dev["k"], dev["v"], p, L, S)
    dq, dk, dv = lb.backward(shape, dev["dout"], bufs)
    torch.cuda.synchronize()
    rng = np.random.default_rng(seed)
    for i in rng.choice(B * H, size=2, replace=False):
        b, h = divmod(int(i), H)
        f = O.forward_head(host["q"][b, h], host["k"][b, h], host["v"][b, h], p, L, S, dt)
        where = f"{name}[{b},{h}]"
        np.testing.assert_array_equal(bufs.sel[b, h].cpu().numpy(), f["sel"], err_msg=where)
        np.testing.assert_array_equal(bufs.pos[b, h].cpu().numpy(), f["pos"], err_msg=where)
        check_close(to_f64(out[b, h]), O.to_f64(f["out"], dt), dt, f"out {where}")
        g = O.backward_head(host["dout"][b, h], f, p, L, dt)
        for nm, got, ref in zip(("dq", "dk", "dv"), (dq, dk, dv), g):
            check_close(to_f64(got[b, h]), ref, dt, f"{nm} {where}")
