"""Robustness: non-finite inputs, concurrent use from several host threads,
and a large number of heads.

Non-finite inputs: NaN and infinity rows in q, k, v.

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
from tests.helpers import check_close, to_device, to_f64

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


def test_concurrent_host_threads_on_separate_streams(gpu_lib):
    """Four host threads run whole steps at the same time, each on its own
    stream with its own buffers (ctypes releases the GIL during the calls):
    every result equals the one-thread run bit for bit.  The library keeps
    no state between calls except each thread's error message."""
    import threading
    lb = gpu_lib
    B, H, N, d, p, L, S = 1, 2, 2048, 64, 4, 4, 300
    host = {t: np.stack([synth.head_tensor(41, t, 0, h, N, d) for h in range(H)])[None]
            for t in ("q", "k", "v", "dout")}
    dev = {t: torch.from_numpy(a).cuda().to(torch.bfloat16) for t, a in host.items()}
    shape = lb.make_shape(B, H, N, d, p, L, S, torch.bfloat16)

    def step(stream):
        bufs = lb.LayerBuffers(shape)
        z = bufs.sizes
        ws = lb.workspace(max(z.ws_forward, z.ws_backward))
        out, dq, dk, dv = (torch.empty_like(dev["q"]) for _ in range(4))
        torch.cuda.synchronize()
        for _ in range(3):
            lb.lh_forward(shape, dev["q"], dev["k"], dev["v"], out, bufs, ws, stream)
            lb.lh_backward(shape, dev["dout"], bufs, dq, dk, dv, ws, stream)
        stream.synchronize()
        return [t.cpu() for t in (out, dq, dk, dv, bufs.sel, bufs.pos)]

    ref = step(torch.cuda.Stream())
    results, errors = [None] * 4, []

    def worker(i):
        try:
            results[i] = step(torch.cuda.Stream())
        except Exception as e:  # noqa: BLE001 - reported below
            errors.append(repr(e))

    threads = [threading.Thread(target=worker, args=(i,)) for i in range(4)]
    for t in threads:
        t.start()
    for t in threads:
        t.join(timeout=120)
    assert not errors, errors
    for r in results:
        assert r is not None
        for a, b in zip(r, ref):
            assert torch.equal(a, b)


@pytest.mark.parametrize("dt", ["bf16", "fp32"])
def test_many_heads(dt, gpu_lib):
    """B*H = 4096 heads of a short sequence (the per-head kernels put B*H on
    the grid's y dimension, the attention kernels flatten it with the query
    or key blocks): 16 sampled heads against the oracle."""
    lb = gpu_lib
    B, H, N, d, p, L, S = 64, 64, 256, 64, 4, 3, 40
    print(f"[robust] many heads {dt}", flush=True)
    rng = np.random.default_rng(5)
    a = {t: rng.standard_normal((B, H, N, d), dtype=np.float32) for t in ("q", "k", "v", "dout")}
    host = {t: synth.bf16_bits_from_f32(x) if dt == "bf16" else x for t, x in a.items()}
    dev = {t: to_device(x, dt) for t, x in host.items()}
    out, bufs, shape = lb.forward(dev["q"], dev["k"], dev["v"], p, L, S)
    dq, dk, dv = lb.backward(shape, dev["dout"], bufs)
    torch.cuda.synchronize()
    for i in rng.choice(B * H, size=16, replace=False):
        b, h = divmod(int(i), H)
        f = O.forward_head(host["q"][b, h], host["k"][b, h], host["v"][b, h], p, L, S, dt)
        np.testing.assert_array_equal(bufs.sel[b, h].cpu().numpy(), f["sel"])
        np.testing.assert_array_equal(bufs.pos[b, h].cpu().numpy(), f["pos"])
        check_close(to_f64(out[b, h]), O.to_f64(f["out"], dt), dt, f"out[{b},{h}]")
        g = O.backward_head(host["dout"][b, h], f, p, L, dt)
        for nm, got, ref in zip(("dq", "dk", "dv"), (dq, dk, dv), g):
            check_close(to_f64(got[b, h]), ref, dt, f"{nm}[{b},{h}]")


# A one-entry subsequence: N = p^(L-1), so the coarsest level holds one entry
# and S = 1 keeps only it.  Its softmax weight is identically 1, so dq and dk
# are exactly zero in the mathematics (the oracle's are 0) while the output
# and dv are not.  A relative bar has no scale there, so dq and dk are held to
# zero on the scale of dv; their values on the GPU are rounding noise of the
# backward's dP - rowsum(dO*O).
@pytest.mark.parametrize("mode", ["span", "causal"])
@pytest.mark.parametrize("dt,d,p,L", [("bf16", 64, 6, 4), ("fp32", 64, 6, 4), ("bf16", 128, 4, 3)])
def test_one_entry_subsequence(dt, d, p, L, mode, gpu_lib):
    lb = gpu_lib
    B, H = 2, 2
    N, S = p ** (L - 1), 1
    print(f"[robust] one entry: N={N} p={p} L={L} d={d} {dt} {mode}", flush=True)
    host = {}
    for t in ("q", "k", "v", "dout"):
        a = np.stack([np.stack([synth.head_tensor(4242, t, b, h, N, d) for h in range(H)])
                      for b in range(B)])
        host[t] = synth.bf16_bits_from_f32(a) if dt == "bf16" else a
    dev = {t: to_device(a, dt) for t, a in host.items()}
    out, bufs, shape = lb.forward(dev["q"], dev["k"], dev["v"], p, L, S, scatter=mode)
    dq, dk, dv = lb.backward(shape, dev["dout"], bufs)
    torch.cuda.synchronize()
    for b in range(B):
        for h in range(H):
            f = O.forward_head(host["q"][b, h], host["k"][b, h], host["v"][b, h], p, L, S, dt, mode)
            np.testing.assert_array_equal(bufs.pos[b, h].cpu().numpy(), f["pos"])
            check_close(to_f64(out[b, h]), O.to_f64(f["out"], dt), dt, f"out[{b},{h}]")
            rq, rk, rv = O.backward_head(host["dout"][b, h], f, p, L, dt)
            assert np.max(np.abs(rq)) == 0.0 and np.max(np.abs(rk)) == 0.0  # the oracle
            check_close(to_f64(dv[b, h]), rv, dt, f"dv[{b},{h}]")
            scale = float(np.max(np.abs(rv)))
            for name, g in (("dq", dq), ("dk", dk)):
                err = float(torch.max(torch.abs(g[b, h].float())))
                assert err <= 1e-4 * scale, f"{name}[{b},{h}]: {err} against dv scale {scale}"
