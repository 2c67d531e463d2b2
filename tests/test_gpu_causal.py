"""GPU parity of the causal scatter reading (R11c: entry (l, j) feeds the p^l
tokens from its end token on; a token nothing feeds gets 0) against the CPU
oracle, stage by stage and end to end, plus a check on the GPU that no output
row reads a later token while the selection is held fixed.

Cases cover the fast power-of-two kernels (p = 4, 64), the generic
ancestor-walk kernels (p = 2, 3, 5), several pooling passes in the scatter
backward (deep pyramids), K = 0 (only the coarsest level: the first
p^(L-1) - 1 tokens get no feeder), L = 1, both dtypes and both head widths.
Bars: bit-exact maps; float32 max-abs <= 1e-4; bfloat16
max|g-r| / max|r| <= 2e-2.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

from oracle import lighthouse as O
from synth import inputs as synth
from tests.helpers import check_close, to_device, to_f64

pytestmark = pytest.mark.gpu

# name, B, H, N, d, p, L, S, dtype
CASES = [
    ("c_tiny_fp32", 1, 2, 256, 64, 4, 3, 40, "fp32"),
    ("c_only_coarse_fp32", 1, 1, 256, 64, 4, 3, 16, "fp32"),   # K = 0
    ("c_n4k_fp32", 1, 2, 4096, 64, 4, 3, 512, "fp32"),
    ("c_d128_bf16", 1, 2, 2048, 128, 4, 4, 300, "bf16"),
    ("c_d64_bf16", 2, 2, 4096, 64, 4, 5, 600, "bf16"),
    ("c_p3_bf16", 1, 2, 729, 64, 3, 4, 100, "bf16"),
    ("c_p5_fp32", 1, 1, 3125, 128, 5, 5, 200, "fp32"),
    ("c_p2_deep_fp32", 2, 1, 1024, 64, 2, 9, 150, "fp32"),     # two pooling passes
    ("c_p2_deep_bf16", 1, 2, 4096, 128, 2, 12, 700, "bf16"),   # several pooling passes
    ("c_p64_bf16", 1, 2, 8192, 64, 64, 3, 400, "bf16"),
    ("c_dense_bf16", 1, 1, 300, 128, 4, 1, 300, "bf16"),        # L = 1
    ("c_lds_p4_L6_d128_bf16", 1, 1, 9216, 128, 4, 6, 700, "bf16"),  # two levels formed in LDS
]
ids = [c[0] for c in CASES]
_cache: dict = {}


def gen(case, tensor, seed=1900):
    name, B, H, N, d, p, L, S, dt = case
    arr = np.stack([np.stack([synth.head_tensor(seed + CASES.index(case), tensor, b, h, N, d)
                              for h in range(H)]) for b in range(B)])
    return synth.bf16_bits_from_f32(arr) if dt == "bf16" else arr


def run_case(case):
    if case[0] in _cache:
        return _cache[case[0]]
    from hierarchical_sparse_attention_pyramid_amd import binding as lb
    name, B, H, N, d, p, L, S, dt = case
    print(f"[gpu-causal] case {name}: B={B} H={H} N={N} d={d} p={p} L={L} S={S} {dt}", flush=True)
    host = {t: gen(case, t) for t in ("q", "k", "v", "dout")}
    orc = [[None] * H for _ in range(B)]
    for b in range(B):
        for h in range(H):
            f = O.forward_head(host["q"][b, h], host["k"][b, h], host["v"][b, h], p, L, S, dt,
                               "causal")
            f["bwd"] = O.backward_stages(host["dout"][b, h], f, p, L, dt)
            orc[b][h] = f
    st = lambda key: np.stack([np.stack([orc[b][h][key] for h in range(H)])  # noqa: E731
                               for b in range(B)])
    dev = {t: to_device(a, dt) for t, a in host.items()}
    shape = lb.make_shape(B, H, N, d, p, L, S, dev["q"].dtype, scatter="causal")
    z = lb.lh_query_sizes(shape)
    opos = torch.from_numpy(np.ascontiguousarray(st("pos"), np.int32)).cuda()
    oos = torch.from_numpy(np.ascontiguousarray(st("os"), np.float32)).cuda()
    r = {}
    # stages on the oracle's inputs
    r["out"] = torch.empty_like(dev["q"])
    lb.lh_scatter(shape, oos, opos, r["out"])
    r["dos"] = torch.empty(B, H, S, d, dtype=dev["q"].dtype, device="cuda")
    lb.lh_scatter_backward(shape, dev["dout"], opos, r["dos"], lb.workspace(z.ws_scatter_backward))
    # the whole layer, twice
    fused = []
    for _ in range(2):
        out, bufs, sh = lb.forward(dev["q"], dev["k"], dev["v"], p, L, S, scatter="causal")
        dq, dk, dv = lb.backward(sh, dev["dout"], bufs)
        fused.append(dict(sel=bufs.sel, pos=bufs.pos, out=out, dq=dq, dk=dk, dv=dv))
    torch.cuda.synchronize()
    print(f"[gpu-causal] case {name}: GPU done", flush=True)
    res = dict(gpu={k: v.cpu() for k, v in r.items()},
               fused=[{k: v.cpu() for k, v in f.items()} for f in fused], orc=orc)
    _cache[name] = res
    return res


def heads(case):
    _, B, H = case[:3]
    return [(b, h) for b in range(B) for h in range(H)]


@pytest.mark.parametrize("case", CASES, ids=ids)
def test_causal_scatter(case, gpu_lib):
    R = run_case(case)
    _, B, H, N, d, p, L, S, dt = case
    for b, h in heads(case):
        o = R["orc"][b][h]
        ref = O.scatter(O.to_f64(o["os"], "fp32"), o["pos"], N, p, L, "causal")
        check_close(to_f64(R["gpu"]["out"][b, h]), ref, dt, f"scatter[{b},{h}]")
        c = O.contributors(o["pos"], N, p, L, "causal")
        assert torch.all(R["gpu"]["out"][b, h][torch.from_numpy(c == 0)] == 0), "unfed tokens must be 0"


@pytest.mark.parametrize("case", CASES, ids=ids)
def test_causal_scatter_backward(case, gpu_lib):
    R = run_case(case)
    dt = case[-1]
    for b, h in heads(case):
        check_close(to_f64(R["gpu"]["dos"][b, h]), R["orc"][b][h]["bwd"]["dos"], dt, f"dos[{b},{h}]")


@pytest.mark.parametrize("case", CASES, ids=ids)
def test_causal_layer(case, gpu_lib):
    R = run_case(case)
    dt = case[-1]
    f, f1 = R["fused"]
    for b, h in heads(case):
        o = R["orc"][b][h]
        np.testing.assert_array_equal(f["sel"][b, h].numpy(), o["sel"])
        np.testing.assert_array_equal(f["pos"][b, h].numpy(), o["pos"])
        check_close(to_f64(f["out"][b, h]), O.to_f64(o["out"], dt), dt, f"out[{b},{h}]")
        for name in ("dq", "dk", "dv"):
            check_close(to_f64(f[name][b, h]), o["bwd"][name], dt, f"{name}[{b},{h}]")
    for key in f:
        assert torch.equal(f[key], f1[key]), f"{key} differs between two identical runs"


@pytest.mark.parametrize("dt", ["fp32", "bf16"])
@pytest.mark.parametrize("mode", ["causal", "span"])
def test_no_look_ahead_on_gpu(gpu_lib, mode, dt):
    """Selection held fixed (the first run's sel), q, k, v of every token from
    t0 on are redrawn: with the causal reading out[:t0] is bit-identical; with
    the span reading the tokens of t0's coarsest span before t0 change (its
    look-ahead, up to p^(L-1) - 1 tokens)."""
    lb = gpu_lib
    B, H, N, d, p, L, S = 1, 2, 4096, 64, 4, 4, 400
    t0 = 1000  # inside the coarsest span [960, 1024)
    host = {t: np.stack([synth.head_tensor(3100, t, 0, h, N, d) for h in range(H)])[None]
            for t in ("q", "k", "v")}
    alt = {t: np.stack([synth.head_tensor(3101, t, 0, h, N, d) for h in range(H)])[None]
           for t in ("q", "k", "v")}
    if dt == "bf16":
        host = {t: synth.bf16_bits_from_f32(a) for t, a in host.items()}
        alt = {t: synth.bf16_bits_from_f32(a) for t, a in alt.items()}
    print(f"[gpu-causal] no look-ahead: {mode} {dt}", flush=True)
    shape = lb.make_shape(B, H, N, d, p, L, S, torch.bfloat16 if dt == "bf16" else torch.float32,
                          scatter=mode)
    z = lb.lh_query_sizes(shape)
    outs = []
    sel = None
    for version in (host, {t: np.concatenate([host[t][:, :, :t0], alt[t][:, :, t0:]], axis=2)
                           for t in host}):
        q, k, v = (to_device(version[t], dt) for t in ("q", "k", "v"))
        bufs = lb.LayerBuffers(shape)
        lb.lh_build_pyramid(shape, q, k, v, bufs.pq, bufs.pk, bufs.pv,
                            lb.workspace(z.ws_build_pyramid))
        if sel is None:
            lb.lh_score(shape, q, k, bufs.score)
            lb.lh_topk(shape, bufs.score, bufs.sel, lb.workspace(z.ws_topk))
            sel = bufs.sel.clone()
        lb.lh_gather(shape, sel, q, k, v, bufs.pq, bufs.pk, bufs.pv, bufs.sub_idx, bufs.pos,
                     bufs.qs, bufs.ks, bufs.vs)
        lb.lh_attention(shape, bufs.qs, bufs.ks, bufs.vs, bufs.os, bufs.lse)
        out = torch.empty_like(q)
        lb.lh_scatter(shape, bufs.os, bufs.pos, out)
        torch.cuda.synchronize()
        outs.append(out.cpu())
    same = torch.all((outs[0] == outs[1]).reshape(B, H, N, -1), dim=-1)[0]  # [H, N]
    if mode == "causal":
        assert bool(same[:, :t0].all()), "a token before t0 changed with the causal scatter"
    else:
        P = p ** (L - 1)
        lo = t0 // P * P
        assert bool(same[:, :lo].all())          # earlier coarsest spans see nothing of it
        assert not bool(same[:, lo:t0].any())    # every token of t0's span before t0 sees it
    assert not bool(same[:, t0:].all())
