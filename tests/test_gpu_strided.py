"""GPU parity of the layer on strided token tensors: q, k, v as views of one
packed token-major [B, N, 3, H, d] buffer (as a model's fused projection
gives them), the output and its gradient token-major [B, N, H, d], and dq,
dk, dv written into one packed [B, N, 3, H, d] gradient buffer.

Every result is compared with the oracle at the layer's bar (the inputs are
the parity cases' seeded tensors), and with the packed-layout run of the
same inputs bit for bit: the layout changes addresses only, never the
arithmetic.  Stage entry points that take token tensors (pyramid, scores,
gather, scatter, scatter backward, gather backward) are run on the same
strided views and compared bit for bit with their packed runs.
"""
from __future__ import annotations

import pytest
import torch

from oracle import lighthouse as O
from tests.helpers import check_close, to_device, to_f64
from tests.test_gpu_parity import CASES, heads, run_case

pytestmark = pytest.mark.gpu

STRIDED = ["d128_ragged_bf16", "p3_bf16", "p2_deep_b2_fp32", "tiny_ragged_fp32", "dense_ragged_bf16",
           "only_coarse_fp32"]


def packed_tokens(ts):
    """[B, N, len(ts), H, d] buffer holding the [B,H,N,d] tensors ts, and
    the [B,H,N,d] views of it."""
    B, H, N, d = ts[0].shape
    buf = torch.empty(B, N, len(ts), H, d, dtype=ts[0].dtype, device="cuda")
    views = [buf[:, :, i].permute(0, 2, 1, 3) for i in range(len(ts))]
    for v_, t in zip(views, ts):
        v_.copy_(t)
    return buf, views


@pytest.mark.parametrize("name", STRIDED)
def test_layer_on_strided_tokens(name, gpu_lib):
    lb = gpu_lib
    case = next(c for c in CASES if c[0] == name)
    R = run_case(case)                   # oracle + packed-layout GPU run of the same inputs
    _, B, H, N, d, p, L, S, dt = case
    print(f"[strided] case {name}", flush=True)
    tdt = torch.bfloat16 if dt == "bf16" else torch.float32
    host = {t: to_device(R["host"][t], dt) for t in ("q", "k", "v", "dout")}
    _, (q, k, v) = packed_tokens([host["q"], host["k"], host["v"]])
    _, (dout,) = packed_tokens([host["dout"]])
    o_buf = torch.full((B, N, 1, H, d), float("nan"), dtype=tdt, device="cuda")
    out = o_buf[:, :, 0].permute(0, 2, 1, 3)
    g_buf = torch.full((B, N, 3, H, d), float("nan"), dtype=tdt, device="cuda")
    dq, dk, dv = (g_buf[:, :, i].permute(0, 2, 1, 3) for i in range(3))
    assert q.stride() == (N * 3 * H * d, d, 3 * H * d, 1)

    _, bufs, shape = lb.forward(q, k, v, p, L, S, out=out)
    # the layout the library was given (strides of extent-1 dimensions are unused: 0)
    assert tuple(shape.qkv_stride) == tuple(0 if q.shape[i] == 1 else q.stride(i) for i in range(3))
    lb.backward(shape, dout, bufs, dq, dk, dv)
    torch.cuda.synchronize()
    f = R["fused"][0]
    for key, t in (("out", out), ("dq", dq), ("dk", dk), ("dv", dv)):
        got = t.cpu()
        assert torch.equal(got, f[key]), f"{key}: strided run differs from the packed run"
    for key in ("sel", "sub_idx", "pos", "qs", "ks", "vs", "os", "lse"):
        assert torch.equal(getattr(bufs, key).cpu(), f[key]), key
    for b, h in heads(case):
        o = R["orc"][b][h]
        check_close(to_f64(out[b, h]), O.to_f64(o["out"], dt), dt, f"out[{b},{h}]")
        for key, t in (("dq", dq), ("dk", dk), ("dv", dv)):
            check_close(to_f64(t[b, h]), o["bwd"][key], dt, f"{key}[{b},{h}]")


@pytest.mark.parametrize("name", ["d128_ragged_bf16", "p3_bf16", "p2_deep_b2_fp32"])
def test_stage_entry_points_on_strided_tokens(name, gpu_lib):
    lb = gpu_lib
    case = next(c for c in CASES if c[0] == name)
    R = run_case(case)
    _, B, H, N, d, p, L, S, dt = case
    print(f"[strided] stages {name}", flush=True)
    tdt = torch.bfloat16 if dt == "bf16" else torch.float32
    host = {t: to_device(R["host"][t], dt) for t in ("q", "k", "v", "dout")}
    _, (q, k, v) = packed_tokens([host["q"], host["k"], host["v"]])
    _, (dout,) = packed_tokens([host["dout"]])
    st = tuple(q.stride()[:3])
    ost = tuple(dout.stride()[:3])
    shape = lb.make_shape(B, H, N, d, p, L, S, tdt, st, ost)
    plain = lb.make_shape(B, H, N, d, p, L, S, tdt)
    z = lb.lh_query_sizes(shape)
    e = lambda *s, dtype=tdt: torch.empty(*s, dtype=dtype, device="cuda")  # noqa: E731

    def both(fn):
        """fn(shape, tensors...) on strided then packed inputs: two results."""
        return fn(shape, q, k, v, dout), fn(plain, *(t.contiguous() for t in (q, k, v, dout)))

    def pyramid(sh, q_, k_, v_, _):
        out = [e(B, H, z.M - N, d) for _ in range(3)]
        lb.lh_build_pyramid(sh, q_, k_, v_, *out, lb.workspace(z.ws_build_pyramid))
        return out

    def score(sh, q_, k_, v_, _):
        s_ = e(B, H, z.M, dtype=torch.float32)
        lb.lh_score(sh, q_, k_, s_, lb.workspace(z.ws_score))
        return [s_]

    sel = R["fused"][0]["sel"].cuda() if z.K else None
    pyr = [R["fused"][0][n].cuda() for n in ("pq", "pk", "pv")]

    def gather(sh, q_, k_, v_, _):
        r = [e(B, H, S, dtype=torch.int32), e(B, H, z.M, dtype=torch.int32)] + [e(B, H, S, d) for _ in range(3)]
        lb.lh_gather(sh, sel, q_, k_, v_, *pyr, *r, lb.workspace(z.ws_gather))
        return r

    pos = R["fused"][0]["pos"].cuda()
    os_ = R["fused"][0]["os"].cuda()
    subs = [torch.randn(B, H, S, d, device="cuda", generator=torch.Generator("cuda").manual_seed(i))
            for i in range(3)]

    def scatter(sh, q_, k_, v_, do_):
        o_buf = torch.full((B, N, 1, H, d), 0.5, dtype=tdt, device="cuda")
        o = o_buf[:, :, 0].permute(0, 2, 1, 3) if sh is shape else torch.full((B, H, N, d), 0.5, dtype=tdt, device="cuda")
        lb.lh_scatter(sh, os_, pos, o)
        return [o.contiguous()]

    def scatter_bwd(sh, q_, k_, v_, do_):
        r = e(B, H, S, d)
        lb.lh_scatter_backward(sh, do_, pos, r, lb.workspace(z.ws_scatter_backward))
        return [r]

    def gather_bwd(sh, q_, k_, v_, do_):
        if sh is shape:
            g_buf = torch.zeros(B, N, 3, H, d, dtype=tdt, device="cuda")
            g = [g_buf[:, :, i].permute(0, 2, 1, 3) for i in range(3)]
        else:
            g = [torch.zeros(B, H, N, d, dtype=tdt, device="cuda") for _ in range(3)]
        lb.lh_gather_backward(sh, *subs, pos, *g)
        return [t.contiguous() for t in g]

    for stage in (pyramid, score, gather, scatter, scatter_bwd, gather_bwd):
        a, b_ = both(stage)
        torch.cuda.synchronize()
        for i, (x, y) in enumerate(zip(a, b_)):
            assert torch.equal(x, y), f"{stage.__name__}[{i}]: strided differs from packed"


@pytest.mark.parametrize("name", ["d128_ragged_bf16", "p3_bf16", "lds_p4_L5_ragged_bf16"])
def test_causal_reading_on_strided_tokens(name, gpu_lib):
    """The causal scatter reading on strided token tensors equals its packed
    run bit for bit (the packed causal runs are compared with the oracle in
    test_gpu_causal.py)."""
    lb = gpu_lib
    case = next(c for c in CASES if c[0] == name)
    R = run_case(case)
    _, B, H, N, d, p, L, S, dt = case
    print(f"[strided] causal {name}", flush=True)
    host = {t: to_device(R["host"][t], dt) for t in ("q", "k", "v", "dout")}
    ref_out, ref_bufs, ref_shape = lb.forward(host["q"], host["k"], host["v"], p, L, S,
                                              scatter="causal")
    ref = (ref_out, *lb.backward(ref_shape, host["dout"], ref_bufs))
    _, (q, k, v) = packed_tokens([host["q"], host["k"], host["v"]])
    _, (dout,) = packed_tokens([host["dout"]])
    o_buf, (out,) = packed_tokens([torch.empty_like(host["q"])])
    g_buf, (dq, dk, dv) = packed_tokens([torch.empty_like(host["q"]) for _ in range(3)])
    out, bufs, shape = lb.forward(q, k, v, p, L, S, out=out, scatter="causal")
    lb.backward(shape, dout, bufs, dq, dk, dv)
    torch.cuda.synchronize()
    for key, got, want in zip(("out", "dq", "dk", "dv"), (out, dq, dk, dv), ref):
        assert torch.equal(got, want), f"{key}: strided causal run differs from the packed run"
