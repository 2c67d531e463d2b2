"""The layer under HIP graph capture: lh_forward + lh_backward captured once
(torch's CUDAGraph API on the HIP stream) and replayed several times, with
eager launches of the same step in between.  Every replay must reproduce
the eager outputs bit for bit; the eager outputs are the ones the parity
tests compare with the oracle.  The library launches kernels only (no
allocation, no memset), so capture needs nothing special from the caller
beyond preallocated buffers and workspace."""
from __future__ import annotations

import pytest
import torch

from tests.helpers import to_device
from tests.test_gpu_parity import CASES, run_case

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("name", ["d128_ragged_bf16", "p2_deep_b2_fp32", "ties_bf16", "only_coarse_fp32",
                                  "ties_n32k_bf16", "lds_p4_L6_d128_fp32"])
def test_graph_replays_match_eager(name, gpu_lib):
    lb = gpu_lib
    case = next(c for c in CASES if c[0] == name)
    R = run_case(case)
    _, B, H, N, d, p, L, S, dt = case
    print(f"[graph] case {name}", flush=True)
    q, k, v, dout = (to_device(R["host"][t], dt) for t in ("q", "k", "v", "dout"))
    shape = lb.make_shape(B, H, N, d, p, L, S, q.dtype)
    bufs = lb.LayerBuffers(shape)
    z = bufs.sizes
    ws = lb.workspace(max(z.ws_forward, z.ws_backward))
    out, dq, dk, dv = (torch.empty_like(q) for _ in range(4))

    def step():
        lb.lh_forward(shape, q, k, v, out, bufs, ws)
        lb.lh_backward(shape, dout, bufs, dq, dk, dv, ws)

    step()
    torch.cuda.synchronize()
    eager = [t.clone() for t in (out, dq, dk, dv)]
    f = R["fused"][0]
    for key, t in zip(("out", "dq", "dk", "dv"), eager):
        assert torch.equal(t.cpu(), f[key]), f"eager {key} differs from the parity run"
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    for rep in range(3):
        for t in (out, dq, dk, dv):
            t.fill_(float("nan"))
        graph.replay()
        torch.cuda.synchronize()
        for key, a, b in zip(("out", "dq", "dk", "dv"), (out, dq, dk, dv), eager):
            assert torch.equal(a, b), f"replay {rep}: {key} differs from the eager step"
        step()  # eager work between replays
        torch.cuda.synchronize()


@pytest.mark.parametrize("kind", ["torch_stream", "raw_handle"])
def test_helpers_on_a_side_stream(kind, gpu_lib):
    """binding.forward / backward with an explicit stream: allocations and
    launches go to that stream and the results equal the default stream's."""
    lb = gpu_lib
    case = next(c for c in CASES if c[0] == "d128_ragged_bf16")
    R = run_case(case)
    _, B, H, N, d, p, L, S, dt = case
    print(f"[stream] {kind}", flush=True)
    q, k, v, dout = (to_device(R["host"][t], dt) for t in ("q", "k", "v", "dout"))
    ref_out, ref_bufs, ref_shape = lb.forward(q, k, v, p, L, S)
    ref = (ref_out, *lb.backward(ref_shape, dout, ref_bufs))
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    handle = side if kind == "torch_stream" else side.cuda_stream
    side.wait_stream(torch.cuda.current_stream())
    for _ in range(2):  # the second call reuses the first call's freed workspace
        out, bufs, shape = lb.forward(q, k, v, p, L, S, stream=handle)
        got = (out, *lb.backward(shape, dout, bufs, stream=handle))
    side.synchronize()
    for g, r in zip(got, ref):
        assert torch.equal(g, r)
