"""lh_backward with bf16 and d = 64 runs the gather backward of dq on a side
stream beside the dK/dV pass and joins it back into the caller's stream.
These tests check that the forked call gives the outputs of the sequential
launch order bit for bit (lh_profile_step runs the same stages in sequence),
that a graph captured by a thread that never ran the layer eagerly (no side
stream exists yet, and none is made inside a capture) replays correctly,
and that host threads on their own streams get identical results (each
thread has its own side stream)."""
from __future__ import annotations

import threading

import pytest
import torch

from tests.helpers import to_device
from tests.test_gpu_parity import CASES, run_case

pytestmark = pytest.mark.gpu

FORK_CASES = ["ties_bf16", "ties_n32k_bf16", "lds_p8_L4_bf16", "all_selected_bf16",
              "dense_n8k_d64_bf16"]


def _layer(lb, name):
    case = next(c for c in CASES if c[0] == name)
    R = run_case(case)
    _, B, H, N, d, p, L, S, dt = case
    assert d == 64 and dt == "bf16"
    q, k, v, dout = (to_device(R["host"][t], dt) for t in ("q", "k", "v", "dout"))
    shape = lb.make_shape(B, H, N, d, p, L, S, q.dtype)
    return R, shape, (q, k, v, dout)


def _buffers(lb, shape, q):
    bufs = lb.LayerBuffers(shape)
    z = bufs.sizes
    ws = lb.workspace(max(z.ws_forward, z.ws_backward))
    return bufs, ws, [torch.empty_like(q) for _ in range(4)]


@pytest.mark.parametrize("name", FORK_CASES)
def test_forked_backward_matches_sequential(name, gpu_lib):
    lb = gpu_lib
    print(f"[fork] case {name}", flush=True)
    R, shape, (q, k, v, dout) = _layer(lb, name)
    bufs, ws, (out, dq, dk, dv) = _buffers(lb, shape, q)
    lb.lh_forward(shape, q, k, v, out, bufs, ws)
    for t in (dq, dk, dv):
        t.fill_(float("nan"))
    lb.lh_backward(shape, dout, bufs, dq, dk, dv, ws)
    torch.cuda.synchronize()
    forked = [t.clone() for t in (out, dq, dk, dv)]
    f = R["fused"][0]  # the parity run, compared with the oracle there
    for key, t in zip(("out", "dq", "dk", "dv"), forked):
        assert torch.equal(t.cpu(), f[key]), f"{key} differs from the parity run"
    for t in (out, dq, dk, dv):
        t.fill_(float("nan"))
    lb.lh_profile_step(shape, q, k, v, out, bufs, dout, dq, dk, dv, ws)  # sequential stages
    torch.cuda.synchronize()
    for key, a, b in zip(("out", "dq", "dk", "dv"), (out, dq, dk, dv), forked):
        assert torch.equal(a, b), f"{key}: forked and sequential launches differ"


def _run_in_thread(fn):
    err = []

    def body():
        try:
            fn()
        except BaseException as e:  # re-raised on the calling thread
            err.append(e)

    t = threading.Thread(target=body)
    t.start()
    t.join()
    if err:
        raise err[0]


def test_capture_on_a_thread_without_eager_calls(gpu_lib):
    lb = gpu_lib
    name = "ties_n32k_bf16"
    print(f"[fork] capture on a fresh thread, case {name}", flush=True)
    R, shape, (q, k, v, dout) = _layer(lb, name)
    f = R["fused"][0]
    dev = torch.cuda.current_device()

    def capture_and_replay():
        torch.cuda.set_device(dev)
        bufs, ws, (out, dq, dk, dv) = _buffers(lb, shape, q)
        torch.cuda.synchronize()

        def step():
            lb.lh_forward(shape, q, k, v, out, bufs, ws)
            lb.lh_backward(shape, dout, bufs, dq, dk, dv, ws)

        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):  # this thread's first call of the layer
            step()
        for rep in range(3):
            for t in (out, dq, dk, dv):
                t.fill_(float("nan"))
            graph.replay()
            torch.cuda.synchronize()
            for key, t in zip(("out", "dq", "dk", "dv"), (out, dq, dk, dv)):
                assert torch.equal(t.cpu(), f[key]), f"replay {rep}: {key} differs"
            step()  # eager: makes the side stream; the graph keeps its launches
            torch.cuda.synchronize()
            for key, t in zip(("out", "dq", "dk", "dv"), (out, dq, dk, dv)):
                assert torch.equal(t.cpu(), f[key]), f"eager after replay {rep}: {key} differs"

    _run_in_thread(capture_and_replay)


def test_two_threads_on_their_own_streams(gpu_lib):
    lb = gpu_lib
    name = "ties_bf16"
    print(f"[fork] two host threads, case {name}", flush=True)
    R, shape, (q, k, v, dout) = _layer(lb, name)
    f = R["fused"][0]
    dev = torch.cuda.current_device()
    results, errors = {}, []
    start = threading.Barrier(2)

    def worker(i):
        try:
            torch.cuda.set_device(dev)
            s = torch.cuda.Stream()
            with torch.cuda.stream(s):
                bufs, ws, (out, dq, dk, dv) = _buffers(lb, shape, q)
                s.wait_stream(torch.cuda.default_stream())
                start.wait()
                for _ in range(4):
                    lb.lh_forward(shape, q, k, v, out, bufs, ws, stream=s)
                    lb.lh_backward(shape, dout, bufs, dq, dk, dv, ws, stream=s)
                s.synchronize()
                results[i] = [t.cpu() for t in (out, dq, dk, dv)]
        except BaseException as e:
            errors.append(e)

    threads = [threading.Thread(target=worker, args=(i,)) for i in range(2)]
    for t in threads:
        t.start()
    for t in threads:
        t.join()
    if errors:
        raise errors[0]
    for i in range(2):
        for key, t in zip(("out", "dq", "dk", "dv"), results[i]):
            assert torch.equal(t, f[key]), f"thread {i}: {key} differs from the parity run"
