"""The C ABI on its own: tests/c_abi/lh_step (C++, HIP runtime and
liblighthouse.so only, no PyTorch) runs lh_forward and lh_backward on
seeded inputs from a file; its outputs are compared with the oracle at the
layer's bar (maps bit-exact, float tensors within the tolerances).

The program is built by hierarchical_sparse_attention_pyramid_amd/build.py
next to its source; the test fails if it is missing."""
from __future__ import annotations

import os
import subprocess

import numpy as np
import pytest

from oracle import lighthouse as O
from synth import inputs as synth
from tests.helpers import check_close

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
STEP = os.path.join(ROOT, "tests", "c_abi", "lh_step")

CASES = [
    # name, B, H, N, d, p, L, S, dtype, stream ("own": a created stream, "null": the default one)
    ("c_abi_bf16", 1, 2, 2048, 128, 4, 4, 300, "bf16", "own"),
    ("c_abi_fp32", 2, 1, 1024, 64, 2, 5, 150, "fp32", "own"),
    # bf16 at d = 64: lh_backward forks the dq gather backward onto its side stream
    ("c_abi_bf16_d64", 1, 2, 4096, 64, 4, 4, 400, "bf16", "own"),
    ("c_abi_bf16_d64_null_stream", 1, 2, 4096, 64, 4, 4, 400, "bf16", "null"),
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_standalone_c_program_matches_oracle(case, tmp_path, gpu_lib):
    assert os.path.exists(STEP), f"{STEP} is missing: build with hierarchical_sparse_attention_pyramid_amd/build.py"
    name, B, H, N, d, p, L, S, dt, stream = case
    print(f"[c-abi] {name}", flush=True)
    seed = 700 + CASES.index(case)
    host = {}
    for t in ("q", "k", "v", "dout"):
        a = np.stack([np.stack([synth.head_tensor(seed, t, b, h, N, d) for h in range(H)])
                      for b in range(B)])
        host[t] = synth.bf16_bits_from_f32(a) if dt == "bf16" else a.astype(np.float32)
    inp, outp = tmp_path / "in.bin", tmp_path / "out.bin"
    with open(inp, "wb") as f:
        np.array([B, H, N, d, p, L, S, 1 if dt == "bf16" else 0], np.int64).tofile(f)
        for t in ("q", "k", "v", "dout"):
            np.ascontiguousarray(host[t]).tofile(f)
    args = [STEP, str(inp), str(outp)] + (["null"] if stream == "null" else [])
    r = subprocess.run(args, capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, f"lh_step failed: {r.stdout}\n{r.stderr}"

    sizes = O.level_sizes(N, p, L)
    M, nc = sum(sizes), sizes[-1]
    K = S - nc
    el = np.uint16 if dt == "bf16" else np.float32
    n = B * H * N * d
    raw = np.fromfile(outp, dtype=np.uint8)
    off = 0

    def take(dtype, count):
        nonlocal off
        nb = np.dtype(dtype).itemsize * count
        a = raw[off:off + nb].view(dtype)
        off += nb
        return a

    out, dq, dk, dv = (take(el, n).reshape(B, H, N, d) for _ in range(4))
    sel = take(np.int32, B * H * K).reshape(B, H, K)
    sub_idx = take(np.int32, B * H * S).reshape(B, H, S)
    pos = take(np.int32, B * H * M).reshape(B, H, M)
    assert off == raw.size
    for b in range(B):
        for h in range(H):
            f = O.forward_head(host["q"][b, h], host["k"][b, h], host["v"][b, h], p, L, S, dt)
            np.testing.assert_array_equal(sel[b, h], f["sel"])
            np.testing.assert_array_equal(sub_idx[b, h], f["sub_idx"])
            np.testing.assert_array_equal(pos[b, h], f["pos"])
            check_close(O.to_f64(out[b, h], dt), O.to_f64(f["out"], dt), dt, f"out[{b},{h}]")
            g = O.backward_head(host["dout"][b, h], f, p, L, dt)
            for nm, got, ref in zip(("dq", "dk", "dv"), (dq, dk, dv), g):
                check_close(O.to_f64(got[b, h], dt), ref, dt, f"{nm}[{b},{h}]")
