"""GPU parity of lh_gather on selections the top-K of the parity workloads
does not produce: K above 131,072 (more selected candidates than the gather's
LDS samples cover at their finest spacing), selections clustered at one end
(gaps of unselected candidates spanning most of the pyramid), single-level
selections, a non-power-of-two factor and an empty selection.

The selection is any strictly ascending subset of the candidates (the
contract of lh_gather); the expected order, position map and rows come from
the oracle's causal_order and gather_rows.  Outputs are pre-filled with a
sentinel so that every slot the gather must write is checked.  Bar:
bit-exact.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

from oracle import lighthouse as O
from tests.helpers import to_device

pytestmark = pytest.mark.gpu

SENTINEL = 0x5A5A5A5A

# name, N, d, p, L, K, selection kind, dtype
CASES = [
    ("large_k", 262144, 64, 2, 2, 140000, "random", "bf16"),
    ("tail_cluster", 65536, 64, 4, 4, 1000, "last", "bf16"),
    ("head_cluster", 65536, 128, 4, 4, 777, "first", "bf16"),
    ("level0_only", 16384, 64, 4, 3, 2000, "level0", "fp32"),
    ("coarse_only", 16384, 64, 4, 4, 1300, "upper", "bf16"),
    ("p3_random", 19683, 64, 3, 5, 3001, "random", "fp32"),
    ("no_candidates", 65536, 64, 4, 4, 0, "random", "bf16"),  # K = 0: pos of every candidate -1
]
ids = [c[0] for c in CASES]


def selection(kind: str, K: int, N: int, p: int, L: int, rng) -> np.ndarray:
    sizes = O.level_sizes(N, p, L)
    C = sum(sizes[:-1])
    if kind == "random":
        return np.sort(rng.choice(C, size=K, replace=False))
    if kind == "last":
        return np.arange(C - K, C)
    if kind == "first":
        return np.arange(K)
    if kind == "level0":
        return np.sort(rng.choice(sizes[0], size=K, replace=False))
    if kind == "upper":  # levels 1..L-2 only
        return np.sort(sizes[0] + rng.choice(C - sizes[0], size=K, replace=False))
    raise ValueError(kind)


@pytest.mark.parametrize("case", CASES, ids=ids)
def test_gather_selection(case, gpu_lib):
    lb = gpu_lib
    name, N, d, p, L, K, kind, dt = case
    rng = np.random.default_rng(1234 + CASES.index(case))
    sizes = O.level_sizes(N, p, L)
    M = sum(sizes)
    S = K + sizes[-1]
    sel = selection(kind, K, N, p, L, rng).astype(np.int32)
    assert len(sel) == K and np.all(np.diff(sel) > 0)
    print(f"[gather] case {name}: N={N} d={d} p={p} L={L} K={K} {kind} {dt}", flush=True)
    # rows are opaque to the gather: arbitrary seeded bit patterns
    if dt == "bf16":
        rows = [rng.integers(0, 1 << 16, size=(n, d), dtype=np.uint16) for n in (N, M - N)]
    else:
        rows = [rng.standard_normal((n, d)).astype(np.float32) for n in (N, M - N)]
    lv0 = {t: rows[0] if t == "q" else np.roll(rows[0], 7 * (t == "k") + 13 * (t == "v"), axis=0)
           for t in "qkv"}
    pyr = {t: np.roll(rows[1], 5 * (t == "k") + 11 * (t == "v"), axis=0) for t in "qkv"}

    sub_idx, pos = O.causal_order(sel, N, p, L)
    bases = O.level_bases(N, p, L)

    def levels(t):
        return [lv0[t]] + [pyr[t][bases[l] - N: bases[l] - N + sizes[l]] for l in range(1, L)]

    dev = lambda a: to_device(a[None, None], dt)  # noqa: E731
    tdt = torch.bfloat16 if dt == "bf16" else torch.float32
    shape = lb.make_shape(1, 1, N, d, p, L, S, tdt)
    z = lb.lh_query_sizes(shape)
    assert (z.M, z.K) == (M, K)
    g_sub = torch.full((1, 1, S), SENTINEL, dtype=torch.int32, device="cuda")
    g_pos = torch.full((1, 1, M), SENTINEL, dtype=torch.int32, device="cuda")
    outs = [torch.empty(1, 1, S, d, dtype=tdt, device="cuda") for _ in range(3)]
    g_sel = torch.from_numpy(sel[None, None].copy()).cuda() if K else None
    lb.lh_gather(shape, g_sel, dev(lv0["q"]),
                 dev(lv0["k"]), dev(lv0["v"]), dev(pyr["q"]), dev(pyr["k"]), dev(pyr["v"]),
                 g_sub, g_pos, outs[0], outs[1], outs[2], lb.workspace(z.ws_gather))
    torch.cuda.synchronize()
    np.testing.assert_array_equal(g_sub[0, 0].cpu().numpy(), sub_idx)
    np.testing.assert_array_equal(g_pos[0, 0].cpu().numpy(), pos)
    for t, o in zip("qkv", outs):
        want = O.gather_rows(levels(t), sub_idx, N, p, L)
        got = o[0, 0].cpu()
        got = got.view(torch.int16).numpy().view(np.uint16) if dt == "bf16" else got.numpy()
        np.testing.assert_array_equal(got, want)
