"""GPU parity of lh_topk on score arrays the parity workloads do not produce:
heads small enough for the single-workgroup path (up to 16384 candidates)
and just above it, candidate counts whose histogram blocks cover several
slices with a partial last block, many exact ties at the threshold (the cut falls inside a run of
equal scores that spans slices), every candidate tied, K = 1, K = C, and a
head whose scores decrease with the flat index (the K selected candidates are
the first K).

The expected selection is the oracle's topk (strict order: score descending,
flat index ascending), compared bit for bit.  sel is pre-filled with a
sentinel, so every slot must be written.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

from oracle import lighthouse as O

pytestmark = pytest.mark.gpu

SENTINEL = 0x5A5A5A5A


def inherited(level0: np.ndarray, p: int, L: int) -> np.ndarray:
    """Flat scores of all levels: coarser entries take the max of their children."""
    lv = [level0.astype(np.float32)]
    for _ in range(1, L):
        lv.append(lv[-1].reshape(-1, p).max(axis=1))
    return np.concatenate(lv)


def head_scores(kind: str, N: int, d: int, p: int, L: int, rng) -> np.ndarray:
    if kind == "norms":  # like the layer: |q| + |k| with log-normal per-token scales
        c = np.sqrt(d - 0.5)
        x = (np.exp(0.5 * rng.standard_normal(N)) * (c + 0.707 * rng.standard_normal(N)) +
             np.exp(0.5 * rng.standard_normal(N)) * (c + 0.707 * rng.standard_normal(N)))
        return inherited(x, p, L)
    if kind == "few_values":  # 7 distinct values: long runs of ties everywhere
        return inherited(rng.integers(0, 7, size=N).astype(np.float32) * 0.25 + 1.0, p, L)
    if kind == "all_equal":
        return inherited(np.full(N, 3.5, np.float32), p, L)
    if kind == "decreasing":  # every level strictly decreasing in the flat index
        M = sum(O.level_sizes(N, p, L))
        return np.linspace(1000.0, 1.0, M, dtype=np.float32)
    raise ValueError(kind)


# name, N, d, p, L, K (None: C), score kinds of the heads
CASES = [
    # C = 305,000 candidates: 75 slices of 4096, histogram blocks of 2 slices, the last with 1
    ("ragged_blocks", 305000, 64, 2, 2, 20000, ("norms", "few_values")),
    # C = 510,000: 125 slices, blocks of 2 (63 blocks, the last with 1); ties cut inside
    # runs spanning slices
    ("ties_many_slices", 510000, 64, 4, 2, 50000, ("few_values", "norms")),
    ("all_equal", 262144, 64, 4, 3, 12345, ("all_equal",)),
    ("k_one", 65536, 64, 4, 4, 1, ("norms", "few_values")),
    ("k_all", 65536, 64, 4, 4, None, ("norms",)),
    ("decreasing", 131072, 64, 2, 5, 30000, ("decreasing",)),
    # heads of at most 16384 candidates: selected in one workgroup's LDS
    ("small_max", 16384, 64, 2, 2, 3000, ("norms", "few_values")),      # C = 16384 exactly
    ("small_all_equal", 4096, 64, 4, 3, 777, ("all_equal",)),
    ("small_k_one", 8192, 64, 2, 2, 1, ("few_values", "norms", "decreasing")),
    ("small_k_all", 12288, 64, 4, 2, None, ("few_values",)),
    # just above: the multi-kernel path with 5 slices, the last holding 2 candidates
    ("large_min", 16386, 64, 2, 2, 9000, ("few_values", "norms")),
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_topk_matches_oracle(case, gpu_lib):
    lb = gpu_lib
    name, N, d, p, L, K, kinds = case
    rng = np.random.default_rng(900 + CASES.index(case))
    sizes = O.level_sizes(N, p, L)
    M, nc = sum(sizes), sizes[-1]
    C = M - nc
    K = C if K is None else K
    S = K + nc
    H = len(kinds)
    print(f"[topk] case {name}: N={N} p={p} L={L} C={C} K={K} heads={kinds}", flush=True)
    score = np.stack([head_scores(k, N, d, p, L, rng) for k in kinds])[None]
    assert score.shape == (1, H, M)
    shape = lb.make_shape(1, H, N, d, p, L, S, torch.bfloat16)
    z = lb.lh_query_sizes(shape)
    assert (z.M, z.C, z.K) == (M, C, K)
    g_score = torch.from_numpy(score).cuda()
    g_sel = torch.full((1, H, K), SENTINEL, dtype=torch.int32, device="cuda")
    lb.lh_topk(shape, g_score, g_sel, lb.workspace(z.ws_topk))
    torch.cuda.synchronize()
    for h in range(H):
        want = O.topk(score[0, h], N, p, L, S)
        np.testing.assert_array_equal(g_sel[0, h].cpu().numpy(), want, err_msg=f"{name} head {h}")


# lh_forward on heads above 16384 candidates: the pooling kernels count the
# first histogram pass as they write the scores (the top-K stage runs only
# its later passes).  name, N, d, p, L, S, row-scale exponent range, tie blocks
FWD_CASES = [
    # row scales 2^-24..2^24: the scores span more coarse bins (top 8 bits)
    # than the counting table has slots, so some go to the global fallback
    ("fwd_wide", 16384, 64, 4, 4, 2000, 24, 1),
    # p = 2, L = 6: level-4 candidates are counted by the second pooling pass
    ("fwd_upper_pass", 16384, 64, 2, 6, 3000, 0, 1),
    # repeated rows: long runs of equal scores around the threshold
    ("fwd_ties", 32768, 128, 4, 3, 3000, 0, 16),
]


@pytest.mark.parametrize("case", FWD_CASES, ids=[c[0] for c in FWD_CASES])
def test_forward_counted_selection(case, gpu_lib):
    from synth import inputs as synth
    lb = gpu_lib
    name, N, d, p, L, S, span, rep = case
    H = 2
    print(f"[topk-fwd] case {name}: N={N} d={d} p={p} L={L} S={S}", flush=True)
    e = np.random.default_rng(61 + FWD_CASES.index(case)).integers(-span, span + 1, size=N)
    scale = np.exp2(e).astype(np.float32)[:, None]
    host = {}
    for t in ("q", "k", "v"):
        rows = [synth.head_tensor(80 + FWD_CASES.index(case), t, 0, h, N, d) for h in range(H)]
        rows = [np.repeat(x[::rep], rep, axis=0) * scale for x in rows]
        host[t] = synth.bf16_bits_from_f32(np.stack(rows)[None])
    dev = {t: torch.from_numpy(host[t].view(np.int16)).view(torch.bfloat16).cuda() for t in host}
    out, bufs, shape = lb.forward(dev["q"], dev["k"], dev["v"], p, L, S)
    torch.cuda.synchronize()
    assert bufs.sizes.C > 16384
    for h in range(H):
        want = O.select_head(host["q"][0, h], host["k"][0, h], p, L, S, "bf16")
        got_score = bufs.score[0, h].cpu().numpy()
        assert np.array_equal(got_score.view(np.uint32), want["score"].view(np.uint32)), name
        for key in ("sel", "sub_idx", "pos"):
            np.testing.assert_array_equal(getattr(bufs, key)[0, h].cpu().numpy(), want[key],
                                          err_msg=f"{name} head {h} {key}")
