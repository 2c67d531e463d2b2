"""Pins of the CPU oracle against facts fixed by the pages and by mathematics.

Each test checks the oracle against something other than itself: a
hand-worked example, a closed form, an invariant, brute force on tiny inputs,
or an independent library routine (torch's CPU attention).
"""
import json
import math
import os

import numpy as np
import pytest
import torch

from oracle import lighthouse as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def rng(seed):
    return np.random.default_rng(seed)


# ---------------------------------------------------------------- rounding

def test_round_to_bf16_matches_torch_on_float32_sources():
    x = rng(0).standard_normal(20000).astype(np.float32) * np.float32(37.0)
    x[:5] = [0.0, -0.0, 1e-39, 3.0e38, -1.0]
    ours = O.round_to(x.astype(np.float64), "bf16")
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(ours, ref)


def test_round_to_bf16_rounds_once_from_float64():
    # 1 + 2^-8 is a tie between bf16 neighbours 1 and 1 + 2^-7: ties to even -> 1.
    # 1 + 2^-8 + 2^-30 is above the tie -> 1 + 2^-7; a float32 detour would
    # first drop the 2^-30 and then round the tie down (double rounding).
    x = np.array([1 + 2.0 ** -8, 1 + 2.0 ** -8 + 2.0 ** -30, -(1 + 3 * 2.0 ** -8)])
    got = O.to_f64(O.round_to(x, "bf16"), "bf16")
    np.testing.assert_array_equal(got, [1.0, 1 + 2.0 ** -7, -(1 + 2 * 2.0 ** -7)])


# ---------------------------------------------------------------- pyramid

@pytest.mark.parametrize("p,L,N", [(2, 4, 32), (3, 3, 27), (4, 3, 64), (4, 1, 8)])
def test_pyramid_levels_are_means_of_children(p, L, N):
    """Closed form (mean of p**l tokens) agrees with the recursive definition
    (mean of p entries of the level below)."""
    x = rng(1).standard_normal((N, 5))
    lv = O.pyramid(x, p, L)
    assert [len(a) for a in lv] == [N // p ** l for l in range(L)]
    np.testing.assert_array_equal(lv[0], x)
    for l in range(1, L):
        for j in range(len(lv[l])):
            kids = lv[l - 1][p * j: p * j + p]
            np.testing.assert_allclose(lv[l][j], sum(kids) / p, rtol=1e-13, atol=1e-13)


def test_pyramid_ramp_closed_form():
    p, L, N = 4, 4, 256
    x = np.arange(N, dtype=np.float64)[:, None] * np.ones((1, 3))
    lv = O.pyramid(x, p, L)
    for l in range(L):
        j = np.arange(N // p ** l)
        expect = j * p ** l + (p ** l - 1) / 2.0   # mean of an arithmetic run
        np.testing.assert_allclose(lv[l][:, 0], expect)


def test_geometry_rejects_ragged_lengths():
    with pytest.raises(ValueError):
        O.level_sizes(30, 4, 3)
    with pytest.raises(ValueError):
        O.level_sizes(32, 1, 2)


# ---------------------------------------------------------------- scores

def test_l2norm_exact_cases():
    v = np.zeros((4, 64), np.float32)
    v[0, 0], v[0, 33] = 3, 4            # 5
    v[1, :] = 1                          # sqrt(64) = 8
    v[2, 63] = -7                        # 7
    np.testing.assert_array_equal(O.l2norm_f32(v), np.float32([5, 8, 7, 0]))


def test_l2norm_close_to_float64_norm():
    x = (rng(2).standard_normal((500, 128)) * 3).astype(np.float32)
    got = O.l2norm_f32(x).astype(np.float64)
    ref = np.linalg.norm(x.astype(np.float64), axis=1)
    np.testing.assert_allclose(got, ref, rtol=2 ** -20)


def _order_rows(d):
    """Rows of tests/golden/score_order.json, widened to d elements (the
    eight values at elements 0, d/8, 2d/8, ...; zeros elsewhere)."""
    g = json.load(open(os.path.join(GOLDEN, "score_order.json")))
    out = {}
    for name, row in g["rows"].items():
        x = np.zeros(d, np.float32)
        for m, ex in enumerate(row["x_pow2_exponents"]):
            if ex is not None:
                x[m * (d // 8)] = np.float32(2.0 ** ex)
        out[name] = (x, row)
    return out


@pytest.mark.parametrize("d", [8, 64, 128])
def test_l2norm_summation_order_golden(d):
    """The halving-tree order of R4, pinned by hand-derived bit patterns that a
    sequential or an adjacent-pair summation would not produce."""
    for name, (x, row) in _order_rows(d).items():
        got = O.l2norm_f32(x[None])[0].view(np.uint32)
        assert got == int(row["norm_bits"], 16), (name, d, hex(got))
        q = np.tile(x, (4, 1))
        s = O.scores(q, q, 2, 2)               # k = q: score = 2 * norm, exact
        assert s[0].view(np.uint32) == int(row["score_q_eq_k_bits"], 16), (name, d)
        assert s[4].view(np.uint32) == s[0].view(np.uint32)   # level 1 inherits the max


def test_l2norm_order_golden_separates_the_orders():
    """The golden's alternative-order bit patterns really differ from the
    halving tree's, so the pin above would catch either mistake."""
    for name, (x, row) in _order_rows(8).items():
        assert row["norm_bits"] != row["sequential_bits"] or \
            row["norm_bits"] != row["adjacent_pairs_bits"], name
    rows = _order_rows(8)
    assert rows["tree_vs_sequential"][1]["sequential_bits"] != rows["tree_vs_sequential"][1]["norm_bits"]
    assert rows["tree_vs_pairs"][1]["adjacent_pairs_bits"] != rows["tree_vs_pairs"][1]["norm_bits"]


def test_golden_tiny_selection():
    g = json.load(open(os.path.join(GOLDEN, "tiny_selection.json")))
    N, p, L, S = g["N"], g["p"], g["L"], g["S"]
    c, b = np.array(g["c"], np.float32), np.array(g["b"], np.float32)
    q = np.stack([3 * c, 4 * c], 1)
    k = np.stack([0 * b, b], 1)
    s = O.scores(q, k, p, L)
    np.testing.assert_array_equal(s, np.float32(g["score"]))
    sel = O.topk(s, N, p, L, S)
    np.testing.assert_array_equal(sel, g["sel"])
    sub_idx, pos = O.causal_order(sel, N, p, L)
    np.testing.assert_array_equal(sub_idx, g["sub_idx"])
    np.testing.assert_array_equal(pos, g["pos"])
    np.testing.assert_array_equal(O.contributors(pos, N, p, L), g["contributors"])
    np.testing.assert_array_equal(O.contributors(pos, N, p, L, "causal"), g["contributors_causal"])
    for t, want in enumerate(g["feeders_causal"]):
        assert [O.level_bases(N, p, L)[l] + int(O.scatter_entry(t, l, p, "causal"))
                for l, _ in O.ancestors(t, pos, N, p, L, "causal")] == want, t
    v = np.stack([np.arange(N), np.ones(N)], 1).astype(np.float64)
    lv = O.pyramid(v, p, L)
    np.testing.assert_array_equal(lv[1], g["v_level1"])
    np.testing.assert_array_equal(lv[2], g["v_level2"])


@pytest.mark.parametrize("p,L", [(2, 5), (4, 4), (3, 3)])
def test_coarse_scores_are_span_maxima(p, L):
    N = p ** (L - 1) * 6
    q = rng(3).standard_normal((N, 16)).astype(np.float32)
    k = rng(4).standard_normal((N, 16)).astype(np.float32)
    s = O.scores(q, k, p, L)
    base = O.level_bases(N, p, L)
    s0 = s[:N]
    for l in range(1, L):
        span = p ** l
        for j in range(N // span):
            assert s[base[l] + j] == s0[j * span:(j + 1) * span].max()
            assert s[base[l] + j] == s[base[l - 1] + p * j: base[l - 1] + p * j + p].max()


# ---------------------------------------------------------------- top-K

def brute_topk(score, C, K):
    """Selected iff fewer than K candidates beat it (higher score, or equal
    score and lower flat index)."""
    out = []
    for i in range(C):
        beat = sum(1 for j in range(C)
                   if score[j] > score[i] or (score[j] == score[i] and j < i))
        if beat < K:
            out.append(i)
    return np.array(out, dtype=np.int64)


@pytest.mark.parametrize("seed", range(6))
def test_topk_matches_brute_force_with_ties(seed):
    p, L = 2, 4
    N = 32
    r = rng(10 + seed)
    # few distinct values -> many exact ties, across levels too
    q = r.integers(0, 3, (N, 4)).astype(np.float32)
    k = r.integers(0, 2, (N, 4)).astype(np.float32)
    s = O.scores(q, k, p, L)
    n_c = N // p ** (L - 1)
    C = len(s) - n_c
    for S in (n_c, n_c + 1, n_c + 7, n_c + C // 2, n_c + C):
        sel = O.topk(s, N, p, L, S)
        np.testing.assert_array_equal(sel, brute_topk(s, C, S - n_c))


def test_topk_rejects_bad_budget():
    s = np.zeros(6, np.float32)   # N=4, p=2, L=2: M = 4 + 2
    with pytest.raises(ValueError):
        O.topk(s, 4, 2, 2, 1)     # S < n_coarse
    with pytest.raises(ValueError):
        O.topk(s, 4, 2, 2, 7)     # S > M


# ---------------------------------------------------------------- causal order

@pytest.mark.parametrize("seed", range(4))
def test_causal_order_invariants(seed):
    p, L, N = 3, 4, 81
    r = rng(20 + seed)
    s = O.scores(r.standard_normal((N, 8)).astype(np.float32),
                 r.standard_normal((N, 8)).astype(np.float32), p, L)
    n_c = N // p ** (L - 1)
    S = n_c + 25
    sel = O.topk(s, N, p, L, S)
    sub_idx, pos = O.causal_order(sel, N, p, L)
    assert len(sub_idx) == S and len(set(sub_idx.tolist())) == S
    lev, j = O.entry_of_flat(sub_idx, N, p, L)
    end = (j + 1) * p ** lev - 1
    key = list(zip(end.tolist(), lev.tolist()))
    # brute force: position == number of chosen entries with a smaller key
    for i, kk in enumerate(key):
        assert sum(1 for o in key if o < kk) == i
    # an entry comes after every chosen entry inside its span (topological)
    for i in range(S):
        lo, hi = j[i] * p ** lev[i], end[i]
        for m in range(S):
            if m != i and lev[m] < lev[i] and lo <= j[m] * p ** lev[m] and end[m] <= hi:
                assert m < i
    assert np.all(pos[sub_idx] == np.arange(S))
    assert (pos >= 0).sum() == S
    c = O.contributors(pos, N, p, L)
    assert c.min() >= 1 and c.max() <= L


# ---------------------------------------------------------------- attention

def sdpa64(q, k, v):
    with torch.no_grad():
        t = [torch.from_numpy(a)[None, None] for a in (q, k, v)]
        return torch.nn.functional.scaled_dot_product_attention(*t, is_causal=True)[0, 0].numpy()


def test_attention_matches_torch_sdpa():
    r = rng(5)
    q, k, v = (r.standard_normal((70, 16)) * 2 for _ in range(3))
    o, lse = O.attention(q, k, v)
    np.testing.assert_allclose(o, sdpa64(q, k, v), rtol=1e-12, atol=1e-12)
    # lse against a direct log-sum-exp
    lg = (q @ k.T) / 4.0
    for i in (0, 10, 69):
        np.testing.assert_allclose(lse[i], np.log(np.exp(lg[i, : i + 1]).sum()), rtol=1e-12)


def test_attention_closed_forms():
    r = rng(6)
    S, d = 40, 8
    v = r.standard_normal((S, d))
    # zero queries: uniform weights over the causal prefix -> running mean
    o, lse = O.attention(np.zeros((S, d)), r.standard_normal((S, d)), v)
    np.testing.assert_allclose(o, np.cumsum(v, 0) / np.arange(1, S + 1)[:, None], atol=1e-12)
    np.testing.assert_allclose(lse, np.log(np.arange(1, S + 1)), atol=1e-12)
    # identical value rows -> that row everywhere
    o, _ = O.attention(r.standard_normal((S, d)), r.standard_normal((S, d)), np.tile(v[:1], (S, 1)))
    np.testing.assert_allclose(o, np.tile(v[:1], (S, 1)), atol=1e-12)
    # rows agree with the per-row version
    q, k = r.standard_normal((S, d)), r.standard_normal((S, d))
    o, lse = O.attention(q, k, v)
    o2, lse2 = O.attention_rows(q, k, v, [0, 7, 39])
    np.testing.assert_allclose(o2, o[[0, 7, 39]], atol=1e-12)
    np.testing.assert_allclose(lse2, lse[[0, 7, 39]], atol=1e-12)


# ---------------------------------------------------------------- whole forward

def test_forward_degenerate_is_dense_causal_attention():
    """L = 1 selects every token (S = N): the layer is dense causal SDPA."""
    r = rng(7)
    N, d = 64, 16
    q, k, v = (r.standard_normal((N, d)) for _ in range(3))
    f = O.forward_head(q, k, v, p=4, L=1, S=N, dtype="f64")
    np.testing.assert_array_equal(f["sub_idx"], np.arange(N))
    np.testing.assert_allclose(f["out"], sdpa64(q, k, v), rtol=1e-12, atol=1e-12)


def test_forward_constant_values_pass_through():
    r = rng(8)
    N, d, p, L = 64, 8, 4, 3
    q, k = r.standard_normal((N, d)), r.standard_normal((N, d))
    v = np.tile(r.standard_normal((1, d)), (N, 1))
    f = O.forward_head(q, k, v, p, L, S=4 + 10, dtype="f64")
    np.testing.assert_allclose(f["out"], v, atol=1e-12)


def test_forward_bf16_storage_and_shapes():
    from synth import bf16_bits_from_f32
    r = rng(9)
    N, d, p, L, S = 256, 64, 4, 3, 40
    q, k, v = (bf16_bits_from_f32(r.standard_normal((N, d)).astype(np.float32)) for _ in range(3))
    f = O.forward_head(q, k, v, p, L, S, "bf16")
    assert f["qs"].dtype == np.uint16 and f["qs"].shape == (S, d)
    assert f["out"].dtype == np.uint16 and f["out"].shape == (N, d)
    assert len(f["pq"]) == L - 1 and f["pq"][0].shape == (N // p, d)
    # the gathered rows are exact copies of level-0 tokens / stored pyramid rows
    for i, fl in enumerate(f["sub_idx"]):
        if fl < N:
            np.testing.assert_array_equal(f["qs"][i], q[fl])


# ---------------------------------------------------------------- backward

@pytest.mark.parametrize("mode", O.SCATTER_MODES)
def test_backward_matches_finite_differences(mode):
    """Selection held fixed: central differences of sum(out * dout)."""
    r = rng(11)
    N, d, p, L, S = 16, 4, 2, 3, 4 + 5
    q, k, v, dout = (r.standard_normal((N, d)) for _ in range(4))
    f = O.forward_head(q, k, v, p, L, S, "f64", mode)
    grads = O.backward_head(dout, f, p, L, "f64")
    h = 1e-6
    for which, g in zip(range(3), grads):
        for t in range(N):
            for c in range(d):
                xs = [q.copy(), k.copy(), v.copy()]
                xs[which][t, c] += h
                fp = (O.forward_fixed(*xs, f["sub_idx"], f["pos"], p, L, mode) * dout).sum()
                xs[which][t, c] -= 2 * h
                fm = (O.forward_fixed(*xs, f["sub_idx"], f["pos"], p, L, mode) * dout).sum()
                assert abs((fp - fm) / (2 * h) - g[t, c]) < 1e-6 * (1 + abs(g[t, c]))


def _dependencies(mode, N, p, L, S, seed, d=4):
    """dep[t, s]: out[t] changes when token s's q, k or v row changes
    (selection held fixed).  float64 results that do not depend on token s
    come out bit-identical, so "changes" is an exact test."""
    r = rng(seed)
    q, k, v = (r.standard_normal((N, d)) for _ in range(3))
    f = O.forward_head(q, k, v, p, L, S, "f64", mode)
    base = O.forward_fixed(q, k, v, f["sub_idx"], f["pos"], p, L, mode)
    dep = np.zeros((N, N), bool)
    for s in range(N):
        for which in range(3):
            xs = [q.copy(), k.copy(), v.copy()]
            xs[which][s] += 1e-3 * r.standard_normal(d)
            out = O.forward_fixed(*xs, f["sub_idx"], f["pos"], p, L, mode)
            dep[:, s] |= np.any(out != base, axis=1)
    return dep, f


@pytest.mark.parametrize("N,p,L,S,seed", [(64, 4, 3, 4 + 12, 30), (54, 3, 3, 6 + 9, 31),
                                          (32, 2, 4, 4 + 20, 32)])
def test_span_scatter_look_ahead_set(N, p, L, S, seed):
    """R11 (span broadcast) is not causal: out[t] depends on exactly the later
    tokens s with t < s <= end of t's coarsest span (the coarsest ancestor is
    always selected, and every selected ancestor's span lies inside it), and
    on no other later token."""
    dep, _ = _dependencies("span", N, p, L, S, seed)
    P = p ** (L - 1)
    for t in range(N):
        E = (t // P + 1) * P - 1
        later = np.arange(t + 1, N)
        np.testing.assert_array_equal(dep[t, later], later <= E, err_msg=f"token {t}")
    # so all but the last token of each coarsest span read the future: 1 - p^-(L-1) of tokens
    reads_future = [t for t in range(N) if dep[t, t + 1:].any()]
    assert len(reads_future) == N - N // P


@pytest.mark.parametrize("N,p,L,S,seed", [(64, 4, 3, 4 + 12, 30), (54, 3, 3, 6 + 9, 31),
                                          (32, 2, 4, 4 + 20, 32), (64, 4, 3, 4, 33)])
def test_causal_scatter_reads_no_later_token(N, p, L, S, seed):
    """R11c: no out[t] depends on any token s > t ([BG] phase 4: the scatter
    keeps causality; [TS-es] §3 item 1: left-to-right causality)."""
    dep, f = _dependencies("causal", N, p, L, S, seed)
    assert not np.triu(dep, 1).any()
    # and every token with a contributor depends on something (no dead rows)
    c = O.contributors(f["pos"], N, p, L, "causal")
    assert all(dep[t].any() for t in range(N) if c[t] > 0)


def test_causal_feeding_windows():
    """Closed form of R11c: entry (l, j) feeds exactly the tokens
    end(l, j) .. end(l, j) + p**l - 1 that exist."""
    N, p, L = 64, 4, 3
    t = np.arange(N)
    for l in range(L):
        j = O.scatter_entry(t, l, p, "causal")
        for jj in range(-1, N // p ** l):
            fed = t[j == jj]
            if jj < 0:
                np.testing.assert_array_equal(fed, np.arange(p ** l - 1))
                continue
            end = (jj + 1) * p ** l - 1
            np.testing.assert_array_equal(fed, np.arange(end, min(end + p ** l, N)))


def test_causal_constant_values_pass_through():
    """Constant V: a token with contributors outputs that row, one without
    outputs 0."""
    r = rng(8)
    N, d, p, L = 64, 8, 4, 3
    q, k = r.standard_normal((N, d)), r.standard_normal((N, d))
    v = np.tile(r.standard_normal((1, d)), (N, 1))
    f = O.forward_head(q, k, v, p, L, S=4 + 10, dtype="f64", mode="causal")
    c = O.contributors(f["pos"], N, p, L, "causal")
    assert (c == 0).any() and (c > 0).any()
    np.testing.assert_allclose(f["out"][c > 0], v[c > 0], atol=1e-12)
    assert np.all(f["out"][c == 0] == 0)


def test_causal_degenerate_is_dense_causal_attention():
    r = rng(7)
    N, d = 64, 16
    q, k, v = (r.standard_normal((N, d)) for _ in range(3))
    f = O.forward_head(q, k, v, p=4, L=1, S=N, dtype="f64", mode="causal")
    np.testing.assert_allclose(f["out"], sdpa64(q, k, v), rtol=1e-12, atol=1e-12)


def test_backward_degenerate_matches_torch_autograd():
    r = rng(12)
    N, d = 48, 8
    q, k, v, dout = (r.standard_normal((N, d)) for _ in range(4))
    f = O.forward_head(q, k, v, 2, 1, N, "f64")
    dq, dk, dv = O.backward_head(dout, f, 2, 1, "f64")
    t = [torch.tensor(a[None, None], requires_grad=True) for a in (q, k, v)]
    out = torch.nn.functional.scaled_dot_product_attention(*t, is_causal=True)
    out.backward(torch.from_numpy(dout[None, None]))
    for mine, tt in zip((dq, dk, dv), t):
        np.testing.assert_allclose(mine, tt.grad[0, 0].numpy(), rtol=1e-10, atol=1e-10)


@pytest.mark.parametrize("mode", O.SCATTER_MODES)
def test_every_token_gets_gradient(mode):
    """No holes: every token's coarsest ancestor is selected and feeds at
    least one token, so every input row gets a gradient path (bitsgeniais
    post, phase 3)."""
    r = rng(13)
    N, d, p, L = 64, 8, 4, 3
    q, k, v, dout = (r.standard_normal((N, d)) for _ in range(4))
    f = O.forward_head(q, k, v, p, L, 4 + 3, "f64", mode)
    dq, dk, dv = O.backward_head(dout, f, p, L, "f64")
    assert np.all(np.abs(dv).sum(1) > 0)


# ---------------------------------------------------------------- sampled forms

def test_row_and_column_forms_match_full_attention():
    """The per-row / per-column evaluations used at full sizes agree with the
    whole-matrix forms (which are pinned above against torch and closed forms)."""
    r = rng(14)
    S, d = 90, 16
    q, k, v, g = (r.standard_normal((S, d)) for _ in range(4))
    o, lse = O.attention(q, k, v)
    o2, lse2 = O.attention_all_rows(q, k, v, block=32)
    np.testing.assert_allclose(o2, o, atol=1e-12)
    np.testing.assert_allclose(lse2, lse, atol=1e-12)
    dq, dk, dv = O.attention_backward(q, k, v, g)
    D = (g * o).sum(axis=1)
    rows = [0, 1, 45, 89]
    np.testing.assert_allclose(O.attention_backward_rows(q, k, v, g, lse, D, rows), dq[rows], atol=1e-10)
    dk2, dv2 = O.attention_backward_cols(q, k, v, g, lse, D, rows)
    np.testing.assert_allclose(dk2, dk[rows], atol=1e-10)
    np.testing.assert_allclose(dv2, dv[rows], atol=1e-10)


def test_selection_and_pooled_rows_forms_match_forward():
    from synth import bf16_bits_from_f32
    r = rng(15)
    N, d, p, L, S = 256, 16, 4, 4, 30
    q, k, v = (bf16_bits_from_f32(r.standard_normal((N, d)).astype(np.float32)) for _ in range(3))
    f = O.forward_head(q, k, v, p, L, S, "bf16")
    sel = O.select_head(q, k, p, L, S, "bf16")
    for key in ("score", "sel", "sub_idx", "pos"):
        np.testing.assert_array_equal(sel[key], f[key])
    rows = O.pooled_rows(O.to_f64(q, "bf16"), f["sub_idx"], p, L, "bf16")
    np.testing.assert_array_equal(rows, O.to_f64(f["qs"], "bf16"))
    c = O.contributors(f["pos"], N, p, L)
    for t in (0, 5, 255):
        anc = O.ancestors(t, f["pos"], N, p, L)
        assert len(anc) == c[t]
        o = np.mean([O.to_f64(f["os"], "fp32")[pos] for _, pos in anc], axis=0)
        np.testing.assert_allclose(o, O.to_f64(f["out"], "bf16")[t], rtol=2 ** -7, atol=1e-6)
