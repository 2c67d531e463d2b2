"""Plain CPU oracle of the Lighthouse attention layer (forward and backward).

TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the CPU-baseline
leg of the benchmark may import this module.  It shares no code with the HIP
library and must never be called on the product path.

Sources (cited by page and section; the pages are web summaries of the
Lighthouse Attention paper, arXiv 2605.06554):
  [TS-es] gist.science technical summary (Spanish), section 2 "Metodología",
          parts A (symmetric pyramid), B (parameter-free scoring and
          selection) and C (dense subsequence attention).
  [TS-ja] gist.science technical summary (Japanese), section 2, parts A-C;
          a near-duplicate of [TS-es] used as corroboration.
  [BG]    bitsgeniais.com.br blog post, the four numbered phases
          "1. Construção da Pirâmide", "2. Pontuação e Seleção Top-K",
          "3. Agrupamento Denso e FlashAttention", "4. Espalhar de Volta".

Readings where the pages leave a step open (R-numbers are the project's
reading list):
  R1  levels are 0..L-1 and L counts level 0 (the token level).
  R2  N must be a multiple of p**(L-1).
  R3  a level-l entry is the mean of the p**l tokens it spans (the closed form
      of "each level averages p consecutive entries of the level below").
  R4  token score = ||q_t||_2 + ||k_t||_2, both norms in float32 with a fixed
      halving-tree summation and correctly rounded square root; pooled
      vectors' own norms are not used.
  R5  coarse score = max of its p children's scores (hence the max over its
      span).
  R6  the whole coarsest level is always selected; the top-K competes over
      levels 0..L-2 with K = S - N/p**(L-1).
  R7  top-K order: score descending, then flat (level-major) index ascending.
  R8  no de-duplication across levels: an entry and its ancestors may both be
      selected.
  R9  causal order of the subsequence: by (end token, level) ascending, where
      end(l, j) = (j+1)*p**l - 1.
  R10 plain causal attention on subsequence positions, scale 1/sqrt(d).
  R11 scatter ("span" mode): a token's output is the mean of the outputs of
      its selected ancestors (itself included at level 0), levels summed in
      ascending order.  A coarse entry's output reaches every token of its
      span, so a token reads up to p**(L-1) - 1 later tokens through its
      coarsest ancestor: NOT causal.
  R11c scatter ("causal" mode): the output of entry (l, j) goes to the p**l
      tokens end(l, j) .. end(l, j) + p**l - 1, i.e. token t receives, per
      level, the last entry completed at or before t: j = (t+1)//p**l - 1
      (level 0: the token itself).  Mean over the selected ones; a token with
      none gets 0.  Every input of out[t] then lies at or before t.
  R12 backward: the exact gradient of R3..R11 (R11c) with the selection held
      fixed.

Precision: every tensor step is computed in float64 from its stored inputs and
rounded once (nearest-even) to the storage type ("fp32", "bf16", or "f64" for
no rounding).  Scores are the exception: they decide integers (the
selection), so they are computed in float32 exactly as R4 states.
"""
from __future__ import annotations

import math

import numpy as np

# ----------------------------------------------------------------------------
# storage helpers


def to_f64(x: np.ndarray, dtype: str) -> np.ndarray:
    """Widen stored values (float64, float32, or bfloat16 bits as uint16) to float64."""
    if dtype == "bf16":
        return (np.asarray(x, np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return np.asarray(x, dtype=np.float64)


def round_to(x: np.ndarray, dtype: str) -> np.ndarray:
    """Round float64 values once, to nearest-even, to the storage type.

    bf16 is rounded directly from float64 (no intermediate float32 step) by
    scaling each value to an integer count of its bf16 quantum.
    """
    x = np.asarray(x, dtype=np.float64)
    if dtype == "f64":
        return x
    if dtype == "fp32":
        return x.astype(np.float32)
    assert dtype == "bf16"
    _, e = np.frexp(x)                      # x = m * 2**e, 0.5 <= |m| < 1
    q = np.ldexp(1.0, np.maximum(e - 8, -133))  # 8 significant bits; subnormal floor
    r = np.rint(x / q) * q                  # np.rint: ties to even
    r32 = r.astype(np.float32)              # exact: r has <= 8 significant bits
    u = r32.view(np.uint32)
    big = np.abs(r) >= 2.0 ** 128 * (1 - 2.0 ** -9)  # rounds up to infinity
    u = np.where(big, (u & 0x80000000) | 0x7F800000, u)
    return (u >> 16).astype(np.uint16)


# ----------------------------------------------------------------------------
# pyramid geometry  [TS-es 2.A], [BG phase 1]


def level_sizes(N: int, p: int, L: int) -> list[int]:
    """N_l = N / p**l entries at level l (R1, R2)."""
    if p < 2 or L < 1 or N % p ** (L - 1):
        raise ValueError("need p >= 2, L >= 1 and N divisible by p**(L-1)")
    return [N // p ** l for l in range(L)]


def level_bases(N: int, p: int, L: int) -> list[int]:
    """Flat index of the first entry of each level (level-major layout)."""
    sizes = level_sizes(N, p, L)
    return [sum(sizes[:l]) for l in range(L)]


def entry_of_flat(f: np.ndarray, N: int, p: int, L: int):
    """(level, index-in-level) of flat indices."""
    bases = np.array(level_bases(N, p, L) + [sum(level_sizes(N, p, L))])
    lev = np.searchsorted(bases, f, side="right") - 1
    return lev, f - bases[lev]


# ----------------------------------------------------------------------------
# stage 1: symmetric average pooling  [TS-es 2.A], [TS-ja 2.A], [BG phase 1]


def pyramid(x: np.ndarray, p: int, L: int) -> list[np.ndarray]:
    """Levels 0..L-1 of one tensor [N, d] (float64): level l entry j is the mean
    of tokens j*p**l .. (j+1)*p**l - 1 (R3)."""
    N, d = x.shape
    level_sizes(N, p, L)
    return [x.reshape(N // p ** l, p ** l, d).mean(axis=1) for l in range(L)]


# ----------------------------------------------------------------------------
# stage 2: parameter-free l2 scores with max inheritance
# [TS-es 2.B "Puntuación"], [BG phase 2], [TS-ja 2.B]


def l2norm_f32(x32: np.ndarray) -> np.ndarray:
    """float32 l2 norm of the rows of x32 [n, d] (d a power of two) in the fixed
    order R4 states: squares rounded to float32, then a halving tree
    y[i] <- y[i] + y[i + w/2] for w = d, d/2, ..., 2, then a correctly rounded
    square root."""
    y = np.asarray(x32, dtype=np.float32)
    y = y * y
    w = y.shape[-1]
    assert w & (w - 1) == 0, "d must be a power of two"
    while w > 1:
        w //= 2
        y = y[..., :w] + y[..., w:2 * w]
    return np.sqrt(y[..., 0])


def scores(q32: np.ndarray, k32: np.ndarray, p: int, L: int) -> np.ndarray:
    """Flat float32 score array [M] for one head (R4, R5).

    q32/k32 are the level-0 rows exactly as stored, widened to float32."""
    N = q32.shape[0]
    s0 = (l2norm_f32(q32) + l2norm_f32(k32)).astype(np.float32)
    levels = [s0]
    for l in range(1, L):
        prev = levels[-1]
        levels.append(prev.reshape(-1, p).max(axis=1))
    assert sum(len(a) for a in levels) == sum(level_sizes(N, p, L))
    return np.concatenate(levels).astype(np.float32)


# ----------------------------------------------------------------------------
# stage 3: joint top-K across levels  [TS-es 2.B "Selección"], [BG phase 1-2]


def topk(score: np.ndarray, N: int, p: int, L: int, S: int) -> np.ndarray:
    """Selected candidate flat indices, ascending (R6, R7, R8).

    Candidates are levels 0..L-2; K = S - n_coarse of them are taken under the
    strict order (score descending, flat index ascending)."""
    sizes = level_sizes(N, p, L)
    n_c = sizes[-1]
    C = sum(sizes) - n_c
    K = S - n_c
    if not (0 <= K <= C):
        raise ValueError("need n_coarse <= S <= M")
    cand = np.asarray(score[:C], dtype=np.float32)
    flat = np.arange(C)
    order = np.lexsort((flat, -cand))  # primary key: -score; ties: flat ascending
    return np.sort(order[:K]).astype(np.int64)


# ----------------------------------------------------------------------------
# stage 4: causal gather  [TS-es 2.C "Recolección"], [BG phase 3], [TS-ja 2.C]


def causal_order(sel: np.ndarray, N: int, p: int, L: int):
    """(sub_idx [S], pos [M]) for the selected candidates plus the whole
    coarsest level, ordered by (end token, level) ascending (R6, R9)."""
    sizes = level_sizes(N, p, L)
    bases = level_bases(N, p, L)
    M = sum(sizes)
    chosen = np.concatenate([np.asarray(sel, np.int64),
                             bases[-1] + np.arange(sizes[-1], dtype=np.int64)])
    lev, j = entry_of_flat(chosen, N, p, L)
    end = (j + 1) * np.power(p, lev) - 1
    order = np.lexsort((lev, end))
    sub_idx = chosen[order]
    pos = np.full(M, -1, dtype=np.int64)
    pos[sub_idx] = np.arange(len(sub_idx))
    return sub_idx, pos


def gather_rows(levels: list[np.ndarray], sub_idx: np.ndarray, N: int, p: int, L: int) -> np.ndarray:
    """Rows of the pyramid (list of per-level arrays) at the given flat indices."""
    lev, j = entry_of_flat(sub_idx, N, p, L)
    return np.stack([levels[a][b] for a, b in zip(lev, j)]) if len(sub_idx) else \
        np.zeros((0, levels[0].shape[1]))


# ----------------------------------------------------------------------------
# stage 5: dense causal attention on the subsequence
# [TS-es 2.C "Atención"], [BG phase 3]


def attention(qs: np.ndarray, ks: np.ndarray, vs: np.ndarray):
    """Causal softmax attention (R10), float64.  Returns (O [S,d], lse [S])."""
    S, d = qs.shape
    tau = 1.0 / math.sqrt(d)
    logits = (qs @ ks.T) * tau
    logits[np.triu_indices(S, 1)] = -np.inf
    m = logits.max(axis=1, keepdims=True)
    e = np.exp(logits - m)
    z = e.sum(axis=1, keepdims=True)
    lse = (m + np.log(z))[:, 0]
    return (e / z) @ vs, lse


def attention_rows(qs, ks, vs, rows):
    """The same attention for a subset of query rows only (for large S)."""
    S, d = qs.shape
    tau = 1.0 / math.sqrt(d)
    out = np.zeros((len(rows), d))
    lse = np.zeros(len(rows))
    for n, i in enumerate(rows):
        lg = (ks[: i + 1] @ qs[i]) * tau
        m = lg.max()
        e = np.exp(lg - m)
        out[n] = (e @ vs[: i + 1]) / e.sum()
        lse[n] = m + math.log(e.sum())
    return out, lse


def attention_block(qs, ks, vs, r0, r1):
    """Rows r0..r1-1 of R10 attention (each row's softmax is independent, so
    this is the same computation as `attention`, restricted to those rows)."""
    S, d = qs.shape
    tau = 1.0 / math.sqrt(d)
    logits = (qs[r0:r1] @ ks[:r1].T) * tau
    rows = np.arange(r0, r1)[:, None]
    logits[np.arange(r1)[None, :] > rows] = -np.inf
    m = logits.max(axis=1, keepdims=True)
    e = np.exp(logits - m)
    z = e.sum(axis=1, keepdims=True)
    return (e / z) @ vs[:r1], (m + np.log(z))[:, 0]


def attention_all_rows(qs, ks, vs, block=2048):
    """(O, lse) of every row, computed `block` rows at a time (bounded memory)."""
    S, d = qs.shape
    O = np.zeros((S, d))
    lse = np.zeros(S)
    for r0 in range(0, S, block):
        r1 = min(S, r0 + block)
        O[r0:r1], lse[r0:r1] = attention_block(qs, ks, vs, r0, r1)
    return O, lse


def attention_backward_rows(qs, ks, vs, dos, lse, D, rows):
    """dQ rows of R10 attention: dQ_i = tau * sum_{j<=i} P_ij (dP_ij - D_i) K_j
    with P_ij = exp(tau q_i.k_j - lse_i), dP_ij = dO_i.v_j, D_i = dO_i.O_i."""
    S, d = qs.shape
    tau = 1.0 / math.sqrt(d)
    out = np.zeros((len(rows), d))
    for n, i in enumerate(rows):
        P = np.exp((ks[: i + 1] @ qs[i]) * tau - lse[i])
        dP = vs[: i + 1] @ dos[i]
        out[n] = tau * (P * (dP - D[i])) @ ks[: i + 1]
    return out


def attention_backward_cols(qs, ks, vs, dos, lse, D, cols):
    """dK and dV rows for key positions `cols`:
    dV_j = sum_{i>=j} P_ij dO_i, dK_j = tau * sum_{i>=j} P_ij (dP_ij - D_i) Q_i."""
    S, d = qs.shape
    tau = 1.0 / math.sqrt(d)
    dk = np.zeros((len(cols), d))
    dv = np.zeros((len(cols), d))
    for n, j in enumerate(cols):
        P = np.exp((qs[j:] @ ks[j]) * tau - lse[j:])
        dP = dos[j:] @ vs[j]
        dv[n] = P @ dos[j:]
        dk[n] = tau * (P * (dP - D[j:])) @ qs[j:]
    return dk, dv


# ----------------------------------------------------------------------------
# stage 6: deterministic scatter back to tokens
# [TS-es 2.C "Dispersión hacia atrás"], [BG phase 4], [TS-ja 2.C]; the
# causal reading follows [BG phase 4] (the scatter keeps causality, no token
# sees the future) and [TS-es 3] item 1 (left-to-right causality preserved)


SCATTER_MODES = ("span", "causal")


def scatter_entry(t, l: int, p: int, mode: str = "span"):
    """Index j of the level-l entry whose output token(s) t receive, or -1.

    span (R11): the entry whose span holds t, t // p**l.
    causal (R11c): the last level-l entry that ends at or before t,
    (t + 1) // p**l - 1 (its output then feeds the p**l tokens from its end
    token on)."""
    if mode == "span":
        return t // p ** l
    assert mode == "causal", mode
    return (t + 1) // p ** l - 1


def _feeds(pos, N, p, L, mode):
    """Per level: (entry index j per token, subsequence position or -1)."""
    bases = level_bases(N, p, L)
    t = np.arange(N)
    out = []
    for l in range(L):
        j = scatter_entry(t, l, p, mode)
        r = np.where(j >= 0, pos[bases[l] + np.maximum(j, 0)], -1)
        out.append((j, r))
    return out


def contributors(pos: np.ndarray, N: int, p: int, L: int, mode: str = "span") -> np.ndarray:
    """c_t: number of selected entries whose output token t receives (span:
    its selected ancestors, 1..L of them; causal: 0..L)."""
    c = np.zeros(N, dtype=np.int64)
    for _, r in _feeds(pos, N, p, L, mode):
        c += r >= 0
    return c


def ancestors(t: int, pos: np.ndarray, N: int, p: int, L: int, mode: str = "span"):
    """[(level, subsequence position)] of the selected entries feeding token t,
    level 0 first (span: t's selected ancestors)."""
    bases = level_bases(N, p, L)
    out = []
    for l in range(L):
        j = int(scatter_entry(t, l, p, mode))
        r = int(pos[bases[l] + j]) if j >= 0 else -1
        if r >= 0:
            out.append((l, r))
    return out


def scatter(os_: np.ndarray, pos: np.ndarray, N: int, p: int, L: int, mode: str = "span") -> np.ndarray:
    """out[t] = mean over the selected entries e feeding t of O_sub[pos(e)]
    (R11 / R11c); 0 for a token that no selected entry feeds (causal mode
    only)."""
    acc = np.zeros((N, os_.shape[1]))
    cnt = np.zeros(N)
    for _, r in _feeds(pos, N, p, L, mode):
        hit = r >= 0
        acc[hit] += os_[r[hit]]
        cnt += hit
    return np.where(cnt[:, None] > 0, acc / np.maximum(cnt, 1)[:, None], 0.0)


# ----------------------------------------------------------------------------
# selection only (scores, top-K, causal order) and pooled rows on demand


def select_head(q, k, p: int, L: int, S: int, dtype: str):
    """score, sel, sub_idx, pos of one head (no attention)."""
    N = q.shape[0]
    score = scores(to_f64(q, dtype).astype(np.float32), to_f64(k, dtype).astype(np.float32), p, L)
    sel = topk(score, N, p, L, S)
    sub_idx, pos = causal_order(sel, N, p, L)
    return dict(score=score, sel=sel, sub_idx=sub_idx, pos=pos)


def pooled_rows(x64: np.ndarray, flat: np.ndarray, p: int, L: int, dtype: str) -> np.ndarray:
    """Stored rows (rounded to dtype, as float64) of entries `flat`: level-0
    tokens as given, level-l entries as the mean of their p**l tokens (R3)."""
    N, d = x64.shape
    lev, j = entry_of_flat(np.asarray(flat), N, p, L)
    out = np.zeros((len(lev), d))
    for n, (a, b) in enumerate(zip(lev, j)):
        span = p ** int(a)
        out[n] = x64[b * span:(b + 1) * span].mean(axis=0)
    return to_f64(round_to(out, dtype), dtype)


# ----------------------------------------------------------------------------
# whole layer, one head


def forward_head(q, k, v, p: int, L: int, S: int, dtype: str, mode: str = "span"):
    """Forward of one head from stored [N, d] inputs; returns every
    intermediate the library exposes, each in its storage form.  `mode`
    selects the scatter reading (R11 "span" or R11c "causal")."""
    N, d = q.shape
    sizes = level_sizes(N, p, L)
    q64, k64, v64 = (to_f64(x, dtype) for x in (q, k, v))
    pyr = {name: [round_to(a, dtype) for a in pyramid(x, p, L)[1:]]
           for name, x in (("q", q64), ("k", k64), ("v", v64))}
    score = scores(q64.astype(np.float32), k64.astype(np.float32), p, L)
    sel = topk(score, N, p, L, S)
    sub_idx, pos = causal_order(sel, N, p, L)
    lv = {name: [x] + [to_f64(a, dtype) for a in pyr[name]]
          for name, x in (("q", q64), ("k", k64), ("v", v64))}
    qs, ks, vs = (gather_rows(lv[n], sub_idx, N, p, L) for n in ("q", "k", "v"))
    o, lse = attention(qs, ks, vs)
    os_ = round_to(o, "f64" if dtype == "f64" else "fp32")   # the layer keeps O in float32
    out = round_to(scatter(to_f64(os_, "fp32"), pos, N, p, L, mode), dtype)
    return dict(pq=pyr["q"], pk=pyr["k"], pv=pyr["v"], score=score, sel=sel,
                sub_idx=sub_idx, pos=pos,
                qs=round_to(qs, dtype), ks=round_to(ks, dtype), vs=round_to(vs, dtype),
                os=os_, lse=lse.astype(np.float32), out=out, M=sum(sizes), mode=mode)


def forward_fixed(q64, k64, v64, sub_idx, pos, p: int, L: int, mode: str = "span"):
    """float64 forward with the selection held fixed (for gradient checks)."""
    N = q64.shape[0]
    lv = {n: pyramid(x, p, L) for n, x in (("q", q64), ("k", k64), ("v", v64))}
    qs, ks, vs = (gather_rows(lv[n], sub_idx, N, p, L) for n in ("q", "k", "v"))
    o, _ = attention(qs, ks, vs)
    return scatter(o, pos, N, p, L, mode)


# ----------------------------------------------------------------------------
# backward, one head  [TS-es 2.B "No Diferenciabilidad"], [TS-ja 2.B]


def attention_backward(qs, ks, vs, dos):
    """Exact float64 gradients of R10 attention: (dQ, dK, dV)."""
    S, d = qs.shape
    tau = 1.0 / math.sqrt(d)
    logits = (qs @ ks.T) * tau
    logits[np.triu_indices(S, 1)] = -np.inf
    m = logits.max(axis=1, keepdims=True)
    P = np.exp(logits - m)
    P /= P.sum(axis=1, keepdims=True)
    dV = P.T @ dos
    dP = dos @ vs.T
    dS = P * (dP - (P * dP).sum(axis=1, keepdims=True))
    return tau * dS @ ks, tau * dS.T @ qs, dV


def scatter_backward(dout, pos, S, N, p, L, mode: str = "span"):
    """dO_sub[pos(e)] = sum over the tokens t that entry e feeds of
    dout[t] / c_t (R11: e's span; R11c: the p**l tokens from e's end on),
    the adjoint of `scatter` (R12)."""
    c = contributors(pos, N, p, L, mode)
    g = np.where(c[:, None] > 0, dout / np.maximum(c, 1)[:, None], 0.0)
    dos = np.zeros((S, dout.shape[1]))
    for j, r in _feeds(pos, N, p, L, mode):
        hit = r >= 0
        np.add.at(dos, r[hit], g[hit])
    return dos


def pool_backward(dxs, pos, N, p, L):
    """dX[t] = sum over t's selected ancestors e of dX_sub[pos(e)] / p**level(e)."""
    bases = level_bases(N, p, L)
    t = np.arange(N)
    acc = np.zeros((N, dxs.shape[1]))
    for l in range(L):
        r = pos[bases[l] + t // p ** l]
        hit = r >= 0
        acc[hit] += dxs[r[hit]] / p ** l
    return acc


def backward_stages(dout, fwd: dict, p: int, L: int, dtype: str) -> dict:
    """Every intermediate of the backward of one head, float64:
    dos (scatter backward), dqs/dks/dvs (attention backward), dq/dk/dv."""
    pos, sub_idx = fwd["pos"], fwd["sub_idx"]
    S = len(sub_idx)
    N = len(dout)
    qs, ks, vs = (to_f64(fwd[n], dtype) for n in ("qs", "ks", "vs"))
    dos = scatter_backward(to_f64(dout, dtype), pos, S, N, p, L, fwd.get("mode", "span"))
    dqs, dks, dvs = attention_backward(qs, ks, vs, dos)
    dq, dk, dv = (pool_backward(x, pos, N, p, L) for x in (dqs, dks, dvs))
    return dict(dos=dos, dqs=dqs, dks=dks, dvs=dvs, dq=dq, dk=dk, dv=dv)


def backward_head(dout, fwd: dict, p: int, L: int, dtype: str):
    """(dq, dk, dv) float64 [N, d] of one head, from the stored forward."""
    st = backward_stages(dout, fwd, p, L, dtype)
    return st["dq"], st["dk"], st["dv"]


# ----------------------------------------------------------------------------
# batched convenience wrappers over [B, H, N, d]


def forward(q, k, v, p, L, S, dtype, mode="span"):
    B, H = q.shape[:2]
    return [[forward_head(q[b, h], k[b, h], v[b, h], p, L, S, dtype, mode) for h in range(H)]
            for b in range(B)]


def backward(dout, fwds, p, L, dtype):
    B, H = dout.shape[:2]
    return [[backward_head(dout[b, h], fwds[b][h], p, L, dtype) for h in range(H)]
            for b in range(B)]
