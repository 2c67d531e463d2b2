"""GPU parity at sizes the oracle finishes in seconds (several tiles, ragged
tails, edge cases).

Two kinds of checks, both against the CPU oracle only:
  * stage by stage: every C-ABI entry point runs on inputs the ORACLE
    computed for that stage (uploaded to the GPU) and is compared with the
    oracle's output for the stage;
  * end to end: lh_forward / lh_backward on the synthetic inputs against the
    oracle's whole chain, run twice to check determinism.
Bars: bit-exact for scores, selections, orders, maps and row copies; float32
tensors max-abs <= 1e-4; bfloat16 tensors max-abs / max|ref| <= 2e-2.
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
    ("tiny_ragged_fp32", 1, 2, 256, 64, 4, 3, 40, "fp32"),
    ("n4k_fp32", 1, 2, 4096, 64, 4, 3, 512, "fp32"),          # the small workload's shape
    ("d128_ragged_bf16", 1, 2, 2048, 128, 4, 4, 300, "bf16"),
    ("p3_bf16", 1, 2, 729, 64, 3, 4, 100, "bf16"),
    ("p2_deep_b2_fp32", 2, 1, 1024, 64, 2, 9, 150, "fp32"),   # two pooling passes
    ("p2_deep_bf16", 1, 2, 4096, 128, 2, 12, 700, "bf16"),   # several pooling passes
    ("only_coarse_fp32", 1, 1, 256, 64, 4, 3, 16, "fp32"),    # K = 0
    ("all_selected_bf16", 1, 1, 64, 64, 4, 3, 84, "bf16"),    # K = C, S = M
    ("dense_ragged_bf16", 1, 2, 300, 128, 4, 1, 300, "bf16"),  # L = 1
    ("dense_fp32", 1, 1, 200, 64, 2, 1, 200, "fp32"),
    ("dense_n2k_bf16", 1, 16, 2048, 128, 4, 1, 2048, "bf16"),  # degenerate S = N workload
    ("dense_n8k_d64_bf16", 1, 1, 8192, 64, 4, 1, 8192, "bf16"),  # the 98K workload's S and d
    ("ties_bf16", 1, 2, 1024, 64, 4, 4, 120, "bf16"),         # duplicated rows: equal scores
    ("p64_bf16", 1, 2, 8192, 64, 64, 3, 400, "bf16"),         # largest pooling factor
    ("deep_L16_fp32", 1, 1, 32768, 64, 2, 16, 300, "fp32"),   # deepest pyramid (one coarse entry)
    ("zeros_bf16", 1, 2, 1024, 64, 4, 4, 200, "bf16"),        # all-zero q, k, v: every score tied
    # above 16384 candidates per head the pooling kernel counts the top-K's
    # first histogram pass; repeated rows tie scores across its slices
    ("ties_n32k_bf16", 1, 2, 32768, 64, 4, 3, 3000, "bf16"),
    # levels above the token pass's registers formed through LDS in its
    # workgroup: one level with a partial last workgroup, two levels, two
    # levels and a further pass, p = 8
    ("lds_p4_L5_ragged_bf16", 1, 2, 4352, 64, 4, 5, 500, "bf16"),
    ("lds_p4_L6_d128_fp32", 1, 1, 9216, 128, 4, 6, 700, "fp32"),
    ("lds_p4_L7_d128_bf16", 1, 1, 16384, 128, 4, 7, 900, "bf16"),
    ("lds_p8_L4_bf16", 1, 2, 4096, 64, 8, 4, 300, "bf16"),
]
ids = [c[0] for c in CASES]
_cache: dict = {}


def gen(case, tensor, seed=900):
    name, B, H, N, d, p, L, S, dt = case
    arr = np.stack([np.stack([synth.head_tensor(seed + CASES.index(case), tensor, b, h, N, d)
                              for h in range(H)]) for b in range(B)])
    if name.startswith("zeros") and tensor != "dout":
        arr = np.zeros_like(arr)
    if name.startswith("ties") and tensor != "dout":
        # repeat blocks of 8 rows: many exact score ties, within and across levels
        arr = np.repeat(arr[:, :, ::8], 8, axis=2)
    return synth.bf16_bits_from_f32(arr) if dt == "bf16" else arr


def stack(case, fn):
    _, B, H = case[:3]
    return np.stack([np.stack([fn(b, h) for h in range(H)]) for b in range(B)])


def run_case(case):
    if case[0] in _cache:
        return _cache[case[0]]
    from hierarchical_sparse_attention_pyramid_amd import binding as lb
    name, B, H, N, d, p, L, S, dt = case
    print(f"[gpu-parity] case {name}: B={B} H={H} N={N} d={d} p={p} L={L} S={S} {dt}", flush=True)
    host = {t: gen(case, t) for t in ("q", "k", "v", "dout")}
    # ---- the oracle's chain, per head
    orc = [[None] * H for _ in range(B)]
    for b in range(B):
        for h in range(H):
            f = O.forward_head(host["q"][b, h], host["k"][b, h], host["v"][b, h], p, L, S, dt)
            f["bwd"] = O.backward_stages(host["dout"][b, h], f, p, L, dt)
            orc[b][h] = f
    o = lambda key: stack(case, lambda b, h: orc[b][h][key])  # noqa: E731
    ob = lambda key: stack(case, lambda b, h: orc[b][h]["bwd"][key])  # noqa: E731
    empty_pyr = np.zeros((0, d), np.uint16 if dt == "bf16" else np.float32)
    pyr = {n: stack(case, lambda b, h, n=n: np.concatenate(orc[b][h][n]) if orc[b][h][n] else empty_pyr)
           for n in ("pq", "pk", "pv")}
    dos_stored = O.round_to(ob("dos"), dt)                              # what the kernel consumes
    odx = {n: O.round_to(ob(n), "fp32") for n in ("dqs", "dks", "dvs")}  # float32 inputs of a9

    dev = {t: to_device(a, dt) for t, a in host.items()}
    tdt = dev["q"].dtype
    shape = lb.make_shape(B, H, N, d, p, L, S, tdt)
    z = lb.lh_query_sizes(shape)
    e = lambda *s, dtype=tdt: torch.empty(*s, dtype=dtype, device="cuda")  # noqa: E731
    i32 = lambda a: torch.from_numpy(np.ascontiguousarray(a, np.int32)).cuda()  # noqa: E731
    f32 = lambda a: torch.from_numpy(np.ascontiguousarray(a, np.float32)).cuda()  # noqa: E731
    q, k, v, dout = dev["q"], dev["k"], dev["v"], dev["dout"]
    r = {}
    # ---- every stage on the oracle's inputs for that stage
    r["pq"], r["pk"], r["pv"] = (e(B, H, z.M - N, d) for _ in range(3))
    lb.lh_build_pyramid(shape, q, k, v, r["pq"], r["pk"], r["pv"], lb.workspace(z.ws_build_pyramid))
    r["score"] = e(B, H, z.M, dtype=torch.float32)
    lb.lh_score(shape, q, k, r["score"], lb.workspace(z.ws_score))
    r["sel"] = e(B, H, z.K, dtype=torch.int32)
    lb.lh_topk(shape, f32(o("score")), r["sel"], lb.workspace(z.ws_topk))
    # sentinel-filled: every slot the gather must write is checked, not inherited
    r["sub_idx"] = torch.full((B, H, S), 0x5A5A5A5A, dtype=torch.int32, device="cuda")
    r["pos"] = torch.full((B, H, z.M), 0x5A5A5A5A, dtype=torch.int32, device="cuda")
    r["qs"], r["ks"], r["vs"] = (e(B, H, S, d) for _ in range(3))
    opyr = {n: to_device(pyr[n], dt) for n in pyr}
    lb.lh_gather(shape, i32(o("sel")) if z.K else None, q, k, v, opyr["pq"], opyr["pk"],
                 opyr["pv"], r["sub_idx"], r["pos"], r["qs"], r["ks"], r["vs"],
                 lb.workspace(z.ws_gather))
    oqs, oks, ovs = (to_device(o(n), dt) for n in ("qs", "ks", "vs"))
    r["os"] = e(B, H, S, d, dtype=torch.float32)
    r["lse"] = e(B, H, S, dtype=torch.float32)
    lb.lh_attention(shape, oqs, oks, ovs, r["os"], r["lse"])
    opos, oos = i32(o("pos")), f32(o("os"))
    r["out"] = e(B, H, N, d)
    lb.lh_scatter(shape, oos, opos, r["out"])
    r["dos"] = e(B, H, S, d)
    lb.lh_scatter_backward(shape, dout, opos, r["dos"], lb.workspace(z.ws_scatter_backward))
    r["dqs"], r["dks"], r["dvs"] = (e(B, H, S, d, dtype=torch.float32) for _ in range(3))
    lb.lh_attention_backward(shape, oqs, oks, ovs, oos, f32(o("lse")), to_device(dos_stored, dt),
                             r["dqs"], r["dks"], r["dvs"], lb.workspace(z.ws_attention_backward))
    r["dq"], r["dk"], r["dv"] = (e(B, H, N, d) for _ in range(3))
    lb.lh_gather_backward(shape, f32(odx["dqs"]), f32(odx["dks"]), f32(odx["dvs"]), opos,
                          r["dq"], r["dk"], r["dv"])
    # ---- the whole layer, twice
    fused = []
    for _ in range(2):
        out, bufs, sh = lb.forward(q, k, v, p, L, S)
        dq, dk, dv = lb.backward(sh, dout, bufs)
        fused.append({n: getattr(bufs, n) for n in bufs.FIELDS} | dict(out=out, dq=dq, dk=dk, dv=dv))
    torch.cuda.synchronize()
    print(f"[gpu-parity] case {name}: GPU done", flush=True)
    res = dict(gpu={kk: vv.cpu() for kk, vv in r.items()},
               fused=[{kk: vv.cpu() for kk, vv in f.items()} for f in fused],
               orc=orc, host=host, pyr=pyr, dos_stored=dos_stored, odx=odx)
    _cache[name] = res
    return res


def heads(case):
    _, B, H = case[:3]
    return [(b, h) for b in range(B) for h in range(H)]


def bits(t: torch.Tensor, dt: str) -> np.ndarray:
    return t.view(torch.int16).numpy().view(np.uint16) if dt == "bf16" else t.numpy()


# ------------------------------------------------------------------ stages

@pytest.mark.parametrize("case", CASES, ids=ids)
def test_build_pyramid(case, gpu_lib):
    R = run_case(case)
    dt = case[-1]
    for b, h in heads(case):
        for n in ("pq", "pk", "pv"):
            check_close(to_f64(R["gpu"][n][b, h]), O.to_f64(R["pyr"][n][b, h], dt), dt, f"{n}[{b},{h}]")


@pytest.mark.parametrize("case", CASES, ids=ids)
def test_score_bit_exact(case, gpu_lib):
    R = run_case(case)
    for b, h in heads(case):
        got = R["gpu"]["score"][b, h].numpy()
        ref = R["orc"][b][h]["score"]
        bad = np.flatnonzero(got.view(np.uint32) != ref.view(np.uint32))
        assert bad.size == 0, f"score mismatch at {bad[:5]}: {got[bad[:5]]} vs {ref[bad[:5]]}"


@pytest.mark.parametrize("case", CASES, ids=ids)
def test_topk_bit_exact(case, gpu_lib):
    R = run_case(case)
    for b, h in heads(case):
        np.testing.assert_array_equal(R["gpu"]["sel"][b, h].numpy(), R["orc"][b][h]["sel"])


@pytest.mark.parametrize("case", CASES, ids=ids)
def test_gather_bit_exact(case, gpu_lib):
    """Maps and rows: the gathered rows are exact copies of the oracle's stored rows."""
    R = run_case(case)
    dt = case[-1]
    for b, h in heads(case):
        o = R["orc"][b][h]
        np.testing.assert_array_equal(R["gpu"]["sub_idx"][b, h].numpy(), o["sub_idx"])
        np.testing.assert_array_equal(R["gpu"]["pos"][b, h].numpy(), o["pos"])
        for n in ("qs", "ks", "vs"):
            np.testing.assert_array_equal(bits(R["gpu"][n][b, h], dt), o[n])


@pytest.mark.parametrize("case", CASES, ids=ids)
def test_attention(case, gpu_lib):
    R = run_case(case)
    dt = case[-1]
    for b, h in heads(case):
        o = R["orc"][b][h]
        ref, lse = O.attention(*(O.to_f64(o[n], dt) for n in ("qs", "ks", "vs")))
        check_close(to_f64(R["gpu"]["os"][b, h]), ref, dt, f"os[{b},{h}]")
        check_close(to_f64(R["gpu"]["lse"][b, h]), lse, dt, f"lse[{b},{h}]")


@pytest.mark.parametrize("case", CASES, ids=ids)
def test_scatter(case, gpu_lib):
    R = run_case(case)
    _, B, H, N, d, p, L, S, dt = case
    for b, h in heads(case):
        o = R["orc"][b][h]
        ref = O.scatter(O.to_f64(o["os"], "fp32"), o["pos"], N, p, L)
        check_close(to_f64(R["gpu"]["out"][b, h]), ref, dt, f"scatter[{b},{h}]")


@pytest.mark.parametrize("case", CASES, ids=ids)
def test_scatter_backward(case, gpu_lib):
    R = run_case(case)
    dt = case[-1]
    for b, h in heads(case):
        check_close(to_f64(R["gpu"]["dos"][b, h]), R["orc"][b][h]["bwd"]["dos"], dt, f"dos[{b},{h}]")


@pytest.mark.parametrize("case", CASES, ids=ids)
def test_attention_backward(case, gpu_lib):
    R = run_case(case)
    dt = case[-1]
    for b, h in heads(case):
        o = R["orc"][b][h]
        qs, ks, vs = (O.to_f64(o[n], dt) for n in ("qs", "ks", "vs"))
        refs = O.attention_backward(qs, ks, vs, O.to_f64(R["dos_stored"][b, h], dt))
        for name, ref in zip(("dqs", "dks", "dvs"), refs):
            check_close(to_f64(R["gpu"][name][b, h]), ref, dt, f"{name}[{b},{h}]")


@pytest.mark.parametrize("case", CASES, ids=ids)
def test_gather_backward(case, gpu_lib):
    R = run_case(case)
    _, B, H, N, d, p, L, S, dt = case
    for b, h in heads(case):
        pos = R["orc"][b][h]["pos"]
        for name, src in (("dq", "dqs"), ("dk", "dks"), ("dv", "dvs")):
            ref = O.pool_backward(O.to_f64(R["odx"][src][b, h], "fp32"), pos, N, p, L)
            check_close(to_f64(R["gpu"][name][b, h]), ref, dt, f"{name}[{b},{h}]")


# ------------------------------------------------------------------ whole layer

@pytest.mark.parametrize("case", CASES, ids=ids)
def test_layer_forward(case, gpu_lib):
    R = run_case(case)
    _, B, H, N, d, p, L, S, dt = case
    f = R["fused"][0]
    for b, h in heads(case):
        o = R["orc"][b][h]
        assert np.array_equal(f["score"][b, h].numpy().view(np.uint32), o["score"].view(np.uint32))
        for key in ("sel", "sub_idx", "pos"):
            np.testing.assert_array_equal(f[key][b, h].numpy(), o[key])
        for key in ("pq", "pk", "pv"):
            check_close(to_f64(f[key][b, h]), O.to_f64(R["pyr"][key][b, h], dt), dt, key)
        for key in ("qs", "ks", "vs"):
            check_close(to_f64(f[key][b, h]), O.to_f64(o[key], dt), dt, key)
        check_close(to_f64(f["os"][b, h]), O.to_f64(o["os"], "fp32"), dt, "os")
        check_close(to_f64(f["lse"][b, h]), O.to_f64(o["lse"], "fp32"), dt, "lse")
        check_close(to_f64(f["out"][b, h]), O.to_f64(o["out"], dt), dt, f"out[{b},{h}]")


@pytest.mark.parametrize("case", CASES, ids=ids)
def test_layer_backward(case, gpu_lib):
    R = run_case(case)
    dt = case[-1]
    f = R["fused"][0]
    for b, h in heads(case):
        for name in ("dq", "dk", "dv"):
            check_close(to_f64(f[name][b, h]), R["orc"][b][h]["bwd"][name], dt, f"{name}[{b},{h}]")


@pytest.mark.parametrize("case", CASES, ids=ids)
def test_layer_is_deterministic(case, gpu_lib):
    R = run_case(case)
    f0, f1 = R["fused"]
    for key in f0:
        assert torch.equal(f0[key], f1[key]), f"{key} differs between two identical runs"
