"""Benchmark of the Lighthouse attention layer on one MI355X.

One step = lh_forward + lh_backward (every stage of the hot path) on one batch
of synthetic input already resident in HBM.  The headline workload is the
98,304-token training context (B=1, H=16, d=64, p=4, L=5, S=8192, bf16);
`value` is its whole-job throughput in tokens/s, with the step captured once
in a HIP graph and replayed (the same kernels, launch for launch; a replay is
checked bit for bit against the eager step first); the eagerly launched step
time is reported beside it (config.eager_ms_per_step).  Alongside:
  * per-stage times from HIP events on the launch stream (mean over the
    profiled steps) and each stage's fraction of its HBM or matrix-core
    roofline (datasheet peaks: 8 TB/s, 2.5 PFLOP/s dense bf16; the float32
    workload's attention computes in float64 on the vector ALUs, so it is
    priced against the 78.6 TFLOP/s fp64 vector peak);
  * `roofline`: the dominant kernel of the step, from the same event times,
    beside the average launch duration of the committed rocprofv3 summary
    (profiles/kernel_avg.json) while that summary matches the kernel's source;
  * per-stage tables of the other workloads: the 4K float32 and 32K forward
    passes and the 1M forward+backward;
  * the 524,288-token layer (H=16, d=128, p=4, L=6, S=16384) forward and
    forward+backward, against the same-GPU dense causal attention (the same
    attention kernels at S = N; median of 3 timed calls after 1 warm-up);
  * both scatter readings: the headline uses the span reading (the C ABI's
    default); `causal_scatter` times the causal one on the 98K and 512K
    workloads;
  * the CPU oracle on the whole headline layer, its 16 heads run concurrently
    in single-threaded processes (cpu_baseline), plus single-thread oracle
    times on the small workloads;
  * reference rates of this GPU measured in the same run (a 1 GiB device
    copy, a large bf16 GEMM through torch), context only: they are not
    ceilings of the kernels;
  * `extras`: the layer inside an attention block with Q/K/V/O projections
    (autograd, D = H*d) at the headline shape; the other workload shapes (32K forward, the degenerate S = N
    2K forward, 1M forward+backward) and the operating points the ablations
    favour (bitsgeniais post, "Configurações e Velocidade"; gist.science
    technical summary §4)
    (L = 3, S = N/p^2 + 1536 for p = 4 and 2 at 98K and 512K, p = 4 at 1M),
    throughput only; the operating points reuse the inputs of the workload
    with the same N, H and d.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-long] [--no-cpu] [--no-extras]
Prints one JSON line on stdout; progress goes to stderr.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM_GBS = 8000.0          # MI355X HBM3E
PEAK_BF16_TFLOPS = 2500.0      # dense MFMA bf16
PEAK_FP64_VALU_TFLOPS = 78.6   # vector fp64: the float32 attention path computes in float64
METRIC = "Lighthouse layer tokens/s fwd+bwd at N=98K/512K; speedup vs dense causal attn"
HEADLINE = "train_n98k_bf16"
LONG = "long_n512k_bf16"
KERNEL_OF_STAGE = {
    "attention_fwd": ("attn_fwd_bf16", "attention_bf16.hip"),
    "attention_dkdv": ("attn_bwd_dkdv_bf16", "attention_bf16.hip"),
    "attention_dq": ("attn_bwd_dq_bf16", "attention_bf16.hip"),
    "scatter": ("bcast_fast", "scatter.hip"),
    "gather_bwd": ("bcast_fast", "scatter.hip"),
    "scatter_bwd": ("pool_bwd_kernel", "pyramid.hip"),
    "pyramid_score": ("pool_fwd_kernel", "pyramid.hip"),
}
FORWARD_STAGES = ("pyramid_score", "topk", "gather", "attention_fwd", "scatter")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def causal_pairs(S):
    return S * (S + 1) / 2.0


def stage_work(cfg, z):
    """Algorithmic HBM bytes or matrix flops of each stage for all B*H heads.

    Bytes count what a stage must read and write once (inputs, outputs), not
    implementation traffic such as the float32 partial sums of deep pyramids.
    Attention flops count causal (i, j <= i) pairs: forward 2 matmuls, the
    backward 5 (recompute of QK^T, dP, dV, dK, dQ), split as 4 in the
    key-block pass and 1 (dQ) in the query-block pass; the query-block pass
    also recomputes QK^T and dP, which is not counted.  With bf16 storage the
    query-block pass also forms rowsum(dO*O) (no kernel of its own then)."""
    BH = cfg.B * cfg.H
    N, d, S, M = cfg.N, cfg.d, cfg.S, z.M
    e = 2 if cfg.dtype == "bf16" else 4
    C, K = z.C, z.K
    pairs = causal_pairs(S)
    return {
        "pyramid_score": ("hbm", BH * (3 * N * d * e + 3 * (M - N) * d * e + 4 * M)),
        "topk": ("hbm", BH * (4 * C + 4 * K)),
        "gather": ("hbm", BH * (2 * 3 * S * d * e + 4 * K + 4 * S + 4 * M)),
        "attention_fwd": ("mfma", BH * 4 * d * pairs),
        "scatter": ("hbm", BH * (4 * S * d + 4 * M + N * d * e)),
        "scatter_bwd": ("hbm", BH * (N * d * e + 4 * M + S * d * e)),
        "attention_delta": ("hbm", BH * (4 * S * d + S * d * e + 4 * S)),
        "attention_dkdv": ("mfma", BH * 8 * d * pairs),
        "attention_dq": ("mfma", BH * 2 * d * pairs),
        "gather_bwd": ("hbm", BH * (3 * 4 * S * d + 4 * M + 3 * N * d * e)),
    }


def roofline_entry(kind, work, ms, dtype):
    ms = max(ms, 1e-6)  # a stage with no work can time as 0
    if kind == "hbm":
        achieved = work / (ms * 1e-3) / 1e9
        peak, unit = PEAK_HBM_GBS, "GB/s"
    elif dtype == "bf16":
        achieved = work / (ms * 1e-3) / 1e12
        peak, unit = PEAK_BF16_TFLOPS, "TFLOP/s"
    else:  # float32 storage: the attention kernels compute in float64 on the VALU
        kind = "alu"
        achieved = work / (ms * 1e-3) / 1e12
        peak, unit = PEAK_FP64_VALU_TFLOPS, "TFLOP/s"
    return {"bound": kind, "achieved": round(achieved, 2), "peak": peak, "unit": unit,
            "frac": round(achieved / peak, 4)}


def stage_table(cfg, z, stages_ms, only=None):
    """Per-stage time with its fraction of the datasheet roofline.  The dQ
    pass also reports the fraction of the products it executes (dQ plus the
    recomputed QK^T and dP: three times its algorithmic flops)."""
    work = stage_work(cfg, z)
    out = {}
    for k, t in stages_ms.items():
        if only is not None and k not in only:
            continue
        kind, w = work[k]
        if k == "attention_delta" and cfg.dtype == "bf16":
            # no kernel of its own: the dQ pass forms rowsum(dO*O)
            out[k] = {"ms": round(t, 4), "in": "attention_dq"}
            continue
        out[k] = {"ms": round(t, 4), **roofline_entry(kind, w, t, cfg.dtype)}
        if k == "attention_dq":
            out[k]["frac_executed"] = round(3 * out[k]["frac"], 4)
    return out


def profile_mean(lay, reps):
    """Mean stage times (ms) over `reps` profiled steps, after one unrecorded
    step (HIP events around each stage on the launch stream)."""
    lay.profile()
    prof = [lay.profile() for _ in range(reps)]
    return {k: sum(p[k] for p in prof) / reps for k in prof[0]}


def src_hash(fname):
    path = os.path.join(ROOT, "hierarchical_sparse_attention_pyramid_amd", "csrc", fname)
    return hashlib.sha256(open(path, "rb").read()).hexdigest()[:16]


def profile_record(json_name, kernel, fname, workload):
    """A kernel's record in a committed profile summary (profiles/<json_name>),
    if it was taken on the current source of that kernel and on this
    workload; else None."""
    path = os.path.join(ROOT, "profiles", json_name)
    if not os.path.exists(path):
        return None
    rec = json.load(open(path)).get(kernel)
    if not rec or rec.get("source_sha256_16") != src_hash(fname) or rec.get("workload") != workload:
        return None
    return rec


def measured_traffic(kernel, fname, workload):
    """HBM bytes per launch from the committed rocprofv3 --pmc summary."""
    rec = profile_record("traffic.json", kernel, fname, workload)
    return rec.get("bytes_per_launch") if rec else None


class Layer:
    """Device tensors of one workload (inputs from the seeded generator)."""

    def __init__(self, cfg, torch, lb, backward=True, scatter="span"):
        from synth import inputs as synth
        t0 = time.time()
        names = ("q", "k", "v", "dout") if backward else ("q", "k", "v")
        host = synth.make_inputs(cfg, tensors=names)
        log(f"[bench] {cfg.name}: inputs drawn in {time.time() - t0:.1f}s")
        self.cfg = cfg
        self.x = {}
        for n in names:
            a = host.pop(n)
            t = torch.from_numpy(a.view("int16")).view(torch.bfloat16) if cfg.dtype == "bf16" \
                else torch.from_numpy(a)
            self.x[n] = t.cuda()
            del a, t
        self.shape = lb.make_shape(cfg.B, cfg.H, cfg.N, cfg.d, cfg.p, cfg.L, cfg.S,
                                   self.x["q"].dtype, scatter=scatter)
        self.bufs = lb.LayerBuffers(self.shape)
        z = self.bufs.sizes
        self.z = z
        self.out = torch.empty_like(self.x["q"])
        if backward:
            self.dq, self.dk, self.dv = (torch.empty_like(self.x["q"]) for _ in range(3))
        self.ws = lb.workspace(max(z.ws_forward, z.ws_backward))
        self.lb = lb

    @classmethod
    def sharing(cls, other, cfg, torch, lb, scatter="span"):
        """A layer of another (p, L, S) or scatter reading on the same input
        tensors (same B, H, N, d)."""
        lay = cls.__new__(cls)
        lay.cfg, lay.x, lay.lb = cfg, other.x, lb
        lay.shape = lb.make_shape(cfg.B, cfg.H, cfg.N, cfg.d, cfg.p, cfg.L, cfg.S,
                                  other.x["q"].dtype, scatter=scatter)
        lay.bufs = lb.LayerBuffers(lay.shape)
        lay.z = lay.bufs.sizes
        lay.out = other.out
        if cfg.backward:
            lay.dq, lay.dk, lay.dv = other.dq, other.dk, other.dv
        lay.ws = lb.workspace(max(lay.z.ws_forward, lay.z.ws_backward))
        return lay

    def forward(self):
        x = self.x
        self.lb.lh_forward(self.shape, x["q"], x["k"], x["v"], self.out, self.bufs, self.ws)

    def step(self):
        self.forward()
        self.lb.lh_backward(self.shape, self.x["dout"], self.bufs, self.dq, self.dk, self.dv,
                            self.ws)

    def outputs(self):
        return (self.out, self.dq, self.dk, self.dv)

    def profile(self):
        x = self.x
        return self.lb.lh_profile_step(self.shape, x["q"], x["k"], x["v"], self.out, self.bufs,
                                       x["dout"], self.dq, self.dk, self.dv, self.ws)


def time_fn(torch, fn, steps, warmup):
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(steps):
        fn()
    b.record()
    torch.cuda.synchronize()
    return a.elapsed_time(b) / steps


def graph_time(torch, lay, steps, warmup):
    """The forward+backward step captured once in a HIP graph and replayed:
    ms per replay (warm-up, then exactly `steps` timed replays), after
    checking that a replay reproduces the eager step's outputs bit for bit.
    The captured work is the eager step's kernels, launch for launch."""
    lay.step()
    torch.cuda.synchronize()
    ref = [t.clone() for t in lay.outputs()]
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        lay.step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        lay.step()
    for t in lay.outputs():
        t.zero_()
    graph.replay()
    torch.cuda.synchronize()
    if not all(torch.equal(a, b) for a, b in zip(lay.outputs(), ref)):
        raise RuntimeError("graph replay differs from the eager step")
    ms = time_fn(torch, graph.replay, steps, warmup)
    del graph
    return ms


def time_median(torch, fn, reps, warmup):
    """Median over `reps` individually timed calls (ms), after `warmup` calls."""
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    ts = []
    for _ in range(reps):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        fn()
        b.record()
        torch.cuda.synchronize()
        ts.append(a.elapsed_time(b))
    return sorted(ts)[len(ts) // 2]


def reference_rates(torch):
    """Rates of plain library work on this GPU, for context (not ceilings of
    the layer's kernels): a 1 GiB device-to-device copy (GB/s, read + write
    bytes) and a 8192^3 bf16 GEMM through torch (TFLOP/s)."""
    a = torch.ones(256 << 20, dtype=torch.float32, device="cuda")
    b = torch.empty_like(a)
    t_copy = time_fn(torch, lambda: b.copy_(a), 10, 2)
    del a, b
    x = torch.randn(8192, 8192, device="cuda").to(torch.bfloat16)
    y = torch.randn(8192, 8192, device="cuda").to(torch.bfloat16)
    t_mm = time_fn(torch, lambda: torch.matmul(x, y), 10, 3)
    del x, y
    torch.cuda.empty_cache()
    return {"copy_GBs": round(2 * (1 << 30) / (t_copy * 1e-3) / 1e9, 1),
            "gemm_bf16_TFLOPs": round(2 * 8192 ** 3 / (t_mm * 1e-3) / 1e12, 1)}


def calibration_copy(torch):
    """A plain 256 MiB device copy, so that HBM counters of a --pmc run can be
    scaled against a kernel of known traffic (256 MiB read + 256 MiB write)."""
    a = torch.ones(64 << 20, dtype=torch.float32, device="cuda")
    b = torch.empty_like(a)
    b.copy_(a)
    torch.cuda.synchronize()


def dense_times(torch, lb, lay, reps, warmup):
    """Same-GPU dense causal attention on the full N (forward, forward+backward):
    median of `reps` timed calls after `warmup` untimed ones."""
    cfg = lay.cfg
    BH, N, d = cfg.B * cfg.H, cfg.N, cfg.d
    shape = lb.make_shape(cfg.B, cfg.H, N, d, cfg.p, 1, N, lay.x["q"].dtype)
    o = torch.empty(cfg.B, cfg.H, N, d, dtype=torch.float32, device="cuda")
    lse = torch.empty(cfg.B, cfg.H, N, dtype=torch.float32, device="cuda")
    q, k, v, g = lay.x["q"], lay.x["k"], lay.x["v"], lay.x["dout"]

    def fwd():
        lb.lh_attention(shape, q, k, v, o, lse)

    t_f = time_median(torch, fwd, reps, warmup)
    log(f"[bench] dense N={N}: forward {t_f:.1f} ms")
    dq, dk, dv = (torch.empty(cfg.B, cfg.H, N, d, dtype=torch.float32, device="cuda")
                  for _ in range(3))
    ws = lb.workspace(lb.lh_query_sizes(shape).ws_attention_backward)

    def fb():
        fwd()
        lb.lh_attention_backward(shape, q, k, v, o, lse, g, dq, dk, dv, ws)

    t_fb = time_median(torch, fb, reps, warmup)
    log(f"[bench] dense N={N}: forward+backward {t_fb:.1f} ms")
    flops_f = BH * 4 * d * causal_pairs(N)
    del o, lse, dq, dk, dv, ws
    torch.cuda.empty_cache()
    return t_f, t_fb, flops_f


def throughput(torch, lay, steps, scatter=None):
    """Forward (and forward+backward where the workload has one) throughput."""
    cfg = lay.cfg
    r = {"workload": cfg.name, "N": cfg.N, "H": cfg.H, "d": cfg.d, "p": cfg.p, "L": cfg.L,
         "S": cfg.S}
    if scatter:
        r["scatter"] = scatter
    t_f = time_fn(torch, lay.forward, steps, 1)
    r["fwd_ms"] = round(t_f, 3)
    r["fwd_tokens_per_s"] = round(cfg.B * cfg.N / (t_f * 1e-3), 1)
    if cfg.backward:
        t_fb = time_fn(torch, lay.step, steps, 1)
        r["fwdbwd_ms"] = round(t_fb, 3)
        r["fwdbwd_tokens_per_s"] = round(cfg.B * cfg.N / (t_fb * 1e-3), 1)
    log(f"[bench] extra {cfg.name}: " + ", ".join(f"{k}={v}" for k, v in r.items()
                                                  if k.endswith("_ms")))
    return r


def block_throughput(torch, cfg, steps):
    """The layer inside an attention block (Q/K/V and output projections,
    autograd through lh_forward / lh_backward), model width D = H * d, at the
    workload's shape; forward+backward including the projection GEMMs."""
    from hierarchical_sparse_attention_pyramid_amd.layer import LighthouseAttention
    from synth import inputs as synth
    D = cfg.H * cfg.d
    m = LighthouseAttention(D, cfg.H, cfg.d, cfg.p, cfg.L, cfg.S)
    x = torch.from_numpy(synth.block_tensor(900, (cfg.B * cfg.N, D), "bf16").view("int16"))
    x = x.view(torch.bfloat16).cuda().view(cfg.B, cfg.N, D).requires_grad_(True)
    dy = torch.randn(cfg.B, cfg.N, D, device="cuda").to(torch.bfloat16)

    def step():
        for t in (x, m.wq, m.wk, m.wv, m.wo):
            t.grad = None
        m(x).backward(dy)

    t = time_fn(torch, step, steps, 2)
    with torch.no_grad():
        t_f = time_fn(torch, lambda: m(x), steps, 1)
    gemm_flops = 3 * 2 * 4 * cfg.B * cfg.N * D * D  # 4 projections, forward + two backward GEMMs each
    r = {"workload": f"block_{cfg.name}", "D": D, "H": cfg.H, "d": cfg.d, "N": cfg.N, "p": cfg.p,
         "L": cfg.L, "S": cfg.S, "fwd_ms": round(t_f, 3), "fwdbwd_ms": round(t, 3),
         "fwdbwd_tokens_per_s": round(cfg.B * cfg.N / (t * 1e-3), 1),
         "projection_gemm_tflop": round(gemm_flops / 1e12, 3)}
    log(f"[bench] block {cfg.name}: forward {t_f:.3f} ms, forward+backward {t:.3f} ms")
    del m, x, dy
    torch.cuda.empty_cache()
    return r


def cpu_single_thread(names):
    """Single-thread oracle forward time on the first head of small workloads."""
    from threadpoolctl import threadpool_limits

    from oracle import lighthouse as O
    from synth import inputs as synth
    out = {}
    with threadpool_limits(limits=1):
        for name in names:
            cfg = synth.CONFIGS[name]
            x = synth.make_inputs(cfg, tensors=("q", "k", "v"), heads=[(0, 0)])
            t0 = time.perf_counter()
            O.forward_head(x["q"][0], x["k"][0], x["v"][0], cfg.p, cfg.L, cfg.S, cfg.dtype)
            out[name] = {"fwd_s_one_head": round(time.perf_counter() - t0, 3), "threads": 1}
    return out


def _oracle_head(args):
    """One head of the oracle, forward+backward, in a single-threaded worker
    process; returns (start, end) wall-clock seconds of the oracle call and
    the BLAS threads used.  Input generation comes before the start."""
    name, b, h = args
    from threadpoolctl import threadpool_info, threadpool_limits

    from oracle import lighthouse as O
    from synth import inputs as synth
    cfg = synth.CONFIGS[name]
    x = synth.make_inputs(cfg, tensors=("q", "k", "v", "dout"), heads=[(b, h)])
    with threadpool_limits(limits=1):
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
        t0 = time.time()
        f = O.forward_head(x["q"][0], x["k"][0], x["v"][0], cfg.p, cfg.L, cfg.S, cfg.dtype)
        O.backward_head(x["dout"][0], f, cfg.p, cfg.L, cfg.dtype)
        return t0, time.time(), threads


def cpu_baseline(cfg, workers=16):
    """The oracle as it stands, forward+backward on every head of the
    headline workload: the B*H heads run concurrently in `workers`
    single-threaded processes (one core each); the layer time is the wall
    time from the first head's oracle start to the last head's end."""
    import multiprocessing
    from concurrent.futures import ProcessPoolExecutor
    heads = [(cfg.name, b, h) for b in range(cfg.B) for h in range(cfg.H)]
    w = min(workers, len(heads), os.cpu_count() or 1)
    with ProcessPoolExecutor(max_workers=w, mp_context=multiprocessing.get_context("spawn")) as ex:
        res = list(ex.map(_oracle_head, heads))
    t_layer = max(r[1] for r in res) - min(r[0] for r in res)
    per_head = [r[1] - r[0] for r in res]
    return {"value": round(cfg.B * cfg.N / t_layer, 2), "unit": "tokens/s", "cores": w,
            "kind": "oracle",
            "sample": f"all {len(heads)} heads of {cfg.name}, forward+backward, run concurrently "
                      f"in {w} single-threaded processes ({max(r[2] for r in res)} BLAS thread "
                      f"each); layer time {t_layer:.1f} s = first head's start to last head's "
                      f"end (one head {min(per_head):.1f}-{max(per_head):.1f} s); "
                      f"{os.cpu_count()} host cpus visible"}


def roofline_of(cfg, z, stages_ms):
    """`roofline` object for the step's dominant kernel: achieved work per
    launch over its mean HIP-event duration, beside the committed rocprofv3
    average of the same kernel on the same workload (when the summary matches
    the kernel's current source)."""
    work = stage_work(cfg, z)
    dom = max((k for k in stages_ms if k in KERNEL_OF_STAGE), key=lambda k: stages_ms[k])
    kname, kfile = KERNEL_OF_STAGE[dom]
    kind, w = work[dom]
    roof = roofline_entry(kind, w, stages_ms[dom], cfg.dtype)
    roof["kernel"] = kname
    roof["timing"] = "hip_events_mean"
    roof["avg_us"] = round(stages_ms[dom] * 1e3, 1)
    roof["traffic"] = measured_traffic(kname, kfile, cfg.name)
    rec = profile_record("kernel_avg.json", kname, kfile, cfg.name)
    if rec:
        rp = roofline_entry(kind, w, rec["avg_us"] * 1e-3, cfg.dtype)
        roof["rocprof_avg_us"] = rec["avg_us"]
        roof["frac_rocprof"] = rp["frac"]
        roof["rocprof_summary"] = rec["summary"]
    return roof


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--profile-reps", type=int, default=10)
    ap.add_argument("--dense-reps", type=int, default=3)
    ap.add_argument("--no-long", action="store_true", help="skip the 512K comparison")
    ap.add_argument("--no-cpu", action="store_true", help="skip the oracle CPU baseline")
    ap.add_argument("--no-extras", action="store_true",
                    help="skip the other workload shapes, the causal scatter lines and the "
                         "ablations' operating points")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py: the layer runs on one GPU per process; --gpus {args.gpus} is not supported "
              "(the layer is not sharded across GPUs)", file=sys.stderr)
        sys.exit(2)

    import torch

    from hierarchical_sparse_attention_pyramid_amd import binding as lb
    from synth import inputs as synth
    lb.load_library()
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    calibration_copy(torch)
    rates = reference_rates(torch)
    log(f"[bench] reference rates (context, not ceilings): {rates}")

    cfg = synth.CONFIGS[HEADLINE]
    lay = Layer(cfg, torch, lb)
    ms_eager = time_fn(torch, lay.step, args.steps, args.warmup)
    ms = graph_time(torch, lay, args.steps, args.warmup)
    tokens = cfg.B * cfg.N
    log(f"[bench] {cfg.name}: {ms:.3f} ms per forward+backward step replayed from a HIP graph "
        f"({ms_eager:.3f} ms launched eagerly)")
    ms_fwd = time_fn(torch, lay.forward, args.steps, 2)
    stages_ms = profile_mean(lay, args.profile_reps)
    stages = stage_table(cfg, lay.z, stages_ms)
    roof = roofline_of(cfg, lay.z, stages_ms)
    log(f"[bench] stages (ms): " + ", ".join(f"{k}={v:.4f}" for k, v in stages_ms.items()))
    extras, causal, workloads = [], {}, {}
    if not args.no_extras:
        c = Layer.sharing(lay, cfg, torch, lb, scatter="causal")
        c_ms = graph_time(torch, c, args.steps, args.warmup)
        causal[cfg.name] = {"fwdbwd_ms": round(c_ms, 4),
                            "fwdbwd_tokens_per_s": round(tokens / (c_ms * 1e-3), 1),
                            "stages": stage_table(cfg, c.z, profile_mean(c, 5),
                                                  only=("scatter", "scatter_bwd"))}
        log(f"[bench] {cfg.name} with the causal scatter: {c_ms:.3f} ms per step (graph replay)")
        del c
        for name in ("op_n98k_p4_bf16", "op_n98k_p2_bf16"):
            e = Layer.sharing(lay, synth.CONFIGS[name], torch, lb)
            extras.append(throughput(torch, e, 5))
            del e
    del lay
    torch.cuda.empty_cache()

    long_ctx = None
    if not args.no_long:
        lcfg = synth.CONFIGS[LONG]
        ll = Layer(lcfg, torch, lb)
        l_fb = time_fn(torch, ll.step, max(3, args.steps // 4), 2)
        l_f = time_fn(torch, ll.forward, max(3, args.steps // 4), 1)
        lprof = profile_mean(ll, 3)
        log(f"[bench] {lcfg.name}: forward {l_f:.2f} ms, forward+backward {l_fb:.2f} ms")
        d_f, d_fb, d_flops = dense_times(torch, lb, ll, args.dense_reps, 1)
        long_ctx = {
            "workload": lcfg.name, "N": lcfg.N, "H": lcfg.H, "d": lcfg.d, "L": lcfg.L,
            "S": lcfg.S,
            "lighthouse_fwd_ms": round(l_f, 3), "lighthouse_fwdbwd_ms": round(l_fb, 3),
            "lighthouse_fwdbwd_tokens_per_s": round(lcfg.B * lcfg.N / (l_fb * 1e-3), 1),
            "lighthouse_stages": stage_table(lcfg, ll.z, lprof),
            "dense_fwd_ms": round(d_f, 2), "dense_fwdbwd_ms": round(d_fb, 2),
            "dense_timing": f"median of {args.dense_reps} calls after 1 warm-up",
            "dense_fwd_tflops": round(d_flops / (d_f * 1e-3) / 1e12, 1),
            "speedup_fwd": round(d_f / l_f, 2), "speedup_fwdbwd": round(d_fb / l_fb, 2),
        }
        if not args.no_extras:
            c = Layer.sharing(ll, lcfg, torch, lb, scatter="causal")
            c_fb = time_fn(torch, c.step, max(3, args.steps // 4), 2)
            causal[lcfg.name] = {"fwdbwd_ms": round(c_fb, 3),
                                 "fwdbwd_tokens_per_s": round(lcfg.B * lcfg.N / (c_fb * 1e-3), 1),
                                 "speedup_fwdbwd": round(d_fb / c_fb, 2)}
            log(f"[bench] {lcfg.name} with the causal scatter: forward+backward {c_fb:.2f} ms")
            del c
            for name in ("op_n512k_p4_bf16", "op_n512k_p2_bf16"):
                e = Layer.sharing(ll, synth.CONFIGS[name], torch, lb)
                extras.append(throughput(torch, e, 3))
                del e
        del ll
        torch.cuda.empty_cache()

    if not args.no_extras:
        extras.append(block_throughput(torch, synth.CONFIGS[HEADLINE], 10))
        # the other workloads: time and per-stage table (forward stages only
        # where the workload is forward only)
        for name in ("fwd_n4k_fp32", "fwd_n32k_bf16", "dense_n2k_bf16", "long_n1m_bf16"):
            wcfg = synth.CONFIGS[name]
            e = Layer(wcfg, torch, lb)  # dout drawn too: the stage profile runs the backward
            reps = 3 if wcfg.N >= 1 << 20 else 10
            r = throughput(torch, e, reps)
            r["stages"] = stage_table(wcfg, e.z, profile_mean(e, 3 if reps == 3 else 5),
                                      only=None if wcfg.backward else FORWARD_STAGES)
            workloads[name] = r
            if name == "long_n1m_bf16":
                o = Layer.sharing(e, synth.CONFIGS["op_n1m_p4_bf16"], torch, lb)
                extras.append(throughput(torch, o, 2))
                del o
            del e
            torch.cuda.empty_cache()

    cpu = None if args.no_cpu else cpu_baseline(cfg)
    if cpu:
        log(f"[bench] cpu oracle: {cpu['value']} tokens/s ({cpu['sample']})")
        cpu["single_thread"] = cpu_single_thread(("fwd_n4k_fp32", "fwd_n32k_bf16", "train_n98k_bf16"))
        log(f"[bench] cpu oracle, one thread: {cpu['single_thread']}")

    rec = {
        "metric": METRIC,
        "value": round(tokens / (ms * 1e-3), 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": cfg.dtype,
        "data": "synthetic",
        "config": {"workload": cfg.name, "B": cfg.B, "H": cfg.H, "N": cfg.N, "d": cfg.d,
                   "p": cfg.p, "L": cfg.L, "S": cfg.S, "pass": "forward+backward",
                   "scatter": "span", "launch": "hip_graph_replay",
                   "eager_ms_per_step": round(ms_eager, 4), "forward_only_ms": round(ms_fwd, 4)},
        "roofline": roof,
        "cpu_baseline": cpu,
        "stages": stages,
        "causal_scatter": causal,
        "long_context": long_ctx,
        "workloads": workloads,
        "reference_rates": rates,
        "extras": extras,
    }
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
