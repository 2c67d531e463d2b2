"""Seeded synthetic inputs shaped like the workloads the Lighthouse pages use.

Recipe (the same for every consumer):
  * one independent numpy Generator per (config seed, tensor, b, h), seeded with
    SeedSequence([1000*cfg + tensor_id, b, h]); tensor ids q=0, k=1, v=2, dout=3;
  * q, k, v rows: z * s with z ~ N(0,1)^d (float32 draws) and one scale
    s = exp(0.5 * N(0,1)) per row (a lognormal(0, 0.5) per token), so that
    norms -- and hence scores -- spread;
  * dout rows: N(0,1)^d, no per-row scale;
  * optional planted rows: 1% of positions, drawn once per config from
    Generator(1000*cfg + 4), shared by all heads and by q/k/v, scaled by 8
    (a power of two, exact in both storage types);
  * fp32 storage keeps the float32 draw; bf16 storage rounds it once, to
    nearest-even, to the upper 16 bits.
Per-head seeding lets a checker regenerate any single head without drawing
the whole tensor.
"""
from __future__ import annotations

import dataclasses
import os
import multiprocessing
from concurrent.futures import ProcessPoolExecutor

import numpy as np

TENSOR_IDS = {"q": 0, "k": 1, "v": 2, "dout": 3}


@dataclasses.dataclass(frozen=True)
class Config:
    name: str
    seed: int          # the "cfg" number in the seed recipe
    B: int
    H: int
    N: int
    d: int
    p: int
    L: int
    S: int
    dtype: str         # "fp32" or "bf16"
    planted: bool = False
    backward: bool = False


# The five workload shapes of the layer (plus the degenerate S = N case).
CONFIGS = {
    "fwd_n4k_fp32": Config("fwd_n4k_fp32", 1, 1, 2, 4096, 64, 4, 3, 512, "fp32"),
    "fwd_n32k_bf16": Config("fwd_n32k_bf16", 2, 1, 16, 32768, 128, 4, 4, 4096, "bf16"),
    "dense_n2k_bf16": Config("dense_n2k_bf16", 6, 1, 16, 2048, 128, 4, 1, 2048, "bf16"),
    "train_n98k_bf16": Config("train_n98k_bf16", 3, 1, 16, 98304, 64, 4, 5, 8192, "bf16",
                              backward=True),
    "long_n512k_bf16": Config("long_n512k_bf16", 4, 1, 16, 524288, 128, 4, 6, 16384, "bf16",
                              backward=True),
    "long_n1m_bf16": Config("long_n1m_bf16", 5, 1, 16, 1048576, 128, 4, 7, 32768, "bf16",
                            planted=True, backward=True),
    # The operating points the ablations favour (bitsgeniais post,
    # "Configurações e Velocidade"; gist.science technical summary §4):
    # L = 3 levels, k = 1536 selected candidates, so S = N / p^2 + 1536 (the
    # whole coarsest level plus k).
    "op_n98k_p4_bf16": Config("op_n98k_p4_bf16", 7, 1, 16, 98304, 64, 4, 3, 98304 // 16 + 1536,
                              "bf16", backward=True),
    "op_n98k_p2_bf16": Config("op_n98k_p2_bf16", 8, 1, 16, 98304, 64, 2, 3, 98304 // 4 + 1536,
                              "bf16", backward=True),
    "op_n512k_p4_bf16": Config("op_n512k_p4_bf16", 9, 1, 16, 524288, 128, 4, 3,
                               524288 // 16 + 1536, "bf16", backward=True),
    "op_n512k_p2_bf16": Config("op_n512k_p2_bf16", 10, 1, 16, 524288, 128, 2, 3,
                               524288 // 4 + 1536, "bf16", backward=True),
    "op_n1m_p4_bf16": Config("op_n1m_p4_bf16", 11, 1, 16, 1048576, 128, 4, 3,
                             1048576 // 16 + 1536, "bf16", backward=True),
}


def bf16_bits_from_f32(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (nearest, ties to even); return uint16 bits."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    r = (u >> 16) & np.uint32(1)
    r += np.uint32(0x7FFF)
    r += u
    r >>= 16
    nan = (u & np.uint32(0x7FFFFFFF)) > np.uint32(0x7F800000)
    if nan.any():
        r[nan] = (u[nan] >> 16) | 0x40
    return r.astype(np.uint16)


def f32_from_bf16_bits(b: np.ndarray) -> np.ndarray:
    """Exact widening of bfloat16 bit patterns to float32."""
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def storage_to_f32(x: np.ndarray, dtype: str) -> np.ndarray:
    return f32_from_bf16_bits(x) if dtype == "bf16" else np.asarray(x, dtype=np.float32)


def planted_positions(cfg_seed: int, N: int) -> np.ndarray:
    rng = np.random.default_rng(1000 * cfg_seed + 4)
    return np.sort(rng.choice(N, N // 100, replace=False))


def head_tensor(cfg_seed: int, tensor: str, b: int, h: int, N: int, d: int,
                planted: bool = False) -> np.ndarray:
    """float32 [N, d] draw for one (tensor, b, h), before storage rounding."""
    tid = TENSOR_IDS[tensor]
    rng = np.random.default_rng(np.random.SeedSequence([1000 * cfg_seed + tid, b, h]))
    z = rng.standard_normal((N, d), dtype=np.float32)
    if tensor == "dout":
        return z
    s = np.exp(0.5 * rng.standard_normal(N)).astype(np.float32)
    z *= s[:, None]
    if planted:
        z[planted_positions(cfg_seed, N)] *= np.float32(8.0)
    return z


def block_tensor(seed: int, shape, dtype: str, scale: float = 1.0) -> np.ndarray:
    """Seeded N(0, scale^2) tensor in storage form (block inputs and projection
    weights of the attention-block tests): float32 draws, bf16 rounded once."""
    x = np.random.default_rng(seed).standard_normal(shape, dtype=np.float32) * np.float32(scale)
    return bf16_bits_from_f32(x) if dtype == "bf16" else x


def _head_storage(args):
    cfg_seed, tensor, b, h, N, d, planted, dtype = args
    x = head_tensor(cfg_seed, tensor, b, h, N, d, planted)
    return bf16_bits_from_f32(x) if dtype == "bf16" else x


def make_inputs(cfg: Config, tensors=("q", "k", "v"), heads=None, N=None,
                workers: int | None = None) -> dict:
    """Storage-typed arrays [B, H', N, d] (uint16 bf16 bits or float32).

    ``heads`` restricts the draw to a list of (b, h) pairs (the result then has
    shape [len(heads), N, d]); ``N`` overrides the config's length.  Large
    draws are spread over worker processes (one job per head and tensor); the
    values do not depend on how the work is split.
    """
    N = cfg.N if N is None else N
    pairs = [(b, h) for b in range(cfg.B) for h in range(cfg.H)] if heads is None else list(heads)
    jobs = [(cfg.seed, t, b, h, N, cfg.d, cfg.planted and t != "dout", cfg.dtype)
            for t in tensors for (b, h) in pairs]
    workers = workers or min(16, os.cpu_count() or 1)
    if len(jobs) > 1 and N * cfg.d >= (1 << 22) and workers > 1:
        ctx = multiprocessing.get_context("spawn")
        with ProcessPoolExecutor(min(workers, len(jobs)), mp_context=ctx) as ex:
            parts = list(ex.map(_head_storage, jobs))
    else:
        parts = [_head_storage(j) for j in jobs]
    out = {}
    for i, t in enumerate(tensors):
        arr = np.stack(parts[i * len(pairs):(i + 1) * len(pairs)])
        out[t] = arr.reshape(cfg.B, cfg.H, N, cfg.d) if heads is None else arr
    return out
