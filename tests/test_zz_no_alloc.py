"""lh_topk_noalloc (the top-K with its scratch in a static device array, for
callers that cannot allocate) against lh_topk with a workspace: bit-identical
selections on two calls in a row, the second on a smaller input, plus the
host-side rejection of shapes whose scratch exceeds the array."""
from __future__ import annotations

import ctypes

import numpy as np
import pytest
import torch

from synth import inputs as synth


def test_oversized_shape_is_rejected_on_the_host():
    from hierarchical_sparse_attention_pyramid_amd import binding as lb
    shape = lb.make_shape(1, 256, 98304, 64, 4, 5, 8192, 1)  # ~140 MB of top-K scratch
    assert lb.lh_query_sizes(shape).ws_topk > 16 << 20
    lib = lb.load_library()
    st = lib.lh_topk_noalloc(ctypes.byref(shape), 4096, 4096, None)
    assert st == 3 and b"static" in lib.lh_last_error()


def _scores(lb, B, H, N, d, p, L, S, seed):
    """Layer-like scores from lh_score on synthetic q, k (plus a tied block)."""
    q = np.stack([np.stack([synth.head_tensor(seed, "q", b, h, N, d) for h in range(H)])
                  for b in range(B)])
    k = np.stack([np.stack([synth.head_tensor(seed, "k", b, h, N, d) for h in range(H)])
                  for b in range(B)])
    q[:, :, 64:128] = q[:, :, 0:1]   # equal scores across a run of tokens: ties at the cut
    k[:, :, 64:128] = k[:, :, 0:1]
    qb, kb = (torch.from_numpy(synth.bf16_bits_from_f32(a).view(np.int16)).view(torch.bfloat16).cuda()
              for a in (q, k))
    shape = lb.make_shape(B, H, N, d, p, L, S, torch.bfloat16)
    z = lb.lh_query_sizes(shape)
    score = torch.empty(B, H, z.M, dtype=torch.float32, device="cuda")
    lb.lh_score(shape, qb, kb, score)
    return shape, z, score


@pytest.mark.gpu
def test_noalloc_topk_matches_topk_twice(gpu_lib):
    lb = gpu_lib
    for B, H, N, d, p, L, S, seed in ((1, 16, 98304, 64, 4, 5, 8192, 61),   # the 98K workload
                                      (2, 3, 24576, 128, 4, 3, 2000, 62),   # a smaller one
                                      (2, 3, 4096, 128, 4, 3, 700, 63)):    # one of <= 16384
                                                                            # candidates a head
        print(f"[gpu-noalloc] B={B} H={H} N={N} p={p} L={L} S={S}", flush=True)
        shape, z, score = _scores(lb, B, H, N, d, p, L, S, seed)
        ref = torch.full((B, H, z.K), -7, dtype=torch.int32, device="cuda")
        lb.lh_topk(shape, score, ref, lb.workspace(z.ws_topk))
        got = torch.full((B, H, z.K), -9, dtype=torch.int32, device="cuda")
        lb.lh_topk_noalloc(shape, score, got)
        torch.cuda.synchronize()
        assert torch.equal(got, ref), "lh_topk_noalloc differs from lh_topk"
        assert bool((ref >= 0).all())
