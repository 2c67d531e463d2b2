"""Host-only checks of the C ABI: the library loads, exports every declared
symbol, sizes agree with the pyramid geometry, and bad arguments are rejected
before anything is launched (no GPU needed)."""
import ctypes
import os
import re

import pytest

from oracle import lighthouse as O

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "lighthouse.h")


@pytest.fixture(scope="module")
def lb():
    from hierarchical_sparse_attention_pyramid_amd import binding
    binding.load_library()
    return binding


def declared_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:lh_status|const char\s*\*)\s*(lh_\w+)\s*\(", text, re.M)))


def test_header_declares_the_layer_calls():
    names = declared_functions()
    for n in ("lh_build_pyramid", "lh_score", "lh_topk", "lh_gather", "lh_attention",
              "lh_scatter", "lh_forward", "lh_backward", "lh_query_sizes", "lh_last_error"):
        assert n in names


def test_every_declared_symbol_is_exported(lb):
    lib = ctypes.CDLL(lb.LIB_PATH)
    for n in declared_functions():
        assert hasattr(lib, n), f"{n} not exported"
    assert set(declared_functions()) == set(lb.EXPORTS)


@pytest.mark.parametrize("N,p,L,S", [(98304, 4, 5, 8192), (4096, 4, 3, 512), (729, 3, 4, 100),
                                     (2048, 4, 1, 2048), (1024, 2, 9, 150)])
def test_sizes_match_geometry(lb, N, p, L, S):
    z = lb.lh_query_sizes(lb.make_shape(1, 16, N, 64, p, L, S, 1))
    sizes = O.level_sizes(N, p, L)
    assert z.M == sum(sizes) and z.n_coarse == sizes[-1]
    assert z.C == z.M - z.n_coarse and z.K == S - z.n_coarse
    assert z.bytes_pos == 16 * z.M * 4 and z.bytes_sub == 16 * S * 64 * 2
    assert z.ws_forward >= z.ws_topk and z.ws_backward > 0


@pytest.mark.parametrize("args,status", [
    ((1, 1, 100, 64, 4, 3, 20, 1), 1),        # N not divisible by p^(L-1)
    ((1, 1, 64, 96, 4, 3, 20, 1), 2),         # unsupported head dim
    ((1, 1, 64, 64, 4, 3, 3, 1), 1),          # S below the coarsest level
    ((1, 1, 64, 64, 4, 3, 85, 1), 1),         # S above M
    ((1, 1, 64, 64, 1, 3, 20, 1), 1),         # p < 2
    ((1, 1, 65 * 65, 64, 65, 3, 80, 1), 2),   # p > 64
    ((1, 1, 64, 64, 4, 0, 20, 1), 1),         # L < 1
    ((1, 1, 1 << 17, 64, 2, 17, 20, 1), 2),   # too many levels
    ((1, 1, 64, 64, 4, 3, 20, 7), 1),         # unknown dtype
    ((0, 1, 64, 64, 4, 3, 20, 1), 1),         # empty batch
    ((1, 4096, 1 << 20, 64, 4, 3, 1 << 16, 1), 2),  # B*H*M >= 2^31
    ((256, 256, 64, 64, 4, 3, 20, 1), 2),     # B*H above the grid's y limit
])
def test_bad_shapes_are_rejected(lb, args, status):
    with pytest.raises(lb.LighthouseError) as ei:
        lb.lh_query_sizes(lb.Shape(*args))
    assert ei.value.status == status
    assert lb.load_library().lh_last_error().decode() != ""


def test_null_pointers_and_small_workspace_are_rejected_without_a_gpu(lb):
    lib = lb.load_library()
    shape = lb.make_shape(1, 2, 256, 64, 4, 3, 40, 1)
    # null q: rejected on the host, nothing launched
    st = lib.lh_build_pyramid(ctypes.byref(shape), None, 1, 1, 1, 1, 1, 1, 1 << 20, None)
    assert st == 1 and b"q is null" in lib.lh_last_error()
    # workspace too small for the top-K (heads above 16384 candidates need one)
    big = lb.make_shape(1, 2, 98304, 64, 4, 5, 8192, 1)
    zb = lb.lh_query_sizes(big)
    assert zb.ws_topk > 0
    st = lib.lh_topk(ctypes.byref(big), 1, 1, 1, zb.ws_topk - 1, None)
    assert st == 3
    z = lb.lh_query_sizes(shape)
    assert z.ws_topk == 0  # small heads: selected in one workgroup's LDS
    st = lib.lh_forward(ctypes.byref(shape), 1, 1, 1, 1, None, 1, z.ws_forward, None)
    assert st == 1 and b"buffers" in lib.lh_last_error()


def test_misaligned_workspace_is_rejected_without_a_gpu(lb):
    lib = lb.load_library()
    big = lb.make_shape(1, 2, 98304, 64, 4, 5, 8192, 1)
    zb = lb.lh_query_sizes(big)
    # nothing is launched: the workspace check fails first
    st = lib.lh_topk(ctypes.byref(big), 4096, 4096, 4096 + 8, zb.ws_topk, None)
    assert st == 1 and b"16-byte aligned" in lib.lh_last_error()
    assert lib.lh_topk(ctypes.byref(big), 4096, 4096, 4096 + 256, zb.ws_topk - 1, None) == 3


def _strided(lb, qkv=None, out=None, B=2, H=4, N=256, d=64, dtype=1):
    return lb.make_shape(B, H, N, d, 4, 3, 40, dtype, qkv, out)


@pytest.mark.parametrize("qkv,out,ok", [
    ((256 * 3 * 4 * 64, 64, 3 * 4 * 64), None, True),           # q/k/v slices of a packed [B,N,3,H,d]
    (None, (256 * 4 * 64, 64, 4 * 64), True),                   # token-major output [B,N,H,d]
    ((4 * 256 * 64, 256 * 64, 64), (4 * 256 * 64, 256 * 64, 64), True),  # packed, given explicitly
    ((256 * 4 * 64, 64, 64), None, False),                      # heads and tokens overlap
    (None, (256 * 4 * 64, 64 * 256, 60), False),                # token rows overlap (60 < d)
    ((256 * 4 * 68, 68, 4 * 68), None, False),                  # 136-byte head stride: not 16-byte multiple
    ((0, 64, 4 * 64), None, False),                             # zero stride on a dimension of extent 2
    ((4 * 256 * 64, 256 * 64, -64), None, False),               # negative stride
])
def test_token_strides_are_validated(lb, qkv, out, ok):
    shape = _strided(lb, qkv, out)
    if ok:
        lb.lh_query_sizes(shape)
    else:
        with pytest.raises(lb.LighthouseError) as ei:
            lb.lh_query_sizes(shape)
        assert ei.value.status == 1 and b"strides" in lb.load_library().lh_last_error()


def test_stride_of_an_extent_one_dimension_is_ignored(lb):
    # B = 1: any batch stride, even one no row layout could use
    lb.lh_query_sizes(_strided(lb, (3, 64, 4 * 64), None, B=1))


def test_misaligned_token_pointer_is_rejected_without_a_gpu(lb):
    lib = lb.load_library()
    shape = lb.make_shape(1, 2, 256, 64, 4, 3, 40, 1)
    st = lib.lh_score(ctypes.byref(shape), 4096 + 8, 4096, 4096, None, 0, None)
    assert st == 1 and b"16-byte aligned" in lib.lh_last_error()


@pytest.mark.parametrize("args", [
    (1, 1, 64 * 64, 64, 64, 2, 64, 1),          # largest pooling factor, p = 64
    (1, 1, 1 << 15, 64, 2, 16, 2, 1),           # deepest pyramid, L = 16 (coarsest level: 2 entries)
    (1, 1, 4096, 128, 4, 3, 5376, 0),           # S = M: every entry selected
    (1, 1, 4096, 128, 4, 3, 256, 0),            # S = n_coarse: K = 0
    (3, 5, 1000, 64, 10, 4, 1, 1),              # non-power-of-two p, one coarse entry per head
])
def test_limit_shapes_are_accepted(lb, args):
    z = lb.lh_query_sizes(lb.Shape(*args))
    B, H, N, d, p, L, S, dt = args
    sizes = O.level_sizes(N, p, L)
    assert z.M == sum(sizes) and z.K == S - sizes[-1]


@pytest.mark.parametrize("N,d,ok", [
    (1 << 23, 128, True),    # S * d * 2 = 2^31 bytes per head: the attention's buffer
                             # descriptors take it as an unsigned 32-bit record count
    (1 << 24, 64, True),     # the same byte count at d = 64
    (1 << 24, 128, False),   # M * d = 2^31: rejected before any launch
])
def test_subsequence_byte_size_limit(lb, N, d, ok):
    """Largest accepted subsequence: M * d < 2^31, so every head's S * d * 2
    bytes stays below 2^32 (dense causal attention, L = 1, S = N)."""
    shape = lb.Shape(1, 1, N, d, 4, 1, N, 1)
    if ok:
        z = lb.lh_query_sizes(shape)
        assert z.bytes_sub == N * d * 2 and z.bytes_sub < 1 << 32
    else:
        with pytest.raises(lb.LighthouseError) as ei:
            lb.lh_query_sizes(shape)
        assert ei.value.status == 2


@pytest.mark.parametrize("B,H,N,d,p,L,S,one_pass", [
    (1, 16, 98304, 64, 4, 5, 8192, True),      # levels 1-3 in registers, 4 through LDS
    (1, 16, 524288, 128, 4, 6, 16384, True),   # levels 4 and 5 through LDS
    (1, 16, 1048576, 128, 4, 7, 32768, False),  # level 6 needs a further pass
    (1, 2, 4096, 128, 2, 12, 700, False),      # p = 2: register levels only
])
def test_pooling_passes_from_the_plan(lb, B, H, N, d, p, L, S, one_pass):
    """The token pass forms the levels whose spans divide its workgroup's rows
    through LDS; only deeper pyramids need float32 sums for a further pass
    (workspace ws_build_pyramid)."""
    z = lb.lh_query_sizes(lb.make_shape(B, H, N, d, p, L, S, 1))  # bf16
    assert (z.ws_build_pyramid == 0) == one_pass
