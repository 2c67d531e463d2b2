"""ctypes binding of liblighthouse.so (include/lighthouse.h).

Argument marshalling only: every entry point takes torch tensors (or None),
passes their device pointers to the C ABI on the current HIP stream, and
raises LighthouseError on a non-zero status.  No step of the layer runs here;
torch is used to allocate device memory in the `alloc_*` helpers.
"""
from __future__ import annotations

import contextlib
import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "liblighthouse.so")

LH_FP32, LH_BF16 = 0, 1
LH_SCATTER_SPAN, LH_SCATTER_CAUSAL = 0, 1
SCATTER = {"span": LH_SCATTER_SPAN, "causal": LH_SCATTER_CAUSAL}
STATUS = {0: "LH_OK", 1: "LH_EINVAL", 2: "LH_EUNSUPPORTED", 3: "LH_EWORKSPACE", 4: "LH_EHIP"}
DTYPES = {torch.float32: LH_FP32, torch.bfloat16: LH_BF16}


class LighthouseError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"{STATUS.get(status, status)}: {msg}")
        self.status = status


class Shape(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int64), ("H", ctypes.c_int64), ("N", ctypes.c_int64),
                ("d", ctypes.c_int64), ("p", ctypes.c_int32), ("L", ctypes.c_int32),
                ("S", ctypes.c_int64), ("dtype", ctypes.c_int32),
                ("qkv_stride", ctypes.c_int64 * 3), ("out_stride", ctypes.c_int64 * 3),
                ("scatter", ctypes.c_int32)]


class Sizes(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int64) for n in ("M", "C", "K", "n_coarse")] + \
               [(n, ctypes.c_size_t) for n in (
                   "bytes_qkv", "bytes_pyramid", "bytes_score", "bytes_sel", "bytes_sub_idx",
                   "bytes_pos", "bytes_sub", "bytes_sub_f32", "bytes_lse",
                   "ws_build_pyramid", "ws_score", "ws_topk", "ws_gather",
                   "ws_attention_backward", "ws_scatter_backward", "ws_forward", "ws_backward")]


class Buffers(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in (
        "pq", "pk", "pv", "score", "sel", "sub_idx", "pos", "qs", "ks", "vs", "os", "lse")]


EXPORTS = ["lh_query_sizes", "lh_last_error", "lh_build_pyramid", "lh_score", "lh_topk",
           "lh_gather", "lh_attention", "lh_scatter", "lh_forward", "lh_scatter_backward",
           "lh_attention_backward", "lh_gather_backward", "lh_backward", "lh_profile_step",
           "lh_topk_noalloc"]

PROFILE_STAGES = ["pyramid_score", "topk", "gather", "attention_fwd", "scatter",
                  "scatter_bwd", "attention_delta", "attention_dkdv", "attention_dq",
                  "gather_bwd"]

_lib = None


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load the built library; fails loudly when it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with `python hierarchical_sparse_attention_pyramid_amd/build.py` "
                           "or hierarchical_sparse_attention_pyramid_amd/build.py")
    lib = ctypes.CDLL(path)
    P, S = ctypes.c_void_p, ctypes.c_size_t
    sp = ctypes.POINTER(Shape)
    sig = {
        "lh_query_sizes": [sp, ctypes.POINTER(Sizes)],
        "lh_build_pyramid": [sp, P, P, P, P, P, P, P, S, P],
        "lh_score": [sp, P, P, P, P, S, P],
        "lh_topk": [sp, P, P, P, S, P],
        "lh_topk_noalloc": [sp, P, P, P],
        "lh_gather": [sp, P, P, P, P, P, P, P, P, P, P, P, P, P, S, P],
        "lh_attention": [sp, P, P, P, P, P, P],
        "lh_scatter": [sp, P, P, P, P],
        "lh_forward": [sp, P, P, P, P, ctypes.POINTER(Buffers), P, S, P],
        "lh_scatter_backward": [sp, P, P, P, P, S, P],
        "lh_attention_backward": [sp, P, P, P, P, P, P, P, P, P, P, S, P],
        "lh_gather_backward": [sp, P, P, P, P, P, P, P, P],
        "lh_backward": [sp, P, ctypes.POINTER(Buffers), P, P, P, P, S, P],
        "lh_profile_step": [sp, P, P, P, P, ctypes.POINTER(Buffers), P, P, P, P, P, S,
                            ctypes.POINTER(ctypes.c_float), P],
    }
    for name, args in sig.items():
        fn = getattr(lib, name)
        fn.argtypes = args
        fn.restype = ctypes.c_int
    lib.lh_last_error.argtypes = []
    lib.lh_last_error.restype = ctypes.c_char_p
    _lib = lib
    return lib


def _ptr(t):
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _nbytes(t):
    return 0 if t is None else t.numel() * t.element_size()


def _stream(stream):
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else stream


def _check(status: int):
    if status != 0:
        raise LighthouseError(status, load_library().lh_last_error().decode())


def make_shape(B, H, N, d, p, L, S, dtype, qkv_stride=None, out_stride=None,
               scatter="span") -> Shape:
    """Shape with optional element strides (b, h, n) of the token tensors:
    qkv_stride for q, k, v, dq, dk, dv; out_stride for out and dout (None =
    packed [B,H,N,d]); scatter: "span" or "causal" (or the LH_SCATTER_* value)."""
    if isinstance(dtype, torch.dtype):
        dtype = DTYPES[dtype]
    sh = Shape(B, H, N, d, p, L, S, dtype)
    sh.scatter = SCATTER.get(scatter, scatter) if isinstance(scatter, str) else scatter
    if qkv_stride is not None:
        sh.qkv_stride = (ctypes.c_int64 * 3)(*qkv_stride)
    if out_stride is not None:
        sh.out_stride = (ctypes.c_int64 * 3)(*out_stride)
    return sh


def token_strides(*ts):
    """Common (b, h, n) element strides of [B,H,N,d] views whose last
    dimension is contiguous, or None if they differ or do not qualify."""
    if any(t.dim() != 4 or t.stride(3) != 1 for t in ts):
        return None
    # the stride of an extent-1 dimension is never used (and may be anything)
    st = {tuple(0 if t.shape[i] == 1 else t.stride(i) for i in range(3)) for t in ts}
    return st.pop() if len(st) == 1 else None


def with_strides(shape: Shape, qkv_stride=None, out_stride=None) -> Shape:
    """A copy of `shape` with the given token strides (None = keep)."""
    return make_shape(shape.B, shape.H, shape.N, shape.d, shape.p, shape.L, shape.S, shape.dtype,
                      tuple(shape.qkv_stride) if qkv_stride is None else qkv_stride,
                      tuple(shape.out_stride) if out_stride is None else out_stride,
                      shape.scatter)


# ------------------------------------------------------------- the C ABI

def lh_query_sizes(shape: Shape) -> Sizes:
    out = Sizes()
    _check(load_library().lh_query_sizes(ctypes.byref(shape), ctypes.byref(out)))
    return out


def lh_build_pyramid(shape, q, k, v, pq, pk, pv, ws=None, stream=None):
    _check(load_library().lh_build_pyramid(ctypes.byref(shape), _ptr(q), _ptr(k), _ptr(v),
                                           _ptr(pq), _ptr(pk), _ptr(pv), _ptr(ws), _nbytes(ws),
                                           _stream(stream)))


def lh_score(shape, q, k, score, ws=None, stream=None):
    _check(load_library().lh_score(ctypes.byref(shape), _ptr(q), _ptr(k), _ptr(score), _ptr(ws),
                                   _nbytes(ws), _stream(stream)))


def lh_topk(shape, score, sel, ws=None, stream=None):
    _check(load_library().lh_topk(ctypes.byref(shape), _ptr(score), _ptr(sel), _ptr(ws),
                                  _nbytes(ws), _stream(stream)))


def lh_topk_noalloc(shape, score, sel, stream=None):
    _check(load_library().lh_topk_noalloc(ctypes.byref(shape), _ptr(score), _ptr(sel),
                                          _stream(stream)))


def lh_gather(shape, sel, q, k, v, pq, pk, pv, sub_idx, pos, qs, ks, vs, ws=None, stream=None):
    _check(load_library().lh_gather(ctypes.byref(shape), _ptr(sel), _ptr(q), _ptr(k), _ptr(v),
                                    _ptr(pq), _ptr(pk), _ptr(pv), _ptr(sub_idx), _ptr(pos),
                                    _ptr(qs), _ptr(ks), _ptr(vs), _ptr(ws), _nbytes(ws),
                                    _stream(stream)))


def lh_attention(shape, qs, ks, vs, os_, lse, stream=None):
    _check(load_library().lh_attention(ctypes.byref(shape), _ptr(qs), _ptr(ks), _ptr(vs),
                                       _ptr(os_), _ptr(lse), _stream(stream)))


def lh_scatter(shape, os_, pos, out, stream=None):
    _check(load_library().lh_scatter(ctypes.byref(shape), _ptr(os_), _ptr(pos), _ptr(out),
                                     _stream(stream)))


def lh_forward(shape, q, k, v, out, bufs: "LayerBuffers", ws, stream=None):
    cb = bufs.as_ctypes()
    _check(load_library().lh_forward(ctypes.byref(shape), _ptr(q), _ptr(k), _ptr(v), _ptr(out),
                                     ctypes.byref(cb), _ptr(ws), _nbytes(ws), _stream(stream)))


def lh_scatter_backward(shape, dout, pos, dos, ws=None, stream=None):
    _check(load_library().lh_scatter_backward(ctypes.byref(shape), _ptr(dout), _ptr(pos),
                                              _ptr(dos), _ptr(ws), _nbytes(ws), _stream(stream)))


def lh_attention_backward(shape, qs, ks, vs, os_, lse, dos, dqs, dks, dvs, ws, stream=None):
    _check(load_library().lh_attention_backward(
        ctypes.byref(shape), _ptr(qs), _ptr(ks), _ptr(vs), _ptr(os_), _ptr(lse), _ptr(dos),
        _ptr(dqs), _ptr(dks), _ptr(dvs), _ptr(ws), _nbytes(ws), _stream(stream)))


def lh_gather_backward(shape, dqs, dks, dvs, pos, dq, dk, dv, stream=None):
    _check(load_library().lh_gather_backward(ctypes.byref(shape), _ptr(dqs), _ptr(dks),
                                             _ptr(dvs), _ptr(pos), _ptr(dq), _ptr(dk), _ptr(dv),
                                             _stream(stream)))


def lh_backward(shape, dout, bufs: "LayerBuffers", dq, dk, dv, ws, stream=None):
    cb = bufs.as_ctypes()
    _check(load_library().lh_backward(ctypes.byref(shape), _ptr(dout), ctypes.byref(cb),
                                      _ptr(dq), _ptr(dk), _ptr(dv), _ptr(ws), _nbytes(ws),
                                      _stream(stream)))


def lh_profile_step(shape, q, k, v, out, bufs: "LayerBuffers", dout, dq, dk, dv, ws,
                    stream=None) -> dict:
    """Per-stage milliseconds of one forward + backward (waits for the stream)."""
    cb = bufs.as_ctypes()
    ms = (ctypes.c_float * len(PROFILE_STAGES))()
    _check(load_library().lh_profile_step(ctypes.byref(shape), _ptr(q), _ptr(k), _ptr(v),
                                          _ptr(out), ctypes.byref(cb), _ptr(dout), _ptr(dq),
                                          _ptr(dk), _ptr(dv), _ptr(ws), _nbytes(ws), ms,
                                          _stream(stream)))
    return dict(zip(PROFILE_STAGES, list(ms)))


# ------------------------------------------------------------- allocation helpers

class LayerBuffers:
    """Device buffers lh_forward fills and lh_backward reads (torch-owned)."""

    FIELDS = ("pq", "pk", "pv", "score", "sel", "sub_idx", "pos", "qs", "ks", "vs", "os", "lse")

    def __init__(self, shape: Shape, device="cuda"):
        z = lh_query_sizes(shape)
        dt = torch.bfloat16 if shape.dtype == LH_BF16 else torch.float32
        B, H, N, d, S = shape.B, shape.H, shape.N, shape.d, shape.S
        kw = dict(device=device)
        self.pq, self.pk, self.pv = (torch.empty(B, H, z.M - N, d, dtype=dt, **kw) for _ in range(3))
        self.score = torch.empty(B, H, z.M, dtype=torch.float32, **kw)
        self.sel = torch.empty(B, H, z.K, dtype=torch.int32, **kw)
        self.sub_idx = torch.empty(B, H, S, dtype=torch.int32, **kw)
        self.pos = torch.empty(B, H, z.M, dtype=torch.int32, **kw)
        self.qs, self.ks, self.vs = (torch.empty(B, H, S, d, dtype=dt, **kw) for _ in range(3))
        self.os = torch.empty(B, H, S, d, dtype=torch.float32, **kw)
        self.lse = torch.empty(B, H, S, dtype=torch.float32, **kw)
        self.sizes = z

    def as_ctypes(self) -> Buffers:
        def p(t):
            return t.data_ptr() if t.numel() else None
        return Buffers(*(p(getattr(self, f)) for f in self.FIELDS))


def _on_stream(stream):
    """Context making `stream` (a torch stream or a raw hipStream_t handle)
    torch's current stream; a no-op for None."""
    if stream is None:
        return contextlib.nullcontext()
    if not isinstance(stream, torch.cuda.Stream):
        stream = torch.cuda.ExternalStream(int(getattr(stream, "cuda_stream", stream)))
    return torch.cuda.stream(stream)


def workspace(nbytes: int, device="cuda") -> torch.Tensor | None:
    return torch.empty(max(int(nbytes), 1), dtype=torch.uint8, device=device) if nbytes else None


def forward(q, k, v, p: int, L: int, S: int, out=None, stream=None, scatter="span"):
    """out, buffers, shape for [B,H,N,d] device tensors (fp32 or bf16).
    scatter: "span" (R11, reads later tokens) or "causal" (R11c).

    q, k, v may be strided views sharing one layout (last dimension
    contiguous), e.g. slices of a packed projection; otherwise they are made
    contiguous.  `out`, if given, is a [B,H,N,d] view to write into (any
    layout with a contiguous last dimension); else a packed tensor is
    allocated.

    With `stream` given, every allocation (out, buffers, workspace, contiguous
    copies) and the launch happen on that stream, so the caching allocator
    reuses the workspace only after the stream's kernels."""
    with _on_stream(stream):
        return _forward(q, k, v, p, L, S, out, scatter)


def _forward(q, k, v, p, L, S, out, scatter):
    B, H, N, d = q.shape
    st = token_strides(q, k, v)
    if st is None:
        q, k, v = (t.contiguous() for t in (q, k, v))
        st = token_strides(q, k, v)
    if out is None:
        out = torch.empty(B, H, N, d, dtype=q.dtype, device=q.device)
    ost = token_strides(out)
    if ost is None:
        raise ValueError("out must be a [B,H,N,d] view with a contiguous last dimension")
    shape = make_shape(B, H, N, d, p, L, S, q.dtype, st, ost, scatter)
    bufs = LayerBuffers(shape, q.device)
    ws = workspace(bufs.sizes.ws_forward, q.device)
    lh_forward(shape, q, k, v, out, bufs, ws)
    return out, bufs, shape


def backward(shape, dout, bufs: LayerBuffers, dq=None, dk=None, dv=None, stream=None):
    """dq, dk, dv of the forward that filled `bufs`.  dout: any [B,H,N,d]
    layout with a contiguous last dimension (else made contiguous); dq, dk,
    dv: views sharing one layout to write into, or None for packed tensors.
    `stream` as in forward()."""
    with _on_stream(stream):
        return _backward(shape, dout, bufs, dq, dk, dv)


def _backward(shape, dout, bufs, dq, dk, dv):
    if token_strides(dout) is None:
        dout = dout.contiguous()
    if dq is None:
        dq, dk, dv = (torch.empty(shape.B, shape.H, shape.N, shape.d, dtype=dout.dtype,
                                  device=dout.device) for _ in range(3))
    gst = token_strides(dq, dk, dv)
    if gst is None:
        raise ValueError("dq, dk, dv must be [B,H,N,d] views sharing one layout")
    call_shape = with_strides(shape, gst, token_strides(dout))
    ws = workspace(bufs.sizes.ws_backward, dout.device)
    lh_backward(call_shape, dout, bufs, dq, dk, dv, ws)
    return dq, dk, dv
