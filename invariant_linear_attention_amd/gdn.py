"""Thin Python binding of the C ABI in include/gdn.h.

Argument marshalling only: every step of the recurrence runs in the HIP kernels of
``libgdn.so``.  torch supplies device memory and the stream.  If the library has
not been built, every call raises; there is no CPU or eager fallback.
"""
from __future__ import annotations

import ctypes
import os
import threading
from typing import Optional, Tuple

PKG = os.path.dirname(os.path.abspath(__file__))
LIBRARY = os.path.join(PKG, "libgdn.so")

GDN_F32, GDN_BF16 = 0, 1
STATUS = {
    0: "GDN_OK", 1: "GDN_ERR_NULL", 2: "GDN_ERR_SHAPE", 3: "GDN_ERR_DTYPE", 4: "GDN_ERR_ALIGN",
    5: "GDN_ERR_ALIAS", 6: "GDN_ERR_UNSUPPORTED", 7: "GDN_ERR_HIP", 8: "GDN_ERR_CAPACITY",
}
GDN_NOALLOC_SCRATCH_BYTES = 64 << 20
EXPORTS = ("gdn_fwd_varlen", "gdn_fwd_varlen_train", "gdn_fwd_varlen_pool", "gdn_decode_step", "gdn_short_conv",
           "gdn_query_plan", "gdn_bwd_workspace_size", "gdn_bwd_varlen", "gdn_bwd_varlen_noalloc", "gdn_fwd_chunked",
           "gdn_chunked_workspace_size", "gdn_bwd_chunked_workspace_size", "gdn_bwd_chunked", "gdn_preprocess",
           "gdn_preprocess_backward", "gdn_short_conv_backward_workspace_size", "gdn_short_conv_backward",
           "gdn_status_string", "gdn_abi_version")

GDN_CHUNK = 16


GDN_PRE_QK_L2NORM, GDN_PRE_GATE_LOGITS = 1, 2


class GdnPreproc(ctypes.Structure):
    """Mirror of ``gdn_preproc``."""
    _fields_ = [("flags", ctypes.c_int32), ("eps", ctypes.c_float),
                ("A_log", ctypes.c_void_p), ("dt_bias", ctypes.c_void_p)]


class GdnDims(ctypes.Structure):
    """Mirror of ``gdn_dims``."""
    _fields_ = [
        ("n_seqs", ctypes.c_int32), ("hk", ctypes.c_int32), ("hv", ctypes.c_int32),
        ("dk", ctypes.c_int32), ("dv", ctypes.c_int32), ("io_dtype", ctypes.c_int32),
        ("total_tokens", ctypes.c_int64), ("pool_size", ctypes.c_int32),
        ("plan_lanes", ctypes.c_int32), ("plan_rows", ctypes.c_int32), ("plan_waves", ctypes.c_int32),
        ("reserved", ctypes.c_int32), ("pre", ctypes.POINTER(GdnPreproc)),
    ]


GDN_CONV_SILU = 1


class GdnConvDims(ctypes.Structure):
    """Mirror of ``gdn_conv_dims``."""
    _fields_ = [
        ("n_seqs", ctypes.c_int32), ("channels", ctypes.c_int32), ("taps", ctypes.c_int32),
        ("io_dtype", ctypes.c_int32), ("total_tokens", ctypes.c_int64), ("pool_size", ctypes.c_int32),
        ("flags", ctypes.c_int32),
    ]


class GdnError(RuntimeError):
    def __init__(self, code: int, message: str):
        super().__init__("%s (%d)" % (message, code))
        self.code = code


_lock = threading.Lock()
_lib = None


class GdnChunkState(ctypes.Structure):
    """Mirror of ``gdn_chunk_state``."""
    _fields_ = [("S", ctypes.c_void_p), ("k", ctypes.c_void_p), ("r", ctypes.c_void_p), ("a", ctypes.c_void_p),
                ("b", ctypes.c_void_p), ("count", ctypes.c_void_p)]


def load_library(path: str = LIBRARY):
    """Load libgdn.so (once).  Raises if it is missing: build it first."""
    global _lib
    with _lock:
        if _lib is not None:
            return _lib
        if not os.path.exists(path):
            raise RuntimeError("libgdn.so is not built (%s); run __graft_entry__.build() first" % path)
        lib = ctypes.CDLL(path)
        vp = ctypes.c_void_p
        lib.gdn_fwd_varlen.restype = ctypes.c_int
        lib.gdn_fwd_varlen.argtypes = [ctypes.POINTER(GdnDims), vp, vp, vp, vp, vp, vp, vp, vp, vp, vp]
        lib.gdn_fwd_varlen_pool.restype = ctypes.c_int
        lib.gdn_fwd_varlen_pool.argtypes = [ctypes.POINTER(GdnDims), vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp,
                                            ctypes.c_int32, ctypes.c_int32, vp, vp]
        lib.gdn_decode_step.restype = ctypes.c_int
        lib.gdn_decode_step.argtypes = [ctypes.POINTER(GdnDims), vp, vp, vp, vp, vp, vp, vp, vp, vp]
        lib.gdn_short_conv.restype = ctypes.c_int
        lib.gdn_short_conv.argtypes = [ctypes.POINTER(GdnConvDims), vp, vp, vp, vp, vp, vp, vp, vp, vp]
        lib.gdn_short_conv_backward_workspace_size.restype = ctypes.c_int
        lib.gdn_short_conv_backward_workspace_size.argtypes = [ctypes.POINTER(GdnConvDims),
                                                               ctypes.POINTER(ctypes.c_uint64)]
        lib.gdn_short_conv_backward.restype = ctypes.c_int
        lib.gdn_short_conv_backward.argtypes = [ctypes.POINTER(GdnConvDims)] + [vp] * 12 + [ctypes.c_uint64, vp]
        lib.gdn_bwd_workspace_size.restype = ctypes.c_int
        lib.gdn_bwd_workspace_size.argtypes = [ctypes.POINTER(GdnDims), ctypes.POINTER(ctypes.c_uint64)]
        lib.gdn_bwd_varlen.restype = ctypes.c_int
        lib.gdn_bwd_varlen.argtypes = [ctypes.POINTER(GdnDims)] + [vp] * 18 + [ctypes.c_uint64, vp]
        lib.gdn_bwd_varlen_noalloc.restype = ctypes.c_int
        lib.gdn_bwd_varlen_noalloc.argtypes = [ctypes.POINTER(GdnDims)] + [vp] * 18
        lib.gdn_fwd_varlen_train.restype = ctypes.c_int
        lib.gdn_fwd_varlen_train.argtypes = [ctypes.POINTER(GdnDims), vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp]
        lib.gdn_fwd_chunked.restype = ctypes.c_int
        lib.gdn_fwd_chunked.argtypes = [ctypes.POINTER(GdnDims), vp, vp, vp, vp, vp, vp,
                                        ctypes.POINTER(GdnChunkState), ctypes.POINTER(GdnChunkState), vp, vp,
                                        ctypes.c_uint64, vp]
        lib.gdn_chunked_workspace_size.restype = ctypes.c_int
        lib.gdn_chunked_workspace_size.argtypes = [ctypes.POINTER(GdnDims), ctypes.POINTER(ctypes.c_uint64)]
        lib.gdn_bwd_chunked_workspace_size.restype = ctypes.c_int
        lib.gdn_bwd_chunked_workspace_size.argtypes = [ctypes.POINTER(GdnDims), ctypes.POINTER(ctypes.c_uint64)]
        lib.gdn_bwd_chunked.restype = ctypes.c_int
        lib.gdn_bwd_chunked.argtypes = [ctypes.POINTER(GdnDims)] + [vp] * 16 + [ctypes.c_uint64, vp]
        lib.gdn_preprocess.restype = ctypes.c_int
        lib.gdn_preprocess.argtypes = [ctypes.POINTER(GdnDims)] + [vp] * 9
        lib.gdn_preprocess_backward.restype = ctypes.c_int
        lib.gdn_preprocess_backward.argtypes = [ctypes.POINTER(GdnDims)] + [vp] * 15
        lib.gdn_query_plan.restype = ctypes.c_int
        lib.gdn_query_plan.argtypes = [ctypes.POINTER(GdnDims), ctypes.c_int32, ctypes.POINTER(ctypes.c_int32)]
        lib.gdn_status_string.restype = ctypes.c_char_p
        lib.gdn_status_string.argtypes = [ctypes.c_int]
        lib.gdn_abi_version.restype = ctypes.c_int32
        lib.gdn_abi_version.argtypes = []
        _lib = lib
        return lib


def status_string(code: int) -> str:
    return load_library().gdn_status_string(int(code)).decode()


def _check(code: int):
    if code != 0:
        raise GdnError(code, status_string(code))


def _ptr(t) -> Optional[int]:
    return None if t is None else int(t.data_ptr())


def _stream_handle(stream) -> Optional[int]:
    import torch
    if stream is None:
        stream = torch.cuda.current_stream()
    if isinstance(stream, int):
        return stream or None
    return int(stream.cuda_stream) or None


def _io_code(t) -> int:
    import torch
    if t.dtype == torch.bfloat16:
        return GDN_BF16
    if t.dtype == torch.float32:
        return GDN_F32
    raise TypeError("q/k/v/out must be bf16 or fp32, got %s" % t.dtype)


def _need(t, name, dtype=None, cuda=True):
    import torch
    if t is None:
        return
    if cuda and not t.is_cuda:
        raise ValueError("%s must be a device tensor" % name)
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)
    if dtype is not None and t.dtype != dtype:
        raise TypeError("%s must be %s, got %s" % (name, dtype, t.dtype))


def _shape(t, name, shape):
    """Raise ValueError unless ``t`` (when given) has exactly ``shape``."""
    if t is None:
        return
    if tuple(int(x) for x in t.shape) != tuple(int(x) for x in shape):
        raise ValueError("%s must have shape %s, got %s" % (name, tuple(shape), tuple(t.shape)))


def _dims_of(q, k, v, g, beta, cu_seqlens=None, require_cu=False):
    """Check the shapes of one packed batch against each other; returns
    (T, hk, dk, hv, dv, N).  The C ABI sizes every buffer from these numbers, so a
    tensor of another shape would be read or written past its end: every such
    mismatch is refused here, before anything is launched."""
    if q is None or v is None:
        raise ValueError("q and v are required")
    if q.dim() != 3 or v.dim() != 3:
        raise ValueError("q must be [T, Hk, dk] and v [T, Hv, dv], got %s and %s" % (tuple(q.shape), tuple(v.shape)))
    T, hk, dk = (int(x) for x in q.shape)
    hv, dv = int(v.shape[1]), int(v.shape[2])
    _shape(k, "k", (T, hk, dk))
    _shape(v, "v", (T, hv, dv))
    _shape(g, "g", (T, hv))
    _shape(beta, "beta", (T, hv))
    N = None
    if cu_seqlens is None and require_cu:
        raise ValueError("cu_seqlens is required")
    if cu_seqlens is not None:
        if cu_seqlens.dim() != 1 or cu_seqlens.numel() < 1:
            raise ValueError("cu_seqlens must be a 1-D [N+1] tensor, got %s" % (tuple(cu_seqlens.shape),))
        N = int(cu_seqlens.numel()) - 1
    return T, hk, dk, hv, dv, N


def _check_pre(pre, hv):
    """The preprocessing arrays A_log / dt_bias must hold one value per value head."""
    if pre is None:
        return
    for name, t in zip(("A_log", "dt_bias"), getattr(pre, "_keep", (None, None))):
        if t is not None and (t.dim() != 1 or int(t.numel()) != hv):
            raise ValueError("%s must be [Hv] = [%d], got %s" % (name, hv, tuple(t.shape)))


def _check_pool(state_pool, hv, dv, dk):
    if state_pool is None or state_pool.dim() != 4 or tuple(int(x) for x in state_pool.shape[1:]) != (hv, dv, dk):
        raise ValueError("state_pool must be [P, Hv, dv, dk] = [P, %d, %d, %d], got %s"
                         % (hv, dv, dk, None if state_pool is None else tuple(state_pool.shape)))


def _check_index(t, name, n):
    if t is not None and (t.dim() != 1 or int(t.numel()) != n):
        raise ValueError("%s must be a 1-D tensor of %d entries, got %s" % (name, n, tuple(t.shape)))


def make_preproc(norm_qk: bool = False, eps: float = 1e-6, A_log=None, dt_bias=None) -> GdnPreproc:
    """Fused preprocessing (see gdn_preproc in include/gdn.h): ``norm_qk`` L2-normalises
    q and k rows in the kernel; with ``A_log`` (fp32 [Hv] on the GPU) the ``g`` and
    ``beta`` arguments of the call are the logits a and b, and the kernel forms
    g = -exp(A_log) softplus(a + dt_bias), beta = sigmoid(b)."""
    import torch
    _need(A_log, "A_log", torch.float32)
    _need(dt_bias, "dt_bias", torch.float32)
    flags = (GDN_PRE_QK_L2NORM if norm_qk else 0) | (GDN_PRE_GATE_LOGITS if A_log is not None else 0)
    pre = GdnPreproc(flags=flags, eps=float(eps), A_log=_ptr(A_log), dt_bias=_ptr(dt_bias))
    pre._keep = (A_log, dt_bias)
    return pre


def make_dims(q, v, n_seqs: int, total_tokens: int, pool_size: int = 0, plan=(0, 0, 0), pre=None) -> GdnDims:
    """``plan`` = (lanes per row, rows per lane, waves per workgroup); 0 = automatic.
    A 2-tuple means (rows, waves) with automatic lanes.  ``pre``: a GdnPreproc or None."""
    plan = tuple(int(x) for x in plan)
    if len(plan) == 2:
        plan = (0,) + plan
    dims = GdnDims(n_seqs=int(n_seqs), hk=int(q.shape[1]), hv=int(v.shape[1]), dk=int(q.shape[2]),
                   dv=int(v.shape[2]), io_dtype=_io_code(q), total_tokens=int(total_tokens),
                   pool_size=int(pool_size), plan_lanes=plan[0], plan_rows=plan[1], plan_waves=plan[2],
                   reserved=0, pre=ctypes.pointer(pre) if pre is not None else None)
    dims._keep = pre
    return dims


def gdn_query_plan(dims: GdnDims, decode: bool = False) -> Tuple[int, int, int]:
    """(lanes per row, rows per lane, waves per workgroup) that gdn_fwd_varlen
    (or gdn_decode_step when ``decode``) would launch for ``dims``.  Host only."""
    shape = (ctypes.c_int32 * 3)()
    _check(load_library().gdn_query_plan(ctypes.byref(dims), int(bool(decode)), shape))
    return tuple(int(x) for x in shape)


def gdn_fwd_varlen(q, k, v, g, beta, h0, cu_seqlens, out=None, hT=None, stream=None, plan=(0, 0, 0),
                   want_state: bool = True, pre=None):
    """Varlen prefill (see include/gdn.h).  Tensors on the GPU, contiguous:
    q, k [T, Hk, dk]; v [T, Hv, dv]; g, beta [T, Hv] fp32; h0 [N, Hv, dv, dk] fp32
    or None; cu_seqlens [N+1] int32.  ``out`` / ``hT`` are allocated when None
    (hT only if ``want_state``).  Returns (out, hT)."""
    import torch
    T, hk, dk, hv, dv, N = _dims_of(q, k, v, g, beta, cu_seqlens, require_cu=True)
    _shape(h0, "h0", (N, hv, dv, dk))
    _shape(out, "out", (T, hv, dv))
    _shape(hT, "hT", (N, hv, dv, dk))
    _check_pre(pre, hv)
    lib = load_library()
    for name, t in (("q", q), ("k", k), ("v", v)):
        _need(t, name, q.dtype)
    _need(g, "g", torch.float32)
    _need(beta, "beta", torch.float32)
    _need(h0, "h0", torch.float32)
    _need(cu_seqlens, "cu_seqlens", torch.int32)
    if out is None:
        out = torch.empty((T, hv, dv), dtype=q.dtype, device=q.device)
    if hT is None and want_state:
        hT = torch.empty((N, hv, dv, dk), dtype=torch.float32, device=q.device)
    _need(out, "out", q.dtype)
    _need(hT, "hT", torch.float32)
    dims = make_dims(q, v, N, T, plan=plan, pre=pre)
    _check(lib.gdn_fwd_varlen(ctypes.byref(dims), _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(h0),
                              _ptr(cu_seqlens), _ptr(out), _ptr(hT), _stream_handle(stream)))
    return out, hT


def gdn_bwd_workspace_size(dims: GdnDims) -> int:
    """Workspace bytes gdn_bwd_varlen needs for ``dims`` (host only)."""
    n = ctypes.c_uint64(0)
    _check(load_library().gdn_bwd_workspace_size(ctypes.byref(dims), ctypes.byref(n)))
    return int(n.value)


def gdn_fwd_varlen_train(q, k, v, g, beta, h0, cu_seqlens, out=None, hT=None, saved_p=None, stream=None):
    """gdn_fwd_varlen that also returns p_t = S_{t-1} k_t [T, Hv, dv] fp32 for the
    backward.  Returns (out, hT, saved_p)."""
    import torch
    T, hk, dk, hv, dv, N = _dims_of(q, k, v, g, beta, cu_seqlens, require_cu=True)
    _shape(h0, "h0", (N, hv, dv, dk))
    _shape(out, "out", (T, hv, dv))
    _shape(hT, "hT", (N, hv, dv, dk))
    _shape(saved_p, "saved_p", (T, hv, dv))
    lib = load_library()
    for name, t in (("q", q), ("k", k), ("v", v)):
        _need(t, name, q.dtype)
    _need(g, "g", torch.float32)
    _need(beta, "beta", torch.float32)
    _need(h0, "h0", torch.float32)
    _need(cu_seqlens, "cu_seqlens", torch.int32)
    if out is None:
        out = torch.empty((T, hv, dv), dtype=q.dtype, device=q.device)
    if hT is None:
        hT = torch.empty((N, hv, dv, dk), dtype=torch.float32, device=q.device)
    if saved_p is None:
        saved_p = torch.empty((T, hv, dv), dtype=torch.float32, device=q.device)
    for name, t, dt in (("out", out, q.dtype), ("hT", hT, torch.float32), ("saved_p", saved_p, torch.float32)):
        _need(t, name, dt)
    dims = make_dims(q, v, N, T)
    _check(lib.gdn_fwd_varlen_train(ctypes.byref(dims), _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(h0),
                                    _ptr(cu_seqlens), _ptr(out), _ptr(hT), _ptr(saved_p), _stream_handle(stream)))
    return out, hT, saved_p


def gdn_bwd_varlen(q, k, v, g, beta, h0, cu_seqlens, dout, dhT=None, workspace=None, grads=None, stream=None,
                   want_dh0: bool = True, saved_p=None, hT=None, noalloc: bool = False):
    """Backward of gdn_fwd_varlen (see include/gdn.h).  Inputs as gdn_fwd_varlen plus
    dout [T, Hv, dv] (dtype of q) and dhT [N, Hv, dv, dk] fp32 or None.  ``workspace``
    (a uint8 device tensor of at least gdn_bwd_workspace_size bytes) and ``grads``
    (a dict of output tensors) are allocated when None.  Returns a dict of fp32
    tensors: dq, dk [T, Hk, dk]; dv [T, Hv, dv]; dg, dbeta [T, Hv]; dh0.  ``saved_p`` (and
    ``hT`` when dhT is given) from gdn_fwd_varlen_train skip the backward's own
    forward recompute.  ``noalloc`` calls gdn_bwd_varlen_noalloc instead: no workspace
    (the library's fixed per-device scratch serves), for calls that fit it; then
    ``grads`` must be given, so that nothing at all is allocated."""
    import torch
    T, hk, dk, hv, dv, N = _dims_of(q, k, v, g, beta, cu_seqlens, require_cu=True)
    if noalloc and (workspace is not None or grads is None):
        raise ValueError("noalloc takes no workspace and needs preallocated grads")
    _shape(h0, "h0", (N, hv, dv, dk))
    _shape(dout, "dout", (T, hv, dv))
    _shape(dhT, "dhT", (N, hv, dv, dk))
    _shape(saved_p, "saved_p", (T, hv, dv))
    _shape(hT, "hT", (N, hv, dv, dk))
    if grads is not None:
        want = {"dq": (T, hk, dk), "dk": (T, hk, dk), "dv": (T, hv, dv), "dg": (T, hv), "dbeta": (T, hv),
                "dh0": (N, hv, dv, dk)}
        for name, shp in want.items():
            if name != "dh0" and grads.get(name) is None:
                raise ValueError("grads[%r] is required" % name)
            _shape(grads.get(name), name, shp)
    if workspace is not None and workspace.dim() != 1:
        raise ValueError("workspace must be a 1-D uint8 tensor")
    lib = load_library()
    for name, t in (("q", q), ("k", k), ("v", v), ("dout", dout)):
        _need(t, name, q.dtype)
    for name, t in (("g", g), ("beta", beta), ("h0", h0), ("dhT", dhT), ("saved_p", saved_p), ("hT", hT)):
        _need(t, name, torch.float32)
    _need(cu_seqlens, "cu_seqlens", torch.int32)
    dims = make_dims(q, v, N, T)
    if noalloc:
        for name, t in grads.items():
            _need(t, name, torch.float32)
        _check(lib.gdn_bwd_varlen_noalloc(ctypes.byref(dims), _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta),
                                          _ptr(h0), _ptr(cu_seqlens), _ptr(dout), _ptr(dhT), _ptr(saved_p), _ptr(hT),
                                          _ptr(grads["dq"]), _ptr(grads["dk"]), _ptr(grads["dv"]), _ptr(grads["dg"]),
                                          _ptr(grads["dbeta"]), _ptr(grads.get("dh0")), _stream_handle(stream)))
        return grads
    if workspace is None:
        workspace = torch.empty(gdn_bwd_workspace_size(dims), dtype=torch.uint8, device=q.device)
    _need(workspace, "workspace", torch.uint8)
    if grads is None:
        f32 = dict(dtype=torch.float32, device=q.device)
        grads = {"dq": torch.empty((T, hk, dk), **f32), "dk": torch.empty((T, hk, dk), **f32),
                 "dv": torch.empty((T, hv, dv), **f32), "dg": torch.empty((T, hv), **f32),
                 "dbeta": torch.empty((T, hv), **f32),
                 "dh0": torch.empty((N, hv, dv, dk), **f32) if want_dh0 else None}
    for name, t in grads.items():
        _need(t, name, torch.float32)
    _check(lib.gdn_bwd_varlen(ctypes.byref(dims), _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(h0),
                              _ptr(cu_seqlens), _ptr(dout), _ptr(dhT), _ptr(saved_p), _ptr(hT),
                              _ptr(grads["dq"]), _ptr(grads["dk"]),
                              _ptr(grads["dv"]), _ptr(grads["dg"]), _ptr(grads["dbeta"]), _ptr(grads.get("dh0")),
                              _ptr(workspace), int(workspace.numel()), _stream_handle(stream)))
    return grads


def gdn_bwd_chunked_workspace_size(dims: GdnDims) -> int:
    """Workspace bytes gdn_bwd_chunked needs for ``dims`` (host only)."""
    n = ctypes.c_uint64(0)
    _check(load_library().gdn_bwd_chunked_workspace_size(ctypes.byref(dims), ctypes.byref(n)))
    return int(n.value)


def gdn_bwd_chunked(q, k, v, g, beta, h0, cu_seqlens, dout, dhT=None, workspace=None, grads=None, stream=None,
                    want_dh0: bool = True, waves: int = 0, parts: int = 0, plain: bool = False):
    """Chunked backward on the matrix cores (see include/gdn.h): the gradients of
    gdn_bwd_varlen, same arguments and results.  ``workspace`` (uint8, at least
    gdn_bwd_chunked_workspace_size bytes) and ``grads`` are allocated when None;
    ``waves`` (0, 1, 2 or 4) is the forward walk's waves per 16-row state tile and
    ``parts`` (0 = automatic, 1 or 2) the reverse walk's workgroups per (sequence,
    value head); ``plain`` turns off its wave specialization (the same bits)."""
    import torch
    T, hk, dk, hv, dv, N = _dims_of(q, k, v, g, beta, cu_seqlens, require_cu=True)
    _shape(h0, "h0", (N, hv, dv, dk))
    _shape(dout, "dout", (T, hv, dv))
    _shape(dhT, "dhT", (N, hv, dv, dk))
    if grads is not None:
        want = {"dq": (T, hk, dk), "dk": (T, hk, dk), "dv": (T, hv, dv), "dg": (T, hv), "dbeta": (T, hv),
                "dh0": (N, hv, dv, dk)}
        for name, shp in want.items():
            if name != "dh0" and grads.get(name) is None:
                raise ValueError("grads[%r] is required" % name)
            _shape(grads.get(name), name, shp)
    if workspace is not None and workspace.dim() != 1:
        raise ValueError("workspace must be a 1-D uint8 tensor")
    lib = load_library()
    for name, t in (("q", q), ("k", k), ("v", v), ("dout", dout)):
        _need(t, name, q.dtype)
    for name, t in (("g", g), ("beta", beta), ("h0", h0), ("dhT", dhT)):
        _need(t, name, torch.float32)
    _need(cu_seqlens, "cu_seqlens", torch.int32)
    dims = make_dims(q, v, N, T, plan=(int(bool(plain)), parts, waves))
    if workspace is None:
        workspace = torch.empty(gdn_bwd_chunked_workspace_size(dims), dtype=torch.uint8, device=q.device)
    _need(workspace, "workspace", torch.uint8)
    if grads is None:
        f32 = dict(dtype=torch.float32, device=q.device)
        grads = {"dq": torch.empty((T, hk, dk), **f32), "dk": torch.empty((T, hk, dk), **f32),
                 "dv": torch.empty((T, hv, dv), **f32), "dg": torch.empty((T, hv), **f32),
                 "dbeta": torch.empty((T, hv), **f32),
                 "dh0": torch.empty((N, hv, dv, dk), **f32) if want_dh0 else None}
    for name, t in grads.items():
        _need(t, name, torch.float32)
    _check(lib.gdn_bwd_chunked(ctypes.byref(dims), _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(h0),
                               _ptr(cu_seqlens), _ptr(dout), _ptr(dhT), _ptr(grads["dq"]), _ptr(grads["dk"]),
                               _ptr(grads["dv"]), _ptr(grads["dg"]), _ptr(grads["dbeta"]), _ptr(grads.get("dh0")),
                               _ptr(workspace), int(workspace.numel()), _stream_handle(stream)))
    return grads


def _pre_dims(q, a, pre) -> GdnDims:
    T, hk, dk = (int(x) for x in q.shape)
    hv = int(a.shape[1])
    dims = GdnDims(n_seqs=0, hk=hk, hv=hv, dk=dk, dv=16, io_dtype=_io_code(q), total_tokens=T, pool_size=0,
                   plan_lanes=0, plan_rows=0, plan_waves=0, reserved=0,
                   pre=ctypes.pointer(pre) if pre is not None else None)
    dims._keep = pre
    return dims


def _pre_shapes(q, k, a, b, pre):
    import torch
    if q is None or q.dim() != 3:
        raise ValueError("q must be [T, Hk, dk], got %s" % (None if q is None else tuple(q.shape),))
    T, hk, dk = (int(x) for x in q.shape)
    _shape(k, "k", (T, hk, dk))
    if a is None or a.dim() != 2 or int(a.shape[0]) != T:
        raise ValueError("a must be [T, Hv] with T = %d, got %s" % (T, None if a is None else tuple(a.shape)))
    hv = int(a.shape[1])
    _shape(b, "b", (T, hv))
    _check_pre(pre, hv)
    return T, hk, dk, hv


def _pre_need(q, k, a, b):
    import torch
    _need(q, "q")
    _need(k, "k", q.dtype)
    _need(a, "a", torch.float32)
    _need(b, "b", torch.float32)


def gdn_preprocess(q, k, a, b, pre=None, out=None, stream=None):
    """The fused preprocessing as a pass of its own (see include/gdn.h): q, k
    [T, Hk, dk] (bf16 or fp32), a, b [T, Hv] fp32 logits (or g, beta when ``pre``
    has no gate logits).  Returns a dict of fp32 tensors qn, kn [T, Hk, dk] and
    g, beta [T, Hv] (``out``, a dict of the same, is filled when given)."""
    import torch
    T, hk, dk, hv = _pre_shapes(q, k, a, b, pre)
    shapes = (("qn", (T, hk, dk)), ("kn", (T, hk, dk)), ("g", (T, hv)), ("beta", (T, hv)))
    if out is not None:
        for name, shp in shapes:
            if out.get(name) is None:
                raise ValueError("out[%r] is required" % name)
            _shape(out[name], name, shp)
    _pre_need(q, k, a, b)
    if out is None:
        f32 = dict(dtype=torch.float32, device=q.device)
        out = {name: torch.empty(shp, **f32) for name, shp in shapes}
    for name, _ in shapes:
        _need(out[name], name, torch.float32)
    dims = _pre_dims(q, a, pre)
    _check(load_library().gdn_preprocess(ctypes.byref(dims), _ptr(q), _ptr(k), _ptr(a), _ptr(b), _ptr(out["qn"]),
                                         _ptr(out["kn"]), _ptr(out["g"]), _ptr(out["beta"]), _stream_handle(stream)))
    return out


def gdn_preprocess_backward(q, k, a, b, dqn, dkn, dg, dbeta, pre=None, grads=None, stream=None):
    """Gradients of gdn_preprocess (see include/gdn.h): given fp32 dqn, dkn
    [T, Hk, dk] and dg, dbeta [T, Hv], returns a dict of fp32 dq, dk [T, Hk, dk],
    da, db [T, Hv] and, with gate logits, dA_log [Hv] and (with dt_bias) ddt_bias
    [Hv]."""
    import torch
    T, hk, dk, hv = _pre_shapes(q, k, a, b, pre)
    ins = (("dqn", dqn, (T, hk, dk)), ("dkn", dkn, (T, hk, dk)), ("dg", dg, (T, hv)), ("dbeta", dbeta, (T, hv)))
    for name, t, shp in ins:
        if t is None:
            raise ValueError("%s is required" % name)
        _shape(t, name, shp)
    gshapes = (("dq", (T, hk, dk)), ("dk", (T, hk, dk)), ("da", (T, hv)), ("db", (T, hv)), ("dA_log", (hv,)),
               ("ddt_bias", (hv,)))
    if grads is not None:
        for name, shp in gshapes:
            if name in ("dq", "dk", "da", "db") and grads.get(name) is None:
                raise ValueError("grads[%r] is required" % name)
            _shape(grads.get(name), name, shp)
    _pre_need(q, k, a, b)
    for name, t, _ in ins:
        _need(t, name, torch.float32)
    gated = pre is not None and (pre.flags & GDN_PRE_GATE_LOGITS)
    has_dtb = gated and pre.dt_bias is not None
    if grads is None:
        f32 = dict(dtype=torch.float32, device=q.device)
        grads = {"dq": torch.empty((T, hk, dk), **f32), "dk": torch.empty((T, hk, dk), **f32),
                 "da": torch.empty((T, hv), **f32), "db": torch.empty((T, hv), **f32),
                 "dA_log": torch.empty((hv,), **f32) if gated else None,
                 "ddt_bias": torch.empty((hv,), **f32) if has_dtb else None}
    for name, _ in gshapes:
        _need(grads.get(name), name, torch.float32)
    dims = _pre_dims(q, a, pre)
    _check(load_library().gdn_preprocess_backward(
        ctypes.byref(dims), _ptr(q), _ptr(k), _ptr(a), _ptr(b), _ptr(dqn), _ptr(dkn), _ptr(dg), _ptr(dbeta),
        _ptr(grads["dq"]), _ptr(grads["dk"]), _ptr(grads["da"]), _ptr(grads["db"]), _ptr(grads.get("dA_log")),
        _ptr(grads.get("ddt_bias")), _stream_handle(stream)))
    return grads


def make_chunk_state(n_seqs: int, hk: int, hv: int, dk: int, dv: int, device, h0=None):
    """A chunked state (see gdn_fwd_chunked): dict of S [N, hv, dv, dk], k [N, 16, hk, dk],
    r [N, 16, hv, dv], a and b [N, 16, hv] (fp32) and count [N] (int32), with an empty
    open chunk and S = h0 (or zeros)."""
    import torch
    f32 = dict(dtype=torch.float32, device=device)
    S = torch.zeros((n_seqs, hv, dv, dk), **f32) if h0 is None else h0.to(device=device, dtype=torch.float32).clone()
    return {"S": S.contiguous(), "k": torch.zeros((n_seqs, GDN_CHUNK, hk, dk), **f32),
            "r": torch.zeros((n_seqs, GDN_CHUNK, hv, dv), **f32), "a": torch.zeros((n_seqs, GDN_CHUNK, hv), **f32),
            "b": torch.zeros((n_seqs, GDN_CHUNK, hv), **f32),
            "count": torch.zeros((n_seqs,), dtype=torch.int32, device=device)}


def _chunk_struct(st):
    if st is None:
        return None
    return GdnChunkState(_ptr(st["S"]), _ptr(st["k"]), _ptr(st["r"]), _ptr(st["a"]), _ptr(st["b"]), _ptr(st["count"]))


def gdn_chunked_workspace_size(dims: GdnDims) -> int:
    """Workspace bytes gdn_fwd_chunked needs for ``dims`` (host only)."""
    n = ctypes.c_uint64(0)
    _check(load_library().gdn_chunked_workspace_size(ctypes.byref(dims), ctypes.byref(n)))
    return int(n.value)


def gdn_fwd_chunked(q, k, v, g, beta, cu_seqlens, state_in, state_out=None, out=None, stream=None, workspace=None,
                    inplace: bool = False, count_out=None, waves: int = 0):
    """Chunked form with a replaying decode (see include/gdn.h).  ``state_in`` is a
    chunked state dict (make_chunk_state) or None for empty states; ``state_out``
    (allocated when None) receives the new states and must not overlap ``state_in``.
    With ``inplace`` (one token per sequence only) the state's S, k, r, a and b are
    updated where they are and the new token counts go to ``count_out`` (int32 [N],
    allocated when None); the returned state shares those arrays with ``state_in``
    and holds the new counts.  ``workspace`` (uint8, at least
    gdn_chunked_workspace_size bytes) is allocated when None.  ``waves`` (0 = automatic,
    else 1, 2 or 4) sets how many waves share a 16-row state tile (never a bit of the
    result).  ``cu_seqlens`` may be None for one token per sequence (a decode step:
    sequence n's token is row n).  Returns (out [T, Hv, dv], state_out)."""
    import torch
    T, hk, dk, hv, dv, N = _dims_of(q, k, v, g, beta, cu_seqlens)
    if N is None:
        N = T  # one token per sequence
    want = {"S": (N, hv, dv, dk), "k": (N, GDN_CHUNK, hk, dk), "r": (N, GDN_CHUNK, hv, dv), "a": (N, GDN_CHUNK, hv),
            "b": (N, GDN_CHUNK, hv), "count": (N,)}
    if inplace and (state_in is None or state_out is not None):
        raise ValueError("inplace updates state_in and takes no state_out")
    for which, st in (("state_in", state_in), ("state_out", state_out)):
        if st is not None:
            for name, shp in want.items():
                if st.get(name) is None:
                    raise ValueError("%s[%r] is required" % (which, name))
                _shape(st[name], "%s.%s" % (which, name), shp)
    _shape(out, "out", (T, hv, dv))
    if workspace is not None and workspace.dim() != 1:
        raise ValueError("workspace must be a 1-D uint8 tensor")
    lib = load_library()
    for name, t in (("q", q), ("k", k), ("v", v)):
        _need(t, name, q.dtype)
    _need(g, "g", torch.float32)
    _need(beta, "beta", torch.float32)
    if cu_seqlens is not None:
        _need(cu_seqlens, "cu_seqlens", torch.int32)
    for st in (state_in, state_out):
        if st is not None:
            for name in ("S", "k", "r", "a", "b"):
                _need(st[name], "state." + name, torch.float32)
            _need(st["count"], "state.count", torch.int32)
    if inplace:
        _shape(count_out, "count_out", (N,))
        _need(count_out, "count_out", torch.int32)
        state_out = dict(state_in)
        state_out["count"] = count_out if count_out is not None else torch.empty_like(state_in["count"])
    if state_out is None:
        state_out = make_chunk_state(N, hk, hv, dk, dv, q.device)
    if out is None:
        out = torch.empty((T, hv, dv), dtype=q.dtype, device=q.device)
    _need(out, "out", q.dtype)
    dims = make_dims(q, v, N, T, plan=(0, 0, int(waves)))
    if workspace is None:
        workspace = torch.empty(gdn_chunked_workspace_size(dims), dtype=torch.uint8, device=q.device)
    _need(workspace, "workspace", torch.uint8)
    sin, sout = _chunk_struct(state_in), _chunk_struct(state_out)
    _check(lib.gdn_fwd_chunked(ctypes.byref(dims), _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(cu_seqlens),
                               ctypes.byref(sin) if sin is not None else None, ctypes.byref(sout), _ptr(out),
                               _ptr(workspace), int(workspace.numel()), _stream_handle(stream)))
    return out, state_out


def gdn_fwd_varlen_pool(q, k, v, g, beta, cu_seqlens, state_pool, src_idx=None, dst_idx=None, pos0=None,
                        snap_idx=None, snap_block: int = 0, out=None, stream=None, plan=(0, 0, 0), pre=None):
    """Varlen prefill against a state pool (see include/gdn.h).  state_pool
    [P, Hv, dv, dk] fp32 is read and written in place; src_idx / dst_idx / pos0
    [N] int32 or None; snap_idx [N, S] int32 (required when snap_block > 0).
    Returns out [T, Hv, dv]."""
    import torch
    T, hk, dk, hv, dv, N = _dims_of(q, k, v, g, beta, cu_seqlens, require_cu=True)
    _check_pool(state_pool, hv, dv, dk)
    for name, t in (("src_idx", src_idx), ("dst_idx", dst_idx), ("pos0", pos0)):
        _check_index(t, name, N)
    _shape(out, "out", (T, hv, dv))
    _check_pre(pre, hv)
    lib = load_library()
    for name, t in (("q", q), ("k", k), ("v", v)):
        _need(t, name, q.dtype)
    _need(g, "g", torch.float32)
    _need(beta, "beta", torch.float32)
    _need(cu_seqlens, "cu_seqlens", torch.int32)
    _need(state_pool, "state_pool", torch.float32)
    for name, t in (("src_idx", src_idx), ("dst_idx", dst_idx), ("pos0", pos0), ("snap_idx", snap_idx)):
        _need(t, name, torch.int32)
    snap_per_seq = 0
    if snap_idx is not None:
        if snap_idx.dim() != 2 or int(snap_idx.shape[0]) != N:
            raise ValueError("snap_idx must be [N, snapshots per sequence]")
        snap_per_seq = int(snap_idx.shape[1])
    if out is None:
        out = torch.empty((T, v.shape[1], v.shape[2]), dtype=q.dtype, device=q.device)
    _need(out, "out", q.dtype)
    dims = make_dims(q, v, N, T, pool_size=int(state_pool.shape[0]), plan=plan, pre=pre)
    _check(lib.gdn_fwd_varlen_pool(ctypes.byref(dims), _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta),
                                   _ptr(cu_seqlens), _ptr(state_pool), _ptr(src_idx), _ptr(dst_idx), _ptr(pos0),
                                   _ptr(snap_idx), int(snap_block), snap_per_seq, _ptr(out),
                                   _stream_handle(stream)))
    return out


def gdn_decode_step(q, k, v, g, beta, state_pool, state_idx=None, out=None, stream=None, plan=(0, 0, 0), pre=None):
    """One decode token per sequence (see include/gdn.h).  q, k [B, Hk, dk];
    v [B, Hv, dv]; g, beta [B, Hv]; state_pool [P, Hv, dv, dk] fp32 updated in
    place; state_idx [B] int32 or None (identity).  Returns out [B, Hv, dv]."""
    import torch
    B, hk, dk, hv, dv, _ = _dims_of(q, k, v, g, beta)
    _check_pool(state_pool, hv, dv, dk)
    _check_index(state_idx, "state_idx", B)
    _shape(out, "out", (B, hv, dv))
    _check_pre(pre, hv)
    lib = load_library()
    for name, t in (("q", q), ("k", k), ("v", v)):
        _need(t, name, q.dtype)
    _need(g, "g", torch.float32)
    _need(beta, "beta", torch.float32)
    _need(state_pool, "state_pool", torch.float32)
    _need(state_idx, "state_idx", torch.int32)
    if out is None:
        out = torch.empty((B, hv, dv), dtype=q.dtype, device=q.device)
    _need(out, "out", q.dtype)
    dims = make_dims(q, v, B, B, pool_size=int(state_pool.shape[0]), plan=plan, pre=pre)
    _check(lib.gdn_decode_step(ctypes.byref(dims), _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta),
                               _ptr(state_pool), _ptr(state_idx), _ptr(out), _stream_handle(stream)))
    return out


def gdn_short_conv(x, w, cu_seqlens, state_pool, bias=None, src_idx=None, dst_idx=None, silu: bool = True,
                   y=None, stream=None):
    """Short causal convolution with a carried state (see include/gdn.h).  x [T, C]
    (bf16 or fp32, on the GPU); w [C, K] fp32; state_pool [P, C, K-1] in x's dtype,
    updated in place; src_idx / dst_idx [N] int32 or None.  Returns y [T, C]."""
    import torch
    if x is None or x.dim() != 2 or w is None or w.dim() != 2:
        raise ValueError("x must be [T, C] and w [C, K]")
    T, C = int(x.shape[0]), int(x.shape[1])
    K = int(w.shape[1])
    _shape(w, "w", (C, K))
    _shape(bias, "bias", (C,))
    if cu_seqlens is None or cu_seqlens.dim() != 1 or cu_seqlens.numel() < 1:
        raise ValueError("cu_seqlens must be a 1-D [N+1] tensor")
    N = int(cu_seqlens.numel()) - 1
    if state_pool is None or state_pool.dim() != 3 or tuple(int(s) for s in state_pool.shape[1:]) != (C, K - 1):
        raise ValueError("state_pool must be [P, C, K-1] = [P, %d, %d], got %s"
                         % (C, K - 1, None if state_pool is None else tuple(state_pool.shape)))
    _check_index(src_idx, "src_idx", N)
    _check_index(dst_idx, "dst_idx", N)
    _shape(y, "y", (T, C))
    lib = load_library()
    _need(x, "x")
    _need(w, "w", torch.float32)
    _need(bias, "bias", torch.float32)
    _need(cu_seqlens, "cu_seqlens", torch.int32)
    _need(state_pool, "state_pool", x.dtype)
    _need(src_idx, "src_idx", torch.int32)
    _need(dst_idx, "dst_idx", torch.int32)
    if y is None:
        y = torch.empty_like(x)
    _need(y, "y", x.dtype)
    dims = GdnConvDims(n_seqs=int(cu_seqlens.numel()) - 1, channels=C, taps=int(w.shape[1]), io_dtype=_io_code(x),
                       total_tokens=T, pool_size=int(state_pool.shape[0]), flags=GDN_CONV_SILU if silu else 0)
    _check(lib.gdn_short_conv(ctypes.byref(dims), _ptr(x), _ptr(w), _ptr(bias), _ptr(cu_seqlens), _ptr(state_pool),
                              _ptr(src_idx), _ptr(dst_idx), _ptr(y), _stream_handle(stream)))
    return y


def gdn_short_conv_backward_workspace_size(dims: GdnConvDims) -> int:
    """Workspace bytes gdn_short_conv_backward needs for ``dims`` (host only)."""
    n = ctypes.c_uint64(0)
    _check(load_library().gdn_short_conv_backward_workspace_size(ctypes.byref(dims), ctypes.byref(n)))
    return int(n.value)


def gdn_short_conv_backward(x, w, cu_seqlens, state_pool, dy, bias=None, src_idx=None, silu: bool = True,
                            workspace=None, grads=None, want_dstate: bool = True, stream=None):
    """Backward of gdn_short_conv (see include/gdn.h): x, w, cu_seqlens, bias, src_idx
    as the forward, ``state_pool`` the states it read, dy [T, C] fp32.  Returns a
    dict of fp32 dx [T, C], dw [C, K], dbias [C] (None without ``bias``) and dstate
    [N, C, K-1] (None unless ``want_dstate``)."""
    import torch
    if x is None or x.dim() != 2 or w is None or w.dim() != 2:
        raise ValueError("x must be [T, C] and w [C, K]")
    T, C = int(x.shape[0]), int(x.shape[1])
    K = int(w.shape[1])
    _shape(w, "w", (C, K))
    _shape(bias, "bias", (C,))
    _shape(dy, "dy", (T, C))
    if cu_seqlens is None or cu_seqlens.dim() != 1 or cu_seqlens.numel() < 1:
        raise ValueError("cu_seqlens must be a 1-D [N+1] tensor")
    N = int(cu_seqlens.numel()) - 1
    if state_pool is None or state_pool.dim() != 3 or tuple(int(s) for s in state_pool.shape[1:]) != (C, K - 1):
        raise ValueError("state_pool must be [P, C, K-1] = [P, %d, %d], got %s"
                         % (C, K - 1, None if state_pool is None else tuple(state_pool.shape)))
    _check_index(src_idx, "src_idx", N)
    gshapes = (("dx", (T, C)), ("dw", (C, K)), ("dbias", (C,)), ("dstate", (N, C, K - 1)))
    if grads is not None:
        for name, shp in gshapes:
            if name in ("dx", "dw") and grads.get(name) is None:
                raise ValueError("grads[%r] is required" % name)
            _shape(grads.get(name), name, shp)
    if dy is None:
        raise ValueError("dy is required")
    _need(x, "x")
    _need(w, "w", torch.float32)
    _need(bias, "bias", torch.float32)
    _need(cu_seqlens, "cu_seqlens", torch.int32)
    _need(state_pool, "state_pool", x.dtype)
    _need(src_idx, "src_idx", torch.int32)
    _need(dy, "dy", torch.float32)
    dims = GdnConvDims(n_seqs=N, channels=C, taps=K, io_dtype=_io_code(x), total_tokens=T,
                       pool_size=int(state_pool.shape[0]), flags=GDN_CONV_SILU if silu else 0)
    if workspace is None:
        workspace = torch.empty(max(gdn_short_conv_backward_workspace_size(dims), 4), dtype=torch.uint8,
                                device=x.device)
    _need(workspace, "workspace", torch.uint8)
    if grads is None:
        f32 = dict(dtype=torch.float32, device=x.device)
        grads = {"dx": torch.empty((T, C), **f32), "dw": torch.empty((C, K), **f32),
                 "dbias": torch.empty((C,), **f32) if bias is not None else None,
                 "dstate": torch.empty((N, C, K - 1), **f32) if want_dstate else None}
    for name, _ in gshapes:
        _need(grads.get(name), name, torch.float32)
    _check(load_library().gdn_short_conv_backward(
        ctypes.byref(dims), _ptr(x), _ptr(w), _ptr(bias), _ptr(cu_seqlens), _ptr(state_pool), _ptr(src_idx),
        _ptr(dy), _ptr(grads["dx"]), _ptr(grads["dw"]), _ptr(grads.get("dbias")), _ptr(grads.get("dstate")),
        _ptr(workspace), int(workspace.numel()), _stream_handle(stream)))
    return grads
