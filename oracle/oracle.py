"""Python front end of the fp64 CPU oracle for the Gated DeltaNet recurrent forward.

TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the benchmark's
CPU-baseline leg may import this module.  The HIP library never calls it and the
two share no code.

The arithmetic lives in ``gdn_oracle.c`` (plain fp64 loops, see its header for
the recurrence and the layouts).  This module only builds that file with gcc if
needed, converts inputs to the exact arrays the GPU receives (bf16 as raw bits,
fp32 as is, fp32 initial state widened to fp64) and calls it through ctypes.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
SOURCE = os.path.join(_HERE, "gdn_oracle.c")
LIBRARY = os.path.join(_HERE, "libgdn_oracle.so")

# Plain build: no fast-math, no FMA contraction, OpenMP over independent units.
CFLAGS = ["-O2", "-fno-fast-math", "-ffp-contract=off", "-fopenmp", "-fPIC", "-shared", "-std=c11"]

_lock = threading.Lock()
_lib = None


def build(source: str = SOURCE, library: str = LIBRARY, extra_flags=()) -> str:
    """Compile the oracle C source into a shared library (always rebuilds)."""
    tmp = library + ".tmp%d" % os.getpid()
    cmd = ["gcc", *CFLAGS, *extra_flags, "-o", tmp, source, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, library)
    return library


def load(library: str = LIBRARY):
    """Load (building on first use if absent) and type the oracle library."""
    lib = ctypes.CDLL(library)
    f = lib.gdn_oracle_forward
    f.restype = ctypes.c_int
    f.argtypes = [
        ctypes.c_int32, ctypes.c_void_p,
        ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
        ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
        ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
        ctypes.c_void_p, ctypes.c_void_p,
        ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
        ctypes.c_int32,
    ]
    p = lib.gdn_oracle_preprocess
    p.restype = ctypes.c_int
    p.argtypes = [
        ctypes.c_int64, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
        ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
        ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int32, ctypes.c_double,
        ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
    ]
    c = lib.gdn_oracle_short_conv
    c.restype = ctypes.c_int
    c.argtypes = [ctypes.c_int32, ctypes.c_void_p, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                  ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int32,
                  ctypes.c_void_p, ctypes.c_void_p]
    pb = lib.gdn_oracle_preprocess_backward
    pb.restype = ctypes.c_int
    pb.argtypes = [
        ctypes.c_int64, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
        ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
        ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int32, ctypes.c_double,
        ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
        ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
    ]
    cb = lib.gdn_oracle_short_conv_backward
    cb.restype = ctypes.c_int
    cb.argtypes = [ctypes.c_int32, ctypes.c_void_p, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                   ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int32,
                   ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]
    b = lib.gdn_oracle_backward
    b.restype = ctypes.c_int
    b.argtypes = [
        ctypes.c_int32, ctypes.c_void_p,
        ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
        ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
        ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
        ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
        ctypes.c_void_p, ctypes.c_void_p,
        ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
        ctypes.c_int32,
    ]
    lib.gdn_oracle_max_threads.restype = ctypes.c_int
    lib.gdn_oracle_max_threads.argtypes = []
    return lib


def _get_lib():
    global _lib
    with _lock:
        if _lib is None:
            if not os.path.exists(LIBRARY) or os.path.getmtime(LIBRARY) < os.path.getmtime(SOURCE):
                build()
            _lib = load(LIBRARY)
        return _lib


def _as_numpy(x):
    """torch tensor or array -> (numpy array, io code). bf16 becomes uint16 bits."""
    try:
        import torch
    except ImportError:  # pragma: no cover - torch is always present here
        torch = None
    if torch is not None and isinstance(x, torch.Tensor):
        x = x.detach().cpu().contiguous()
        if x.dtype == torch.bfloat16:
            return x.view(torch.int16).numpy().view(np.uint16), 1
        if x.dtype == torch.float32:
            return x.numpy(), 0
        if x.dtype == torch.float64:
            return x.numpy(), 2
        if x.dtype == torch.int32:
            return x.numpy(), 3
        raise TypeError("unsupported tensor dtype %s" % x.dtype)
    x = np.ascontiguousarray(x)
    if x.dtype == np.uint16:
        return x, 1
    if x.dtype == np.float32:
        return x, 0
    if x.dtype == np.float64:
        return x, 2
    if x.dtype == np.int32:
        return x, 3
    raise TypeError("unsupported array dtype %s" % x.dtype)


def gdn_forward(q, k, v, g, beta, cu_seqlens, h0=None, n_threads=None, library=None):
    """Run the fp64 oracle.

    q, k: [T, Hk, dk] and v: [T, Hv, dv], each fp32, bf16 (torch bf16 or raw
    uint16 bits) or fp64 (q and k share one dtype); g, beta: [T, Hv] fp32 or fp64
    (one dtype); cu_seqlens: [N+1] int32; h0: optional [N, Hv, dv, dk] fp32 or
    fp64.  Every input is widened exactly.

    Returns (out [T, Hv, dv] float64, hT [N, Hv, dv, dk] float64).
    """
    qn, qc = _as_numpy(q)
    kn, kc = _as_numpy(k)
    vn, vc = _as_numpy(v)
    if not (qc == kc and qc in (0, 1, 2) and vc in (0, 1, 2)):
        raise TypeError("q and k must share one dtype; q, k, v must be fp32, bf16 or fp64")
    gn, gc = _as_numpy(g)
    bn, bc = _as_numpy(beta)
    if gc != bc or gc not in (0, 2):
        raise TypeError("g and beta must both be fp32 or both fp64")
    cu, cc = _as_numpy(cu_seqlens)
    if cc != 3:
        raise TypeError("cu_seqlens must be int32")
    if qn.ndim != 3 or kn.shape != qn.shape or vn.ndim != 3:
        raise ValueError("q, k must be [T, Hk, dk] and v [T, Hv, dv]")
    T, hk, dk = qn.shape
    hv, dv = vn.shape[1], vn.shape[2]
    if vn.shape[0] != T or gn.shape != (T, hv) or bn.shape != (T, hv):
        raise ValueError("inconsistent token / head shapes")
    n = cu.shape[0] - 1
    if n < 0 or (n > 0 and int(cu[-1]) != T):
        raise ValueError("cu_seqlens[-1] must equal T")
    h0n = None
    if h0 is not None:
        h0n, hc = _as_numpy(h0)
        if hc not in (0, 2):
            raise TypeError("h0 must be fp32 or fp64")
        h0n = np.ascontiguousarray(h0n, dtype=np.float64)
        if h0n.shape != (n, hv, dv, dk):
            raise ValueError("h0 must be [N, Hv, dv, dk]")
    out = np.zeros((T, hv, dv), dtype=np.float64)
    hT = np.zeros((max(n, 0), hv, dv, dk), dtype=np.float64)
    lib = load(library) if library is not None else _get_lib()
    if n_threads is None:
        n_threads = os.cpu_count() or 1

    def ptr(a):
        return None if a is None or a.size == 0 else a.ctypes.data

    rc = lib.gdn_oracle_forward(
        n, ptr(cu), hk, hv, dk, dv, qc, vc, gc,
        ptr(qn), ptr(kn), ptr(vn), ptr(gn), ptr(bn),
        ptr(h0n), ptr(out), ptr(hT), int(n_threads))
    if rc != 0:
        raise ValueError("oracle rejected its arguments (code %d)" % rc)
    return out, hT


def preprocess(q, k, a, b, A_log=None, dt_bias=None, norm_qk=True, eps=1e-6, library=None):
    """fp64 preprocessing of the fused path (see gdn_oracle_preprocess).

    q, k: [T, Hk, dk] fp32 or bf16 (one dtype); a, b: [T, Hv] fp32; A_log, dt_bias:
    [Hv] fp32 or None.  Returns (q', k', g, beta), all float64.
    """
    qn, qc = _as_numpy(q)
    kn, kc = _as_numpy(k)
    if not (qc == kc and qc in (0, 1)):
        raise TypeError("q and k must share one dtype: fp32 or bf16")
    an, ac = _as_numpy(a)
    bn, bc = _as_numpy(b)
    if ac != 0 or bc != 0:
        raise TypeError("a and b must be fp32")
    T, hk, dk = qn.shape
    hv = an.shape[1]
    if kn.shape != qn.shape or an.shape != (T, hv) or bn.shape != (T, hv):
        raise ValueError("inconsistent shapes")
    Ln = Dn = None
    if A_log is not None:
        Ln, lc = _as_numpy(A_log)
        if lc != 0 or Ln.shape != (hv,):
            raise ValueError("A_log must be fp32 [Hv]")
    if dt_bias is not None:
        Dn, dc = _as_numpy(dt_bias)
        if dc != 0 or Dn.shape != (hv,):
            raise ValueError("dt_bias must be fp32 [Hv]")
    q2 = np.zeros((T, hk, dk), dtype=np.float64)
    k2 = np.zeros((T, hk, dk), dtype=np.float64)
    g2 = np.zeros((T, hv), dtype=np.float64)
    b2 = np.zeros((T, hv), dtype=np.float64)
    lib = load(library) if library is not None else _get_lib()

    def ptr(x):
        return None if x is None or x.size == 0 else x.ctypes.data

    rc = lib.gdn_oracle_preprocess(T, hk, hv, dk, qc, ptr(qn), ptr(kn), ptr(an), ptr(bn), ptr(Ln), ptr(Dn),
                                   1 if norm_qk else 0, float(eps), ptr(q2), ptr(k2), ptr(g2), ptr(b2))
    if rc != 0:
        raise ValueError("oracle rejected its arguments (code %d)" % rc)
    return q2, k2, g2, b2


def _f64(x, shape, name):
    """Gradient input (torch or numpy, fp32, bf16 or fp64) as a contiguous float64 array."""
    xn, xc = _as_numpy(x)
    if xc == 1:
        import torch
        xn = torch.from_numpy(xn.view(np.int16)).view(torch.bfloat16).double().numpy()
    elif xc not in (0, 2):
        raise TypeError("%s must be fp32, bf16 or fp64" % name)
    xn = np.ascontiguousarray(xn, dtype=np.float64)
    if xn.shape != tuple(shape):
        raise ValueError("%s must have shape %s" % (name, tuple(shape)))
    return xn


def preprocess_backward(q, k, a, b, dqn, dkn, dg, dbeta, A_log=None, dt_bias=None, norm_qk=True, eps=1e-6,
                        library=None):
    """fp64 gradients of preprocess() (see gdn_oracle_preprocess_backward).

    q, k, a, b, A_log, dt_bias as preprocess(); dqn, dkn [T, Hk, dk] and dg, dbeta
    [T, Hv]: the loss's gradients with respect to preprocess()'s four outputs.
    Returns a dict of float64 arrays: dq, dk [T, Hk, dk]; da, db [T, Hv]; and, with
    A_log, dA_log and ddt_bias [Hv].
    """
    qn, qc = _as_numpy(q)
    kn, kc = _as_numpy(k)
    if not (qc == kc and qc in (0, 1)):
        raise TypeError("q and k must share one dtype: fp32 or bf16")
    an, ac = _as_numpy(a)
    bn, bc = _as_numpy(b)
    if ac != 0 or bc != 0:
        raise TypeError("a and b must be fp32")
    T, hk, dk = qn.shape
    hv = an.shape[1]
    if kn.shape != qn.shape or an.shape != (T, hv) or bn.shape != (T, hv):
        raise ValueError("inconsistent shapes")
    Ln = Dn = None
    if A_log is not None:
        Ln, lc = _as_numpy(A_log)
        if lc != 0 or Ln.shape != (hv,):
            raise ValueError("A_log must be fp32 [Hv]")
    if dt_bias is not None:
        Dn, dc = _as_numpy(dt_bias)
        if dc != 0 or Dn.shape != (hv,):
            raise ValueError("dt_bias must be fp32 [Hv]")
    gq, gk = _f64(dqn, (T, hk, dk), "dqn"), _f64(dkn, (T, hk, dk), "dkn")
    gg, gb = _f64(dg, (T, hv), "dg"), _f64(dbeta, (T, hv), "dbeta")
    res = {"dq": np.zeros((T, hk, dk)), "dk": np.zeros((T, hk, dk)), "da": np.zeros((T, hv)),
           "db": np.zeros((T, hv))}
    if A_log is not None:
        res["dA_log"] = np.zeros(hv)
        res["ddt_bias"] = np.zeros(hv)
    lib = load(library) if library is not None else _get_lib()

    def ptr(x):
        return None if x is None or x.size == 0 else x.ctypes.data

    rc = lib.gdn_oracle_preprocess_backward(
        T, hk, hv, dk, qc, ptr(qn), ptr(kn), ptr(an), ptr(bn), ptr(Ln), ptr(Dn), 1 if norm_qk else 0, float(eps),
        ptr(gq), ptr(gk), ptr(gg), ptr(gb), ptr(res["dq"]), ptr(res["dk"]), ptr(res["da"]), ptr(res["db"]),
        ptr(res.get("dA_log")), ptr(res.get("ddt_bias")))
    if rc != 0:
        raise ValueError("oracle rejected its arguments (code %d)" % rc)
    return res


def gdn_forward_fused(q, k, v, a, b, cu_seqlens, h0=None, A_log=None, dt_bias=None, norm_qk=True, eps=1e-6,
                      n_threads=None, library=None):
    """preprocess() followed by gdn_forward() on its fp64 results."""
    q2, k2, g2, b2 = preprocess(q, k, a, b, A_log, dt_bias, norm_qk, eps, library=library)
    return gdn_forward(q2, k2, v, g2, b2, cu_seqlens, h0, n_threads=n_threads, library=library)


def max_threads() -> int:
    return int(_get_lib().gdn_oracle_max_threads())


def short_conv(x, w, cu_seqlens, bias=None, state=None, silu=True, library=None):
    """fp64 short causal convolution with a carried state (see gdn_oracle_short_conv).

    x: [T, C] fp32 or bf16; w: [C, K] fp32; bias: [C] fp32 or None; state:
    [N, C, K-1] (fp32, bf16 or fp64; widened exactly) or None.
    Returns (y [T, C] float64, state_out [N, C, K-1] float64).
    """
    xn, xc = _as_numpy(x)
    if xc not in (0, 1):
        raise TypeError("x must be fp32 or bf16")
    wn, wc = _as_numpy(w)
    if wc != 0 or wn.ndim != 2:
        raise TypeError("w must be fp32 [C, K]")
    cu, cc = _as_numpy(cu_seqlens)
    if cc != 3:
        raise TypeError("cu_seqlens must be int32")
    T, C = xn.shape
    K = wn.shape[1]
    if wn.shape[0] != C:
        raise ValueError("w must be [C, K]")
    n = cu.shape[0] - 1
    bn = None
    if bias is not None:
        bn, bc = _as_numpy(bias)
        if bc != 0 or bn.shape != (C,):
            raise ValueError("bias must be fp32 [C]")
    sn = None
    if state is not None:
        sn, sc = _as_numpy(state)
        if sc == 1:
            import torch
            sn = torch.from_numpy(sn.view(np.int16)).view(torch.bfloat16).float().numpy()
        sn = np.ascontiguousarray(sn, dtype=np.float64)
        if sn.shape != (n, C, K - 1):
            raise ValueError("state must be [N, C, K-1]")
    y = np.zeros((T, C), dtype=np.float64)
    so = np.zeros((max(n, 0), C, K - 1), dtype=np.float64)
    lib = load(library) if library is not None else _get_lib()

    def ptr(a):
        return None if a is None or a.size == 0 else a.ctypes.data

    rc = lib.gdn_oracle_short_conv(n, ptr(cu), C, K, xc, ptr(xn), ptr(wn), ptr(bn), ptr(sn), 1 if silu else 0,
                                   ptr(y), ptr(so))
    if rc != 0:
        raise ValueError("oracle rejected its arguments (code %d)" % rc)
    return y, so


def gdn_backward(q, k, v, g, beta, cu_seqlens, dout, h0=None, dhT=None, n_threads=None, library=None):
    """fp64 gradients of gdn_forward (see gdn_oracle_backward).

    Inputs as gdn_forward, plus dout [T, Hv, dv] (fp32, bf16 or fp64) and dhT
    (optional [N, Hv, dv, dk], fp32 or fp64): the gradient of the loss with respect
    to the outputs and to the final state.  Returns a dict of float64 arrays:
    dq, dk [T, Hk, dk]; dv [T, Hv, dv]; dg, dbeta [T, Hv]; dh0 [N, Hv, dv, dk].
    """
    qn, qc = _as_numpy(q)
    kn, kc = _as_numpy(k)
    vn, vc = _as_numpy(v)
    if not (qc == kc and qc in (0, 1, 2) and vc in (0, 1, 2)):
        raise TypeError("q and k must share one dtype; q, k, v must be fp32, bf16 or fp64")
    gn, gc = _as_numpy(g)
    bn, bc = _as_numpy(beta)
    if gc != bc or gc not in (0, 2):
        raise TypeError("g and beta must both be fp32 or both fp64")
    dn, dc = _as_numpy(dout)
    if dc not in (0, 1, 2):
        raise TypeError("dout must be fp32, bf16 or fp64")
    cu, cc = _as_numpy(cu_seqlens)
    if cc != 3:
        raise TypeError("cu_seqlens must be int32")
    T, hk, dk = qn.shape
    hv, dv = vn.shape[1], vn.shape[2]
    if kn.shape != qn.shape or vn.shape[0] != T or gn.shape != (T, hv) or bn.shape != (T, hv) or \
            dn.shape != (T, hv, dv):
        raise ValueError("inconsistent shapes")
    n = cu.shape[0] - 1
    if n < 0 or (n > 0 and int(cu[-1]) != T):
        raise ValueError("cu_seqlens[-1] must equal T")

    def state(x, name):
        if x is None:
            return None
        xn, xc = _as_numpy(x)
        if xc not in (0, 2):
            raise TypeError("%s must be fp32 or fp64" % name)
        xn = np.ascontiguousarray(xn, dtype=np.float64)
        if xn.shape != (n, hv, dv, dk):
            raise ValueError("%s must be [N, Hv, dv, dk]" % name)
        return xn

    h0n, dhn = state(h0, "h0"), state(dhT, "dhT")
    res = {"dq": np.zeros((T, hk, dk)), "dk": np.zeros((T, hk, dk)), "dv": np.zeros((T, hv, dv)),
           "dg": np.zeros((T, hv)), "dbeta": np.zeros((T, hv)), "dh0": np.zeros((max(n, 0), hv, dv, dk))}
    lib = load(library) if library is not None else _get_lib()
    if n_threads is None:
        n_threads = os.cpu_count() or 1

    def ptr(a):
        return None if a is None or a.size == 0 else a.ctypes.data

    rc = lib.gdn_oracle_backward(
        n, ptr(cu), hk, hv, dk, dv, qc, vc, gc, dc,
        ptr(qn), ptr(kn), ptr(vn), ptr(gn), ptr(bn), ptr(h0n), ptr(dn), ptr(dhn),
        ptr(res["dq"]), ptr(res["dk"]), ptr(res["dv"]), ptr(res["dg"]), ptr(res["dbeta"]), ptr(res["dh0"]),
        int(n_threads))
    if rc != 0:
        raise ValueError("oracle rejected its arguments (code %d)" % rc)
    return res


def short_conv_backward(x, w, cu_seqlens, dy, bias=None, state=None, silu=True, library=None):
    """fp64 gradients of short_conv() (see gdn_oracle_short_conv_backward).

    x, w, cu_seqlens, bias, state as short_conv(); dy [T, C] (fp32, bf16 or fp64):
    dL/dy.  Returns a dict of float64 arrays: dx [T, C], dw [C, K], dbias [C] and
    dstate [N, C, K-1] (the gradient of the carried state taken in).
    """
    xn, xc = _as_numpy(x)
    if xc not in (0, 1):
        raise TypeError("x must be fp32 or bf16")
    wn, wc = _as_numpy(w)
    if wc != 0 or wn.ndim != 2:
        raise TypeError("w must be fp32 [C, K]")
    cu, cc = _as_numpy(cu_seqlens)
    if cc != 3:
        raise TypeError("cu_seqlens must be int32")
    T, C = xn.shape
    K = wn.shape[1]
    if wn.shape[0] != C:
        raise ValueError("w must be [C, K]")
    n = cu.shape[0] - 1
    bn = None
    if bias is not None:
        bn, bc = _as_numpy(bias)
        if bc != 0 or bn.shape != (C,):
            raise ValueError("bias must be fp32 [C]")
    sn = None
    if state is not None:
        sn = _f64(state, (n, C, K - 1), "state")
    gy = _f64(dy, (T, C), "dy")
    res = {"dx": np.zeros((T, C)), "dw": np.zeros((C, K)), "dbias": np.zeros(C),
           "dstate": np.zeros((max(n, 0), C, K - 1))}
    lib = load(library) if library is not None else _get_lib()

    def ptr(a):
        return None if a is None or a.size == 0 else a.ctypes.data

    rc = lib.gdn_oracle_short_conv_backward(n, ptr(cu), C, K, xc, ptr(xn), ptr(wn), ptr(bn), ptr(sn),
                                            1 if silu else 0, ptr(gy), ptr(res["dx"]), ptr(res["dw"]),
                                            ptr(res["dbias"]), ptr(res["dstate"]))
    if rc != 0:
        raise ValueError("oracle rejected its arguments (code %d)" % rc)
    return res
