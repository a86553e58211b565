"""gdn_bwd_varlen_noalloc (the allocation-free backward) against gdn_bwd_varlen.

Both run the same kernels; the only difference is where the workspace lives (a
fixed per-device array instead of the caller's buffer), so the gradients must be
bit-identical.  Two calls in a row, the second with a smaller input, check that the
array's leftover contents from the first call do not leak into the second.
"""
import ctypes

import pytest
import torch

from gpu_helpers import bit_equal, say
from invariant_linear_attention_amd import synth

pytestmark = pytest.mark.gpu
DEV = "cuda"


def grads_like(w, hk, hv, dk, dv):
    T, N = w.total_tokens, w.n_seqs
    f = dict(dtype=torch.float32, device=DEV)
    return {"dq": torch.empty((T, hk, dk), **f), "dk": torch.empty((T, hk, dk), **f), "dv": torch.empty((T, hv, dv), **f),
            "dg": torch.empty((T, hv), **f), "dbeta": torch.empty((T, hv), **f), "dh0": torch.empty((N, hv, dv, dk), **f)}


def run_both(gdn, seed, lengths, hk, hv, dk, dv, io):
    w = synth.make_workload(seed, lengths, hk=hk, hv=hv, dk=dk, dv=dv, io_dtype=io, h0_std=0.1)
    gen = torch.Generator().manual_seed(seed)
    dout = torch.randn(tuple(w.v.shape), generator=gen).to(io).to(DEV)
    dhT = torch.randn((w.n_seqs, hv, dv, dk), generator=gen).to(DEV)
    d = [t.to(DEV) for t in (w.q, w.k, w.v, w.g, w.beta, w.h0, w.cu_seqlens)]
    ref = gdn.gdn_bwd_varlen(*d, dout, dhT)
    got = grads_like(w, hk, hv, dk, dv)
    for t in got.values():
        t.fill_(float("nan"))
    # straight through the C ABI (the binding only marshals the pointers)
    lib = gdn.load_library()
    dims = gdn.make_dims(d[0], d[2], w.n_seqs, w.total_tokens)
    ptr = lambda t: ctypes.c_void_p(t.data_ptr())
    rc = lib.gdn_bwd_varlen_noalloc(ctypes.byref(dims), *(ptr(t) for t in d), ptr(dout), ptr(dhT), None, None,
                                    ptr(got["dq"]), ptr(got["dk"]), ptr(got["dv"]), ptr(got["dg"]), ptr(got["dbeta"]),
                                    ptr(got["dh0"]), ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert rc == 0, gdn.status_string(rc)
    torch.cuda.synchronize()
    for name in got:
        assert bit_equal(got[name], ref[name]), name
    return w


def test_noalloc_backward_matches_workspace_backward(gpu):
    # first call: 2 sequences, 700 tokens, hv = 32, dk = dv = 128 (about 48 MB of the 64 MiB scratch)
    w1 = run_both(gpu, 401, [500, 200], 16, 32, 128, 128, torch.bfloat16)
    need = gpu.gdn_bwd_workspace_size(gpu.make_dims(w1.q, w1.v, w1.n_seqs, w1.total_tokens))
    assert need <= gpu.GDN_NOALLOC_SCRATCH_BYTES
    # second call, smaller: the first call's leftovers must not reach it
    run_both(gpu, 402, [37, 1, 64], 2, 4, 64, 32, torch.float32)
    # through the binding as well
    w = synth.make_workload(403, [90], hk=2, hv=2, dk=32, dv=32, io_dtype=torch.float32, h0_std=0.1)
    d = [t.to(DEV) for t in (w.q, w.k, w.v, w.g, w.beta, w.h0, w.cu_seqlens)]
    dout = torch.ones(tuple(w.v.shape), device=DEV)
    ref = gpu.gdn_bwd_varlen(*d, dout)
    got = gpu.gdn_bwd_varlen(*d, dout, grads=grads_like(w, 2, 2, 32, 32), noalloc=True)
    torch.cuda.synchronize()
    assert all(bit_equal(got[n], ref[n]) for n in ref)
    say("noalloc backward: bit-identical to the workspace backward on 3 calls (%d bytes needed on the first)" % need)


def test_noalloc_refuses_what_does_not_fit(gpu):
    w = synth.make_workload(404, [1100], io_dtype=torch.bfloat16, h0_std=0.1)
    d = [t.to(DEV) for t in (w.q, w.k, w.v, w.g, w.beta, w.h0, w.cu_seqlens)]
    dout = torch.zeros(tuple(w.v.shape), dtype=torch.bfloat16, device=DEV)
    with pytest.raises(gpu.GdnError) as e:
        gpu.gdn_bwd_varlen(*d, dout, grads=grads_like(w, 16, 32, 128, 128), noalloc=True)
    assert e.value.code == 8
