"""Chunked backward (gdn_bwd_chunked, the matrix-core WY form) on the GPU.

Parity: every gradient against the fp64 gradient oracle (oracle.gdn_backward,
pinned by finite differences and closed forms), with the gates of the recurrent
backward's tests (1e-4 normwise per sequence; dg against the scale of its terms).
The chunked form computes the same gradients in another order, so it is compared
with the oracle, not bitwise with gdn_bwd_varlen.  Determinism, batch invariance
and independence from the forward walk's launch shape are bitwise.
"""
import pytest
import torch

from gpu_helpers import say, to_dev
from invariant_linear_attention_amd import synth
from test_backward import check_grads, grad_inputs

pytestmark = pytest.mark.gpu
DEV = "cuda"


def run_cbwd(gdn, w, dout, dhT, d=None, **kw):
    d = d if d is not None else to_dev(w)
    r = gdn.gdn_bwd_chunked(d["q"], d["k"], d["v"], d["g"], d["beta"], d["h0"], d["cu_seqlens"], dout.to(DEV),
                            None if dhT is None else dhT.to(DEV), **kw)
    torch.cuda.synchronize()
    return r


@pytest.mark.parametrize("hk,hv,dk,dv,io", [
    (2, 4, 128, 128, torch.bfloat16),
    (2, 4, 64, 64, torch.float32),
    (1, 4, 64, 128, torch.bfloat16),   # four value heads per key head
    (2, 2, 128, 32, torch.float32),    # one value head per key head: dq, dk written directly
    (1, 2, 64, 32, torch.bfloat16),
    (1, 1, 128, 64, torch.bfloat16),
])
@pytest.mark.parametrize("with_h0,with_dhT", [(True, True), (False, False)])
def test_parity_small(gpu, hk, hv, dk, dv, io, with_h0, with_dhT):
    from oracle import oracle
    # lengths: ragged tails, an empty sequence, exact chunks, a lone token
    w = synth.make_workload(500 + dk + dv, [37, 1, 100, 0, 16, 33], hk=hk, hv=hv, dk=dk, dv=dv, io_dtype=io,
                            h0_std=0.1 if with_h0 else 0.0)
    dout, dhT = grad_inputs(w, 21, dhT=with_dhT)
    r = run_cbwd(gpu, w, dout, dhT)
    ref = oracle.gdn_backward(w.q, w.k, w.v, w.g, w.beta, w.cu_seqlens, dout, h0=w.h0, dhT=dhT)
    check_grads(w, r, ref, "chunked bwd hk=%d hv=%d dk=%d dv=%d %s h0=%s dhT=%s"
                % (hk, hv, dk, dv, io, with_h0, with_dhT), dout)


@pytest.mark.parametrize("hk,hv,dk,dv", [(2, 4, 128, 128), (2, 2, 64, 64), (1, 1, 128, 128), (1, 2, 64, 128)])
@pytest.mark.parametrize("parts", [1, 2])
def test_parity_row_parts(gpu, hk, hv, dk, dv, parts):
    """The reverse walk with the state rows in one workgroup or split over two (each
    part's sums over its rows added afterwards), against the oracle."""
    from oracle import oracle
    w = synth.make_workload(570 + dk + dv + hv, [45, 0, 130, 16, 3], hk=hk, hv=hv, dk=dk, dv=dv, h0_std=0.1)
    dout, dhT = grad_inputs(w, 22)
    r = run_cbwd(gpu, w, dout, dhT, parts=parts)
    ref = oracle.gdn_backward(w.q, w.k, w.v, w.g, w.beta, w.cu_seqlens, dout, h0=w.h0, dhT=dhT)
    check_grads(w, r, ref, "chunked bwd parts=%d hk=%d hv=%d dk=%d dv=%d" % (parts, hk, hv, dk, dv), dout)


def test_parity_benchmark_batch(gpu):
    """The benchmark batch (8 sequences, 17,459 tokens, 16/32 heads, dk = dv = 128),
    every gradient of every head against the oracle."""
    from oracle import oracle
    w = synth.varlen_prefill(1001)
    dout, dhT = grad_inputs(w, 12)
    r = run_cbwd(gpu, w, dout, dhT)
    ref = oracle.gdn_backward(w.q, w.k, w.v, w.g, w.beta, w.cu_seqlens, dout, h0=w.h0, dhT=dhT)
    check_grads(w, r, ref, "chunked bwd benchmark batch", dout)


@pytest.mark.parametrize("parts", [0, 1, 2])
def test_deterministic_batch_invariant_any_walk_shape(gpu, parts):
    """Repeat, alone vs in a batch, and the forward walk at 1, 2 and 4 waves per
    state tile: all bitwise equal for each split of the reverse walk's rows."""
    w = synth.make_workload(521, [70, 5, 33, 0, 130], hk=2, hv=4, dk=128, dv=128, h0_std=0.1)
    dout, dhT = grad_inputs(w, 13)
    r1 = run_cbwd(gpu, w, dout, dhT, parts=parts)
    for waves in (0, 1, 2, 4):
        r2 = run_cbwd(gpu, w, dout, dhT, waves=waves, parts=parts)
        for key in r1:
            assert torch.equal(r1[key], r2[key]), (waves, key)
    cu = w.cu_seqlens.tolist()
    for n in (0, 2, 4):
        s = synth.select(w, [n])
        a, b = cu[n], cu[n + 1]
        rs = run_cbwd(gpu, s, dout[a:b].contiguous(), dhT[n:n + 1].contiguous(), parts=parts)
        for key in ("dq", "dk", "dv", "dg", "dbeta"):
            assert torch.equal(rs[key], r1[key][a:b]), (n, key)
        assert torch.equal(rs["dh0"][0], r1["dh0"][n]), n
    if parts == 0:  # the automatic split for dv = 128 is two parts
        r2 = run_cbwd(gpu, w, dout, dhT, parts=2)
        for key in r1:
            assert torch.equal(r1[key], r2[key]), ("auto", key)
    say("chunked backward parts=%d: repeat, walk shapes and alone-vs-batch bitwise equal" % parts)


@pytest.mark.parametrize("dk,io", [(128, torch.bfloat16), (64, torch.float32)])
def test_wave_specialization_same_bits(gpu, dk, io):
    """dv = 128 in two parts runs with state and gradient waves by default; the plain
    walk (every wave does a whole chunk) gives the same bits."""
    w = synth.make_workload(581 + dk, [70, 0, 16, 33, 1, 130], hk=2, hv=4, dk=dk, dv=128, io_dtype=io, h0_std=0.1)
    dout, dhT = grad_inputs(w, 23)
    r1 = run_cbwd(gpu, w, dout, dhT, parts=2)
    r2 = run_cbwd(gpu, w, dout, dhT, parts=2, plain=True)
    for key in r1:
        assert torch.equal(r1[key], r2[key]), key
    say("chunked backward dk=%d: specialized and plain reverse walks bitwise equal" % dk)


def test_empty_and_single_token_sequences(gpu):
    from oracle import oracle
    w = synth.make_workload(531, [0, 1, 0, 2, 1, 17], hk=1, hv=2, dk=64, dv=64, h0_std=0.1)
    dout, dhT = grad_inputs(w, 14)
    r = run_cbwd(gpu, w, dout, dhT)
    ref = oracle.gdn_backward(w.q, w.k, w.v, w.g, w.beta, w.cu_seqlens, dout, h0=w.h0, dhT=dhT)
    check_grads(w, r, ref, "chunked bwd short sequences", dout)
    # an empty sequence hands dhT straight back as dh0
    assert torch.equal(r["dh0"][0].cpu(), dhT[0]) and torch.equal(r["dh0"][2].cpu(), dhT[2])


def test_long_sequence(gpu):
    """One 8192-token sequence (512 chunks): the adjoint state and the gate
    gradient's running sum are carried longest here."""
    from oracle import oracle
    w = synth.make_workload(541, [8192], hk=1, hv=2, dk=128, dv=128, h0_std=0.1)
    dout, dhT = grad_inputs(w, 15)
    r = run_cbwd(gpu, w, dout, dhT)
    ref = oracle.gdn_backward(w.q, w.k, w.v, w.g, w.beta, w.cu_seqlens, dout, h0=w.h0, dhT=dhT)
    check_grads(w, r, ref, "chunked bwd 8192 tokens", dout)


def test_workspace_contents_do_not_matter(gpu):
    """A NaN-filled workspace gives the same bits as a zeroed one; dh0 may be skipped."""
    from invariant_linear_attention_amd import gdn
    w = synth.make_workload(551, [40, 0, 17, 64], hk=2, hv=4, dk=128, dv=64, h0_std=0.1)
    dout, dhT = grad_inputs(w, 16)
    d = to_dev(w)
    dims = gdn.make_dims(d["q"], d["v"], w.n_seqs, int(w.q.shape[0]))
    nbytes = gdn.gdn_bwd_chunked_workspace_size(dims)
    ws0 = torch.zeros(nbytes, dtype=torch.uint8, device=DEV)
    ws1 = torch.full((nbytes // 4,), float("nan"), dtype=torch.float32, device=DEV).view(torch.uint8)
    args = (d["q"], d["k"], d["v"], d["g"], d["beta"], d["h0"], d["cu_seqlens"], dout.to(DEV), dhT.to(DEV))
    r0 = gdn.gdn_bwd_chunked(*args, workspace=ws0)
    r1 = gdn.gdn_bwd_chunked(*args, workspace=ws1, want_dh0=False)
    torch.cuda.synchronize()
    assert r1["dh0"] is None
    for key in ("dq", "dk", "dv", "dg", "dbeta"):
        assert torch.equal(r0[key], r1[key]), key
    assert all(bool(torch.isfinite(r0[key]).all()) for key in r0)


def test_agrees_with_recurrent_backward(gpu):
    """The two backward forms on one batch: the same gradients to fp32 rounding."""
    w = synth.make_workload(561, [300, 77, 512], hk=2, hv=4, dk=128, dv=128, h0_std=0.1)
    dout, dhT = grad_inputs(w, 18)
    d = to_dev(w)
    rc = run_cbwd(gpu, w, dout, dhT, d=d)
    rr = gpu.gdn_bwd_varlen(d["q"], d["k"], d["v"], d["g"], d["beta"], d["h0"], d["cu_seqlens"], dout.to(DEV),
                            dhT.to(DEV))
    torch.cuda.synchronize()
    for key in ("dq", "dk", "dv", "dbeta", "dh0"):
        a, b = rc[key].double(), rr[key].double()
        err = float((a - b).norm() / b.norm())
        say("chunked vs recurrent %s: %.2e" % (key, err))
        assert err <= 2e-4, key
