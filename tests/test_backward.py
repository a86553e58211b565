"""Backward of the recurrent forward (gdn_bwd_varlen) on the GPU.

Parity: every gradient against the fp64 gradient oracle (oracle.gdn_backward, pinned
by finite differences and closed forms) on the same inputs.  The GPU works in fp32
from exactly the values the oracle widens, so the gap is fp32 rounding only; the
gate is 1e-4 normwise per sequence for each gradient (the fp32 state's gate).  dg
is formed as a running sum, over the rest of the sequence, of the terms
dO_s . o_s - dv_s . v_s, which largely cancel: its error scales with those terms,
not with dg (which is exactly 0 for a one-token sequence from a zero state), so its
gate is 1e-4 of the larger of ||dg|| and the norm of the terms in the sequence (the
measured worst is ~2e-6).
Determinism and batch invariance are bitwise: every sum has a fixed order and
nothing crosses sequences.
"""
import numpy as np
import pytest
import torch

from gpu_helpers import say, seq_errors, state_errors, to_dev
from invariant_linear_attention_amd import synth

pytestmark = pytest.mark.gpu
DEV = "cuda"
GRAD_TOL = {"dq": 1e-4, "dk": 1e-4, "dv": 1e-4, "dbeta": 1e-4, "dg": 1e-4}
DH0_TOL = 1e-4


def grad_inputs(w, seed, dhT=True):
    gen = torch.Generator().manual_seed(seed)
    T, hv, dv = w.v.shape
    dout = torch.randn((T, hv, dv), generator=gen).to(w.q.dtype)
    dh = torch.randn((w.n_seqs, hv, dv, w.q.shape[2]), generator=gen) if dhT else None
    return dout, dh


def run_bwd(gdn, w, dout, dhT, d=None):
    d = d if d is not None else to_dev(w)
    r = gdn.gdn_bwd_varlen(d["q"], d["k"], d["v"], d["g"], d["beta"], d["h0"], d["cu_seqlens"], dout.to(DEV),
                           None if dhT is None else dhT.to(DEV))
    torch.cuda.synchronize()
    return r


def gate_term_scale(w, ref, dout):
    """Per sequence: the 2-norm over (token, head) of |dO.o| + |dv.v| (oracle values)."""
    from oracle import oracle
    out, _ = oracle.gdn_forward(w.q, w.k, w.v, w.g, w.beta, w.cu_seqlens, w.h0)
    terms = np.abs((dout.double().numpy() * out).sum(-1)) + np.abs((ref["dv"] * w.v.double().numpy()).sum(-1))
    cu = w.cu_seqlens.tolist()
    return [float(np.linalg.norm(terms[cu[n]:cu[n + 1]])) for n in range(w.n_seqs) if cu[n + 1] > cu[n]]


def check_grads(w, r, ref, label, dout):
    cu = w.cu_seqlens.tolist()
    worst = {}
    for key, tol in GRAD_TOL.items():
        if key == "dg":
            x, y = r[key].cpu().double().numpy(), ref[key]
            nz = [n for n in range(w.n_seqs) if cu[n + 1] > cu[n]]
            errs = [float(np.linalg.norm(x[cu[n]:cu[n + 1]] - y[cu[n]:cu[n + 1]]) /
                          max(np.linalg.norm(y[cu[n]:cu[n + 1]]), s, 1e-300))
                    for n, s in zip(nz, gate_term_scale(w, ref, dout))]
        else:
            errs = seq_errors(r[key].cpu().numpy(), ref[key], cu)
        worst[key] = max(errs) if errs else 0.0
    worst["dh0"] = max(state_errors(r["dh0"].cpu().numpy(), ref["dh0"])) if w.n_seqs else 0.0
    say("%s: %s" % (label, " ".join("%s %.1e" % kv for kv in worst.items())))
    for key, tol in GRAD_TOL.items():
        assert worst[key] <= tol, (label, key, worst[key])
    assert worst["dh0"] <= DH0_TOL, (label, "dh0", worst["dh0"])


@pytest.mark.parametrize("hk,hv,dk,dv,io", [
    (2, 4, 128, 128, torch.bfloat16),
    (2, 4, 64, 64, torch.float32),
    (1, 4, 32, 128, torch.bfloat16),   # four value heads per key head
    (2, 2, 128, 32, torch.float32),
])
@pytest.mark.parametrize("with_h0,with_dhT", [(True, True), (False, False)])
def test_parity_small(gpu, hk, hv, dk, dv, io, with_h0, with_dhT):
    from oracle import oracle
    w = synth.make_workload(300 + dk + dv, [37, 1, 100, 0, 16], hk=hk, hv=hv, dk=dk, dv=dv, io_dtype=io,
                            h0_std=0.1 if with_h0 else 0.0)
    dout, dhT = grad_inputs(w, 11, dhT=with_dhT)
    r = run_bwd(gpu, w, dout, dhT)
    ref = oracle.gdn_backward(w.q, w.k, w.v, w.g, w.beta, w.cu_seqlens, dout, h0=w.h0, dhT=dhT)
    check_grads(w, r, ref, "bwd hk=%d hv=%d dk=%d dv=%d %s h0=%s dhT=%s" % (hk, hv, dk, dv, io, with_h0, with_dhT),
                dout)


def test_parity_benchmark_batch(gpu):
    """The benchmark batch (8 sequences, 17,459 tokens, 16/32 heads, dk = dv = 128),
    every gradient of every head against the oracle."""
    from oracle import oracle
    w = synth.varlen_prefill(1001)
    dout, dhT = grad_inputs(w, 12)
    r = run_bwd(gpu, w, dout, dhT)
    ref = oracle.gdn_backward(w.q, w.k, w.v, w.g, w.beta, w.cu_seqlens, dout, h0=w.h0, dhT=dhT)
    check_grads(w, r, ref, "bwd benchmark batch", dout)


def test_deterministic_and_batch_invariant(gpu):
    w = synth.make_workload(321, [70, 5, 33, 0, 130], hk=2, hv=4, dk=128, dv=128, h0_std=0.1)
    dout, dhT = grad_inputs(w, 13)
    r1 = run_bwd(gpu, w, dout, dhT)
    r2 = run_bwd(gpu, w, dout, dhT)
    for key in r1:
        assert torch.equal(r1[key], r2[key]), key
    cu = w.cu_seqlens.tolist()
    for n in (0, 2, 4):
        s = synth.select(w, [n])
        a, b = cu[n], cu[n + 1]
        rs = run_bwd(gpu, s, dout[a:b].contiguous(), dhT[n:n + 1].contiguous())
        for key in ("dq", "dk", "dv", "dg", "dbeta"):
            assert torch.equal(rs[key], r1[key][a:b]), (n, key)
        assert torch.equal(rs["dh0"][0], r1["dh0"][n]), n
    say("backward: repeat and alone-vs-batch bitwise equal")


def test_empty_and_single_token_sequences(gpu):
    from oracle import oracle
    w = synth.make_workload(331, [0, 1, 0, 2, 1], hk=1, hv=2, dk=64, dv=64, h0_std=0.1)
    dout, dhT = grad_inputs(w, 14)
    r = run_bwd(gpu, w, dout, dhT)
    ref = oracle.gdn_backward(w.q, w.k, w.v, w.g, w.beta, w.cu_seqlens, dout, h0=w.h0, dhT=dhT)
    check_grads(w, r, ref, "bwd short sequences", dout)
    # an empty sequence hands dhT straight back as dh0
    assert torch.equal(r["dh0"][0].cpu(), dhT[0]) and torch.equal(r["dh0"][2].cpu(), dhT[2])


def test_long_sequence(gpu):
    """One 8192-token sequence (the chunked-prefill size): the gate gradient's
    running sum is longest here."""
    from oracle import oracle
    w = synth.make_workload(341, [8192], hk=1, hv=2, dk=128, dv=128, h0_std=0.1)
    dout, dhT = grad_inputs(w, 15)
    r = run_bwd(gpu, w, dout, dhT)
    ref = oracle.gdn_backward(w.q, w.k, w.v, w.g, w.beta, w.cu_seqlens, dout, h0=w.h0, dhT=dhT)
    check_grads(w, r, ref, "bwd 8192 tokens", dout)


def test_workspace_contents_do_not_matter(gpu):
    """A workspace filled with NaN gives the same bits as a fresh one: every
    workspace entry is written before it is read.  dh0 = None skips that output."""
    from invariant_linear_attention_amd import gdn
    w = synth.make_workload(351, [40, 0, 17, 64], hk=2, hv=4, dk=128, dv=64, h0_std=0.1)
    dout, dhT = grad_inputs(w, 16)
    d = to_dev(w)
    dims = gdn.make_dims(d["q"], d["v"], w.n_seqs, int(w.q.shape[0]))
    nbytes = gdn.gdn_bwd_workspace_size(dims)
    ws0 = torch.zeros(nbytes, dtype=torch.uint8, device=DEV)
    ws1 = torch.full((nbytes // 4,), float("nan"), dtype=torch.float32, device=DEV).view(torch.uint8)
    args = (d["q"], d["k"], d["v"], d["g"], d["beta"], d["h0"], d["cu_seqlens"], dout.to(DEV), dhT.to(DEV))
    r0 = gdn.gdn_bwd_varlen(*args, workspace=ws0)
    r1 = gdn.gdn_bwd_varlen(*args, workspace=ws1, want_dh0=False)
    torch.cuda.synchronize()
    assert r1["dh0"] is None
    for key in ("dq", "dk", "dv", "dg", "dbeta"):
        assert torch.equal(r0[key], r1[key]), key
    assert all(bool(torch.isfinite(r0[key]).all()) for key in r0)


def test_training_forward_and_saved_p(gpu):
    """gdn_fwd_varlen_train: out and hT bit-identical to gdn_fwd_varlen; saved_p
    equals p_t = S_{t-1} k_t from the oracle (its state after the first t-1 tokens,
    times k_t); the backward fed saved_p (and hT) meets the same gates."""
    from invariant_linear_attention_amd import gdn
    from oracle import oracle
    w = synth.make_workload(361, [23, 0, 9], hk=2, hv=4, dk=64, dv=64, io_dtype=torch.float32, h0_std=0.1)
    d = to_dev(w)
    out0, hT0 = gdn.gdn_fwd_varlen(d["q"], d["k"], d["v"], d["g"], d["beta"], d["h0"], d["cu_seqlens"])
    out1, hT1, sp = gdn.gdn_fwd_varlen_train(d["q"], d["k"], d["v"], d["g"], d["beta"], d["h0"], d["cu_seqlens"])
    torch.cuda.synchronize()
    assert torch.equal(out0, out1) and torch.equal(hT0, hT1)
    cu = w.cu_seqlens.tolist()
    sp_c = sp.cpu().double().numpy()
    kk = w.k.double().numpy()
    worst = 0.0
    for n in (0, 2):
        for t in range(cu[n + 1] - cu[n]):
            pre = synth.token_slice(synth.select(w, [n]), 0, t, h0=w.h0[n:n + 1])
            if t == 0:
                S = w.h0[n].double().numpy()
            else:
                _, S = oracle.gdn_forward(pre.q, pre.k, pre.v, pre.g, pre.beta, pre.cu_seqlens, pre.h0)
                S = S[0]
            for h in range(4):
                ref = S[h] @ kk[cu[n] + t, h // 2]
                got = sp_c[cu[n] + t, h]
                worst = max(worst, float(np.linalg.norm(got - ref) / np.linalg.norm(ref)))
    say("saved p_t vs oracle: max rel err %.2e" % worst)
    assert worst <= 1e-4
    dout, dhT = grad_inputs(w, 17)
    ref = oracle.gdn_backward(w.q, w.k, w.v, w.g, w.beta, w.cu_seqlens, dout, h0=w.h0, dhT=dhT)
    r = gdn.gdn_bwd_varlen(d["q"], d["k"], d["v"], d["g"], d["beta"], d["h0"], d["cu_seqlens"], dout.to(DEV),
                           dhT.to(DEV), saved_p=sp, hT=hT1)
    torch.cuda.synchronize()
    check_grads(w, r, ref, "bwd with saved p", dout)
