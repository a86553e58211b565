"""The fused preprocessing as a pass of its own (gdn_preprocess) and its gradients
(gdn_preprocess_backward), on the GPU.

Parity: against the fp64 oracle (oracle.preprocess, oracle.preprocess_backward;
pinned by exactly representable finite differences, closed forms and the whole
fused layer).  The forward pass uses the fused kernels' fp32 operations, so the
recurrence on its outputs gives the fused call's state bit for bit, and its
outputs before their rounding to bf16.  The whole fused layer's gradients (the
pass, the chunked backward on its outputs, the pass's backward) are checked
against the oracle's chain in fp64 with the backward's gates.
"""
import numpy as np
import pytest
import torch

from gpu_helpers import say, to_dev
from invariant_linear_attention_amd import synth

pytestmark = pytest.mark.gpu
DEV = "cuda"


def raw(seed, lengths, hk=2, hv=4, dk=128, dv=128, io=torch.bfloat16, h0=0.1):
    return synth.make_raw_workload(seed, lengths, hk=hk, hv=hv, dk=dk, dv=dv, io_dtype=io, h0_std=h0)


def make_pre(gdn, w, norm, gate, dtb=True, eps=1e-6):
    A = w.meta["A_log"].to(DEV) if gate else None
    D = w.meta["dt_bias"].to(DEV) if (gate and dtb) else None
    return gdn.make_preproc(norm_qk=norm, eps=eps, A_log=A, dt_bias=D), (A, D)


def rel(x, r):
    x = np.asarray(x, dtype=np.float64)
    r = np.asarray(r, dtype=np.float64)
    return float(np.linalg.norm(x - r) / max(np.linalg.norm(r), 1e-300))


def row_rel(x, r):
    """Worst relative error over the last axis' rows."""
    x = np.asarray(x, dtype=np.float64).reshape(-1, np.shape(x)[-1])
    r = np.asarray(r, dtype=np.float64).reshape(-1, np.shape(r)[-1])
    den = np.maximum(np.linalg.norm(r, axis=1), 1e-300)
    return float((np.linalg.norm(x - r, axis=1) / den).max()) if len(r) else 0.0


@pytest.mark.parametrize("norm,gate", [(True, True), (True, False), (False, True), (False, False)])
@pytest.mark.parametrize("dk,io", [(128, torch.bfloat16), (64, torch.float32), (32, torch.bfloat16),
                                   (16, torch.float32)])
def test_preprocess_matches_oracle(gpu, norm, gate, dk, io):
    from oracle import oracle
    w = raw(601 + dk, [37, 0, 100, 16], dk=dk, dv=32, io=io)
    pre, keep = make_pre(gpu, w, norm, gate)
    d = to_dev(w)
    out = gpu.gdn_preprocess(d["q"], d["k"], d["g"], d["beta"], pre=pre)
    torch.cuda.synchronize()
    qn, kn, g, b = oracle.preprocess(w.q, w.k, w.g, w.beta, A_log=w.meta["A_log"] if gate else None,
                                     dt_bias=w.meta["dt_bias"] if gate else None, norm_qk=norm)
    errs = {"qn": row_rel(out["qn"].cpu(), qn), "kn": row_rel(out["kn"].cpu(), kn),
            "g": rel(out["g"].cpu(), g), "beta": rel(out["beta"].cpu(), b)}
    say("preprocess norm=%s gate=%s dk=%d %s: %s" % (norm, gate, dk, io, errs))
    for key, e in errs.items():
        assert e <= 2e-6, (key, e)
    if not norm:  # no norm: the rows are the inputs, widened exactly
        assert torch.equal(out["qn"], d["q"].float()) and torch.equal(out["kn"], d["k"].float())
    if not gate:
        assert torch.equal(out["g"], d["g"]) and torch.equal(out["beta"], d["beta"])


@pytest.mark.parametrize("dk", [128, 64])
def test_preprocess_reproduces_fused_forward(gpu, dk):
    """gdn_fwd_varlen on gdn_preprocess's outputs (fp32 io, v widened) gives the fused
    bf16 call's state bit for bit, and its outputs before rounding."""
    w = raw(611 + dk, [70, 1, 130, 16, 0], dk=dk, dv=dk)
    pre, keep = make_pre(gpu, w, True, True)
    d = to_dev(w)
    o_f, h_f = gpu.gdn_fwd_varlen(d["q"], d["k"], d["v"], d["g"], d["beta"], d["h0"], d["cu_seqlens"], pre=pre)
    p = gpu.gdn_preprocess(d["q"], d["k"], d["g"], d["beta"], pre=pre)
    o_p, h_p = gpu.gdn_fwd_varlen(p["qn"], p["kn"], d["v"].float().contiguous(), p["g"], p["beta"], d["h0"],
                                  d["cu_seqlens"])
    torch.cuda.synchronize()
    assert torch.equal(h_f, h_p)
    assert torch.equal(o_f, o_p.to(torch.bfloat16))
    say("preprocess dk=%d: plain fp32 forward on its outputs = fused bf16 forward, bitwise" % dk)


@pytest.mark.parametrize("norm,gate,dtb", [(True, True, True), (True, True, False), (True, False, True),
                                           (False, True, True)])
@pytest.mark.parametrize("dk,io", [(128, torch.bfloat16), (64, torch.float32), (16, torch.bfloat16)])
def test_preprocess_backward_matches_oracle(gpu, norm, gate, dtb, dk, io):
    from oracle import oracle
    w = raw(621 + dk, [37, 0, 100, 16], dk=dk, dv=32, io=io)
    pre, keep = make_pre(gpu, w, norm, gate, dtb=dtb)
    gen = torch.Generator().manual_seed(22)
    T, hk, hv = w.q.shape[0], w.q.shape[1], w.g.shape[1]
    dqn, dkn = torch.randn((T, hk, dk), generator=gen), torch.randn((T, hk, dk), generator=gen)
    dg, db = torch.randn((T, hv), generator=gen), torch.randn((T, hv), generator=gen)
    d = to_dev(w)
    r = gpu.gdn_preprocess_backward(d["q"], d["k"], d["g"], d["beta"], dqn.to(DEV), dkn.to(DEV), dg.to(DEV),
                                    db.to(DEV), pre=pre)
    torch.cuda.synchronize()
    ref = oracle.preprocess_backward(w.q, w.k, w.g, w.beta, dqn, dkn, dg, db,
                                     A_log=w.meta["A_log"] if gate else None,
                                     dt_bias=w.meta["dt_bias"] if (gate and dtb) else None, norm_qk=norm)
    errs = {"dq": row_rel(r["dq"].cpu(), ref["dq"]), "dk": row_rel(r["dk"].cpu(), ref["dk"]),
            "da": rel(r["da"].cpu(), ref["da"]), "db": rel(r["db"].cpu(), ref["db"])}
    if gate:
        errs["dA_log"] = rel(r["dA_log"].cpu(), ref["dA_log"])
        if dtb:
            errs["ddt_bias"] = rel(r["ddt_bias"].cpu(), ref["ddt_bias"])
        else:
            assert r["ddt_bias"] is None
    say("preprocess backward norm=%s gate=%s dtb=%s dk=%d %s: %s" % (norm, gate, dtb, dk, io, errs))
    for key, e in errs.items():
        assert e <= 1e-5, (key, e)


def test_parameter_gradients_many_heads(gpu):
    """More value heads than a wave has lanes (the block sums take two head groups), a
    token count that ends mid-block, and every parameter gradient against the oracle;
    a repeat gives the same bits."""
    from oracle import oracle
    w = raw(651, [70, 1, 129, 33], hk=4, hv=96, dk=32, dv=16)
    pre, keep = make_pre(gpu, w, True, True)
    gen = torch.Generator().manual_seed(24)
    T, hk, dk, hv = w.q.shape[0], 4, 32, 96
    dqn, dkn = torch.randn((T, hk, dk), generator=gen), torch.randn((T, hk, dk), generator=gen)
    dg, db = torch.randn((T, hv), generator=gen), torch.randn((T, hv), generator=gen)
    d = to_dev(w)
    args = (d["q"], d["k"], d["g"], d["beta"], dqn.to(DEV), dkn.to(DEV), dg.to(DEV), db.to(DEV))
    r1 = gpu.gdn_preprocess_backward(*args, pre=pre)
    r2 = gpu.gdn_preprocess_backward(*args, pre=pre)
    torch.cuda.synchronize()
    for key in r1:
        if r1[key] is not None:
            assert torch.equal(r1[key], r2[key]), key
    ref = oracle.preprocess_backward(w.q, w.k, w.g, w.beta, dqn, dkn, dg, db, A_log=w.meta["A_log"],
                                     dt_bias=w.meta["dt_bias"], norm_qk=True)
    errs = {key: rel(r1[key].cpu(), ref[key]) for key in ("da", "db", "dA_log", "ddt_bias")}
    say("preprocess backward, 96 value heads: %s" % errs)
    for key, e in errs.items():
        assert e <= 1e-5, (key, e)


def test_fused_layer_gradients(gpu):
    """The whole fused layer: preprocessing, the chunked backward on its outputs (fp32
    io, v and dO widened) and the preprocessing's backward, against the oracle's
    fp64 chain, with the backward's gates."""
    from oracle import oracle
    w = raw(631, [45, 0, 130, 16, 3], hk=2, hv=4, dk=128, dv=128)
    pre, keep = make_pre(gpu, w, True, True)
    gen = torch.Generator().manual_seed(23)
    T, hv, dv = w.v.shape
    dout = torch.randn((T, hv, dv), generator=gen).to(torch.bfloat16)
    dhT = torch.randn((w.n_seqs, hv, dv, w.q.shape[2]), generator=gen)
    d = to_dev(w)
    p = gpu.gdn_preprocess(d["q"], d["k"], d["g"], d["beta"], pre=pre)
    gb = gpu.gdn_bwd_chunked(p["qn"], p["kn"], d["v"].float().contiguous(), p["g"], p["beta"], d["h0"],
                             d["cu_seqlens"], dout.to(DEV).float().contiguous(), dhT.to(DEV))
    gp = gpu.gdn_preprocess_backward(d["q"], d["k"], d["g"], d["beta"], gb["dq"], gb["dk"], gb["dg"], gb["dbeta"],
                                     pre=pre)
    torch.cuda.synchronize()
    A, D = w.meta["A_log"], w.meta["dt_bias"]
    qn, kn, g, b = oracle.preprocess(w.q, w.k, w.g, w.beta, A_log=A, dt_bias=D, norm_qk=True)
    rb = oracle.gdn_backward(qn, kn, w.v, g, b, w.cu_seqlens, dout, h0=w.h0, dhT=dhT)
    rp = oracle.preprocess_backward(w.q, w.k, w.g, w.beta, rb["dq"], rb["dk"], rb["dg"], rb["dbeta"], A_log=A,
                                    dt_bias=D, norm_qk=True)
    errs = {"dq": rel(gp["dq"].cpu(), rp["dq"]), "dk": rel(gp["dk"].cpu(), rp["dk"]),
            "dv": rel(gb["dv"].cpu(), rb["dv"]), "da": rel(gp["da"].cpu(), rp["da"]),
            "db": rel(gp["db"].cpu(), rp["db"]), "dA_log": rel(gp["dA_log"].cpu(), rp["dA_log"]),
            "ddt_bias": rel(gp["ddt_bias"].cpu(), rp["ddt_bias"]), "dh0": rel(gb["dh0"].cpu(), rb["dh0"])}
    say("fused layer gradients: %s" % errs)
    for key, e in errs.items():
        assert e <= 1e-4, (key, e)


def test_empty_and_refusals(gpu):
    w = raw(641, [5, 3], dk=64, dv=32)
    pre, keep = make_pre(gpu, w, True, True)
    d = to_dev(w)
    e = torch.empty((0, 2, 64), dtype=torch.bfloat16, device=DEV)
    z = torch.empty((0, 4), device=DEV)
    out = gpu.gdn_preprocess(e, e, z, z, pre=pre)
    assert out["qn"].shape == (0, 2, 64)
    # no tokens: the parameter gradients are sums over nothing
    r = gpu.gdn_preprocess_backward(e, e, z, z, torch.empty((0, 2, 64), device=DEV),
                                    torch.empty((0, 2, 64), device=DEV), z, z, pre=pre)
    torch.cuda.synchronize()
    assert float(r["dA_log"].abs().sum()) == 0.0 and float(r["ddt_bias"].abs().sum()) == 0.0
    # an output overlapping an input
    with pytest.raises(gpu.GdnError):
        gpu.gdn_preprocess(d["q"], d["k"], d["g"], d["beta"], pre=pre,
                           out={"qn": torch.empty((8, 2, 64), device=DEV), "kn": torch.empty((8, 2, 64), device=DEV),
                                "g": d["g"], "beta": torch.empty((8, 4), device=DEV)})
