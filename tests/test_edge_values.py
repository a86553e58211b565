"""The method's special cases, through the HIP kernels (prefill and decode), against
the oracle and against what the rule itself fixes.

The recurrence S_t = exp(g_t) S_{t-1} (I - beta_t k_t k_t^T) + beta_t v_t k_t^T,
o_t = S_t q_t (gated delta rule) reduces, for particular gates, to results that
need no oracle to state:
  * beta = 0 and g = 0: the step is the identity, so the state is unchanged;
  * beta = 1 and a unit key: (I - k k^T) k = 0, so S_t k_t = v_t (the written
    association is recalled exactly);
  * exp(g) -> 0 (g = -1e4): the old state is forgotten, S_t = beta_t v_t k_t^T and
    o_t = beta_t (k_t . q_t) v_t;
  * beta outside (0, 1) is not clamped (the rule is a gradient step of size beta);
  * rows of the state never interact, so a NaN written into one value row stays
    in that row (and in that sequence and head).
"""
import numpy as np
import pytest
import torch

from gpu_helpers import bit_equal, check_parity, run_prefill, say, to_dev
from invariant_linear_attention_amd import synth

pytestmark = pytest.mark.gpu
DEV = "cuda"


def oracle_of(w):
    from oracle import oracle
    return oracle.gdn_forward(w.q, w.k, w.v, w.g, w.beta, w.cu_seqlens, w.h0)


def with_gates(w, g=None, beta=None):
    return synth.Workload(w.q, w.k, w.v, w.g if g is None else g.contiguous(),
                          w.beta if beta is None else beta.contiguous(), w.cu_seqlens, w.h0, meta=w.meta)


def decode_one(gpu, w, pool, state_idx=None):
    """One decode step of a workload whose sequences are one token each."""
    d = to_dev(w)
    o = gpu.gdn_decode_step(d["q"], d["k"], d["v"], d["g"], d["beta"], pool, state_idx=state_idx)
    torch.cuda.synchronize()
    return o


@pytest.mark.parametrize("io", [torch.bfloat16, torch.float32])
def test_beta0_g0_is_identity(gpu, io):
    """beta = 0, g = 0 everywhere: hT has h0's bits, o_t = h0 q_t (oracle gates),
    in prefill and in decode; and such tokens in the middle of a sequence leave
    the state where the tokens before them put it."""
    w = synth.make_workload(201, [37, 1, 200, 16], hk=2, hv=4, dk=128, dv=128, io_dtype=io, h0_std=0.1)
    z = with_gates(w, g=torch.zeros_like(w.g), beta=torch.zeros_like(w.beta))
    out, hT = run_prefill(gpu, z)
    assert bit_equal(hT, z.h0.to(DEV)), "prefill: beta = g = 0 changed the state"
    ro, rh = oracle_of(z)
    check_parity(z, out, hT, ro, rh, "beta=g=0 prefill %s" % io)
    # decode: every row of a pool of states, one identity token each
    dz = synth.make_workload(202, [1] * 64, hk=2, hv=4, dk=128, dv=128, io_dtype=io, h0_std=0.1)
    dz = with_gates(dz, g=torch.zeros_like(dz.g), beta=torch.zeros_like(dz.beta))
    pool = dz.h0.to(DEV).clone()
    o = decode_one(gpu, dz, pool)
    assert bit_equal(pool, dz.h0.to(DEV)), "decode: beta = g = 0 changed the state"
    rdo, rdh = oracle_of(dz)
    check_parity(dz, o, pool, rdo, rdh, "beta=g=0 decode %s" % io)
    # identity tokens [80, 130) inside a 200-token sequence
    s = synth.select(w, [2])
    g = s.g.clone()
    b = s.beta.clone()
    g[80:130] = 0.0
    b[80:130] = 0.0
    s = with_gates(s, g=g, beta=b)
    _, h80 = run_prefill(gpu, synth.token_slice(s, 0, 80, h0=s.h0))
    _, h130 = run_prefill(gpu, synth.token_slice(s, 0, 130, h0=s.h0))
    assert bit_equal(h80, h130), "identity tokens inside a sequence moved the state"


def test_beta1_unit_key_recall(gpu):
    """beta = 1 with fp32 unit keys: after each token S_t k_t = v_t to fp32
    rounding, in prefill (final state, every sequence and head) and in decode."""
    w = synth.make_workload(211, [1, 9, 64, 301], hk=2, hv=4, dk=128, dv=64, io_dtype=torch.float32, h0_std=0.1)
    w = with_gates(w, beta=torch.ones_like(w.beta))
    out, hT = run_prefill(gpu, w)
    ro, rh = oracle_of(w)
    check_parity(w, out, hT, ro, rh, "beta=1 unit keys")
    cu = w.cu_seqlens.tolist()
    grp = 2
    worst = 0.0
    for n in range(w.n_seqs):
        t = cu[n + 1] - 1
        for h in range(4):
            k = w.k[t, h // grp].double()
            v = w.v[t, h].double()
            recall = hT[n, h].double().cpu() @ k
            worst = max(worst, float((recall - v).norm() / v.norm()))
    say("prefill recall |S_T k_T - v_T| / |v_T| <= %.2e" % worst)
    assert worst <= 1e-5
    # decode: one more token per sequence with beta = 1
    dw = synth.make_workload(212, [1] * 4, hk=2, hv=4, dk=128, dv=64, io_dtype=torch.float32)
    dw = with_gates(dw, beta=torch.ones_like(dw.beta))
    pool = hT.clone()
    decode_one(gpu, dw, pool)
    worst = 0.0
    for n in range(4):
        for h in range(4):
            recall = pool[n, h].double().cpu() @ dw.k[n, h // grp].double()
            worst = max(worst, float((recall - dw.v[n, h].double()).norm() / dw.v[n, h].double().norm()))
    say("decode recall <= %.2e" % worst)
    assert worst <= 1e-5


@pytest.mark.parametrize("io", [torch.bfloat16, torch.float32])
def test_full_forget(gpu, io):
    """g = -1e4 (exp(g) = 0 in fp32): S_t = beta_t v_t k_t^T whatever came before,
    o_t = beta_t (k_t . q_t) v_t, in prefill and decode; against the oracle too."""
    w = synth.make_workload(221, [1, 17, 100], hk=2, hv=4, dk=128, dv=128, io_dtype=io, h0_std=0.1)
    w = with_gates(w, g=torch.full_like(w.g, -1e4))
    out, hT = run_prefill(gpu, w)
    ro, rh = oracle_of(w)
    check_parity(w, out, hT, ro, rh, "g=-1e4 prefill %s" % io)
    assert bool(torch.isfinite(hT).all()) and bool(torch.isfinite(out.float()).all())
    cu = w.cu_seqlens.tolist()
    for n in range(w.n_seqs):
        t = cu[n + 1] - 1
        for h in range(4):
            k = w.k[t, h // 2].double()
            v = w.v[t, h].double()
            b = float(w.beta[t, h])
            closed = b * torch.outer(v, k)
            got = hT[n, h].double().cpu()
            assert float((got - closed).norm() / closed.norm()) <= 1e-6, (n, h)
            o_closed = b * float(k @ w.q[t, h // 2].double()) * v
            assert float((out[t, h].double().cpu() - o_closed).norm() / o_closed.norm()) <= 8e-3, (n, h)
    # decode from arbitrary states
    dw = synth.make_workload(222, [1] * 16, hk=2, hv=4, dk=128, dv=128, io_dtype=io, h0_std=0.1)
    dw = with_gates(dw, g=torch.full_like(dw.g, -1e4))
    pool = dw.h0.to(DEV).clone()
    o = decode_one(gpu, dw, pool)
    rdo, rdh = oracle_of(dw)
    check_parity(dw, o, pool, rdo, rdh, "g=-1e4 decode %s" % io)


@pytest.mark.parametrize("beta_value", [1.5, -0.2])
def test_beta_outside_unit_interval(gpu, beta_value):
    """beta is not clamped: beta = 1.5 and -0.2 against the oracle, and decode
    continuing a prefill gives the full prefill's bits."""
    w = synth.make_workload(231, [5, 130, 64], hk=2, hv=4, dk=128, dv=128, h0_std=0.1)
    w = with_gates(w, beta=torch.full_like(w.beta, beta_value))
    out, hT = run_prefill(gpu, w)
    ro, rh = oracle_of(w)
    check_parity(w, out, hT, ro, rh, "beta=%g" % beta_value)
    s = synth.select(w, [1])
    _, h129 = run_prefill(gpu, synth.token_slice(s, 0, 129, h0=s.h0))
    pool = h129.clone()
    o = decode_one(gpu, synth.token_slice(s, 129, 130), pool)
    cu = w.cu_seqlens.tolist()
    assert bit_equal(o, out[cu[2] - 1:cu[2]]) and bit_equal(pool[0], hT[1])


def test_nan_in_one_value_row_stays_there(gpu):
    """A NaN in v[t, h, j] of one sequence makes o[t', h, j] (t' >= t) and row j of
    that sequence's state NaN; every other element keeps the clean run's bits."""
    w = synth.make_workload(241, [40, 90, 33], hk=2, hv=4, dk=128, dv=128, h0_std=0.1)
    clean_out, clean_hT = run_prefill(gpu, w)
    n, t_rel, h, j = 1, 25, 3, 77
    cu = w.cu_seqlens.tolist()
    t = cu[n] + t_rel
    v = w.v.clone()
    v[t, h, j] = float("nan")
    bad = synth.Workload(w.q, w.k, v, w.g, w.beta, w.cu_seqlens, w.h0, meta=w.meta)
    out, hT = run_prefill(gpu, bad)
    mask_o = torch.zeros(out.shape, dtype=torch.bool)
    mask_o[t:cu[n + 1], h, j] = True
    mask_s = torch.zeros(hT.shape, dtype=torch.bool)
    mask_s[n, h, j, :] = True
    oc, oo = out.cpu(), clean_out.cpu()
    assert bool(torch.isnan(oc[mask_o].float()).all()), "the NaN did not reach its row's later outputs"
    assert bit_equal(oc[~mask_o], oo[~mask_o]), "the NaN leaked out of its row"
    hc, hh = hT.cpu(), clean_hT.cpu()
    assert bool(torch.isnan(hc[mask_s]).all())
    assert bit_equal(hc[~mask_s], hh[~mask_s])
    # decode: a NaN in one value row of one batch row
    dw = synth.make_workload(242, [1] * 32, hk=2, hv=4, dk=128, dv=128, h0_std=0.1)
    pool_c = dw.h0.to(DEV).clone()
    o_c = decode_one(gpu, dw, pool_c)
    v = dw.v.clone()
    b, h, j = 9, 2, 5
    v[b, h, j] = float("nan")
    dbad = synth.Workload(dw.q, dw.k, v, dw.g, dw.beta, dw.cu_seqlens, dw.h0, meta=dw.meta)
    pool = dw.h0.to(DEV).clone()
    o = decode_one(gpu, dbad, pool)
    m_o = torch.zeros(o.shape, dtype=torch.bool)
    m_o[b, h, j] = True
    m_s = torch.zeros(pool.shape, dtype=torch.bool)
    m_s[b, h, j, :] = True
    assert bool(torch.isnan(o.cpu()[m_o].float()).all()) and bool(torch.isnan(pool.cpu()[m_s]).all())
    assert bit_equal(o.cpu()[~m_o], o_c.cpu()[~m_o]) and bit_equal(pool.cpu()[~m_s], pool_c.cpu()[~m_s])


def test_nan_gate_stays_in_its_head(gpu):
    """A NaN gate g[t, h] poisons head h of its own sequence from token t on (every
    row decays by it); other heads, sequences and earlier tokens keep their bits."""
    w = synth.make_workload(251, [40, 90, 33], hk=2, hv=4, dk=128, dv=128, h0_std=0.1)
    clean_out, clean_hT = run_prefill(gpu, w)
    n, t_rel, h = 1, 60, 1
    cu = w.cu_seqlens.tolist()
    t = cu[n] + t_rel
    g = w.g.clone()
    g[t, h] = float("nan")
    out, hT = run_prefill(gpu, with_gates(w, g=g))
    mask_o = torch.zeros(out.shape, dtype=torch.bool)
    mask_o[t:cu[n + 1], h, :] = True
    mask_s = torch.zeros(hT.shape, dtype=torch.bool)
    mask_s[n, h] = True
    assert bool(torch.isnan(out.cpu()[mask_o].float()).all()) and bool(torch.isnan(hT.cpu()[mask_s]).all())
    assert bit_equal(out.cpu()[~mask_o], clean_out.cpu()[~mask_o])
    assert bit_equal(hT.cpu()[~mask_s], clean_hT.cpu()[~mask_s])
