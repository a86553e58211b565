"""Pins for the fp64 oracle: checks against things other than the oracle itself.

Each ``pin_*`` function takes a ``forward`` callable with the signature of
``oracle.gdn_forward`` and raises AssertionError when the forward disagrees with

  * brute-force products of the per-token transition matrices (a closed form of
    the gated delta rule, evaluated with numpy matrix products);
  * a finite-difference gradient of the delta-rule regression loss (the
    Widrow-Hoff reading of the rule);
  * hand-derived scalar values (tests/golden/scalar_delta_rule.json);
  * invariants: identity when beta = g = 0, exact recall of a written value,
    exact chunk-split carry, closed forms for beta = 0 and for a vanishing decay,
    associative recall with orthonormal keys, linearity in (h0, v), and grouped
    heads equal to duplicated key heads.

The rule being pinned is the gated delta rule of Yang, Kautz and Hatamizadeh
("Gated Delta Networks", ICLR 2025): S_t = exp(g_t) S_{t-1} (I - beta_t k_t k_t^T)
+ beta_t v_t k_t^T, o_t = S_t q_t, with S a dv x dk matrix, walked token by token
per sequence as in the page "Defending Against the Training-Inference Numeric
Mismatch in RL (Especially Linear Attention)", section 3.2.

The tests run every pin on the real oracle (all must pass) and on deliberately
broken copies of it (each copy must fail at least one pin).
"""
from __future__ import annotations

import json
import math
import os

import numpy as np

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")
RTOL = 1e-11


# ------------------------------------------------------------------ helpers

def _rng(seed):
    return np.random.default_rng(seed)


def _unit(x):
    return x / np.linalg.norm(x, axis=-1, keepdims=True)


def random_case(seed, lengths, hk, hv, dk, dv, with_h0=True, g_scale=1.0):
    """fp32 inputs with the workload's distributions (numpy, for small pins)."""
    r = _rng(seed)
    T = int(sum(lengths))
    q = _unit(r.standard_normal((T, hk, dk))).astype(np.float32)
    k = _unit(r.standard_normal((T, hk, dk))).astype(np.float32)
    v = r.standard_normal((T, hv, dv)).astype(np.float32)
    g = (-np.log1p(np.exp(r.standard_normal((T, hv)))) * g_scale).astype(np.float32)
    beta = (1.0 / (1.0 + np.exp(-r.standard_normal((T, hv))))).astype(np.float32)
    cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)
    h0 = (0.5 * r.standard_normal((len(lengths), hv, dv, dk))).astype(np.float32) if with_h0 else None
    return dict(q=q, k=k, v=v, g=g, beta=beta, cu_seqlens=cu, h0=h0)


def _rel(a, b):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    den = max(np.linalg.norm(b), 1e-300)
    return float(np.linalg.norm(a - b) / den)


def _close(a, b, tol=RTOL, what=""):
    e = _rel(a, b)
    assert e <= tol, "%s: relative error %.3e > %.1e" % (what, e, tol)


def bruteforce(case):
    """Closed form via transition products.

    With A_t = exp(g_t) (I - beta_t k_t k_t^T) (dk x dk) the rule reads
    S_t = S_{t-1} A_t + beta_t v_t k_t^T, hence
    S_t = S_0 A_1 ... A_t + sum_{s<=t} beta_s v_s k_s^T A_{s+1} ... A_t.
    Every S_t is rebuilt from scratch from that sum (no recurrence is run).
    """
    q = case["q"].astype(np.float64)
    k = case["k"].astype(np.float64)
    v = case["v"].astype(np.float64)
    g = case["g"].astype(np.float64)
    beta = case["beta"].astype(np.float64)
    cu = case["cu_seqlens"]
    T, hk, dk = q.shape
    hv, dv = v.shape[1], v.shape[2]
    grp = hv // hk
    N = len(cu) - 1
    out = np.zeros((T, hv, dv))
    hT = np.zeros((N, hv, dv, dk))
    for n in range(N):
        t0, t1 = int(cu[n]), int(cu[n + 1])
        for h in range(hv):
            kh = h // grp
            S0 = np.zeros((dv, dk)) if case["h0"] is None else case["h0"][n, h].astype(np.float64)
            A = [math.exp(g[t, h]) * (np.eye(dk) - beta[t, h] * np.outer(k[t, kh], k[t, kh]))
                 for t in range(t0, t1)]
            W = [beta[t, h] * np.outer(v[t, h], k[t, kh]) for t in range(t0, t1)]

            def prod(a, b):
                m = np.eye(dk)
                for x in A[a:b]:
                    m = m @ x
                return m

            St = S0
            for t in range(t0, t1):
                m = t - t0 + 1
                St = S0 @ prod(0, m)
                for s in range(m):
                    St = St + W[s] @ prod(s + 1, m)
                out[t, h] = St @ q[t, kh]
            hT[n, h] = St
    return out, hT


# ---------------------------------------------------------------------- pins

def pin_bruteforce_plain(forward):
    """One sequence, no grouping, dk != dv (catches transposed state indexing)."""
    c = random_case(11, [7], hk=1, hv=1, dk=5, dv=3)
    out, hT = forward(**c)
    bo, bh = bruteforce(c)
    _close(out, bo, what="out vs transition products")
    _close(hT, bh, what="hT vs transition products")


def pin_bruteforce_grouped_varlen(forward):
    """Grouped heads (2 value heads per key head), several sequences incl. an empty one."""
    c = random_case(12, [3, 0, 6, 1], hk=2, hv=4, dk=4, dv=6)
    out, hT = forward(**c)
    bo, bh = bruteforce(c)
    _close(out, bo, what="out vs transition products (grouped)")
    _close(hT, bh, what="hT vs transition products (grouped)")
    # the empty sequence hands its initial state through unchanged
    assert np.array_equal(hT[1], c["h0"][1].astype(np.float64)), "empty sequence must return h0"


def pin_bruteforce_no_h0(forward):
    c = random_case(13, [5, 4], hk=1, hv=2, dk=3, dv=4, with_h0=False)
    out, hT = forward(**c)
    bo, bh = bruteforce(c)
    _close(out, bo, what="out vs transition products (zero h0)")
    _close(hT, bh, what="hT vs transition products (zero h0)")


def _loss_grad_fd(S, kv, vv, eps=1e-3):
    """Central finite-difference gradient of L(S) = 0.5 * ||S k - v||^2."""
    G = np.zeros_like(S)
    for j in range(S.shape[0]):
        for i in range(S.shape[1]):
            E = np.zeros_like(S)
            E[j, i] = eps
            lp = 0.5 * np.sum(((S + E) @ kv - vv) ** 2)
            lm = 0.5 * np.sum(((S - E) @ kv - vv) ** 2)
            G[j, i] = (lp - lm) / (2 * eps)
    return G


def pin_gradient_step(forward):
    """One token: the new state is one gradient step of size beta on the regression
    loss 0.5 ||S k - v||^2, taken at the decayed state exp(g) S_0 (the delta /
    Widrow-Hoff rule with a decay applied first).  Gradient by finite differences."""
    c = random_case(21, [1], hk=1, hv=1, dk=4, dv=3)
    out, hT = forward(**c)
    a = math.exp(float(c["g"][0, 0]))
    b = float(c["beta"][0, 0])
    S = a * c["h0"][0, 0].astype(np.float64)
    kv = c["k"][0, 0].astype(np.float64)
    vv = c["v"][0, 0].astype(np.float64)
    expect = S - b * _loss_grad_fd(S, kv, vv)
    _close(hT[0, 0], expect, tol=1e-9, what="gradient-step reading")
    _close(out[0, 0], expect @ c["q"][0, 0].astype(np.float64), tol=1e-9, what="read-out of the new state")


def pin_scalar_golden(forward):
    """dk = dv = 1 hand-derived values (tests/golden/scalar_delta_rule.json)."""
    with open(os.path.join(GOLDEN, "scalar_delta_rule.json")) as f:
        fx = json.load(f)
    for case in fx["cases"]:
        T = len(case["v"])
        c = dict(q=np.array(case["q"], np.float32).reshape(T, 1, 1),
                 k=np.array(case["k"], np.float32).reshape(T, 1, 1),
                 v=np.array(case["v"], np.float32).reshape(T, 1, 1),
                 g=np.array(case["g"], np.float32).reshape(T, 1),
                 beta=np.array(case["beta"], np.float32).reshape(T, 1),
                 cu_seqlens=np.array([0, T], np.int32),
                 h0=np.array(case["s0"], np.float32).reshape(1, 1, 1, 1))
        out, hT = forward(**c)
        np.testing.assert_allclose(out.reshape(-1), case["o"], rtol=case["rtol"], atol=0,
                                   err_msg="scalar golden %s: outputs" % case["name"])
        np.testing.assert_allclose(hT.reshape(-1), [case["s"][-1]], rtol=case["rtol"], atol=0,
                                   err_msg="scalar golden %s: final state" % case["name"])


def pin_identity_when_idle(forward):
    """beta = 0 and g = 0: the state never changes (exactly) and o_t = h0 q_t."""
    c = random_case(31, [6], hk=1, hv=2, dk=4, dv=5)
    c["beta"][:] = 0.0
    c["g"][:] = 0.0
    out, hT = forward(**c)
    assert np.array_equal(hT, c["h0"].astype(np.float64)), "state must be unchanged"
    for t in range(6):
        for h in range(2):
            _close(out[t, h], c["h0"][0, h].astype(np.float64) @ c["q"][t, 0].astype(np.float64),
                   what="idle read-out")


def pin_exact_recall(forward):
    """beta = 1 and a unit key: S_t k_t = v_t, since (I - k k^T) k = 0."""
    c = random_case(32, [5], hk=1, hv=1, dk=6, dv=4)
    k = _unit(_rng(33).standard_normal((5, 1, 6)))
    c["k"] = k.astype(np.float32)
    c["beta"][:] = 1.0
    kk = c["k"].astype(np.float64)
    for t in range(1, 6):
        cc = dict(c)
        cc["cu_seqlens"] = np.array([0, t], np.int32)
        for key in ("q", "k", "v", "g", "beta"):
            cc[key] = c[key][:t].copy()
        _, hT = forward(**cc)
        # the key is unit only up to fp32 rounding of its entries: renormalise
        kt = kk[t - 1, 0]
        nk = float(kt @ kt)
        # S_t k = a S_{t-1}(k - k (k.k)) + v (k.k) -> v when k.k = 1; allow for the fp32 key norm
        resid = hT[0, 0] @ kt - c["v"][t - 1, 0].astype(np.float64) * nk
        assert np.linalg.norm(resid) <= 1e-6 * (1 + np.linalg.norm(c["v"][t - 1, 0])), \
            "S_t k_t must equal v_t (residual %.3e)" % np.linalg.norm(resid)


def pin_chunk_carry(forward):
    """Splitting a sequence and carrying the fp64 state reproduces the full run exactly."""
    c = random_case(41, [9], hk=1, hv=2, dk=4, dv=3)
    out, hT = forward(**c)
    cuts = [0, 4, 5, 9]
    state = c["h0"].astype(np.float64)
    outs = []
    for a, b in zip(cuts[:-1], cuts[1:]):
        cc = dict(q=c["q"][a:b], k=c["k"][a:b], v=c["v"][a:b], g=c["g"][a:b], beta=c["beta"][a:b],
                  cu_seqlens=np.array([0, b - a], np.int32), h0=state)
        o, state = forward(**cc)
        outs.append(o)
    assert np.array_equal(np.concatenate(outs), out), "chunked outputs must be bit-identical"
    assert np.array_equal(state, hT), "chunked final state must be bit-identical"


def pin_no_write_closed_form(forward):
    """beta = 0: o_t = exp(g_1 + ... + g_t) S_0 q_t (pure decay)."""
    c = random_case(51, [6], hk=1, hv=2, dk=3, dv=4)
    c["beta"][:] = 0.0
    out, hT = forward(**c)
    g = c["g"].astype(np.float64)
    for h in range(2):
        S0 = c["h0"][0, h].astype(np.float64)
        for t in range(6):
            _close(out[t, h], math.exp(g[:t + 1, h].sum()) * (S0 @ c["q"][t, 0].astype(np.float64)),
                   what="pure decay read-out")
        _close(hT[0, h], math.exp(g[:, h].sum()) * S0, what="pure decay state")


def pin_full_forget(forward):
    """exp(g) underflows to 0: S_t = beta_t v_t k_t^T and o_t = beta_t (k_t.q_t) v_t."""
    c = random_case(52, [4], hk=1, hv=1, dk=5, dv=3)
    c["g"][:] = -1.0e4
    out, hT = forward(**c)
    for t in range(4):
        b = float(c["beta"][t, 0])
        kv = c["k"][t, 0].astype(np.float64)
        qv = c["q"][t, 0].astype(np.float64)
        vv = c["v"][t, 0].astype(np.float64)
        _close(out[t, 0], b * float(kv @ qv) * vv, what="full-forget read-out")
    _close(hT[0, 0], float(c["beta"][3, 0]) * np.outer(c["v"][3, 0].astype(np.float64),
                                                      c["k"][3, 0].astype(np.float64)),
           what="full-forget state")


def pin_associative_recall(forward):
    """g = 0, beta = 1, orthonormal keys, zero start: every stored value is recalled."""
    dk, dv, m = 6, 4, 5
    r = _rng(61)
    K, _ = np.linalg.qr(r.standard_normal((dk, dk)))
    keys = K[:, :m].T  # m orthonormal rows
    c = random_case(62, [m], hk=1, hv=1, dk=dk, dv=dv, with_h0=False)
    c["k"] = keys.reshape(m, 1, dk).astype(np.float32)
    c["g"][:] = 0.0
    c["beta"][:] = 1.0
    _, hT = forward(**c)
    kk = c["k"].astype(np.float64)[:, 0]
    # fp32 rounding of the keys breaks exact orthonormality slightly
    for j in range(m):
        _close(hT[0, 0] @ kk[j], c["v"][j, 0].astype(np.float64), tol=1e-6, what="recall of item %d" % j)


def pin_linearity(forward):
    """For fixed q, k, g, beta the map (h0, v) -> (out, hT) is linear."""
    c1 = random_case(71, [5, 3], hk=1, hv=2, dk=3, dv=3)
    c2 = random_case(72, [5, 3], hk=1, hv=2, dk=3, dv=3)
    for key in ("q", "k", "g", "beta"):
        c2[key] = c1[key]
    a, b = 0.75, -1.25
    mix = dict(c1)
    mix["v"] = (a * c1["v"].astype(np.float64) + b * c2["v"].astype(np.float64))
    mix["h0"] = (a * c1["h0"].astype(np.float64) + b * c2["h0"].astype(np.float64))
    # feed the mixture in fp64 through the fp32 interface: keep it exactly representable
    mix["v"] = mix["v"].astype(np.float32)
    mix["h0"] = mix["h0"].astype(np.float32)
    o1, s1 = forward(**c1)
    o2, s2 = forward(**c2)
    om, sm = forward(**mix)
    # v/h0 mixtures rounded to fp32: compare against the same rounding applied on the right
    _close(om, a * o1 + b * o2, tol=1e-6, what="linearity (out)")
    _close(sm, a * s1 + b * s2, tol=1e-6, what="linearity (hT)")


def pin_grouped_equals_duplicated(forward):
    """Value head h reads key head h // (hv/hk): same bits as duplicating key heads."""
    c = random_case(81, [4, 2], hk=2, hv=4, dk=3, dv=2)
    out, hT = forward(**c)
    d = dict(c)
    d["q"] = np.repeat(c["q"], 2, axis=1)
    d["k"] = np.repeat(c["k"], 2, axis=1)
    out2, hT2 = forward(**d)
    assert np.array_equal(out, out2) and np.array_equal(hT, hT2), "grouped heads must equal duplicated keys"


def pin_gate_and_beta_per_value_head(forward):
    """g and beta index the value head: value heads sharing a key head but with
    different gates must evolve differently, each matching its own brute force."""
    c = random_case(91, [5], hk=1, hv=2, dk=3, dv=3)
    c["g"][:, 1] = c["g"][:, 0] * 3.0
    c["beta"][:, 1] = 1.0 - c["beta"][:, 0]
    out, hT = forward(**c)
    bo, bh = bruteforce(c)
    _close(out, bo, what="per-head gate/beta (out)")
    _close(hT, bh, what="per-head gate/beta (hT)")


def pin_bf16_inputs_widened_exactly(forward):
    """bf16 inputs are read as their exact values (bits << 16)."""
    import torch
    c = random_case(95, [4], hk=1, hv=2, dk=4, dv=4)
    cb = dict(c)
    for key in ("q", "k", "v"):
        cb[key] = torch.from_numpy(c[key]).to(torch.bfloat16)
    out_b, hT_b = forward(**cb)
    cf = dict(c)
    for key in ("q", "k", "v"):
        cf[key] = cb[key].to(torch.float32).numpy()
    out_f, hT_f = forward(**cf)
    assert np.array_equal(out_b, out_f) and np.array_equal(hT_b, hT_f), "bf16 must widen exactly"


ALL_PINS = [
    pin_bruteforce_plain,
    pin_bruteforce_grouped_varlen,
    pin_bruteforce_no_h0,
    pin_gradient_step,
    pin_scalar_golden,
    pin_identity_when_idle,
    pin_exact_recall,
    pin_chunk_carry,
    pin_no_write_closed_form,
    pin_full_forget,
    pin_associative_recall,
    pin_linearity,
    pin_grouped_equals_duplicated,
    pin_gate_and_beta_per_value_head,
    pin_bf16_inputs_widened_exactly,
]


# ------------------------------------------------- fused-path preprocessing
#
# Pins for oracle.preprocess (q/k L2 normalisation and the gate / write strength
# from raw logits).  Each takes (preprocess, forward) callables with the
# signatures of oracle.preprocess and oracle.gdn_forward and checks values that
# mathematics fixes: norms, the constants softplus(0) = ln 2 and sigmoid(ln 3) =
# 3/4, the asymptotes of softplus, and the full-forget closed form of the rule.

def _raw_case(seed, T, hk, hv, dk, scale=3.0):
    r = _rng(seed)
    q = (scale * r.standard_normal((T, hk, dk))).astype(np.float32)
    k = (scale * r.standard_normal((T, hk, dk))).astype(np.float32)
    a = r.standard_normal((T, hv)).astype(np.float32)
    b = r.standard_normal((T, hv)).astype(np.float32)
    return q, k, a, b


def pin_pre_norm_closed_form(preprocess, forward):
    """|q'|^2 = |q|^2 / (|q|^2 + eps), q' parallel to q (eps large enough to see)."""
    q, k, a, b = _raw_case(101, 5, 2, 2, 8, scale=0.05)
    eps = 1e-2
    q2, k2, _, _ = preprocess(q, k, a, b, norm_qk=True, eps=eps)
    for x, x2 in ((q, q2), (k, k2)):
        x = x.astype(np.float64)
        ss = np.sum(x * x, axis=-1)
        _close(np.sum(x2 * x2, axis=-1), ss / (ss + eps), 1e-13, "normalised length")
        cos = np.sum(x * x2, axis=-1) / (np.sqrt(ss) * np.linalg.norm(x2, axis=-1))
        _close(cos, np.ones_like(cos), 1e-14, "direction")


def pin_pre_unit_rows(preprocess, forward):
    """With the default tiny eps, rows of moderate size come out of unit length."""
    q, k, a, b = _raw_case(102, 4, 3, 3, 16)
    q2, k2, _, _ = preprocess(q, k, a, b)
    for x2 in (q2, k2):
        _close(np.linalg.norm(x2, axis=-1), np.ones(x2.shape[:2]), 1e-7, "unit rows")


def pin_pre_norm_off_is_widening(preprocess, forward):
    q, k, a, b = _raw_case(103, 3, 1, 2, 4)
    q2, k2, g2, b2 = preprocess(q, k, a, b, norm_qk=False)
    assert np.array_equal(q2, q.astype(np.float64)) and np.array_equal(k2, k.astype(np.float64))
    assert np.array_equal(g2, a.astype(np.float64)) and np.array_equal(b2, b.astype(np.float64))


def pin_pre_gate_constants(preprocess, forward):
    """softplus(0) = ln 2; softplus(x) -> x (x large), -> exp(x) (x very negative);
    sigmoid(0) = 1/2, sigmoid(+-ln 3) = 3/4, 1/4; A_log and dt_bias per value head."""
    hv = 4
    A_log = np.array([0.0, math.log(2.0), -1.0, 0.5], dtype=np.float32)
    dt_bias = np.array([0.0, 1.0, -2.0, 0.25], dtype=np.float32)
    x = np.array([0.0, 40.0, -40.0], dtype=np.float64)
    a = (x[:, None] - dt_bias[None, :].astype(np.float64)).astype(np.float32)   # a + dt_bias = x (exactly here)
    b = np.array([[0.0, math.log(3.0), -math.log(3.0), 0.0]] * 3, dtype=np.float32)
    q = np.ones((3, 1, 2), dtype=np.float32)
    _, _, g2, b2 = preprocess(q, q, a, b, A_log=A_log, dt_bias=dt_bias, norm_qk=False)
    amp = np.exp(A_log.astype(np.float64))
    xs = a.astype(np.float64) + dt_bias.astype(np.float64)[None, :]
    _close(g2[0], -amp * math.log(2.0) * np.ones(hv), 1e-15, "softplus(0) = ln 2")
    _close(g2[1], -amp * xs[1], 1e-15, "softplus(x) ~ x")
    _close(g2[2], -amp * np.exp(xs[2]), 1e-12, "softplus(x) ~ exp(x)")
    want_b = 1.0 / (1.0 + np.exp(-b.astype(np.float64)))
    _close(b2[:, 0], 0.5 * np.ones(3), 1e-16, "sigmoid(0)")
    _close(b2[:, 1], want_b[:, 1], 1e-15, "sigmoid(ln 3)")
    assert abs(b2[0, 1] - 0.75) < 1e-7 and abs(b2[0, 2] - 0.25) < 1e-7


def pin_pre_gate_without_A_log_passes_through(preprocess, forward):
    q, k, a, b = _raw_case(104, 3, 1, 3, 4)
    _, _, g2, b2 = preprocess(q, k, a, b, A_log=None, norm_qk=True)
    assert np.array_equal(g2, a.astype(np.float64)) and np.array_equal(b2, b.astype(np.float64))


def pin_pre_full_forget_through_the_rule(preprocess, forward):
    """A huge a + dt_bias makes exp(g) vanish: the state after a token is
    beta v k'^T and o = beta (k'.q') v, with beta = sigmoid(b) and q', k' unit."""
    T, hk, hv, dk, dv = 2, 1, 2, 4, 3
    q, k, _, b = _raw_case(105, T, hk, hv, dk)
    a = np.full((T, hv), 800.0, dtype=np.float32)
    A_log = np.zeros(hv, dtype=np.float32)
    v = _rng(106).standard_normal((T, hv, dv)).astype(np.float32)
    q2, k2, g2, b2 = preprocess(q, k, a, b, A_log=A_log, eps=0.0)   # exact unit rows
    cu = np.array([0, T], dtype=np.int32)
    h0 = _rng(107).standard_normal((1, hv, dv, dk)).astype(np.float32)
    out, hT = forward(q2, k2, v, g2, b2, cu, h0)
    t = T - 1
    for h in range(hv):
        bt = 1.0 / (1.0 + math.exp(-float(b[t, h])))
        kk = k[t, 0].astype(np.float64) / np.linalg.norm(k[t, 0].astype(np.float64))
        qq = q[t, 0].astype(np.float64) / np.linalg.norm(q[t, 0].astype(np.float64))
        vv = v[t, h].astype(np.float64)
        _close(hT[0, h], bt * np.outer(vv, kk), 1e-12, "state after a full forget")
        _close(out[t, h], bt * float(kk @ qq) * vv, 1e-12, "output after a full forget")


def pin_pre_bf16_rows(preprocess, forward):
    """bf16 raw q/k are widened exactly before normalising."""
    import torch
    q, k, a, b = _raw_case(108, 3, 2, 2, 8)
    qb = torch.from_numpy(q).to(torch.bfloat16)
    kb = torch.from_numpy(k).to(torch.bfloat16)
    q2b, k2b, _, _ = preprocess(qb, kb, a, b)
    q2f, k2f, _, _ = preprocess(qb.float().numpy(), kb.float().numpy(), a, b)
    assert np.array_equal(q2b, q2f) and np.array_equal(k2b, k2f)


PRE_PINS = [
    pin_pre_norm_closed_form,
    pin_pre_unit_rows,
    pin_pre_norm_off_is_widening,
    pin_pre_gate_constants,
    pin_pre_gate_without_A_log_passes_through,
    pin_pre_full_forget_through_the_rule,
    pin_pre_bf16_rows,
]


# ------------------------------------------------------------ short conv
#
# Pins for oracle.short_conv (causal depthwise convolution with a carried state,
# then SiLU).  Each takes a ``conv`` callable with its signature.

def _conv_case(seed, lengths, C, K, with_state=True):
    r = _rng(seed)
    T = int(sum(lengths))
    x = r.standard_normal((T, C)).astype(np.float32)
    w = r.standard_normal((C, K)).astype(np.float32)
    bias = r.standard_normal(C).astype(np.float32)
    cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)
    state = r.standard_normal((len(lengths), C, K - 1)) if with_state else None
    return x, w, bias, cu, state


def pin_conv_impulse_response(conv):
    """A unit impulse at token t0 (zero state) comes out as the taps, newest tap first."""
    C, K, T, t0 = 3, 4, 12, 5
    x = np.zeros((T, C), dtype=np.float32)
    x[t0] = 1.0
    w = _rng(201).standard_normal((C, K)).astype(np.float32)
    y, _ = conv(x, w, np.array([0, T], dtype=np.int32), silu=False)
    for d in range(K):
        _close(y[t0 + d], w[:, K - 1 - d].astype(np.float64), 1e-15, "impulse tap %d" % d)
    assert not y[:t0].any() and not y[t0 + K:].any(), "response outside the taps"


def pin_conv_matches_numpy_convolve(conv):
    """Per channel, y is numpy's full convolution of [old state, x] with the taps."""
    x, w, bias, cu, state = _conv_case(202, [9, 1, 5], C=4, K=4)
    y, so = conv(x, w, cu, bias=bias, state=state, silu=False)
    for n in range(len(cu) - 1):
        a, b = int(cu[n]), int(cu[n + 1])
        for c in range(x.shape[1]):
            sig = np.concatenate([state[n, c], x[a:b, c].astype(np.float64)])
            full = np.convolve(sig, w[c, ::-1].astype(np.float64))
            want = full[w.shape[1] - 1:w.shape[1] - 1 + (b - a)] + float(bias[c])
            _close(y[a:b, c], want, 1e-13, "channel %d of sequence %d" % (c, n))
            _close(so[n, c], sig[len(sig) - (w.shape[1] - 1):], 0.0 + 1e-300, "state out")


def pin_conv_state_carry(conv):
    """Cutting a sequence and carrying the fp64 state reproduces it exactly."""
    x, w, bias, cu, state = _conv_case(203, [17], C=5, K=4)
    y, so = conv(x, w, cu, bias=bias, state=state)
    st = state
    parts = []
    for a, b in ((0, 2), (2, 3), (3, 11), (11, 17)):
        yp, st = conv(x[a:b], w, np.array([0, b - a], dtype=np.int32), bias=bias, state=st)
        parts.append(yp)
    assert np.array_equal(np.concatenate(parts), y) and np.array_equal(st, so)


def pin_conv_causal(conv):
    x, w, bias, cu, state = _conv_case(204, [10], C=2, K=4)
    y, _ = conv(x, w, cu, bias=bias, state=state)
    x2 = x.copy()
    x2[6:] = 7.0
    y2, _ = conv(x2, w, cu, bias=bias, state=state)
    assert np.array_equal(y[:6], y2[:6]) and not np.array_equal(y[6:], y2[6:])


def pin_conv_constant_and_silu(conv):
    """Constant input a, zero state, no bias: a * sum(w) once the window is full;
    SiLU values silu(0) = 0 and silu(ln 3) = (3/4) ln 3 from bias alone."""
    C, K, T = 2, 4, 8
    w = _rng(205).standard_normal((C, K)).astype(np.float32)
    x = np.full((T, C), 1.5, dtype=np.float32)
    y, _ = conv(x, w, np.array([0, T], dtype=np.int32), silu=False)
    _close(y[K - 1:], np.tile(1.5 * w.astype(np.float64).sum(axis=1), (T - K + 1, 1)), 1e-15, "constant input")
    bias = np.array([0.0, math.log(3.0)], dtype=np.float32)
    y0, _ = conv(np.zeros((3, C), dtype=np.float32), w, np.array([0, 3], dtype=np.int32), bias=bias)
    assert np.all(y0[:, 0] == 0.0)
    # bias[1] is ln 3 rounded to fp32, which moves silu by ~5e-9 relative
    _close(y0[:, 1], np.full(3, 0.75 * math.log(3.0)), 1e-7, "silu(ln 3)")


def pin_conv_short_sequence_state(conv):
    """A sequence shorter than K-1 keeps the newest part of the old state."""
    C, K = 1, 4
    w = np.ones((C, K), dtype=np.float32)
    state = np.array([[[10.0, 20.0, 30.0]]])
    x = np.array([[1.0]], dtype=np.float32)
    y, so = conv(x, w, np.array([0, 1], dtype=np.int32), state=state, silu=False)
    assert y[0, 0] == 61.0 and np.array_equal(so[0, 0], [20.0, 30.0, 1.0])


CONV_PINS = [
    pin_conv_impulse_response,
    pin_conv_matches_numpy_convolve,
    pin_conv_state_carry,
    pin_conv_causal,
    pin_conv_constant_and_silu,
    pin_conv_short_sequence_state,
]


# ----------------------------------------------------- gradient (backward) pins
#
# Each takes ``backward`` (signature of oracle.gdn_backward) and ``forward``
# (oracle.gdn_forward, itself pinned above).  The loss is
# L = sum(dout * out) + sum(dhT * hT), so backward(...) must return dL/d(input).

def _grad_case(seed, lengths, hk, hv, dk, dv, with_h0=True, with_dhT=True):
    c = random_case(seed, lengths, hk, hv, dk, dv, with_h0=with_h0)
    c = {k: (v.astype(np.float64) if isinstance(v, np.ndarray) and v.dtype == np.float32 else v)
         for k, v in c.items()}
    r = _rng(seed + 1)
    T, N = int(sum(lengths)), len(lengths)
    c_d = dict(dout=r.standard_normal((T, hv, dv)),
               dhT=r.standard_normal((N, hv, dv, dk)) if with_dhT else None)
    return c, c_d


def _loss(forward, c, d):
    out, hT = forward(**c)
    L = float((out * d["dout"]).sum())
    if d["dhT"] is not None:
        L += float((hT * d["dhT"]).sum())
    return L


GRAD_NAMES = {"q": "dq", "k": "dk", "v": "dv", "g": "dg", "beta": "dbeta", "h0": "dh0"}


def pin_grad_finite_differences(backward, forward):
    """Every gradient against central differences of the (pinned) forward, on a
    grouped varlen case with an empty sequence, h0 and dhT, all in fp64."""
    c, d = _grad_case(61, [4, 0, 6], hk=1, hv=2, dk=3, dv=2)
    r = backward(**c, **d)
    eps = 1e-6
    for name, gname in GRAD_NAMES.items():
        x = c[name]
        fd = np.zeros_like(x)
        for idx in np.ndindex(x.shape):
            keep = x[idx]
            x[idx] = keep + eps
            lp = _loss(forward, c, d)
            x[idx] = keep - eps
            lm = _loss(forward, c, d)
            x[idx] = keep
            fd[idx] = (lp - lm) / (2 * eps)
        _close(r[gname], fd, tol=1e-7, what="d%s vs finite differences" % name)


def pin_grad_one_token_closed_form(backward, forward):
    """One token from a zero state: out = b (k.q) v and hT = b v k^T, so
    L = b (k.q)(v.dO) + b v^T dhT k and each gradient is a short formula."""
    c, d = _grad_case(62, [1], hk=1, hv=1, dk=4, dv=3, with_h0=False)
    r = backward(**c, **d)
    q, k, v = c["q"][0, 0], c["k"][0, 0], c["v"][0, 0]
    a, b = math.exp(c["g"][0, 0]), c["beta"][0, 0]
    dO, W = d["dout"][0, 0], d["dhT"][0, 0]
    # L = b (k.q)(v.dO) + b v^T W k
    _close(r["dq"][0, 0], b * (v @ dO) * k, what="one-token dq")
    _close(r["dk"][0, 0], b * (v @ dO) * q + b * (W.T @ v), what="one-token dk")
    _close(r["dv"][0, 0], b * (k @ q) * dO + b * (W @ k), what="one-token dv")
    _close(r["dbeta"][0, 0], (k @ q) * (v @ dO) + v @ W @ k, what="one-token dbeta")
    assert r["dg"][0, 0] == 0.0, "the gate cannot act on a zero state"
    # dL/dS0 = a (I - b k k^T)^T-side: D = dO q^T + W, du = D k, dh0 = a (D - b du k^T)
    D = np.outer(dO, q) + W
    _close(r["dh0"][0, 0], a * (D - b * np.outer(D @ k, k)), what="one-token dh0")


def pin_grad_no_write_closed_form(backward, forward):
    """beta = 0 (pure decay, o_t = A_t S0 q_t with A_t = exp(g_1 + ... + g_t)):
    dq_t = A_t S0^T dO_t, dk = dv = 0, dg_t = sum_{s>=t} A_s dO_s.S0 q_s + A_T <dhT, S0>,
    dh0 = sum_s A_s dO_s q_s^T + A_T dhT, dbeta_t = (D_t k_t).(v_t - A_t S0 k_t)
    with D_t = sum_{s>=t} (A_s / A_t) dO_s q_s^T + (A_T / A_t) dhT."""
    c, d = _grad_case(63, [5], hk=1, hv=1, dk=3, dv=4)
    c["beta"][:] = 0.0
    r = backward(**c, **d)
    g = c["g"][:, 0]
    A = np.exp(np.cumsum(g))
    S0 = c["h0"][0, 0]
    q, k, v, dO, W = c["q"][:, 0], c["k"][:, 0], c["v"][:, 0], d["dout"][:, 0], d["dhT"][0, 0]
    T = 5
    for t in range(T):
        _close(r["dq"][t, 0], A[t] * (S0.T @ dO[t]), what="pure decay dq")
        dg = sum(A[s] * dO[s] @ S0 @ q[s] for s in range(t, T)) + A[-1] * float((W * S0).sum())
        _close(r["dg"][t, 0], dg, what="pure decay dg")
        D = sum((A[s] / A[t]) * np.outer(dO[s], q[s]) for s in range(t, T)) + (A[-1] / A[t]) * W
        _close(r["dbeta"][t, 0], (D @ k[t]) @ (v[t] - A[t] * (S0 @ k[t])), what="pure decay dbeta")
    assert not r["dk"].any() and not r["dv"].any()
    _close(r["dh0"][0, 0], sum(A[s] * np.outer(dO[s], q[s]) for s in range(T)) + A[-1] * W, what="pure decay dh0")


def pin_grad_gate_identity(backward, forward):
    """dg_t = <dhT, hT> + sum_{s >= t} (dO_s . o_s - dv_s . v_s) within a sequence:
    scaling S_{t-1} by a_t telescopes through <dL/dS, S> (derivation: with
    Phi_t = <D_t, S_t>, Phi_{t-1} = dO_{t-1}.o_{t-1} + dg_t and Phi_t = dg_t + beta_t du_t.v_t)."""
    c, d = _grad_case(64, [7, 3], hk=1, hv=2, dk=3, dv=3)
    r = backward(**c, **d)
    out, hT = forward(**c)
    cu = c["cu_seqlens"]
    for n in range(2):
        for h in range(2):
            tb, te = int(cu[n]), int(cu[n + 1])
            acc = float((d["dhT"][n, h] * hT[n, h]).sum())
            for t in range(te - 1, tb - 1, -1):
                acc += float(d["dout"][t, h] @ out[t, h] - r["dv"][t, h] @ c["v"][t, h])
                _close(r["dg"][t, h], acc, tol=1e-10, what="gate identity")


def pin_grad_split_sequence(backward, forward):
    """Cutting a sequence in two and chaining the halves through (hT -> h0,
    dh0 of the second -> dhT of the first) reproduces the whole backward."""
    c, d = _grad_case(65, [9], hk=1, hv=2, dk=2, dv=3)
    whole = backward(**c, **d)
    cut = 4
    first = {k: (v[:cut] if k in ("q", "k", "v", "g", "beta") else v) for k, v in c.items()}
    first["cu_seqlens"] = np.array([0, cut], dtype=np.int32)
    _, hmid = forward(**first)
    second = {k: (v[cut:] if k in ("q", "k", "v", "g", "beta") else v) for k, v in c.items()}
    second["cu_seqlens"] = np.array([0, 9 - cut], dtype=np.int32)
    second["h0"] = hmid
    r2 = backward(**second, dout=d["dout"][cut:], dhT=d["dhT"])
    r1 = backward(**first, dout=d["dout"][:cut], dhT=r2["dh0"])
    for key in ("dq", "dk", "dv", "dg", "dbeta"):
        _close(np.concatenate([r1[key], r2[key]]), whole[key], tol=1e-10, what="split %s" % key)
    _close(r1["dh0"], whole["dh0"], tol=1e-10, what="split dh0")


def pin_grad_grouped_heads(backward, forward):
    """Two key heads, each read by two value heads: dq and dk of a key head are
    the sums of what its value heads give with every key head duplicated."""
    c, d = _grad_case(66, [5, 2], hk=2, hv=4, dk=3, dv=2)
    r = backward(**c, **d)
    dup = dict(c)
    dup["q"] = np.repeat(c["q"], 2, axis=1)
    dup["k"] = np.repeat(c["k"], 2, axis=1)
    rd = backward(**dup, **d)
    for kh in range(2):
        _close(r["dq"][:, kh], rd["dq"][:, 2 * kh:2 * kh + 2].sum(axis=1), tol=1e-12, what="grouped dq")
        _close(r["dk"][:, kh], rd["dk"][:, 2 * kh:2 * kh + 2].sum(axis=1), tol=1e-12, what="grouped dk")
    for key in ("dv", "dg", "dbeta", "dh0"):
        _close(r[key], rd[key], tol=1e-12, what="grouped %s" % key)


GRAD_PINS = [
    pin_grad_finite_differences,
    pin_grad_one_token_closed_form,
    pin_grad_no_write_closed_form,
    pin_grad_gate_identity,
    pin_grad_split_sequence,
    pin_grad_grouped_heads,
]


# ------------------------------------- gradients of the preprocessing and the conv
#
# Finite differences on exact perturbations: inputs sit on the grid of multiples
# of 2^-12, so x + j h with h = 2^-10 and j = -2..2 is an fp32 number and the
# forward is evaluated exactly there (in fp64).  The five-point stencil
# (f(x-2h) - 8 f(x-h) + 8 f(x+h) - f(x+2h)) / 12h then has an O(h^4) truncation
# error, about 1e-12 of the derivative's scale for these smooth maps.

FD_H = 2.0 ** -10


def _grid(x):
    return (np.round(np.asarray(x, dtype=np.float64) * 4096.0) / 4096.0).astype(np.float32)


def _fd5(loss, x):
    """dloss/dx for every element of x (modified in place and restored)."""
    out = np.zeros(x.shape)
    for idx in np.ndindex(x.shape):
        keep = x[idx]
        vals = []
        for j in (-2, -1, 1, 2):
            x[idx] = keep + j * FD_H
            assert float(x[idx]) == float(keep) + j * FD_H, "perturbation not exact"
            vals.append(loss())
        x[idx] = keep
        out[idx] = (vals[0] - 8.0 * vals[1] + 8.0 * vals[2] - vals[3]) / (12.0 * FD_H)
    return out


def _pre_grad_case(seed, T, hk, hv, dk, gate=True, bias=True):
    r = _rng(seed)
    c = dict(q=_grid(1.5 * r.standard_normal((T, hk, dk))), k=_grid(1.5 * r.standard_normal((T, hk, dk))),
             a=_grid(2.0 * r.standard_normal((T, hv))), b=_grid(2.0 * r.standard_normal((T, hv))),
             A_log=_grid(r.uniform(-1.0, 1.5, hv)) if gate else None,
             dt_bias=_grid(r.standard_normal(hv)) if (gate and bias) else None)
    w = dict(dqn=r.standard_normal((T, hk, dk)), dkn=r.standard_normal((T, hk, dk)),
             dg=r.standard_normal((T, hv)), dbeta=r.standard_normal((T, hv)))
    return c, w


def pin_pre_grad_finite_differences(pre_backward, preprocess):
    """Every gradient of the preprocessing against five-point differences of the
    (pinned) preprocessing, for L = sum of random weights times its four outputs;
    with the norm and gate maps on and off, with and without dt_bias, eps small and
    large."""
    for seed, gate, bias, norm, eps in ((81, True, True, True, 1e-6), (82, True, False, True, 0.25),
                                        (83, False, False, True, 1e-6), (84, True, True, False, 1e-6)):
        c, w = _pre_grad_case(seed, T=3, hk=2, hv=4, dk=5, gate=gate, bias=bias)

        def loss():
            qn, kn, g, beta = preprocess(c["q"], c["k"], c["a"], c["b"], c["A_log"], c["dt_bias"],
                                         norm_qk=norm, eps=eps)
            return float((qn * w["dqn"]).sum() + (kn * w["dkn"]).sum() + (g * w["dg"]).sum()
                         + (beta * w["dbeta"]).sum())

        r = pre_backward(c["q"], c["k"], c["a"], c["b"], w["dqn"], w["dkn"], w["dg"], w["dbeta"],
                         A_log=c["A_log"], dt_bias=c["dt_bias"], norm_qk=norm, eps=eps)
        names = [("q", "dq"), ("k", "dk"), ("a", "da"), ("b", "db")]
        if gate:
            names.append(("A_log", "dA_log"))
            if bias:
                names.append(("dt_bias", "ddt_bias"))
        for name, gname in names:
            _close(r[gname], _fd5(loss, c[name]), tol=1e-9,
                   what="%s vs finite differences (seed %d)" % (gname, seed))


def pin_pre_grad_constants(pre_backward, preprocess):
    """At a = dt_bias = A_log = 0 and b = 0: softplus'(0) = sigmoid(0) = 1/2 and
    g = -ln 2, so da = -dg / 2, dA_log = -ln 2 * sum_t dg, ddt_bias = sum_t da and
    db = dbeta / 4.  A unit row with eps = 0 has dq = dqn - q (q . dqn)."""
    T, hv = 3, 2
    z = np.zeros((T, hv), dtype=np.float32)
    q = np.array([[[0.5, 0.5, 0.5, 0.5]], [[1.0, 0.0, 0.0, 0.0]], [[0.0, 0.0, -1.0, 0.0]]], dtype=np.float32)
    dg = np.array([[1.0, -2.0], [0.5, 3.0], [-1.0, 0.25]])
    dbeta = np.array([[2.0, 4.0], [-8.0, 1.0], [0.0, 0.5]])
    dqn = np.arange(12, dtype=np.float64).reshape(T, 1, 4) / 7.0
    r = pre_backward(q, q, z, z, dqn, dqn, dg, dbeta, A_log=np.zeros(hv, np.float32),
                     dt_bias=np.zeros(hv, np.float32), norm_qk=True, eps=0.0)
    _close(r["da"], -0.5 * dg, tol=1e-15, what="da at zero logits")
    _close(r["db"], 0.25 * dbeta, tol=1e-15, what="db at zero logits")
    _close(r["dA_log"], -math.log(2.0) * dg.sum(axis=0), tol=1e-15, what="dA_log at zero logits")
    _close(r["ddt_bias"], -0.5 * dg.sum(axis=0), tol=1e-15, what="ddt_bias at zero logits")
    qq = q.astype(np.float64)
    expect = dqn - qq * (qq * dqn).sum(axis=-1, keepdims=True)
    _close(r["dq"], expect, tol=1e-14, what="dq of a unit row")
    _close(r["dk"], expect, tol=1e-14, what="dk of a unit row")


def pin_pre_grad_norm_is_scale_invariant(pre_backward, preprocess):
    """With eps = 0 the normalised row does not change along x, so the gradient
    is orthogonal to x whatever dL/dq' is: x . dq = 0."""
    c, w = _pre_grad_case(85, T=4, hk=3, hv=3, dk=6)
    r = pre_backward(c["q"], c["k"], c["a"], c["b"], w["dqn"], w["dkn"], w["dg"], w["dbeta"],
                     A_log=c["A_log"], dt_bias=c["dt_bias"], norm_qk=True, eps=0.0)
    for x, g in ((c["q"], r["dq"]), (c["k"], r["dk"])):
        dots = (x.astype(np.float64) * g).sum(axis=-1)
        scale = np.linalg.norm(x, axis=-1) * np.linalg.norm(g, axis=-1)
        assert np.all(np.abs(dots) <= 1e-14 * scale), "norm gradient not orthogonal to its row"


PRE_GRAD_PINS = [
    pin_pre_grad_finite_differences,
    pin_pre_grad_constants,
    pin_pre_grad_norm_is_scale_invariant,
]


def pin_conv_grad_finite_differences(conv_backward, conv):
    """dx, dw, dbias and dstate against five-point differences of the (pinned)
    convolution, with SiLU on and off, a sequence shorter than K - 1, an empty one,
    and with and without a carried state."""
    for seed, silu, with_state in ((91, True, True), (92, False, True), (93, True, False)):
        r = _rng(seed)
        lengths, C, K = [5, 0, 2], 3, 4
        x, w, bias, cu, state = _conv_case(seed, lengths, C, K, with_state=with_state)
        x, w, bias = _grid(x), _grid(0.5 * w), _grid(bias)
        if state is not None:
            state = _grid(state).astype(np.float64)
        dy = r.standard_normal(x.shape)

        def loss():
            y, _ = conv(x, w, cu, bias=bias, state=state, silu=silu)
            return float((y * dy).sum())

        g = conv_backward(x, w, cu, dy, bias=bias, state=state, silu=silu)
        arrays = [("x", x, "dx"), ("w", w, "dw"), ("bias", bias, "dbias")]
        if state is not None:
            arrays.append(("state", state, "dstate"))
        for name, arr, gname in arrays:
            _close(g[gname], _fd5(loss, arr), tol=1e-9, what="%s vs finite differences (seed %d)" % (gname, seed))


def pin_conv_grad_adjoint(conv_backward, conv):
    """Without SiLU, bias and state the convolution is linear in x and in w, so
    <dy, conv(x)> = <dx, x> = <dw, w> (the adjoint identity)."""
    r = _rng(94)
    lengths, C, K = [7, 3, 1], 5, 3
    x, w, _, cu, _ = _conv_case(94, lengths, C, K, with_state=False)
    dy = r.standard_normal(x.shape)
    y, _ = conv(x, w, cu, bias=None, state=None, silu=False)
    g = conv_backward(x, w, cu, dy, bias=None, state=None, silu=False)
    lhs = float((dy * y).sum())
    for name, arr, gname in (("x", x, "dx"), ("w", w, "dw")):
        rhs = float((g[gname] * arr.astype(np.float64)).sum())
        assert abs(lhs - rhs) <= 1e-12 * (1.0 + abs(lhs)), "adjoint identity fails for %s" % name


CONV_GRAD_PINS = [
    pin_conv_grad_finite_differences,
    pin_conv_grad_adjoint,
]


def pin_fused_layer_chain(pre_backward, preprocess, backward, forward):
    """The fused layer end to end: raw q, k, a, b, A_log, dt_bias -> preprocessing
    -> the rule -> L = sum(dout * out) + sum(dhT * hT).  The chained gradients
    (the rule's backward, then the preprocessing's) against five-point differences
    of the whole forward, on two sequences with grouped heads and h0."""
    r = _rng(95)
    lengths, hk, hv, dk, dv = [3, 2], 1, 2, 3, 2
    T = sum(lengths)
    c, _ = _pre_grad_case(95, T=T, hk=hk, hv=hv, dk=dk)
    v = _grid(r.standard_normal((T, hv, dv)))
    cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)
    h0 = 0.5 * r.standard_normal((len(lengths), hv, dv, dk))
    dout = r.standard_normal((T, hv, dv))
    dhT = r.standard_normal((len(lengths), hv, dv, dk))

    def pre():
        return preprocess(c["q"], c["k"], c["a"], c["b"], c["A_log"], c["dt_bias"], norm_qk=True, eps=1e-6)

    def loss():
        qn, kn, g, beta = pre()
        out, hT = forward(qn, kn, v, g, beta, cu, h0)
        return float((out * dout).sum() + (hT * dhT).sum())

    qn, kn, g, beta = pre()
    gb = backward(qn, kn, v, g, beta, cu, dout, h0=h0, dhT=dhT)
    gp = pre_backward(c["q"], c["k"], c["a"], c["b"], gb["dq"], gb["dk"], gb["dg"], gb["dbeta"],
                      A_log=c["A_log"], dt_bias=c["dt_bias"], norm_qk=True, eps=1e-6)
    for name, gname in (("q", "dq"), ("k", "dk"), ("a", "da"), ("b", "db"), ("A_log", "dA_log"),
                        ("dt_bias", "ddt_bias")):
        _close(gp[gname], _fd5(loss, c[name]), tol=1e-8, what="fused-layer %s vs finite differences" % gname)
