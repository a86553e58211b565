"""Shared helpers for the GPU tests: moving synthetic workloads to the device,
running them through the C ABI, and the error metrics of the parity gates.

Parity metric.  For each sequence n, over all its tokens and heads,
e_n = ||x_n - r_n||_2 / ||r_n||_2 against the fp64 oracle, and the gate is on
max_n e_n: <= 2e-3 for bf16 outputs (rounding fp32 to bf16 alone costs about
1.7e-3 on these distributions; on samples so small that rounding the exact
result to bf16 already exceeds 2e-3, the gate is that rounding floor + 1e-4),
<= 1e-4 for fp32 outputs and for the fp32 final state.  bf16 outputs are also checked element-wise: each one that is not tiny
(|r| >= 1% of the RMS) must be within one bf16 ulp of the oracle value rounded
to nearest even.
"""
from __future__ import annotations

import sys

import numpy as np
import torch

OUT_TOL = {torch.bfloat16: 2e-3, torch.float32: 1e-4}
STATE_TOL = 1e-4


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def to_dev(w, dev="cuda"):
    h0 = None if w.h0 is None else w.h0.to(dev)
    return dict(q=w.q.to(dev), k=w.k.to(dev), v=w.v.to(dev), g=w.g.to(dev), beta=w.beta.to(dev), h0=h0,
                cu_seqlens=w.cu_seqlens.to(dev))


def run_prefill(gdn, w, plan=(0, 0), dev="cuda", d=None):
    d = d if d is not None else to_dev(w, dev)
    out, hT = gdn.gdn_fwd_varlen(d["q"], d["k"], d["v"], d["g"], d["beta"], d["h0"], d["cu_seqlens"], plan=plan)
    torch.cuda.synchronize()
    return out, hT


def seq_errors(x, ref, cu):
    """Per-sequence normwise relative error of token-major arrays [T, ...]."""
    x = np.asarray(x, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    errs = []
    for n in range(len(cu) - 1):
        a, b = int(cu[n]), int(cu[n + 1])
        if b == a:
            continue
        den = np.linalg.norm(ref[a:b])
        errs.append(float(np.linalg.norm(x[a:b] - ref[a:b]) / max(den, 1e-300)))
    return errs


def state_errors(x, ref):
    x = np.asarray(x, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    return [float(np.linalg.norm(x[n] - ref[n]) / max(np.linalg.norm(ref[n]), 1e-300)) for n in range(ref.shape[0])]


def bf16_ulp_distance(x_bf16: torch.Tensor, ref: np.ndarray, rel_floor: float = 1e-2):
    """Distance, in bf16 ulps, between GPU bf16 outputs and RNE(oracle).

    Returns (max over elements with |ref| >= rel_floor * rms(ref), count of all
    elements more than one ulp away).  Outputs near zero through cancellation
    carry an fp32 error that is large in their own ulps, hence the floor."""
    ref = np.asarray(ref, dtype=np.float64)
    r = torch.from_numpy(ref).to(torch.float32).to(torch.bfloat16)
    a = x_bf16.cpu().contiguous().view(torch.int16).to(torch.int32)
    b = r.contiguous().view(torch.int16).to(torch.int32)
    # map sign-magnitude bf16 bit patterns onto a monotone integer line
    a = torch.where(a < 0, -32768 - a, a)
    b = torch.where(b < 0, -32768 - b, b)
    d = (a - b).abs()
    if d.numel() == 0:
        return 0, 0
    rms = float(np.sqrt(np.mean(ref * ref)))
    big = torch.from_numpy(np.abs(ref) >= rel_floor * rms)
    dm = d[big]
    return (int(dm.max()) if dm.numel() else 0), int((d > 1).sum())


def check_parity(w, out, hT, ref_out, ref_hT, label=""):
    """Assert the gates; returns a dict of the measured errors."""
    cu = w.cu_seqlens.tolist()
    tol = OUT_TOL[out.dtype]
    eo = seq_errors(out.float().cpu().numpy(), ref_out, cu)
    es = state_errors(hT.cpu().numpy(), ref_hT) if hT is not None else []
    res = dict(out_max=max(eo) if eo else 0.0, state_max=max(es) if es else 0.0)
    if out.dtype == torch.bfloat16:
        res["ulp"], res["n_beyond_1ulp"] = bf16_ulp_distance(out, ref_out)
        res["floor"] = max(seq_errors(torch.from_numpy(ref_out).float().to(torch.bfloat16).float().numpy(),
                                      ref_out, cu) or [0.0])
    if out.dtype == torch.bfloat16:
        # On a handful of elements, rounding the exact result to bf16 can by itself
        # exceed 2e-3; the gate is then that floor plus the fp32 allowance.
        tol = max(tol, res["floor"] + STATE_TOL)
    res["gate"] = tol
    say("%s: %s" % (label, res))
    assert res["out_max"] <= tol, "%s: output error %.3e > %.1e" % (label, res["out_max"], tol)
    assert res["state_max"] <= STATE_TOL, "%s: state error %.3e > %.1e" % (label, res["state_max"], STATE_TOL)
    if "ulp" in res:
        assert res["ulp"] <= 1, "%s: a bf16 output is %d ulps from RNE(oracle)" % (label, res["ulp"])
    return res


def bit_equal(a: torch.Tensor, b: torch.Tensor) -> bool:
    """Exact equality of the bit patterns (distinguishes -0 from +0, compares NaNs)."""
    if a.shape != b.shape or a.dtype != b.dtype:
        return False
    iv = {torch.float32: torch.int32, torch.bfloat16: torch.int16}[a.dtype]
    return torch.equal(a.contiguous().view(iv), b.contiguous().view(iv))
