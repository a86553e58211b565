"""Seeded synthetic workloads for the Gated DeltaNet recurrent forward.

This module only draws inputs; it holds none of the recurrence's arithmetic, so
both the HIP path and the CPU oracle may be fed from it.  Every tensor is made on
the CPU with a seeded ``torch.Generator`` and is returned on the CPU.

Distributions (the same for every workload):
  * q, k : N(0, 1), L2-normalised per (token, head) vector in fp32, then cast to
           the io dtype with round-to-nearest-even (so bf16 keys are only
           approximately unit length);
  * v    : N(0, 1), cast to the io dtype;
  * g    : -softplus(N(0, 1)), fp32 (log of the per-token decay, always < 0);
  * beta : sigmoid(N(0, 1)), fp32 (write strength in (0, 1));
  * h0   : N(0, std^2) fp32 where a sequence resumes from a cached state, else 0.

Shapes are the Qwen3.5-style GDN layer shape used throughout: 16 query/key heads,
32 value heads (two value heads per key head), dk = dv = 128.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import List, Optional

import torch

HK, HV, DK, DV = 16, 32, 128, 128


@dataclass
class Workload:
    """One packed varlen batch (all tensors on the CPU)."""
    q: torch.Tensor            # [T, Hk, dk]
    k: torch.Tensor            # [T, Hk, dk]
    v: torch.Tensor            # [T, Hv, dv]
    g: torch.Tensor            # [T, Hv] fp32
    beta: torch.Tensor         # [T, Hv] fp32
    cu_seqlens: torch.Tensor   # [N+1] int32
    h0: Optional[torch.Tensor]  # [N, Hv, dv, dk] fp32 or None (zero state)
    name: str = ""
    meta: dict = field(default_factory=dict)

    @property
    def n_seqs(self) -> int:
        return int(self.cu_seqlens.numel()) - 1

    @property
    def total_tokens(self) -> int:
        return int(self.q.shape[0])

    @property
    def lengths(self) -> List[int]:
        cu = self.cu_seqlens.tolist()
        return [cu[i + 1] - cu[i] for i in range(len(cu) - 1)]

    @property
    def dims(self):
        return dict(hk=self.q.shape[1], hv=self.v.shape[1], dk=self.q.shape[2], dv=self.v.shape[2])


def _normal(gen, shape):
    return torch.randn(*shape, generator=gen, dtype=torch.float32)


def _unit_rows(x: torch.Tensor) -> torch.Tensor:
    return x / x.norm(dim=-1, keepdim=True)


def cu_from_lengths(lengths) -> torch.Tensor:
    cu = [0]
    for n in lengths:
        cu.append(cu[-1] + int(n))
    return torch.tensor(cu, dtype=torch.int32)


def make_workload(seed: int, lengths, hk=HK, hv=HV, dk=DK, dv=DV, io_dtype=torch.bfloat16,
                  h0_std: float = 0.0, h0_rows=None, name: str = "") -> Workload:
    """Draw one packed batch.

    ``lengths``: tokens per sequence.  ``h0_std`` > 0 gives resuming sequences an
    N(0, h0_std^2) initial state; ``h0_rows`` (a list of booleans, one per
    sequence) says which sequences resume; by default all do when h0_std > 0 and
    none otherwise (h0 is then None, the zero state).
    """
    gen = torch.Generator().manual_seed(int(seed))
    lengths = [int(n) for n in lengths]
    T = sum(lengths)
    q = _unit_rows(_normal(gen, (T, hk, dk))).to(io_dtype)
    k = _unit_rows(_normal(gen, (T, hk, dk))).to(io_dtype)
    v = _normal(gen, (T, hv, dv)).to(io_dtype)
    g = -torch.nn.functional.softplus(_normal(gen, (T, hv)))
    beta = torch.sigmoid(_normal(gen, (T, hv)))
    h0 = None
    if h0_std > 0:
        h0 = _normal(gen, (len(lengths), hv, dv, dk)) * float(h0_std)
        if h0_rows is not None:
            mask = torch.tensor([bool(r) for r in h0_rows], dtype=torch.bool)
            h0[~mask] = 0.0
    return Workload(q.contiguous(), k.contiguous(), v.contiguous(), g.contiguous(),
                    beta.contiguous(), cu_from_lengths(lengths), h0, name=name,
                    meta=dict(seed=int(seed)))


def make_raw_workload(seed: int, lengths, hk=HK, hv=HV, dk=DK, dv=DV, io_dtype=torch.bfloat16,
                      h0_std: float = 0.0, name: str = "") -> Workload:
    """Raw inputs for the fused-preprocessing path.

    q, k: N(0, 1) rows scaled by a per-(token, head) factor in [0.25, 4], not
    normalised; v: N(0, 1); the ``g`` and ``beta`` fields hold the logits a, b
    ~ N(0, 1); meta["A_log"] = log U(1, 16) and meta["dt_bias"] ~ U(ln 1e-3, ln 0.1)
    per value head (fp32), the usual initial ranges of a decay amplitude and of
    its time-step bias.
    """
    gen = torch.Generator().manual_seed(int(seed) + 104729)
    lengths = [int(n) for n in lengths]
    T = sum(lengths)

    def rows(shape):
        x = _normal(gen, shape)
        scale = torch.exp2(torch.rand(shape[:-1] + (1,), generator=gen) * 4.0 - 2.0)
        return (x * scale).to(io_dtype)

    q = rows((T, hk, dk))
    k = rows((T, hk, dk))
    v = _normal(gen, (T, hv, dv)).to(io_dtype)
    a = _normal(gen, (T, hv))
    b = _normal(gen, (T, hv))
    A_log = torch.log(1.0 + 15.0 * torch.rand((hv,), generator=gen))
    dt_bias = math.log(1e-3) + (math.log(0.1) - math.log(1e-3)) * torch.rand((hv,), generator=gen)
    h0 = _normal(gen, (len(lengths), hv, dv, dk)) * float(h0_std) if h0_std > 0 else None
    return Workload(q.contiguous(), k.contiguous(), v.contiguous(), a.contiguous(), b.contiguous(),
                    cu_from_lengths(lengths), h0, name=name or "raw",
                    meta=dict(seed=int(seed), A_log=A_log.float(), dt_bias=dt_bias.float(), raw=True))


# ---------------------------------------------------------------- the workloads

def tiny(seed: int = 1000) -> Workload:
    """1 sequence, T=64, 2 heads (no grouping), dk=dv=16, all fp32, zero state."""
    return make_workload(seed, [64], hk=2, hv=2, dk=16, dv=16, io_dtype=torch.float32,
                         name="tiny_T64_H2_d16_fp32")


def varlen_prefill(seed: int = 1001) -> Workload:
    """8 sequences, lengths uniform in [256, 4096], bf16 io, h0 ~ N(0, 0.1^2)."""
    gen = torch.Generator().manual_seed(int(seed) + 7919)
    lengths = torch.randint(256, 4097, (8,), generator=gen).tolist()
    return make_workload(seed, lengths, h0_std=0.1, name="varlen_prefill_8seq_256to4096")


def long_context(seed: int = 1003, T: int = 65536) -> Workload:
    """1 sequence of 65,536 tokens from the zero state, bf16 io."""
    return make_workload(seed, [T], name="long_context_T%d" % T)


def decode_history(seed: int = 1002, batch: int = 256, prefix: int = 512, steps: int = 1) -> Workload:
    """``batch`` sequences of ``prefix + steps`` tokens from the zero state.

    The first ``prefix`` tokens of each sequence build its cached state by
    prefill; the remaining ``steps`` tokens are fed one decode step at a time.
    """
    return make_workload(seed, [prefix + steps] * batch, name="decode_B%d_prefix%d" % (batch, prefix))


def mixed_batch(seed: int = 1004) -> Workload:
    """64 sequences: 32 prefill chunks with log-uniform lengths in [16, 8192] and
    32 single-token decodes, shuffled; all decodes and 16 of the prefill chunks
    resume from a nonzero cached state, the other 16 chunks start from zero."""
    gen = torch.Generator().manual_seed(int(seed) + 7919)
    u = torch.rand(32, generator=gen, dtype=torch.float64)
    lo, hi = math.log(16.0), math.log(8192.0)
    pre = [int(round(math.exp(lo + float(x) * (hi - lo)))) for x in u]
    cached_pre = torch.randperm(32, generator=gen)[:16].tolist()
    kinds = [("prefill", n, i in cached_pre) for i, n in enumerate(pre)] + [("decode", 1, True)] * 32
    order = torch.randperm(64, generator=gen).tolist()
    kinds = [kinds[i] for i in order]
    w = make_workload(seed, [n for _, n, _ in kinds], h0_std=0.1, h0_rows=[c for _, _, c in kinds],
                      name="mixed_64seq_32prefill_32decode")
    w.meta["kinds"] = [kd for kd, _, _ in kinds]
    w.meta["cached"] = [c for _, _, c in kinds]
    return w


# ------------------------------------------------------------- batch surgery

def permute(w: Workload, perm) -> Workload:
    """Reorder whole sequences (their token segments and h0 rows): pure data movement."""
    perm = [int(i) for i in perm]
    cu = w.cu_seqlens.tolist()
    idx = torch.cat([torch.arange(cu[i], cu[i + 1]) for i in perm]) if perm else torch.zeros(0, dtype=torch.long)
    lengths = [cu[i + 1] - cu[i] for i in perm]
    h0 = None if w.h0 is None else w.h0[perm].contiguous()
    return Workload(w.q[idx].contiguous(), w.k[idx].contiguous(), w.v[idx].contiguous(),
                    w.g[idx].contiguous(), w.beta[idx].contiguous(), cu_from_lengths(lengths), h0,
                    name=w.name + "_perm", meta=dict(w.meta, perm=perm))


def select(w: Workload, seqs) -> Workload:
    """Sub-batch made of the listed sequences, in the listed order."""
    return permute(w, seqs)


def token_slice(w: Workload, start: int, stop: int, h0=None) -> Workload:
    """Tokens [start, stop) of a single-sequence workload as a new one-sequence batch."""
    assert w.n_seqs == 1
    sl = slice(start, stop)
    return Workload(w.q[sl].contiguous(), w.k[sl].contiguous(), w.v[sl].contiguous(),
                    w.g[sl].contiguous(), w.beta[sl].contiguous(), cu_from_lengths([stop - start]),
                    h0, name="%s[%d:%d]" % (w.name, start, stop), meta=dict(w.meta))


def head_slice(w: Workload, kh: int) -> Workload:
    """Only key head ``kh`` and its value heads (for sampled oracle checks)."""
    d = w.dims
    grp = d["hv"] // d["hk"]
    vs = slice(kh * grp, (kh + 1) * grp)
    h0 = None if w.h0 is None else w.h0[:, vs].contiguous()
    return Workload(w.q[:, kh:kh + 1].contiguous(), w.k[:, kh:kh + 1].contiguous(), w.v[:, vs].contiguous(),
                    w.g[:, vs].contiguous(), w.beta[:, vs].contiguous(), w.cu_seqlens.clone(), h0,
                    name="%s_kh%d" % (w.name, kh), meta=dict(w.meta))
