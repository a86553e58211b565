"""GPU vs the fp64 oracle, element by element, through the C ABI.

Small cases are checked in full (several row tiles, ragged sequence tails, empty
sequences, every head dim and io dtype).  The full-size workloads run on the GPU
at full size in the launch shape the benchmark uses, and the oracle recomputes a
sample of them (whole key heads, whole sequences) one by one.
"""
import numpy as np
import pytest
import torch

from gpu_helpers import check_parity, run_prefill, say, to_dev
from invariant_linear_attention_amd import synth
from oracle import oracle

pytestmark = pytest.mark.gpu


def oracle_of(w):
    return oracle.gdn_forward(w.q, w.k, w.v, w.g, w.beta, w.cu_seqlens, w.h0)


def test_tiny_fp32(gpu):
    """1 sequence, T=64, 2 heads, dk=dv=16, fp32 io, zero initial state."""
    w = synth.tiny(1000)
    out, hT = run_prefill(gpu, w)
    ro, rh = oracle_of(w)
    check_parity(w, out, hT, ro, rh, "tiny fp32")


SMALL = [
    # (name, lengths, hk, hv, dk, dv, io, h0)
    ("dk128_bf16_gqa", [0, 1, 15, 16, 17, 100, 33], 2, 4, 128, 128, torch.bfloat16, 0.1),
    ("dk128_fp32", [5, 40, 1], 1, 2, 128, 128, torch.float32, 0.1),
    ("dk128_bf16_dv64", [31, 9], 2, 2, 128, 64, torch.bfloat16, 0.0),
    ("dk64_bf16", [23, 64, 2], 2, 4, 64, 64, torch.bfloat16, 0.1),
    ("dk32_fp32_g4", [19, 0, 48], 1, 4, 32, 32, torch.float32, 0.1),
    ("dk16_bf16_dv48", [70, 3], 2, 2, 16, 48, torch.bfloat16, 0.1),
    ("dk128_bf16_dv16", [12], 1, 1, 128, 16, torch.bfloat16, 0.1),
]


@pytest.mark.parametrize("name,lengths,hk,hv,dk,dv,io,h0", SMALL, ids=[c[0] for c in SMALL])
def test_small_shapes(gpu, name, lengths, hk, hv, dk, dv, io, h0):
    w = synth.make_workload(77, lengths, hk=hk, hv=hv, dk=dk, dv=dv, io_dtype=io, h0_std=h0)
    out, hT = run_prefill(gpu, w)
    ro, rh = oracle_of(w)
    check_parity(w, out, hT, ro, rh, name)


def _sampled(gpu, w, key_heads, label):
    """Full-size GPU run; oracle on the listed key heads (and their value heads)."""
    out, hT = run_prefill(gpu, w)
    grp = w.dims["hv"] // w.dims["hk"]
    for kh in key_heads:
        s = synth.head_slice(w, kh)
        ro, rh = oracle_of(s)
        vs = slice(kh * grp, (kh + 1) * grp)
        check_parity(s, out[:, vs].contiguous(), hT[:, vs].contiguous(), ro, rh, "%s kh=%d" % (label, kh))
    return out, hT


def test_varlen_prefill_full_size_sampled(gpu):
    """8 sequences of 256..4096 tokens, 16/32 heads, dk=dv=128, bf16 io, random h0."""
    w = synth.varlen_prefill(1001)
    say("lengths %s" % w.lengths)
    _sampled(gpu, w, [0, 7, 15], "varlen_prefill")


def test_mixed_batch_full_size_sampled(gpu):
    """64 sequences: 32 prefill chunks (16..8192 tokens) and 32 single-token decodes."""
    w = synth.mixed_batch(1004)
    _sampled(gpu, w, [3], "mixed_batch")


def test_long_context_full_size_sampled(gpu):
    """One sequence of 65,536 tokens from the zero state; oracle on one key head."""
    w = synth.long_context(1003)
    _sampled(gpu, w, [9], "long_context")


def test_decode_after_prefill_vs_oracle(gpu):
    """512-token prefill, then one decode step per sequence, against the oracle's
    513-token run (sampled sequences of a 64-sequence batch)."""
    w = synth.decode_history(1002, batch=64, prefix=512, steps=1)
    pre = synth.permute(w, range(64))
    # split each sequence into its 512-token prefix and its last token
    cu = w.cu_seqlens.tolist()
    first = torch.cat([torch.arange(cu[i], cu[i] + 512) for i in range(64)])
    last = torch.tensor([cu[i] + 512 for i in range(64)])
    dev = "cuda"
    d = to_dev(w, dev)
    cu_pre = torch.arange(0, 64 * 512 + 1, 512, dtype=torch.int32, device=dev)
    _, pool = gpu.gdn_fwd_varlen(d["q"][first.to(dev)].contiguous(), d["k"][first.to(dev)].contiguous(),
                                 d["v"][first.to(dev)].contiguous(), d["g"][first.to(dev)].contiguous(),
                                 d["beta"][first.to(dev)].contiguous(), None, cu_pre)
    li = last.to(dev)
    o = gpu.gdn_decode_step(d["q"][li].contiguous(), d["k"][li].contiguous(), d["v"][li].contiguous(),
                            d["g"][li].contiguous(), d["beta"][li].contiguous(), pool)
    torch.cuda.synchronize()
    for s in (0, 37, 63):
        sw = synth.select(pre, [s])
        ro, rh = oracle_of(sw)
        # the decode output is the sequence's last token; the pool holds its final state
        one = synth.token_slice(sw, 0, 1)  # shape carrier for the metric (one token)
        check_parity(one, o[s:s + 1], pool[s:s + 1], ro[-1:], rh, "decode seq %d" % s)
