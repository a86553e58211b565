"""GPU vs the fp64 oracle, element by element, through the C ABI.

Small cases are checked in full (several row tiles, ragged sequence tails, empty
sequences, every head dim and io dtype).  The full-size workloads run on the GPU
at full size in the launch shape the benchmark uses, and the oracle recomputes
all of them: every sequence, head and token, and every sequence of the B = 256
decode step against its 513-token oracle run.
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


def _full(gpu, w, label):
    """Full-size GPU run in the benchmark's launch shape; the oracle recomputes
    every sequence, key head and token (one call, so its threads spread over all
    (sequence, value head) units), and the gates apply to every element."""
    out, hT = run_prefill(gpu, w)
    say("%s: GPU done (%d tokens, %d sequences); oracle on every head" % (label, w.total_tokens, w.n_seqs))
    ro, rh = oracle_of(w)
    check_parity(w, out, hT, ro, rh, label)
    return out, hT


def test_varlen_prefill_full_size(gpu):
    """8 sequences of 256..4096 tokens, 16/32 heads, dk=dv=128, bf16 io, random h0:
    all 32 value heads against the oracle."""
    w = synth.varlen_prefill(1001)
    say("lengths %s" % w.lengths)
    _full(gpu, w, "varlen_prefill")


def test_mixed_batch_full_size(gpu):
    """64 sequences: 32 prefill chunks (16..8192 tokens) and 32 single-token
    decodes, a quarter resuming from cached states: every head against the oracle."""
    w = synth.mixed_batch(1004)
    _full(gpu, w, "mixed_batch")


def test_long_context_full_size(gpu):
    """One sequence of 65,536 tokens from the zero state: every head against the oracle."""
    w = synth.long_context(1003)
    _full(gpu, w, "long_context")


def test_decode_after_prefill_vs_oracle(gpu):
    """512-token prefill of 256 sequences, then one decode step at B = 256, against
    the oracle's 513-token run of every sequence (outputs and final states)."""
    B = 256
    w = synth.decode_history(1002, batch=B, prefix=512, steps=1)
    cu = w.cu_seqlens.tolist()
    first = torch.cat([torch.arange(cu[i], cu[i] + 512) for i in range(B)])
    last = torch.tensor([cu[i] + 512 for i in range(B)])
    dev = "cuda"
    d = to_dev(w, dev)
    fi, li = first.to(dev), last.to(dev)
    cu_pre = torch.arange(0, B * 512 + 1, 512, dtype=torch.int32, device=dev)
    _, pool = gpu.gdn_fwd_varlen(d["q"][fi].contiguous(), d["k"][fi].contiguous(), d["v"][fi].contiguous(),
                                 d["g"][fi].contiguous(), d["beta"][fi].contiguous(), None, cu_pre)
    o = gpu.gdn_decode_step(d["q"][li].contiguous(), d["k"][li].contiguous(), d["v"][li].contiguous(),
                            d["g"][li].contiguous(), d["beta"][li].contiguous(), pool)
    torch.cuda.synchronize()
    say("decode B=%d: GPU done; oracle on %d x 513 tokens" % (B, B))
    ro, rh = oracle_of(w)
    # the decode outputs are each sequence's last token; the pool holds its final state
    one = synth.make_workload(0, [1] * B, hk=1, hv=1, dk=16, dv=16)  # carrier of cu_seqlens = 0..B
    check_parity(one, o, pool, ro[last.numpy()], rh, "decode B=%d after 512-token prefill" % B)
