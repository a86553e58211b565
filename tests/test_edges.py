"""Edge and size cases of the recurrent forward: many short sequences (past the
longest-first ordering limit), uncommon head shapes, and a sequence much longer
than the benchmark's, each against the oracle where it finishes in seconds and
bitwise against a cut or permuted run otherwise."""
import numpy as np
import pytest
import torch

from gpu_helpers import bit_equal, check_parity, run_prefill, say, to_dev
from invariant_linear_attention_amd import synth

pytestmark = pytest.mark.gpu


def test_many_short_sequences(gpu):
    """2048 sequences of 0..20 tokens (the workgroups then keep batch order)."""
    from oracle import oracle
    gen = torch.Generator().manual_seed(77)
    lengths = torch.randint(0, 21, (2048,), generator=gen).tolist()
    w = synth.make_workload(78, lengths, hk=2, hv=4, dk=64, dv=64, h0_std=0.1)
    out, hT = run_prefill(gpu, w)
    ro, rh = oracle.gdn_forward(w.q, w.k, w.v, w.g, w.beta, w.cu_seqlens, w.h0)
    check_parity(w, out, hT, ro, rh, label="2048 short sequences")
    perm = torch.randperm(len(lengths), generator=gen).tolist()
    po, ph = run_prefill(gpu, synth.permute(w, perm))
    cu = w.cu_seqlens.tolist()
    pcu = synth.permute(w, perm).cu_seqlens.tolist()
    for i, n in enumerate(perm[:200]):
        assert bit_equal(po[pcu[i]:pcu[i + 1]], out[cu[n]:cu[n + 1]]) and bit_equal(ph[i], hT[n])


@pytest.mark.parametrize("hk,hv,dk,dv,io", [
    (1, 8, 32, 48, torch.bfloat16),     # 8 value heads per key head, dv = 48
    (4, 4, 16, 16, torch.float32),      # no grouping, the smallest head
    (2, 6, 64, 80, torch.bfloat16),     # dv = 80
])
def test_uncommon_shapes(gpu, hk, hv, dk, dv, io):
    from oracle import oracle
    w = synth.make_workload(90 + dv, [33, 1, 70, 0, 17], hk=hk, hv=hv, dk=dk, dv=dv, io_dtype=io, h0_std=0.1)
    out, hT = run_prefill(gpu, w)
    ro, rh = oracle.gdn_forward(w.q, w.k, w.v, w.g, w.beta, w.cu_seqlens, w.h0)
    check_parity(w, out, hT, ro, rh, label="shape hk=%d hv=%d dk=%d dv=%d" % (hk, hv, dk, dv))
    # decode of one more token reproduces a prefill of it
    d = to_dev(synth.token_slice(synth.select(w, [2]), 69, 70, h0=None))
    _, h69 = run_prefill(gpu, synth.token_slice(synth.select(w, [2]), 0, 69, h0=w.h0[2:3]))
    pool = h69.clone()
    o = gpu.gdn_decode_step(d["q"], d["k"], d["v"], d["g"], d["beta"], pool)
    torch.cuda.synchronize()
    cu = w.cu_seqlens.tolist()
    assert bit_equal(o, out[cu[2] + 69:cu[2] + 70]) and bit_equal(pool[0], hT[2])


def test_very_long_sequence_cut_in_two(gpu):
    """131,072 tokens (twice the long-context workload): one call vs two calls
    carrying the state, bit for bit, and the state still bounded."""
    T = 131072
    w = synth.make_workload(95, [T], hk=2, hv=4, dk=128, dv=128)
    d = to_dev(w)
    out, hT = run_prefill(gpu, w, d=d)
    half = T // 2 + 123
    a = synth.token_slice(w, 0, half)
    o1, h1 = run_prefill(gpu, a)
    b = synth.token_slice(w, half, T, h0=h1.cpu())
    o2, h2 = run_prefill(gpu, b)
    assert bit_equal(torch.cat([o1, o2]), out) and bit_equal(h2, hT)
    assert bool(torch.isfinite(hT).all()) and float(hT.abs().max()) < 1e3
    say("131072 tokens: cut == whole, max |S| = %.3g" % float(hT.abs().max()))
