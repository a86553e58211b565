"""Fused preprocessing (gdn_dims.pre): in-kernel q/k L2 normalisation and the gate
and write strength formed from logits.

Parity: the GPU path with raw inputs against the fp64 oracle run on the same raw
inputs (oracle.preprocess, then the recurrence), under the same gates as the
plain path.  Invariance: the preprocessing is part of the fixed per-row
arithmetic, so decode reproduces prefill, and batch-mates, launch shape, chunking
and the state pool change no bit.
"""
import pytest
import torch

from gpu_helpers import bit_equal, check_parity, say, to_dev
from invariant_linear_attention_amd import synth

pytestmark = pytest.mark.gpu
DEV = "cuda"


def raw(seed, lengths, hk=4, hv=8, dk=128, dv=128, io=torch.bfloat16, h0=0.1):
    return synth.make_raw_workload(seed, lengths, hk=hk, hv=hv, dk=dk, dv=dv, io_dtype=io, h0_std=h0)


def pre_for(gdn, w, norm=True, gate=True, eps=1e-6):
    A = w.meta["A_log"].to(DEV) if gate else None
    D = w.meta["dt_bias"].to(DEV) if gate else None
    return gdn.make_preproc(norm_qk=norm, eps=eps, A_log=A, dt_bias=D), (A, D)


def run(gdn, w, pre, plan=(0, 0, 0), d=None):
    d = d if d is not None else to_dev(w)
    out, hT = gdn.gdn_fwd_varlen(d["q"], d["k"], d["v"], d["g"], d["beta"], d["h0"], d["cu_seqlens"], plan=plan,
                                 pre=pre)
    torch.cuda.synchronize()
    return out, hT


def oracle_ref(w, norm=True, gate=True, eps=1e-6):
    from oracle import oracle
    return oracle.gdn_forward_fused(w.q, w.k, w.v, w.g, w.beta, w.cu_seqlens, w.h0,
                                    A_log=w.meta["A_log"] if gate else None,
                                    dt_bias=w.meta["dt_bias"] if gate else None, norm_qk=norm, eps=eps)


@pytest.mark.parametrize("norm,gate", [(True, True), (True, False), (False, True)])
@pytest.mark.parametrize("dk,io", [(128, torch.bfloat16), (64, torch.bfloat16), (16, torch.float32)])
def test_parity_small(gpu, norm, gate, dk, io):
    w = raw(51, [37, 1, 100, 0, 16], dk=dk, dv=dk if dk >= 64 else 32, io=io)
    if not gate:   # the plain gate and beta ranges
        w = synth.Workload(w.q, w.k, w.v, -torch.nn.functional.softplus(w.g), torch.sigmoid(w.beta),
                           w.cu_seqlens, w.h0, meta=w.meta)
    if not norm:   # plain path takes unit rows
        w = synth.Workload((w.q.float() / w.q.float().norm(dim=-1, keepdim=True)).to(io),
                           (w.k.float() / w.k.float().norm(dim=-1, keepdim=True)).to(io),
                           w.v, w.g, w.beta, w.cu_seqlens, w.h0, meta=w.meta)
    pre, keep = pre_for(gpu, w, norm=norm, gate=gate)
    out, hT = run(gpu, w, pre)
    ro, rh = oracle_ref(w, norm=norm, gate=gate)
    check_parity(w, out, hT, ro, rh, label="pre norm=%s gate=%s dk=%d %s" % (norm, gate, dk, io))


def test_parity_benchmark_shape(gpu):
    """Raw inputs at the benchmark batch's shape; oracle on two key heads."""
    from oracle import oracle
    w = synth.make_raw_workload(1001, synth.varlen_prefill(1001).lengths, h0_std=0.1)
    pre, keep = pre_for(gpu, w)
    out, hT = run(gpu, w, pre)
    for kh in (0, 11):
        s = synth.head_slice(w, kh)
        A, D = w.meta["A_log"][2 * kh:2 * kh + 2], w.meta["dt_bias"][2 * kh:2 * kh + 2]
        ro, rh = oracle.gdn_forward_fused(s.q, s.k, s.v, s.g, s.beta, s.cu_seqlens, s.h0, A_log=A, dt_bias=D)
        vs = slice(2 * kh, 2 * kh + 2)
        check_parity(s, out[:, vs].contiguous(), hT[:, vs].contiguous(), ro, rh, label="pre bench kh%d" % kh)


def test_decode_reproduces_prefill(gpu):
    """Token L of a sequence by decode, from the prefill state of its first L
    tokens, equals the (L+1)-token prefill bit for bit, with preprocessing."""
    for dk, io in ((128, torch.bfloat16), (64, torch.float32), (16, torch.bfloat16)):
        L = 40
        w = raw(61, [L + 1], dk=dk, dv=64, io=io)
        pre, keep = pre_for(gpu, w)
        full_out, full_hT = run(gpu, w, pre)
        _, hL = run(gpu, synth.token_slice(w, 0, L, h0=w.h0), pre)
        d = to_dev(synth.token_slice(w, L, L + 1))
        pool = hL.clone()
        o = gpu.gdn_decode_step(d["q"], d["k"], d["v"], d["g"], d["beta"], pool, pre=pre)
        torch.cuda.synchronize()
        assert bit_equal(o, full_out[L:]) and bit_equal(pool, full_hT), (dk, io)


def test_alone_vs_in_batch_and_shapes(gpu):
    w = raw(71, [50, 3, 130, 17], hv=8)
    pre, keep = pre_for(gpu, w)
    ref_out, ref_hT = run(gpu, w, pre)
    cu = w.cu_seqlens.tolist()
    for n in range(w.n_seqs):
        o, h = run(gpu, synth.select(w, [n]), pre)
        assert bit_equal(o, ref_out[cu[n]:cu[n + 1]]) and bit_equal(h[0], ref_hT[n]), n
    for plan in [(8, 1, 1), (16, 1, 4), (16, 2, 4), (4, 1, 4), (4, 2, 1), (8, 2, 2), (16, 4, 1), (8, 1, 8), (8, 2, 4),
                 (16, 2, 8)]:
        o, h = run(gpu, w, pre, plan=plan)
        assert bit_equal(o, ref_out) and bit_equal(h, ref_hT), plan


def test_chunked_and_pool_paths(gpu):
    L = 150
    w = raw(81, [L])
    pre, keep = pre_for(gpu, w)
    ref_out, ref_hT = run(gpu, w, pre)
    state = w.h0.clone()
    outs = []
    for a, b in ((0, 37), (37, 38), (38, 130), (130, L)):
        o, state = run(gpu, synth.token_slice(w, a, b, h0=state.cpu()), pre)
        outs.append(o)
    assert bit_equal(torch.cat(outs), ref_out) and bit_equal(state, ref_hT)
    d = to_dev(w)
    pool = torch.zeros((3, 8, 128, 128), device=DEV)
    pool[0] = d["h0"][0]
    snap = torch.tensor([[1, 2]], dtype=torch.int32, device=DEV)
    o = gpu.gdn_fwd_varlen_pool(d["q"], d["k"], d["v"], d["g"], d["beta"], d["cu_seqlens"], pool,
                                src_idx=torch.tensor([0], dtype=torch.int32, device=DEV),
                                dst_idx=torch.tensor([0], dtype=torch.int32, device=DEV),
                                snap_idx=snap, snap_block=64, pre=pre)
    torch.cuda.synchronize()
    assert bit_equal(o, ref_out) and bit_equal(pool[0], ref_hT[0])
    _, h64 = run(gpu, synth.token_slice(w, 0, 64, h0=w.h0), pre)
    assert bit_equal(pool[1], h64[0])


def test_decode_batch_sizes(gpu):
    """Each decode row's bits do not depend on the batch it rides in."""
    B = 64
    w = raw(91, [1] * B, h0=0.1)
    pre, keep = pre_for(gpu, w)
    d = to_dev(w)
    pool = d["h0"].clone()
    o_all = gpu.gdn_decode_step(d["q"], d["k"], d["v"], d["g"], d["beta"], pool, pre=pre)
    torch.cuda.synchronize()
    for Bs in (1, 8):
        p2 = d["h0"][:Bs].clone()
        o = gpu.gdn_decode_step(d["q"][:Bs], d["k"][:Bs], d["v"][:Bs], d["g"][:Bs].contiguous(),
                                d["beta"][:Bs].contiguous(), p2, pre=pre)
        torch.cuda.synchronize()
        assert bit_equal(o, o_all[:Bs]) and bit_equal(p2, pool[:Bs]), Bs
    say("decode with preprocessing: batch sizes 1/8/64 agree bitwise")


def _very_negative_logits(seed, lengths, hv=8, io=torch.bfloat16):
    """Raw inputs whose gate argument a + dt_bias lies in [-30, -5] (softplus far
    below 1, where log(1 + e^x) must not be formed from a rounded 1 + e^x), with a
    large decay amplitude exp(A_log) in [1e3, 1e4] so that g = -exp(A_log)
    softplus(a + dt_bias) spans (-67, 0) and the decay's accuracy reaches the state."""
    w = raw(seed, lengths, hv=hv, io=io)
    gen = torch.Generator().manual_seed(seed + 1)
    A_log = torch.log(1e3 + 9e3 * torch.rand((hv,), generator=gen))
    x = -30.0 + 25.0 * torch.rand(tuple(w.g.shape), generator=gen)
    a = (x - w.meta["dt_bias"][None, :]).contiguous()
    meta = dict(w.meta, A_log=A_log.float())
    return synth.Workload(w.q, w.k, w.v, a, w.beta, w.cu_seqlens, w.h0, meta=meta)


def test_gate_from_very_negative_logits(gpu):
    """a + dt_bias in [-30, -5]: the fused gate against the fp64 oracle, which
    evaluates log1p(exp(x)) there."""
    w = _very_negative_logits(101, [37, 200, 1, 64])
    pre, keep = pre_for(gpu, w)
    out, hT = run(gpu, w, pre)
    ro, rh = oracle_ref(w)
    check_parity(w, out, hT, ro, rh, label="gate logits in [-30, -5]")


def test_decay_from_very_negative_logits_one_token(gpu):
    """With beta = sigmoid(-200) = 0 a decode step only decays: S_1 = a S_0, so a
    state of ones returns the kernel's decay a = exp(g) itself.  Its error against
    exp(-exp(A_log) log1p(exp(x))) in fp64 stays at the rounding of g (about
    2e-6 relative from the arguments of the two exponentials, scaled by |g|), for
    x down to -30; forming log(1 + e^x) from a rounded 1 + e^x misses it by up to
    6e-4 at x = -12."""
    import numpy as np
    hv, B = 8, 256
    w = _very_negative_logits(111, [1] * B, hv=hv)
    b = torch.full((B, hv), -200.0)
    pre, keep = pre_for(gpu, w, norm=False)
    d = to_dev(w)
    pool = torch.ones((B, hv, 128, 128), device=DEV)
    gpu.gdn_decode_step(d["q"], d["k"], d["v"], d["g"], b.to(DEV), pool, pre=pre)
    torch.cuda.synchronize()
    got = pool[:, :, 0, 0].double().cpu().numpy()
    assert bool((pool == pool[:, :, :1, :1]).all()), "a decay-only step must scale every element alike"
    x = (w.g + w.meta["dt_bias"][None, :]).double().numpy()
    g = -np.exp(w.meta["A_log"].double().numpy())[None, :] * np.log1p(np.exp(x))
    ref = np.exp(g)
    err = np.abs(got - ref) / ref
    bound = 2e-6 + 4e-6 * np.abs(g)
    say("decay from logits in [-30, -5]: max rel err %.3e (|g| up to %.1f)" % (err.max(), np.abs(g).max()))
    assert (err <= bound).all(), "decay error %.3e at g=%.3e" % (err.max(), g.flat[int(np.argmax(err / bound))])
