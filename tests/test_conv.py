"""The short causal convolution with a carried state (gdn_short_conv).

Parity: y against the fp64 oracle (bf16 within one ulp of the rounded oracle
value, normwise within the output gate), the new state exactly.  Invariance: every
output depends only on its own sequence, so decode (one token per sequence),
cutting a sequence, batch-mates and in-place state updates change no bit.
End to end: convolution, then the recurrence with fused preprocessing, against
the same chain in fp64.
"""
import numpy as np
import pytest
import torch

from gpu_helpers import bf16_ulp_distance, bit_equal, check_parity, say, seq_errors
from invariant_linear_attention_amd import synth

pytestmark = pytest.mark.gpu
DEV = "cuda"


def conv_case(seed, lengths, C, K, io=torch.bfloat16):
    gen = torch.Generator().manual_seed(seed)
    T = sum(lengths)
    x = torch.randn((T, C), generator=gen).to(io)
    w = (torch.randn((C, K), generator=gen) * 0.5).float()
    bias = (torch.randn((C,), generator=gen) * 0.1).float()
    state = torch.randn((len(lengths), C, K - 1), generator=gen).to(io)
    cu = synth.cu_from_lengths(lengths)
    return x, w, bias, state, cu


def gpu_conv(gdn, x, w, bias, state, cu, silu=True, src=None, dst=None):
    pool = state.to(DEV).clone()
    y = gdn.gdn_short_conv(x.to(DEV), w.to(DEV), cu.to(DEV), pool, bias=None if bias is None else bias.to(DEV),
                           src_idx=src, dst_idx=dst, silu=silu)
    torch.cuda.synchronize()
    return y, pool


@pytest.mark.parametrize("K", [2, 4, 8])
@pytest.mark.parametrize("io", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("silu", [True, False])
def test_parity(gpu, K, io, silu):
    from oracle import oracle
    lengths = [37, 1, 2, 0, 100, 9]
    x, w, bias, state, cu = conv_case(7 + K, lengths, C=320, K=K, io=io)
    y, pool = gpu_conv(gpu, x, w, bias, state, cu, silu=silu)
    ry, rs = oracle.short_conv(x, w, cu, bias=bias, state=state, silu=silu)
    errs = seq_errors(y.float().cpu().numpy(), ry, cu.tolist())
    tol = 2e-3 if io == torch.bfloat16 else 1e-5
    say("conv K=%d %s silu=%s: max normwise %.2e" % (K, io, silu, max(errs)))
    assert max(errs) <= tol
    if io == torch.bfloat16:
        ulp, _ = bf16_ulp_distance(y, ry)
        assert ulp <= 1
    assert np.array_equal(pool.float().cpu().numpy().astype(np.float64), rs)   # the state holds inputs exactly


def test_chunked_decode_and_batch(gpu):
    C, K = 192, 4
    lengths = [50, 7, 33]
    x, w, bias, state, cu = conv_case(21, lengths, C, K)
    y_ref, pool_ref = gpu_conv(gpu, x, w, bias, state, cu)
    cuL = cu.tolist()
    # alone vs in the batch
    for n in range(len(lengths)):
        xs = x[cuL[n]:cuL[n + 1]]
        y1, p1 = gpu_conv(gpu, xs, w, bias, state[n:n + 1], synth.cu_from_lengths([lengths[n]]))
        assert bit_equal(y1, y_ref[cuL[n]:cuL[n + 1]]) and bit_equal(p1[0], pool_ref[n]), n
    # sequence 0 cut into calls (1-token calls are decode steps), state in place
    xs = x[:50].to(DEV)
    pool = state[0:1].to(DEV).clone()
    parts = []
    for a, b in ((0, 1), (1, 2), (2, 19), (19, 49), (49, 50)):
        parts.append(gpu.gdn_short_conv(xs[a:b].contiguous(), w.to(DEV), synth.cu_from_lengths([b - a]).to(DEV),
                                        pool, bias=bias.to(DEV)))
    torch.cuda.synchronize()
    assert bit_equal(torch.cat(parts), y_ref[:50]) and bit_equal(pool[0], pool_ref[0])
    # decode batch: the first token of every sequence at once, rows in a permuted
    # order, each row reading and updating its own sequence's slot
    B = 3
    pool = state.to(DEV).clone()
    order = (2, 0, 1)
    idx = torch.tensor(order, dtype=torch.int32, device=DEV)
    xt = torch.stack([x[cuL[n]] for n in order]).to(DEV)
    yt = gpu.gdn_short_conv(xt, w.to(DEV), synth.cu_from_lengths([1] * B).to(DEV), pool, bias=bias.to(DEV),
                            src_idx=idx, dst_idx=idx)
    torch.cuda.synchronize()
    for row, n in enumerate(order):
        assert bit_equal(yt[row], y_ref[cuL[n]]), n
        one, p1 = gpu_conv(gpu, x[cuL[n]:cuL[n] + 1], w, bias, state[n:n + 1], synth.cu_from_lengths([1]))
        assert bit_equal(pool[n], p1[0]), n


def test_slots_none_and_out_of_place(gpu):
    C, K = 64, 4
    x, w, bias, state, cu = conv_case(31, [5, 3], C, K)
    pool = torch.zeros((4, C, K - 1), dtype=torch.bfloat16, device=DEV)
    pool[1] = state[0].to(DEV)
    pool[2] = state[1].to(DEV)
    before = pool.clone()
    y = gpu.gdn_short_conv(x.to(DEV), w.to(DEV), cu.to(DEV), pool, bias=bias.to(DEV),
                           src_idx=torch.tensor([1, -1], dtype=torch.int32, device=DEV),
                           dst_idx=torch.tensor([3, 9], dtype=torch.int32, device=DEV))
    torch.cuda.synchronize()
    st = state.clone()
    st[1] = 0
    y_ref, p_ref = gpu_conv(gpu, x, w, bias, st, cu)
    assert bit_equal(y, y_ref) and bit_equal(pool[3], p_ref[0]) and bit_equal(pool[:3], before[:3])


def test_layer_end_to_end(gpu):
    """conv -> split into q, k, v -> recurrence with in-kernel L2 norm and gate from
    logits, against the same chain in fp64 (the oracle rounds its conv output to
    bf16 as the layer's forward does)."""
    from oracle import oracle
    hk, hv, dk, dv, K = 2, 4, 64, 64, 4
    lengths = [40, 1, 23]
    C = 2 * hk * dk + hv * dv
    x, w, bias, state, cu = conv_case(41, lengths, C, K)
    raw = synth.make_raw_workload(42, lengths, hk=hk, hv=hv, dk=dk, dv=dv, h0_std=0.1)
    y, _ = gpu_conv(gpu, x, w, bias, state, cu)
    T = sum(lengths)
    q = y[:, :hk * dk].reshape(T, hk, dk).contiguous()
    k = y[:, hk * dk:2 * hk * dk].reshape(T, hk, dk).contiguous()
    v = y[:, 2 * hk * dk:].reshape(T, hv, dv).contiguous()
    A, D = raw.meta["A_log"].to(DEV), raw.meta["dt_bias"].to(DEV)
    pre = gpu.make_preproc(norm_qk=True, eps=1e-6, A_log=A, dt_bias=D)
    out, hT = gpu.gdn_fwd_varlen(q, k, v, raw.g.to(DEV), raw.beta.to(DEV), raw.h0.to(DEV), cu.to(DEV), pre=pre)
    torch.cuda.synchronize()
    ry, _ = oracle.short_conv(x, w, cu, bias=bias, state=state)
    yb = torch.from_numpy(ry).float().to(torch.bfloat16)          # the forward's bf16 activations
    rq = yb[:, :hk * dk].reshape(T, hk, dk).contiguous()
    rk = yb[:, hk * dk:2 * hk * dk].reshape(T, hk, dk).contiguous()
    rv = yb[:, 2 * hk * dk:].reshape(T, hv, dv).contiguous()
    ro, rh = oracle.gdn_forward_fused(rq, rk, rv, raw.g, raw.beta, cu, raw.h0, A_log=raw.meta["A_log"],
                                      dt_bias=raw.meta["dt_bias"])
    ref = synth.Workload(rq, rk, rv, raw.g, raw.beta, cu, raw.h0)
    check_parity(ref, out, hT, ro, rh, label="layer end to end")
