"""Backward of the short causal convolution (gdn_short_conv_backward).

Parity: every gradient (inputs, taps, bias, carried state) against the fp64
oracle (oracle.short_conv_backward, pinned by exactly representable finite
differences and the adjoint identity), normwise 1e-5: the GPU recomputes z in the
forward's fp32 order and sums in fp32.  dx and dstate depend only on their own
sequence (tested bitwise alone vs in a batch); dw and dbias sum over the call's
tokens in a fixed order (repeat bitwise).
"""
import numpy as np
import pytest
import torch

from gpu_helpers import say
from invariant_linear_attention_amd import synth

pytestmark = pytest.mark.gpu
DEV = "cuda"


def case(seed, lengths, C, K, io=torch.bfloat16):
    gen = torch.Generator().manual_seed(seed)
    T = sum(lengths)
    x = torch.randn((T, C), generator=gen).to(io)
    w = (torch.randn((C, K), generator=gen) * 0.5).float()
    bias = (torch.randn((C,), generator=gen) * 0.1).float()
    state = torch.randn((len(lengths), C, K - 1), generator=gen).to(io)
    dy = torch.randn((T, C), generator=gen).float()
    return x, w, bias, state, dy, synth.cu_from_lengths(lengths)


def rel(x, r):
    x = np.asarray(x, dtype=np.float64)
    r = np.asarray(r, dtype=np.float64)
    return float(np.linalg.norm(x - r) / max(np.linalg.norm(r), 1e-300))


def run(gdn, x, w, bias, state, dy, cu, silu=True, src=None):
    r = gdn.gdn_short_conv_backward(x.to(DEV), w.to(DEV), cu.to(DEV), state.to(DEV), dy.to(DEV),
                                    bias=None if bias is None else bias.to(DEV), src_idx=src, silu=silu)
    torch.cuda.synchronize()
    return r


@pytest.mark.parametrize("K", [2, 4, 8])
@pytest.mark.parametrize("io", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("silu", [True, False])
def test_parity(gpu, K, io, silu):
    from oracle import oracle
    # lengths: shorter than K - 1, empty, one token, across 64-token blocks
    lengths = [37, 1, 2, 0, 150, 9, 64]
    x, w, bias, state, dy, cu = case(17 + K, lengths, C=320, K=K, io=io)
    r = run(gpu, x, w, bias, state, dy, cu, silu=silu)
    ref = oracle.short_conv_backward(x, w, cu, dy, bias=bias, state=state, silu=silu)
    errs = {k: rel(r[k].cpu(), ref[k]) for k in ("dx", "dw", "dbias", "dstate")}
    say("conv backward K=%d %s silu=%s: %s" % (K, io, silu, errs))
    for k, e in errs.items():
        assert e <= 1e-5, (k, e)


@pytest.mark.parametrize("io", [torch.bfloat16, torch.float32])
def test_channels_off_the_four_channel_grid(gpu, io):
    """A channel count that is no multiple of four takes the one-channel-a-thread
    kernel; it gives the same gradients."""
    from oracle import oracle
    lengths = [37, 1, 0, 150, 3]
    x, w, bias, state, dy, cu = case(23, lengths, C=13, K=4, io=io)
    r = run(gpu, x, w, bias, state, dy, cu)
    ref = oracle.short_conv_backward(x, w, cu, dy, bias=bias, state=state, silu=True)
    for k in ("dx", "dw", "dbias", "dstate"):
        assert rel(r[k].cpu(), ref[k]) <= 1e-5, k


def test_slots_no_bias_and_no_state_gradient(gpu):
    """src_idx picks state slots (an out-of-range entry is the zero state); without
    bias and dstate only dx and dw are written."""
    from oracle import oracle
    C, K = 64, 4
    lengths = [5, 70, 2]
    x, w, bias, state, dy, cu = case(31, lengths, C=C, K=K)
    pool = torch.randn((6, C, K - 1), generator=torch.Generator().manual_seed(5)).to(torch.bfloat16)
    src = torch.tensor([4, -1, 1], dtype=torch.int32)
    eff = torch.zeros((3, C, K - 1), dtype=torch.bfloat16)
    eff[0], eff[2] = pool[4], pool[1]
    r = gpu.gdn_short_conv_backward(x.to(DEV), w.to(DEV), cu.to(DEV), pool.to(DEV), dy.to(DEV),
                                    src_idx=src.to(DEV), want_dstate=False)
    torch.cuda.synchronize()
    assert r["dbias"] is None and r["dstate"] is None
    ref = oracle.short_conv_backward(x, w, cu, dy, bias=None, state=eff, silu=True)
    for k in ("dx", "dw"):
        assert rel(r[k].cpu(), ref[k]) <= 1e-5, k


def test_alone_vs_batch_and_repeat(gpu):
    C, K = 128, 4
    lengths = [70, 3, 130]
    x, w, bias, state, dy, cu = case(41, lengths, C=C, K=K)
    r1 = run(gpu, x, w, bias, state, dy, cu)
    r2 = run(gpu, x, w, bias, state, dy, cu)
    for k in r1:
        assert torch.equal(r1[k], r2[k]), k
    c = cu.tolist()
    for n in range(3):
        a, b = c[n], c[n + 1]
        rs = run(gpu, x[a:b].contiguous(), w, bias, state[n:n + 1].contiguous(), dy[a:b].contiguous(),
                 torch.tensor([0, b - a], dtype=torch.int32))
        assert torch.equal(rs["dx"], r1["dx"][a:b]), n
        assert torch.equal(rs["dstate"][0], r1["dstate"][n]), n
    say("conv backward: repeat bitwise; dx and dstate alone = in the batch")


def test_benchmark_shape_sampled(gpu):
    """The benchmark batch's q|k|v channels (8192 x 17,459 tokens, K = 4): every
    gradient of the first 256 channels against the oracle."""
    from oracle import oracle
    w0 = synth.varlen_prefill(1001)
    cu = w0.cu_seqlens
    T, C, K = int(cu[-1]), 8192, 4
    gen = torch.Generator().manual_seed(1007)
    x = torch.randn((T, C), generator=gen).to(torch.bfloat16)
    w = (0.5 * torch.randn((C, K), generator=gen)).float()
    bias = (0.1 * torch.randn((C,), generator=gen)).float()
    state = torch.randn((w0.n_seqs, C, K - 1), generator=gen).to(torch.bfloat16)
    dy = torch.randn((T, C), generator=gen).float()
    r = run(gpu, x, w, bias, state, dy, cu)
    sl = slice(0, 256)
    ref = oracle.short_conv_backward(x[:, sl].contiguous(), w[sl].contiguous(), cu, dy[:, sl].contiguous(),
                                     bias=bias[sl].contiguous(), state=state[:, sl].contiguous())
    errs = {"dx": rel(r["dx"][:, sl].cpu(), ref["dx"]), "dw": rel(r["dw"][sl].cpu(), ref["dw"]),
            "dbias": rel(r["dbias"][sl].cpu(), ref["dbias"]), "dstate": rel(r["dstate"][:, sl].cpu(), ref["dstate"])}
    say("conv backward benchmark shape, first 256 channels: %s" % errs)
    for k, e in errs.items():
        assert e <= 1e-5, (k, e)
