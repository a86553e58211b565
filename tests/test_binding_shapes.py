"""The Python binding refuses tensors whose shapes do not match each other, before
anything reaches the C ABI.

The ABI sizes every buffer from the dimensions it is given (T and N from q and
cu_seqlens, heads and head dims from q and v), so a k, g, beta, h0, hT, out,
pool or index array of another shape would be read or written past its end.
These checks run on host tensors: the shape checks come before the device and
dtype checks and before the library is touched, so nothing here needs a GPU.
"""
import pytest
import torch

from invariant_linear_attention_amd import gdn

T, N, HK, HV, DK, DV = 10, 2, 2, 4, 16, 32


def batch():
    bf = dict(dtype=torch.bfloat16)
    return dict(q=torch.zeros((T, HK, DK), **bf), k=torch.zeros((T, HK, DK), **bf), v=torch.zeros((T, HV, DV), **bf),
                g=torch.zeros((T, HV)), beta=torch.zeros((T, HV)), h0=torch.zeros((N, HV, DV, DK)),
                cu_seqlens=torch.tensor([0, 4, T], dtype=torch.int32))


WRONG = {
    "k": torch.zeros((T, HK + 1, DK), dtype=torch.bfloat16),
    "v": torch.zeros((T - 1, HV, DV), dtype=torch.bfloat16),
    "g": torch.zeros((T, HK)),
    "beta": torch.zeros((T + 1, HV)),
    "h0": torch.zeros((N, HV, DV, DK + 1)),
    "cu_seqlens": torch.zeros((1, N + 1), dtype=torch.int32),
}


def expect_shape_error(fn, *a, **kw):
    with pytest.raises(ValueError) as e:
        fn(*a, **kw)
    assert "must" in str(e.value) or "required" in str(e.value)


@pytest.mark.parametrize("name", sorted(WRONG))
def test_fwd_varlen_refuses(name):
    b = batch()
    b[name] = WRONG[name]
    expect_shape_error(gdn.gdn_fwd_varlen, b["q"], b["k"], b["v"], b["g"], b["beta"], b["h0"], b["cu_seqlens"])


@pytest.mark.parametrize("which,shape", [("out", (T, HV, DV + 16)), ("hT", (N + 1, HV, DV, DK))])
def test_fwd_varlen_refuses_outputs(which, shape):
    b = batch()
    kw = {which: torch.zeros(shape, dtype=torch.bfloat16 if which == "out" else torch.float32)}
    expect_shape_error(gdn.gdn_fwd_varlen, b["q"], b["k"], b["v"], b["g"], b["beta"], b["h0"], b["cu_seqlens"], **kw)


def test_fwd_varlen_train_refuses_saved_p():
    b = batch()
    expect_shape_error(gdn.gdn_fwd_varlen_train, b["q"], b["k"], b["v"], b["g"], b["beta"], b["h0"], b["cu_seqlens"],
                       saved_p=torch.zeros((T, HV, DK + 1)))


@pytest.mark.parametrize("name", sorted(WRONG))
def test_pool_refuses(name):
    b = batch()
    b[name] = WRONG[name]
    pool = torch.zeros((3, HV, DV, DK))
    expect_shape_error(gdn.gdn_fwd_varlen_pool, b["q"], b["k"], b["v"], b["g"], b["beta"], b["cu_seqlens"], pool)


@pytest.mark.parametrize("kw", [
    dict(state_pool=torch.zeros((3, HV, DK, DV + 16))),
    dict(src_idx=torch.zeros((N + 1,), dtype=torch.int32)),
    dict(dst_idx=torch.zeros((N, 1), dtype=torch.int32)),
    dict(pos0=torch.zeros((1,), dtype=torch.int32)),
])
def test_pool_refuses_pool_and_indices(kw):
    b = batch()
    pool = kw.pop("state_pool", torch.zeros((3, HV, DV, DK)))
    expect_shape_error(gdn.gdn_fwd_varlen_pool, b["q"], b["k"], b["v"], b["g"], b["beta"], b["cu_seqlens"], pool, **kw)


def decode_args(B=3):
    bf = dict(dtype=torch.bfloat16)
    return [torch.zeros((B, HK, DK), **bf), torch.zeros((B, HK, DK), **bf), torch.zeros((B, HV, DV), **bf),
            torch.zeros((B, HV)), torch.zeros((B, HV)), torch.zeros((5, HV, DV, DK))]


@pytest.mark.parametrize("pos,bad", [
    (1, torch.zeros((3, HK, DK + 16), dtype=torch.bfloat16)),
    (2, torch.zeros((2, HV, DV), dtype=torch.bfloat16)),
    (3, torch.zeros((3, HK))),
    (4, torch.zeros((3, HV, 1))),
    (5, torch.zeros((5, HV, DV, DK + 4))),
])
def test_decode_refuses(pos, bad):
    a = decode_args()
    a[pos] = bad
    expect_shape_error(gdn.gdn_decode_step, *a)


@pytest.mark.parametrize("kw", [dict(state_idx=torch.zeros((2,), dtype=torch.int32)),
                                dict(out=torch.zeros((3, HV, DK + 16), dtype=torch.bfloat16))])
def test_decode_refuses_index_and_out(kw):
    expect_shape_error(gdn.gdn_decode_step, *decode_args(), **kw)


def test_preproc_arrays_must_cover_every_value_head():
    b = batch()
    pre = gdn.GdnPreproc(flags=gdn.GDN_PRE_GATE_LOGITS, eps=1e-6, A_log=None, dt_bias=None)
    pre._keep = (torch.zeros((HV - 1,)), None)
    expect_shape_error(gdn.gdn_fwd_varlen, b["q"], b["k"], b["v"], b["g"], b["beta"], b["h0"], b["cu_seqlens"], pre=pre)


@pytest.mark.parametrize("name,shape", [("dout", (T, HV, DV + 1)), ("dhT", (N, HV, DV, 1)), ("saved_p", (1, HV, DV)),
                                        ("hT", (N, HV + 1, DV, DK))])
def test_backward_refuses(name, shape):
    b = batch()
    kw = dict(dout=torch.zeros((T, HV, DV), dtype=torch.bfloat16))
    kw[name] = torch.zeros(shape, dtype=torch.bfloat16 if name == "dout" else torch.float32)
    dout = kw.pop("dout")
    expect_shape_error(gdn.gdn_bwd_varlen, b["q"], b["k"], b["v"], b["g"], b["beta"], b["h0"], b["cu_seqlens"], dout,
                       **kw)


def test_backward_refuses_gradient_buffers():
    b = batch()
    f = torch.zeros
    grads = {"dq": f((T, HK, DK)), "dk": f((T, HK, DK)), "dv": f((T, HV, DV)), "dg": f((T, HV)),
             "dbeta": f((T, HV, 1)), "dh0": None}
    expect_shape_error(gdn.gdn_bwd_varlen, b["q"], b["k"], b["v"], b["g"], b["beta"], b["h0"], b["cu_seqlens"],
                       torch.zeros((T, HV, DV), dtype=torch.bfloat16), grads=grads)


def test_chunked_refuses_state_shapes():
    b = batch()
    st = {"S": torch.zeros((N, HV, DV, DK)), "k": torch.zeros((N, 16, HK, DK)), "r": torch.zeros((N, 16, HV, DV)),
          "a": torch.zeros((N, 16, HV)), "b": torch.zeros((N, 16, HV)), "count": torch.zeros((N,), dtype=torch.int32)}
    for name, shape in (("S", (N, HV, DV, DK * 2)), ("k", (N, 8, HK, DK)), ("r", (N, 16, HK, DV)),
                        ("a", (N, 16)), ("b", (N, 17, HV)), ("count", (N + 1,))):
        bad = dict(st)
        bad[name] = torch.zeros(shape, dtype=st[name].dtype)
        expect_shape_error(gdn.gdn_fwd_chunked, b["q"], b["k"], b["v"], b["g"], b["beta"], b["cu_seqlens"], bad)


@pytest.mark.parametrize("kw", [dict(bias=torch.zeros((7,))), dict(src_idx=torch.zeros((3,), dtype=torch.int32)),
                                dict(y=torch.zeros((T, 16), dtype=torch.bfloat16))])
def test_short_conv_refuses(kw):
    C, K = 32, 4
    x = torch.zeros((T, C), dtype=torch.bfloat16)
    w = torch.zeros((C, K))
    pool = torch.zeros((N, C, K - 1), dtype=torch.bfloat16)
    expect_shape_error(gdn.gdn_short_conv, x, w, torch.tensor([0, 4, T], dtype=torch.int32), pool, **kw)


def test_short_conv_refuses_state_pool():
    C, K = 32, 4
    expect_shape_error(gdn.gdn_short_conv, torch.zeros((T, C), dtype=torch.bfloat16), torch.zeros((C, K)),
                       torch.tensor([0, 4, T], dtype=torch.int32), torch.zeros((N, C, K), dtype=torch.bfloat16))


def test_matching_shapes_pass_the_shape_checks():
    """With every shape right, the call gets past the shape checks and stops at the
    first device check (host tensors), so the checks above are what refused."""
    b = batch()
    with pytest.raises(ValueError, match="device tensor"):
        gdn.gdn_fwd_varlen(b["q"], b["k"], b["v"], b["g"], b["beta"], b["h0"], b["cu_seqlens"])
    with pytest.raises(ValueError, match="device tensor"):
        gdn.gdn_decode_step(*decode_args())


@pytest.mark.parametrize("name,shape", [("dout", (T, HV, DV + 1)), ("dhT", (N, HV, DV, 1)), ("h0", (N, HV, 1, DK))])
def test_chunked_backward_refuses(name, shape):
    b = batch()
    kw = dict(dout=torch.zeros((T, HV, DV), dtype=torch.bfloat16), dhT=None)
    if name == "h0":
        b["h0"] = torch.zeros(shape)
    else:
        kw[name] = torch.zeros(shape, dtype=torch.bfloat16 if name == "dout" else torch.float32)
    expect_shape_error(gdn.gdn_bwd_chunked, b["q"], b["k"], b["v"], b["g"], b["beta"], b["h0"], b["cu_seqlens"],
                       kw["dout"], kw["dhT"])


def test_chunked_backward_refuses_gradient_buffers():
    b = batch()
    f = torch.zeros
    grads = {"dq": f((T, HK, DK)), "dk": f((T, HK, DK + 4)), "dv": f((T, HV, DV)), "dg": f((T, HV)),
             "dbeta": f((T, HV)), "dh0": None}
    expect_shape_error(gdn.gdn_bwd_chunked, b["q"], b["k"], b["v"], b["g"], b["beta"], b["h0"], b["cu_seqlens"],
                       torch.zeros((T, HV, DV), dtype=torch.bfloat16), grads=grads)


# ------------------------------------------------ the fused layer's training passes

def expect_shape_only(fn, *a, **kw):
    """A shape error, raised before the device checks (which CPU tensors would fail)."""
    with pytest.raises(ValueError) as e:
        fn(*a, **kw)
    msg = str(e.value)
    assert ("must" in msg or "required" in msg) and "device tensor" not in msg, msg


def pre_inputs():
    bf = dict(dtype=torch.bfloat16)
    return dict(q=torch.zeros((T, HK, DK), **bf), k=torch.zeros((T, HK, DK), **bf), a=torch.zeros((T, HV)),
                b=torch.zeros((T, HV)))


def gated_pre(n=HV):
    pre = gdn.GdnPreproc(flags=gdn.GDN_PRE_QK_L2NORM | gdn.GDN_PRE_GATE_LOGITS, eps=1e-6)
    pre._keep = (torch.zeros((n,)), None)
    return pre


PRE_WRONG = {"k": torch.zeros((T, HK, DK + 1), dtype=torch.bfloat16), "a": torch.zeros((T - 1, HV)),
             "b": torch.zeros((T, HV + 1)), "q": torch.zeros((T, HK * DK), dtype=torch.bfloat16)}


@pytest.mark.parametrize("name", sorted(PRE_WRONG))
def test_preprocess_refuses(name):
    i = pre_inputs()
    i[name] = PRE_WRONG[name]
    expect_shape_only(gdn.gdn_preprocess, i["q"], i["k"], i["a"], i["b"], pre=gated_pre())


def test_preprocess_refuses_outputs_and_parameters():
    i = pre_inputs()
    out = {"qn": torch.zeros((T, HK, DK)), "kn": torch.zeros((T, HK, DK)), "g": torch.zeros((T, HV)),
           "beta": torch.zeros((T, HV + 1))}
    expect_shape_only(gdn.gdn_preprocess, i["q"], i["k"], i["a"], i["b"], pre=gated_pre(), out=out)
    del out["beta"]
    expect_shape_only(gdn.gdn_preprocess, i["q"], i["k"], i["a"], i["b"], pre=gated_pre(), out=out)
    expect_shape_only(gdn.gdn_preprocess, i["q"], i["k"], i["a"], i["b"], pre=gated_pre(HV + 1))


@pytest.mark.parametrize("which,shape", [("dqn", (T, HK, DK + 1)), ("dkn", (T + 1, HK, DK)), ("dg", (T, HK)),
                                         ("dbeta", (T, HV, 1))])
def test_preprocess_backward_refuses(which, shape):
    i = pre_inputs()
    g = {"dqn": torch.zeros((T, HK, DK)), "dkn": torch.zeros((T, HK, DK)), "dg": torch.zeros((T, HV)),
         "dbeta": torch.zeros((T, HV))}
    g[which] = torch.zeros(shape)
    expect_shape_only(gdn.gdn_preprocess_backward, i["q"], i["k"], i["a"], i["b"], g["dqn"], g["dkn"], g["dg"],
                      g["dbeta"], pre=gated_pre())


@pytest.mark.parametrize("which,shape", [("dq", (T, HK, DK - 1)), ("da", (T, HV + 1)), ("dA_log", (HV + 1,)),
                                         ("db", None)])
def test_preprocess_backward_refuses_gradient_buffers(which, shape):
    i = pre_inputs()
    grads = {"dq": torch.zeros((T, HK, DK)), "dk": torch.zeros((T, HK, DK)), "da": torch.zeros((T, HV)),
             "db": torch.zeros((T, HV)), "dA_log": torch.zeros((HV,)), "ddt_bias": None}
    grads[which] = None if shape is None else torch.zeros(shape)
    expect_shape_only(gdn.gdn_preprocess_backward, i["q"], i["k"], i["a"], i["b"], torch.zeros((T, HK, DK)),
                      torch.zeros((T, HK, DK)), torch.zeros((T, HV)), torch.zeros((T, HV)), pre=gated_pre(),
                      grads=grads)


C, K = 24, 4


def conv_inputs():
    return dict(x=torch.zeros((T, C), dtype=torch.bfloat16), w=torch.zeros((C, K)),
                cu_seqlens=torch.tensor([0, 4, T], dtype=torch.int32),
                state_pool=torch.zeros((3, C, K - 1), dtype=torch.bfloat16), dy=torch.zeros((T, C)),
                bias=torch.zeros((C,)))


CONV_WRONG = {"w": torch.zeros((C + 1, K)), "dy": torch.zeros((T, C + 4)), "bias": torch.zeros((C - 1,)),
              "state_pool": torch.zeros((3, C, K)), "cu_seqlens": torch.zeros((1, N + 1), dtype=torch.int32),
              "src_idx": torch.zeros((N + 1,), dtype=torch.int32)}


@pytest.mark.parametrize("name", sorted(CONV_WRONG))
def test_conv_backward_refuses(name):
    i = conv_inputs()
    i["src_idx"] = None
    i[name] = CONV_WRONG[name]
    expect_shape_only(gdn.gdn_short_conv_backward, i["x"], i["w"], i["cu_seqlens"], i["state_pool"], i["dy"],
                      bias=i["bias"], src_idx=i["src_idx"])


@pytest.mark.parametrize("which,shape", [("dx", (T, C + 1)), ("dw", (C, K + 1)), ("dstate", (N, C, K)),
                                         ("dx", None)])
def test_conv_backward_refuses_gradient_buffers(which, shape):
    i = conv_inputs()
    grads = {"dx": torch.zeros((T, C)), "dw": torch.zeros((C, K)), "dbias": torch.zeros((C,)),
             "dstate": torch.zeros((N, C, K - 1))}
    grads[which] = None if shape is None else torch.zeros(shape)
    expect_shape_only(gdn.gdn_short_conv_backward, i["x"], i["w"], i["cu_seqlens"], i["state_pool"], i["dy"],
                      bias=i["bias"], grads=grads)
