"""Bitwise GPU-vs-GPU invariance of the recurrent forward.

The order follows the verification ladder of the page "Train-inference
consistency" summary (a request alone vs in mixed batches first, then whole
prefill vs token-by-token decode) and the bitwise goals of the page "Defending
Against the Training-Inference Numeric Mismatch in RL (Especially Linear
Attention)" (sections 2 and 3.2): a sequence's outputs and final state must not
change by a single bit with its batch-mates, its position in the batch, the
launch shape, the chunking of its prefill, or whether its tokens arrive by
prefill or by decode.
"""
import itertools

import pytest
import torch

from gpu_helpers import bit_equal, run_prefill, say, to_dev
from invariant_linear_attention_amd import synth

pytestmark = pytest.mark.gpu
DEV = "cuda"


def seq_rows(w, n):
    cu = w.cu_seqlens.tolist()
    return slice(cu[n], cu[n + 1])


def small_batch(seed=5, lengths=(37, 1, 160, 0, 64, 17, 300, 2), h0=0.1):
    return synth.make_workload(seed, list(lengths), hk=4, hv=8, dk=128, dv=128, h0_std=h0)


def test_run_to_run(gpu):
    w = small_batch()
    o1, s1 = run_prefill(gpu, w)
    o2, s2 = run_prefill(gpu, w)
    assert bit_equal(o1, o2) and bit_equal(s1, s2)


def test_alone_vs_in_batch(gpu):
    w = small_batch()
    ob, sb = run_prefill(gpu, w)
    for n in range(w.n_seqs):
        a = synth.select(w, [n])
        oa, sa = run_prefill(gpu, a)
        assert bit_equal(oa, ob[seq_rows(w, n)]), "sequence %d output changed in the batch" % n
        assert bit_equal(sa[0], sb[n]), "sequence %d state changed in the batch" % n


PLANS = [(4, 1, 1), (4, 1, 2), (4, 1, 4), (4, 2, 1), (4, 2, 2), (4, 2, 4), (4, 4, 1), (4, 4, 2),
         (8, 1, 1), (8, 1, 2), (8, 1, 4), (8, 1, 8), (8, 2, 1), (8, 2, 2), (8, 2, 4),
         (16, 1, 2), (16, 1, 4), (16, 2, 1), (16, 2, 2), (16, 2, 4), (16, 2, 8),
         (16, 4, 1), (16, 4, 2), (16, 4, 4), (0, 0, 0)]


def test_every_launch_shape_gives_the_same_bits(gpu):
    """Lanes per row, rows per lane and waves per workgroup move rows around the
    chip; none of them may change a bit."""
    w = small_batch()
    ref_o, ref_s = run_prefill(gpu, w, plan=(4, 1, 1))
    for plan in PLANS:
        o, s = run_prefill(gpu, w, plan=plan)
        assert bit_equal(o, ref_o) and bit_equal(s, ref_s), "plan %s changed the bits" % (plan,)


def test_launch_shapes_dk64(gpu):
    w = synth.make_workload(6, [33, 0, 70], hk=2, hv=4, dk=64, dv=64, h0_std=0.1)
    ref_o, ref_s = run_prefill(gpu, w, plan=(4, 1, 1))
    for plan in [(4, 2, 2), (8, 1, 1), (8, 2, 4), (0, 0, 0)]:
        o, s = run_prefill(gpu, w, plan=plan)
        assert bit_equal(o, ref_o) and bit_equal(s, ref_s), "plan %s changed the bits" % (plan,)


def test_grouped_heads_equal_duplicated_key_heads(gpu):
    w = small_batch(lengths=(50, 9))
    o, s = run_prefill(gpu, w)
    d = synth.Workload(w.q.repeat_interleave(2, dim=1).contiguous(), w.k.repeat_interleave(2, dim=1).contiguous(),
                       w.v, w.g, w.beta, w.cu_seqlens, w.h0)
    o2, s2 = run_prefill(gpu, d)
    assert bit_equal(o, o2) and bit_equal(s, s2)


def test_in_place_state(gpu):
    w = small_batch()
    o, s = run_prefill(gpu, w)
    d = to_dev(w)
    st = d["h0"].clone()
    o2, s2 = gpu.gdn_fwd_varlen(d["q"], d["k"], d["v"], d["g"], d["beta"], st, d["cu_seqlens"], hT=st)
    torch.cuda.synchronize()
    assert s2.data_ptr() == st.data_ptr()
    assert bit_equal(o, o2) and bit_equal(s, st)


def test_empty_sequence_passes_state_through(gpu):
    w = small_batch(lengths=(0, 5, 0))
    o, s = run_prefill(gpu, w)
    assert bit_equal(s[0], w.h0[0].to(DEV)) and bit_equal(s[2], w.h0[2].to(DEV))
    wz = small_batch(lengths=(0,), h0=0.0)
    _, sz = run_prefill(gpu, wz)
    assert torch.count_nonzero(sz) == 0


def _chunked(gpu, w, cuts, d=None):
    """Run a one-sequence workload as consecutive calls split at `cuts`, carrying hT -> h0."""
    d = d if d is not None else to_dev(w)
    state = d["h0"]
    outs = []
    for a, b in zip(cuts[:-1], cuts[1:]):
        cu = torch.tensor([0, b - a], dtype=torch.int32, device=DEV)
        o, state = gpu.gdn_fwd_varlen(d["q"][a:b].contiguous(), d["k"][a:b].contiguous(), d["v"][a:b].contiguous(),
                                      d["g"][a:b].contiguous(), d["beta"][a:b].contiguous(), state, cu)
        outs.append(o)
    torch.cuda.synchronize()
    return torch.cat(outs), state


@pytest.mark.parametrize("cuts", [[0, 1, 300], [0, 15, 16, 17, 33, 300], [0, 128, 129, 255, 300], [0, 299, 300]])
def test_chunked_prefill_is_bitwise_unchunked(gpu, cuts):
    w = synth.make_workload(9, [300], hk=2, hv=4, dk=128, dv=128, h0_std=0.1)
    o, s = run_prefill(gpu, w)
    oc, sc = _chunked(gpu, w, cuts)
    assert bit_equal(o, oc) and bit_equal(s, sc[0:1] if sc.dim() == 4 else sc)


def test_prefill_then_decode_is_bitwise_full_prefill(gpu):
    """Prefill 40 tokens, then decode 25 tokens one step at a time through the pool
    entry of that sequence; every output and the final state equal a 65-token prefill."""
    w = synth.make_workload(10, [65, 65, 65], hk=2, hv=4, dk=128, dv=128, h0_std=0.1)
    o_full, s_full = run_prefill(gpu, w)
    d = to_dev(w)
    cu = w.cu_seqlens.tolist()
    idx_pre = torch.cat([torch.arange(cu[n], cu[n] + 40) for n in range(3)]).to(DEV)
    cu_pre = torch.tensor([0, 40, 80, 120], dtype=torch.int32, device=DEV)
    o_pre, st = gpu.gdn_fwd_varlen(d["q"][idx_pre].contiguous(), d["k"][idx_pre].contiguous(),
                                   d["v"][idx_pre].contiguous(), d["g"][idx_pre].contiguous(),
                                   d["beta"][idx_pre].contiguous(), d["h0"], cu_pre)
    # scatter the three states into a larger pool at permuted slots
    pool = torch.zeros((7,) + tuple(st.shape[1:]), dtype=torch.float32, device=DEV)
    slots = torch.tensor([5, 0, 3], dtype=torch.int32, device=DEV)
    pool[slots.long()] = st
    outs = []
    for t in range(40, 65):
        rows = torch.tensor([cu[n] + t for n in range(3)], device=DEV)
        outs.append(gpu.gdn_decode_step(d["q"][rows].contiguous(), d["k"][rows].contiguous(),
                                        d["v"][rows].contiguous(), d["g"][rows].contiguous(),
                                        d["beta"][rows].contiguous(), pool, slots))
    torch.cuda.synchronize()
    for n in range(3):
        full = o_full[seq_rows(w, n)]
        assert bit_equal(o_pre[40 * n:40 * (n + 1)], full[:40])
        dec = torch.stack([outs[i][n] for i in range(25)])
        assert bit_equal(dec, full[40:]), "decode outputs of sequence %d differ from prefill" % n
        assert bit_equal(pool[int(slots[n])], s_full[n]), "decode state of sequence %d differs" % n


def test_decode_padding_rows(gpu):
    w = synth.make_workload(11, [1, 1, 1], hk=2, hv=4, dk=128, dv=128)
    d = to_dev(w)
    pool = torch.randn((2, 4, 128, 128), device=DEV)
    before = pool.clone()
    idx = torch.tensor([-1, 1, 2], dtype=torch.int32, device=DEV)  # rows 0 and 2 are padding
    o = gpu.gdn_decode_step(d["q"], d["k"], d["v"], d["g"], d["beta"], pool, idx)
    torch.cuda.synchronize()
    assert torch.count_nonzero(o[0]) == 0 and torch.count_nonzero(o[2]) == 0
    assert bit_equal(pool[0], before[0]) and not bit_equal(pool[1], before[1])


def test_decode_across_batch_sizes(gpu):
    """Config: 256 sequences with 512-token prefilled states, one decode step at
    B = 1, 8, 64, 256 (the first B sequences) and once at B = 256 permuted; every
    sequence's output and state are bit-identical in every batch that holds it,
    and equal a 513-token full prefill."""
    w = synth.decode_history(1002, batch=256, prefix=512, steps=1)
    d = to_dev(w)
    cu = w.cu_seqlens.tolist()
    first = torch.cat([torch.arange(cu[i], cu[i] + 512) for i in range(256)]).to(DEV)
    last = torch.tensor([cu[i] + 512 for i in range(256)], device=DEV)
    cu_pre = torch.arange(0, 256 * 512 + 1, 512, dtype=torch.int32, device=DEV)
    _, states = gpu.gdn_fwd_varlen(d["q"][first].contiguous(), d["k"][first].contiguous(),
                                   d["v"][first].contiguous(), d["g"][first].contiguous(),
                                   d["beta"][first].contiguous(), None, cu_pre)
    o_full, s_full = gpu.gdn_fwd_varlen(d["q"], d["k"], d["v"], d["g"], d["beta"], None, d["cu_seqlens"])
    torch.cuda.synchronize()
    res = {}
    for B in (1, 8, 64, 256):
        pool = states[:B].clone()
        li = last[:B]
        o = gpu.gdn_decode_step(d["q"][li].contiguous(), d["k"][li].contiguous(), d["v"][li].contiguous(),
                                d["g"][li].contiguous(), d["beta"][li].contiguous(), pool)
        torch.cuda.synchronize()
        res[B] = (o, pool)
    perm = torch.randperm(256, generator=torch.Generator().manual_seed(3)).to(DEV)
    pool_p = states[perm].clone()
    lp = last[perm]
    o_p = gpu.gdn_decode_step(d["q"][lp].contiguous(), d["k"][lp].contiguous(), d["v"][lp].contiguous(),
                              d["g"][lp].contiguous(), d["beta"][lp].contiguous(), pool_p)
    torch.cuda.synchronize()
    o256, p256 = res[256]
    for B in (1, 8, 64):
        o, p = res[B]
        assert bit_equal(o, o256[:B]) and bit_equal(p, p256[:B]), "batch size %d changed the bits" % B
    inv = torch.argsort(perm)
    assert bit_equal(o_p[inv], o256) and bit_equal(pool_p[inv], p256), "permuted batch changed the bits"
    assert bit_equal(o256, o_full[last]), "decode output differs from the full prefill"
    assert bit_equal(p256, s_full), "decode state differs from the full prefill"


def test_mixed_batch_permutations(gpu):
    """64-sequence continuous batch (prefill chunks and single-token decodes, some
    resuming from cached states) under three seeded permutations: per-sequence bits
    identical."""
    w = synth.mixed_batch(1004)
    o, s = run_prefill(gpu, w)
    for seed in (2000, 2001, 2002):
        perm = torch.randperm(64, generator=torch.Generator().manual_seed(seed)).tolist()
        wp = synth.permute(w, perm)
        op, sp = run_prefill(gpu, wp)
        for new, old in enumerate(perm):
            assert bit_equal(op[seq_rows(wp, new)], o[seq_rows(w, old)]), "seed %d seq %d output" % (seed, old)
            assert bit_equal(sp[new], s[old]), "seed %d seq %d state" % (seed, old)


def test_long_context_chunked_8x8192(gpu):
    """One 65,536-token sequence, unchunked vs 8 chunked-prefill calls of 8,192 tokens."""
    w = synth.long_context(1003)
    d = to_dev(w)
    o, s = run_prefill(gpu, w, d=d)
    oc, sc = _chunked(gpu, w, list(range(0, 65536 + 1, 8192)), d=d)
    say("long context: chunked equal = %s" % (bit_equal(o, oc) and bit_equal(s, sc)))
    assert bit_equal(o, oc) and bit_equal(s, sc)


@pytest.mark.parametrize("dk,dv,io", [(16, 16, torch.float32), (16, 48, torch.bfloat16), (32, 32, torch.bfloat16),
                                      (64, 64, torch.float32), (64, 128, torch.bfloat16), (128, 128, torch.float32)])
def test_decode_equals_prefill_every_head_dim(gpu, dk, dv, io):
    """For every supported key dim and io dtype: prefill 20 tokens, then decode 3
    steps; each step's output and the final state equal a 23-token prefill."""
    w = synth.make_workload(21, [23, 23], hk=2, hv=4, dk=dk, dv=dv, io_dtype=io, h0_std=0.1)
    o_full, s_full = run_prefill(gpu, w)
    d = to_dev(w)
    idx_pre = torch.cat([torch.arange(23 * n, 23 * n + 20) for n in range(2)]).to(DEV)
    cu_pre = torch.tensor([0, 20, 40], dtype=torch.int32, device=DEV)
    _, pool = gpu.gdn_fwd_varlen(d["q"][idx_pre].contiguous(), d["k"][idx_pre].contiguous(),
                                 d["v"][idx_pre].contiguous(), d["g"][idx_pre].contiguous(),
                                 d["beta"][idx_pre].contiguous(), d["h0"], cu_pre)
    for t in range(20, 23):
        rows = torch.tensor([t, 23 + t], device=DEV)
        o = gpu.gdn_decode_step(d["q"][rows].contiguous(), d["k"][rows].contiguous(), d["v"][rows].contiguous(),
                                d["g"][rows].contiguous(), d["beta"][rows].contiguous(), pool)
        torch.cuda.synchronize()
        assert bit_equal(o, o_full[rows]), "dk=%d step %d output" % (dk, t)
    assert bit_equal(pool, s_full), "dk=%d final state" % dk


def test_all_empty_batch_with_null_inputs(gpu):
    """T = 0 with sequences present: q/k/v/g/beta/out may be NULL; hT = h0."""
    h0 = torch.randn((3, 4, 128, 128), device=DEV)
    hT = torch.empty_like(h0)
    cu = torch.zeros(4, dtype=torch.int32, device=DEV)
    dims = gpu.GdnDims(n_seqs=3, hk=2, hv=4, dk=128, dv=128, io_dtype=gpu.GDN_BF16, total_tokens=0,
                       pool_size=0, plan_lanes=0, plan_rows=0, plan_waves=0, reserved=0)
    import ctypes
    lib = gpu.load_library()
    rc = lib.gdn_fwd_varlen(ctypes.byref(dims), None, None, None, None, None, h0.data_ptr(), cu.data_ptr(),
                            None, hT.data_ptr(), None)
    torch.cuda.synchronize()
    assert rc == 0 and bit_equal(hT, h0)
