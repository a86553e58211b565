"""Varlen prefill against a state pool (gdn_fwd_varlen_pool): slot routing and
block-aligned state snapshots for prefix caching.

The page "Defending Against the Training-Inference Numeric Mismatch in RL
(Especially Linear Attention)" (section 3.2, "Solution") keeps its serving
stack's state cache, including the state snapshots that stack takes at
block-aligned positions so that prefix caching keeps working.  What must hold:

* routing states through pool slots changes no bit of any output or state
  relative to gdn_fwd_varlen with the same initial states gathered by hand;
* a snapshot taken at absolute position p holds exactly the bits that hT holds
  for a run cut at p, and resuming from it reproduces the uncut run bit for bit;
* none of this depends on the launch shape or on how many tokens came before.

Bitwise expectations come from gdn_fwd_varlen on the same GPU; the snapshot
values are also checked against the fp64 oracle within the fp32 state gate.
"""
import pytest
import torch

from gpu_helpers import STATE_TOL, bit_equal, run_prefill, say, state_errors, to_dev
from invariant_linear_attention_amd import synth

pytestmark = pytest.mark.gpu
DEV = "cuda"
HK, HV, DK, DV = 4, 8, 128, 128


def batch(lengths, seed=11, h0=0.1):
    return synth.make_workload(seed, list(lengths), hk=HK, hv=HV, dk=DK, dv=DV, h0_std=h0)


def i32(x):
    return torch.tensor(list(x), dtype=torch.int32, device=DEV)


def random_pool(P, seed=3):
    gen = torch.Generator().manual_seed(seed)
    return (torch.randn((P, HV, DV, DK), generator=gen) * 0.1).to(DEV)


def pool_call(gdn, w, pool, d=None, plan=(0, 0, 0), **kw):
    d = d if d is not None else to_dev(w)
    out = gdn.gdn_fwd_varlen_pool(d["q"], d["k"], d["v"], d["g"], d["beta"], d["cu_seqlens"], pool, plan=plan, **kw)
    torch.cuda.synchronize()
    return out


def with_h0(w, h0):
    return synth.Workload(w.q, w.k, w.v, w.g, w.beta, w.cu_seqlens, h0, name=w.name, meta=dict(w.meta))


def prefix_state(gdn, w, n, k, h0_row):
    """hT of gdn_fwd_varlen over the first k tokens of sequence n, from h0_row."""
    s = synth.token_slice(synth.select(w, [n]), 0, k, h0=h0_row.unsqueeze(0).cpu())
    _, hT = run_prefill(gdn, s)
    return hT[0]


def test_slots_match_plain_call(gpu):
    lengths = (37, 100, 5, 64, 0, 130, 1)
    w = batch(lengths, h0=0.0)
    N, P = len(lengths), 12
    pool = random_pool(P)
    before = pool.clone()
    src = [3, 0, 7, 7, 2, 11, 5]        # a slot may be read by several sequences (7)
    dst = [8, 1, 4, 6, 9, 10, 5]        # written slots are distinct; sequence 6 works in place
    out = pool_call(gpu, w, pool, src_idx=i32(src), dst_idx=i32(dst))
    ref_out, ref_hT = run_prefill(gpu, with_h0(w, before[src].cpu()))
    assert bit_equal(out, ref_out)
    for n in range(N):
        assert bit_equal(pool[dst[n]], ref_hT[n]), n
    untouched = sorted(set(range(P)) - set(dst))
    assert bit_equal(pool[untouched], before[untouched])


def test_none_slots(gpu):
    """src outside [0, P): the zero state; dst outside [0, P): nothing written."""
    lengths = (20, 33, 8)
    w = batch(lengths, h0=0.0)
    P = 4
    pool = random_pool(P, seed=4)
    before = pool.clone()
    out = pool_call(gpu, w, pool, src_idx=i32([-1, 1, P]), dst_idx=i32([0, -5, 2 * P]))
    h0 = torch.zeros((3, HV, DV, DK))
    h0[1] = before[1].cpu()
    ref_out, ref_hT = run_prefill(gpu, with_h0(w, h0))
    assert bit_equal(out, ref_out)
    assert bit_equal(pool[0], ref_hT[0])
    assert bit_equal(pool[1:], before[1:])


def test_identity_slots_and_in_place(gpu):
    """NULL index arrays mean slot n; src == dst updates in place."""
    w = batch((50, 17, 96))
    pool = w.h0.clone().to(DEV)
    ref_out, ref_hT = run_prefill(gpu, w)
    out = pool_call(gpu, w, pool)
    assert bit_equal(out, ref_out) and bit_equal(pool, ref_hT)
    pool2 = torch.cat([torch.zeros((2, HV, DV, DK), device=DEV), w.h0.to(DEV)])
    out2 = pool_call(gpu, w, pool2, src_idx=i32([2, 3, 4]), dst_idx=i32([2, 3, 4]))
    assert bit_equal(out2, ref_out) and bit_equal(pool2[2:], ref_hT)


def boundaries(pos0, length, block):
    """Absolute positions p = m * block with pos0 < p <= pos0 + length."""
    first = (pos0 // block + 1) * block
    return list(range(first, pos0 + length + 1, block))


def snapshot_case(gpu, lengths, pos0, block, plan=(0, 0, 0), seed=21, per_seq=None):
    w = batch(lengths, seed=seed)
    N = len(lengths)
    bnds = [boundaries(pos0[n], lengths[n], block) for n in range(N)]
    S = per_seq if per_seq is not None else max(1, max(len(b) for b in bnds))
    P = 2 * N + N * S
    pool = torch.zeros((P, HV, DV, DK), device=DEV)
    pool[:N] = w.h0.to(DEV)
    snap = [[2 * N + n * S + j for j in range(S)] for n in range(N)]
    out = pool_call(gpu, w, pool, plan=plan, src_idx=i32(range(N)), dst_idx=i32(range(N, 2 * N)),
                    pos0=i32(pos0), snap_idx=torch.tensor(snap, dtype=torch.int32, device=DEV), snap_block=block)
    return w, bnds, snap, pool, out


@pytest.mark.parametrize("block", [16, 64])
def test_snapshots_equal_cut_runs(gpu, block):
    lengths = (200, 77, 0, 130, 33, 16, 1)
    pos0 = (0, 5, 9, 16, 250, 31, 47)
    w, bnds, snap, pool, out = snapshot_case(gpu, lengths, pos0, block)
    ref_out, ref_hT = run_prefill(gpu, w)
    assert bit_equal(out, ref_out)                       # snapshots change no output
    N = len(lengths)
    assert bit_equal(pool[N:2 * N], ref_hT)
    n_checked = 0
    for n in range(N):
        for j, p in enumerate(bnds[n]):
            got = pool[snap[n][j]]
            want = prefix_state(gpu, w, n, p - pos0[n], w.h0[n])
            assert bit_equal(got, want), (n, j, p)
            n_checked += 1
        for j in range(len(bnds[n]), len(snap[n])):   # slots past the last boundary stay untouched
            assert not bool(pool[snap[n][j]].abs().sum()), (n, j)
    say("block %d: %d snapshots bitwise equal to cut runs" % (block, n_checked))
    assert n_checked > 0


def test_snapshots_against_oracle(gpu):
    from oracle import oracle
    lengths = (90, 41)
    pos0 = (7, 0)
    block = 32
    w, bnds, snap, pool, _ = snapshot_case(gpu, lengths, pos0, block)
    for n in range(len(lengths)):
        for j, p in enumerate(bnds[n]):
            s = synth.token_slice(synth.select(w, [n]), 0, p - pos0[n], h0=w.h0[n:n + 1])
            _, ref = oracle.gdn_forward(s.q, s.k, s.v, s.g, s.beta, s.cu_seqlens, s.h0)
            e = state_errors(pool[snap[n][j]].unsqueeze(0).cpu().numpy(), ref)[0]
            say("seq %d snapshot at %d: state error %.2e" % (n, p, e))
            assert e <= STATE_TOL


PLANS = [(8, 1, 4), (8, 1, 1), (16, 1, 4), (16, 2, 4), (16, 1, 2), (4, 1, 4), (4, 2, 1), (4, 1, 1), (8, 1, 8),
         (8, 2, 4), (16, 2, 8)]


def test_snapshots_across_launch_shapes(gpu):
    """Odd and even starting offsets, blocks of 8 (one wave) and 16 tokens."""
    lengths = (61, 130, 3, 95)
    pos0 = (3, 16, 13, 1)
    ref = snapshot_case(gpu, lengths, pos0, 16, plan=PLANS[0])
    for plan in PLANS[1:]:
        got = snapshot_case(gpu, lengths, pos0, 16, plan=plan)
        assert bit_equal(got[4], ref[4]), plan
        assert bit_equal(got[3], ref[3]), plan


def test_resume_from_snapshot(gpu):
    """Prefix caching: a second request resumes from a snapshot of the first and
    reproduces the uncut run's outputs and final state bit for bit."""
    L, cut_at, block = 300, 128, 64
    w = batch((L,), seed=31)
    pool = torch.zeros((4, HV, DV, DK), device=DEV)
    pool[0] = w.h0[0].to(DEV)
    snap = torch.tensor([[1, 2, 3, -1]], dtype=torch.int32, device=DEV)
    full_out = pool_call(gpu, w, pool, src_idx=i32([0]), dst_idx=i32([-1]), snap_idx=snap, snap_block=block)
    # the snapshot at absolute position 128 is j = 1 (boundaries 64, 128, 192, 256)
    rest = synth.token_slice(w, cut_at, L)
    out2 = pool_call(gpu, rest, pool, src_idx=i32([2]), dst_idx=i32([0]), pos0=i32([cut_at]),
                     snap_idx=torch.tensor([[3, -1]], dtype=torch.int32, device=DEV), snap_block=block)
    assert bit_equal(out2, full_out[cut_at:])
    _, ref_hT = run_prefill(gpu, w)
    assert bit_equal(pool[0], ref_hT[0])
    # the resumed call's first snapshot (position 192) rewrote slot 3 with the same bits
    want = prefix_state(gpu, w, 0, 192, w.h0[0])
    assert bit_equal(pool[3], want)


def test_snapshot_then_decode(gpu):
    """A snapshot at the end of a prefill feeds decode exactly like hT does."""
    L, block = 64, 32
    w = batch((L + 1,), seed=41)
    pre = synth.token_slice(w, 0, L, h0=w.h0)
    pool = torch.zeros((3, HV, DV, DK), device=DEV)
    pool[0] = w.h0[0].to(DEV)
    pool_call(gpu, pre, pool, src_idx=i32([0]), dst_idx=i32([-1]),
              snap_idx=torch.tensor([[-1, 1]], dtype=torch.int32, device=DEV), snap_block=block)
    d = to_dev(synth.token_slice(w, L, L + 1))
    o = gpu.gdn_decode_step(d["q"], d["k"], d["v"], d["g"], d["beta"], pool, state_idx=i32([1]))
    torch.cuda.synchronize()
    ref_out, ref_hT = run_prefill(gpu, w)
    assert bit_equal(o, ref_out[L:]) and bit_equal(pool[1], ref_hT[0])


def test_snapshots_at_benchmark_size(gpu):
    """The 8-sequence benchmark batch with a snapshot every 256 tokens: outputs and
    final states unchanged, and sampled snapshots equal to cut runs."""
    w = synth.varlen_prefill(1001)
    N = w.n_seqs
    block = 256
    S = max(len(boundaries(0, L, block)) for L in w.lengths)
    d = to_dev(w)
    pool = torch.zeros((2 * N + N * S, 32, 128, 128), device=DEV)
    pool[:N] = d["h0"]
    snap = torch.tensor([[2 * N + n * S + j for j in range(S)] for n in range(N)], dtype=torch.int32, device=DEV)
    out = gpu.gdn_fwd_varlen_pool(d["q"], d["k"], d["v"], d["g"], d["beta"], d["cu_seqlens"], pool,
                                  src_idx=i32(range(N)), dst_idx=i32(range(N, 2 * N)), snap_idx=snap,
                                  snap_block=block)
    torch.cuda.synchronize()
    ref_out, ref_hT = run_prefill(gpu, w, d=d)
    assert bit_equal(out, ref_out) and bit_equal(pool[N:2 * N], ref_hT)
    for n, j in ((7, 0), (7, 14), (2, 5), (1, 0)):
        p = (j + 1) * block
        if p > w.lengths[n]:
            continue
        got = pool[2 * N + n * S + j]
        s = synth.token_slice(synth.select(w, [n]), 0, p, h0=w.h0[n:n + 1])
        _, want = run_prefill(gpu, s)
        assert bit_equal(got, want[0]), (n, j)
