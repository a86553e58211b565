"""The chunked form with a replaying decode (gdn_fwd_chunked).

Parity: outputs against the fp64 recurrence oracle (the chunked form is the same
rule written from each chunk's start), and the final state, rebuilt on the host in
fp64 from the chunked state (S at the open chunk's start plus its u, k and decay
factors a), against the oracle's hT, under the same gates as the recurrent path.
Bitwise: any split of a sequence into calls, one-token decode steps included (in
place or not), and any batch give the same outputs and chunked states.
"""
import numpy as np
import pytest
import torch

from gpu_helpers import OUT_TOL, STATE_TOL, bit_equal, say, seq_errors, state_errors, to_dev
from invariant_linear_attention_amd import synth

pytestmark = pytest.mark.gpu
DEV = "cuda"
CK = 16


def final_state(st):
    """fp64 state after the open chunk's tokens, rebuilt from the chunked state: the
    open chunk's u from its R rows by forward substitution (u_m = R_m - sum_{r<m}
    beta_m Gam_{m,r} (k_m . k_r) u_r), then Gam_{c-1} S0 + sum_s Gam_{c-1,s} u_s k_s^T,
    with Gam_{m,s} = a_m ... a_{s+1} and Gam_{c-1} = a_{c-1} ... a_0."""
    S0 = st["S"].double().cpu().numpy()
    K = st["k"].double().cpu().numpy()
    R = st["r"].double().cpu().numpy()
    A = st["a"].double().cpu().numpy()
    B = st["b"].double().cpu().numpy()
    cnt = st["count"].cpu().numpy()
    N, hv = S0.shape[0], S0.shape[1]
    hk = K.shape[2]
    out = S0.copy()
    for n in range(N):
        c = int(cnt[n])
        if c == 0:
            continue
        for h in range(hv):
            kh = h // (hv // hk)
            u = []
            for m in range(c):
                um = R[n, m, h].copy()
                for r in range(m):
                    um -= B[n, m, h] * np.prod(A[n, r + 1:m + 1, h]) * (K[n, m, kh] @ K[n, r, kh]) * u[r]
                u.append(um)
            acc = np.prod(A[n, :c, h]) * S0[n, h]
            for s in range(c):
                acc += np.prod(A[n, s + 1:c, h]) * np.outer(u[s], K[n, s, kh])
            out[n, h] = acc
    return out


def run(gdn, w, st_in=None, d=None, inplace=False, waves=0):
    d = d if d is not None else to_dev(w)
    out, st = gdn.gdn_fwd_chunked(d["q"], d["k"], d["v"], d["g"], d["beta"], d["cu_seqlens"], st_in, inplace=inplace,
                                  waves=waves)
    torch.cuda.synchronize()
    return out, st


def start_state(gdn, w):
    return gdn.make_chunk_state(w.n_seqs, w.q.shape[1], w.v.shape[1], w.q.shape[2], w.v.shape[2], DEV,
                                h0=w.h0)


def states_equal(a, b):
    """Same count and S, and the same k, u and G in the open chunk's slots."""
    if not torch.equal(a["count"], b["count"]) or not bit_equal(a["S"], b["S"]):
        return False
    for n, c in enumerate(a["count"].cpu().tolist()):
        for key in ("k", "r", "a", "b"):
            if not bit_equal(a[key][n, :c], b[key][n, :c]):
                return False
    return True


@pytest.mark.parametrize("dk,dv,io", [(128, 128, torch.bfloat16), (64, 64, torch.float32), (128, 32, torch.bfloat16),
                                      (64, 48, torch.bfloat16)])
@pytest.mark.parametrize("h0", [0.0, 0.1])
def test_parity(gpu, dk, dv, io, h0):
    from oracle import oracle
    lengths = [37, 0, 1, 16, 15, 17, 100, 33]
    w = synth.make_workload(500 + dk + dv, lengths, hk=2, hv=4, dk=dk, dv=dv, io_dtype=io, h0_std=h0)
    out, st = run(gpu, w, start_state(gpu, w) if h0 > 0 else None)
    ro, rh = oracle.gdn_forward(w.q, w.k, w.v, w.g, w.beta, w.cu_seqlens, w.h0)
    errs = seq_errors(out.float().cpu().numpy(), ro, w.cu_seqlens.tolist())
    serr = state_errors(final_state(st), rh)
    say("chunked dk=%d dv=%d %s h0=%.1f: out %.2e state %.2e" % (dk, dv, io, h0, max(errs), max(serr)))
    assert max(errs) <= OUT_TOL[io] and max(serr) <= STATE_TOL
    assert st["count"].cpu().tolist() == [n % CK for n in lengths]


def test_parity_benchmark_batch(gpu):
    """The benchmark batch (8 sequences, 17,459 tokens, 16/32 heads, dk = dv = 128):
    every head against the oracle, outputs and rebuilt final states."""
    from oracle import oracle
    w = synth.varlen_prefill(1001)
    out, st = run(gpu, w, start_state(gpu, w))
    fs = final_state(st)
    ro, rh = oracle.gdn_forward(w.q, w.k, w.v, w.g, w.beta, w.cu_seqlens, w.h0)
    e = max(seq_errors(out.float().cpu().numpy(), ro, w.cu_seqlens.tolist()))
    es = max(state_errors(fs, rh))
    say("chunked benchmark batch, all heads: out %.2e state %.2e" % (e, es))
    assert e <= OUT_TOL[torch.bfloat16] and es <= STATE_TOL


def test_parity_long_sequence_and_extreme_gates(gpu):
    """A 2,000-token sequence against the oracle, plus gates the chunk products must
    survive: g = -1e4 (full forget inside a chunk), g = 0, beta = 0 and beta = 1.5."""
    from oracle import oracle
    w = synth.make_workload(541, [2000, 77], hk=2, hv=4, dk=128, dv=128, h0_std=0.1)
    g, b = w.g.clone(), w.beta.clone()
    g[100:103] = -1e4
    g[300:340] = 0.0
    b[500:530] = 0.0
    b[700:760] = 1.5
    w = synth.Workload(w.q, w.k, w.v, g, b, w.cu_seqlens, w.h0)
    out, st = run(gpu, w, start_state(gpu, w))
    ro, rh = oracle.gdn_forward(w.q, w.k, w.v, w.g, w.beta, w.cu_seqlens, w.h0)
    e = max(seq_errors(out.float().cpu().numpy(), ro, w.cu_seqlens.tolist()))
    es = max(state_errors(final_state(st), rh))
    say("chunked extreme gates: out %.2e state %.2e" % (e, es))
    assert e <= OUT_TOL[torch.bfloat16] and es <= STATE_TOL


@pytest.mark.parametrize("hk,hv", [(2, 4), (1, 8)])
def test_split_calls_and_decode_replay(gpu, hk, hv):
    """One call over the whole sequences == the same tokens in several calls
    (cuts inside and at chunk boundaries, one-token decode steps), bit for bit;
    with 8 value heads on one key head the key cache has one writer for eight readers."""
    lengths = [70, 23, 48]
    w = synth.make_workload(601, lengths, hk=hk, hv=hv, dk=128, dv=64, h0_std=0.1)
    st0 = start_state(gpu, w)
    ref_out, ref_st = run(gpu, w, st0)
    cuts = [0, 1, 2, 5, 16, 17, 31, 32, 33, 40, 47, 48, 61, 70]
    cu = w.cu_seqlens.tolist()
    st = st0
    outs = {n: [] for n in range(len(lengths))}
    for a, b in zip(cuts[:-1], cuts[1:]):
        # every sequence advances by its share of [a, b) (clipped to its length)
        segs = [(min(a, L), min(b, L)) for L in lengths]
        q, k, v, g, beta, cs = [], [], [], [], [], [0]
        for n, (x, y) in enumerate(segs):
            sl = slice(cu[n] + x, cu[n] + y)
            q.append(w.q[sl]); k.append(w.k[sl]); v.append(w.v[sl]); g.append(w.g[sl]); beta.append(w.beta[sl])
            cs.append(cs[-1] + (y - x))
        part = synth.Workload(torch.cat(q), torch.cat(k), torch.cat(v), torch.cat(g), torch.cat(beta),
                              torch.tensor(cs, dtype=torch.int32), None)
        o, st = run(gpu, part, st)
        for n in range(len(lengths)):
            outs[n].append(o[cs[n]:cs[n + 1]])
    for n in range(len(lengths)):
        assert bit_equal(torch.cat(outs[n]), ref_out[cu[n]:cu[n + 1]]), n
    assert states_equal(st, ref_st)
    say("chunked: %d calls (decode steps included) == one call, bitwise" % (len(cuts) - 1))


def test_alone_vs_in_batch(gpu):
    w = synth.make_workload(611, [50, 3, 130, 0, 17], hk=2, hv=4, dk=128, dv=128, h0_std=0.1)
    ref_out, ref_st = run(gpu, w, start_state(gpu, w))
    cu = w.cu_seqlens.tolist()
    for n in range(w.n_seqs):
        s = synth.select(w, [n])
        o, st = run(gpu, s, start_state(gpu, s))
        assert bit_equal(o, ref_out[cu[n]:cu[n + 1]]), n
        assert bit_equal(st["S"][0], ref_st["S"][n]) and int(st["count"][0]) == int(ref_st["count"][n])
        c = int(st["count"][0])
        for key in ("k", "r", "a", "b"):
            assert bit_equal(st[key][0, :c], ref_st[key][n, :c]), (n, key)


def test_empty_call_keeps_state(gpu):
    w = synth.make_workload(621, [20, 5], hk=1, hv=2, dk=64, dv=64, h0_std=0.1)
    _, st = run(gpu, w, start_state(gpu, w))
    e = synth.Workload(w.q[:0], w.k[:0], w.v[:0], w.g[:0], w.beta[:0], torch.tensor([0, 0, 0], dtype=torch.int32), None)
    _, st2 = run(gpu, e, st)
    assert states_equal(st, st2)


def test_decode_replay_benchmark_heads(gpu):
    """16/32 heads, dk = dv = 128: a 512-token prefill then 9 one-token decode steps
    (crossing a chunk end) equal a 521-token prefill, outputs and state bit for bit,
    for a batch of 3 sequences."""
    L0, steps = 512, 9
    w = synth.make_workload(631, [L0 + steps] * 3, h0_std=0.1)
    ref_out, ref_st = run(gpu, w, start_state(gpu, w))
    cu = w.cu_seqlens.tolist()

    def part(a, b):
        idx = torch.cat([torch.arange(cu[n] + a, cu[n] + b) for n in range(3)])
        return synth.Workload(w.q[idx], w.k[idx], w.v[idx], w.g[idx], w.beta[idx],
                              synth.cu_from_lengths([b - a] * 3), None)

    out0, st = run(gpu, part(0, L0), start_state(gpu, w))
    for n in range(3):
        assert bit_equal(out0[n * L0:(n + 1) * L0], ref_out[cu[n]:cu[n] + L0]), n
    for j in range(steps):
        o, st = run(gpu, part(L0 + j, L0 + j + 1), st)
        for n in range(3):
            assert bit_equal(o[n:n + 1], ref_out[cu[n] + L0 + j:cu[n] + L0 + j + 1]), (n, j)
    assert states_equal(st, ref_st)
    say("chunked: 512-token prefill + 9 decode steps == 521-token prefill, 32 heads, bitwise")


def test_inplace_decode_equals_out_of_place(gpu):
    """One-token steps with the state updated in place (S written only when a chunk
    closes) give the bits of out-of-place steps and of one prefill, across a chunk end."""
    L0, steps = 40, 12
    w = synth.make_workload(641, [L0 + steps] * 4, hk=2, hv=4, dk=128, dv=64, h0_std=0.1)
    ref_out, ref_st = run(gpu, w, start_state(gpu, w))
    cu = w.cu_seqlens.tolist()

    def part(a, b):
        idx = torch.cat([torch.arange(cu[n] + a, cu[n] + b) for n in range(4)])
        return synth.Workload(w.q[idx], w.k[idx], w.v[idx], w.g[idx], w.beta[idx],
                              synth.cu_from_lengths([b - a] * 4), None)

    _, st = run(gpu, part(0, L0), start_state(gpu, w))
    S_addr = st["S"].data_ptr()
    for j in range(steps):
        o, st = run(gpu, part(L0 + j, L0 + j + 1), st, inplace=True)
        for n in range(4):
            assert bit_equal(o[n:n + 1], ref_out[cu[n] + L0 + j:cu[n] + L0 + j + 1]), (n, j)
    assert st["S"].data_ptr() == S_addr
    assert states_equal(st, ref_st)


def test_nan_stays_in_its_chunk_and_row(gpu):
    """A NaN in v[t, h, j] reaches row j of head h from the start of t's 16-token
    chunk on (0 x NaN in the chunk's tile products), never an earlier chunk, another
    row, head or sequence; everything else keeps the clean run's bits."""
    w = synth.make_workload(651, [45, 30], hk=2, hv=4, dk=128, dv=64, h0_std=0.1)
    clean, _ = run(gpu, w, start_state(gpu, w))
    t, h, j = 21, 3, 9     # position 21: inside the second chunk (16 .. 31) of sequence 0
    v = w.v.clone()
    v[t, h, j] = float("nan")
    bad = synth.Workload(w.q, w.k, v, w.g, w.beta, w.cu_seqlens, w.h0)
    out, _ = run(gpu, bad, start_state(gpu, bad))
    mask = torch.zeros(out.shape, dtype=torch.bool)
    mask[16:45, h, j] = True
    assert bool(torch.isnan(out.cpu()[mask].float()).all())
    assert bit_equal(out.cpu()[~mask], clean.cpu()[~mask])


@pytest.mark.parametrize("dk,io", [(128, torch.bfloat16), (64, torch.float32)])
def test_every_wave_split_gives_the_same_bits(gpu, dk, io):
    """1, 2 or 4 waves per 16-row tile (the dk quarters spread over them) give the
    same outputs and states, and so do a prefill and one-token steps under each."""
    w = synth.make_workload(661, [70, 1, 33, 16], hk=2, hv=4, dk=dk, dv=64, io_dtype=io, h0_std=0.1)
    ref_out, ref_st = run(gpu, w, start_state(gpu, w), waves=1)
    for W in (2, 4):
        o, st = run(gpu, w, start_state(gpu, w), waves=W)
        assert bit_equal(o, ref_out) and states_equal(st, ref_st), W
    one = synth.select(w, [0])
    _, st1 = run(gpu, synth.token_slice(one, 0, 69, h0=one.h0), start_state(gpu, one), waves=4)
    o, st2 = run(gpu, synth.token_slice(one, 69, 70), st1, waves=2)
    assert bit_equal(o, ref_out[69:70])


def test_decode_without_cu_seqlens(gpu):
    """A one-token-per-sequence call may pass no cu_seqlens (sequence n's token is
    row n): the same bits as with cu_seqlens = 0, 1, ..., N, out of place and in
    place, across a chunk end, for a batch of 5 sequences at different offsets."""
    w = synth.make_workload(661, [30 + 3 * n for n in range(5)], hk=2, hv=4, dk=128, dv=64, h0_std=0.1)
    cu = w.cu_seqlens.tolist()
    N = w.n_seqs
    pre = synth.Workload(*(torch.cat([getattr(w, nm)[cu[n]:cu[n + 1] - 4] for n in range(N)])
                           for nm in ("q", "k", "v", "g", "beta")),
                         synth.cu_from_lengths([cu[n + 1] - cu[n] - 4 for n in range(N)]), w.h0)
    _, st = run(gpu, pre, start_state(gpu, w))
    st_a = {k: v.clone() for k, v in st.items()}
    st_b = {k: v.clone() for k, v in st.items()}
    for step in range(4):
        idx = torch.tensor([cu[n + 1] - 4 + step for n in range(N)])
        d = {nm: getattr(w, nm)[idx].contiguous().to(DEV) for nm in ("q", "k", "v", "g", "beta")}
        ar = torch.arange(N + 1, dtype=torch.int32, device=DEV)
        o1, s1 = gpu.gdn_fwd_chunked(d["q"], d["k"], d["v"], d["g"], d["beta"], ar, st)
        o2, s2 = gpu.gdn_fwd_chunked(d["q"], d["k"], d["v"], d["g"], d["beta"], None, st)
        o3, st_a = gpu.gdn_fwd_chunked(d["q"], d["k"], d["v"], d["g"], d["beta"], None, st_a, inplace=True)
        o4, st_b = gpu.gdn_fwd_chunked(d["q"], d["k"], d["v"], d["g"], d["beta"], ar, st_b, inplace=True)
        torch.cuda.synchronize()
        assert bit_equal(o1, o2) and bit_equal(o1, o3) and bit_equal(o1, o4), step
        assert states_equal(s1, s2) and states_equal(s1, st_a) and states_equal(s1, st_b), step
        st = s1
        st_a = {k: v.clone() for k, v in st_a.items()}
        st_b = {k: v.clone() for k, v in st_b.items()}
    say("chunked decode without cu_seqlens: same bits as with it, in place and out of place")
