#!/usr/bin/env python3
"""Benchmark of the batch-invariant Gated DeltaNet recurrent forward on one MI355X.

A step is one varlen prefill pass (gdn_fwd_varlen) over the 8-sequence batch with
lengths drawn uniformly from [256, 4096] (16 query/key heads, 32 value heads,
dk = dv = 128, bf16 q/k/v/out, fp32 gates and state, random initial states).
``value`` is that pass's throughput in tokens/s with every input already in HBM.

Order of work.  Every GPU line is timed first, back to back, and the outputs of
each timed configuration are kept; the fp64 oracle then re-checks them, and the
CPU baseline runs last.  So no CPU work sits between GPU measurements (the GPU
clock does not drop in an idle gap), and the benchmark step is timed last, after
its own warm-up launches, on a GPU that has been busy.

Also reported on the same line:
  roofline      prefill kernel against the fp32 vector peak (7 dk dv flops per
                token and value head: decay, key read-out, rank-1 write, query
                read-out), from per-launch HIP events on the launch stream, with
                the per-launch durations and their percentiles;
  decode        one decode step at B = 1, 8, 64 and 256 from states made by a
                512-token prefill, against the HBM peak (state read + written in
                place).  Its launches are queued behind a GPU-side hold, so every
                launch starts when the previous one ends and no host issue time
                enters a duration; state pools rotate over >= 1 GiB so the 256 MB
                Infinity Cache cannot hold them;
  workloads     the same prefill kernel on the 65,536-token sequence (whole, and
                as 8 chunks of 8,192 carried in place through the state), on
                the 64-sequence mixed batch, through the state pool with
                snapshots, and with fused preprocessing, against the same fp32
                roofline; the short convolution on the batch's q|k|v channels
                against the HBM roofline; the backward (gdn_bwd_varlen) on the
                benchmark batch against the fp32 roofline on its 18 flops per
                state element and token; the chunked form with its replaying
                decode (gdn_fwd_chunked) on the same batch and at B = 256;
  cpu_baseline  the fp64 oracle on the host cores, on a bounded sample;
  parity        the timed outputs re-checked against the oracle: every head of
                the benchmark step, the long context and the mixed batch.

Usage: python bench.py [--gpus 1] [--steps 20] [--warmup 50] [--no-cpu] [--no-decode] [--no-workloads]
"""
import argparse
import hashlib
import json
import os
import subprocess
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

FP32_VECTOR_PEAK_TFLOPS = 157.3   # MI355X: 256 CUs x 2.4 GHz x 256 flop/clk
FP32_MATRIX_PEAK_TFLOPS = 157.3   # MI355X dense fp32 MFMA (the same figure)
HBM_PEAK_GBS = 8000.0             # MI355X HBM3E
METRIC = "GDN recurrent fwd tokens/s (prefill, decode) + % HBM/FP32-VALU roofline"
HEADS = dict(hk=16, hv=32, dk=128, dv=128)
FLOPS_PER_TOKEN = 7.0 * 128 * 128 * 32
DECODE_BYTES_PER_SEQ = 2 * 32 * 128 * 128 * 4 + 24832


def kernel_source_hash():
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "invariant_linear_attention_amd", "csrc")
    for name in sorted(os.listdir(csrc)):
        with open(os.path.join(csrc, name), "rb") as f:
            h.update(name.encode() + f.read())
    return h.hexdigest()[:16]


def traffic_from_profile(kind, src_hash):
    """HBM bytes per launch from a committed rocprofv3 PMC summary, if it was taken
    on the current kernel sources (else None)."""
    path = os.path.join(ROOT, "profiles", "%s_traffic.json" % kind)
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("kernel_source_hash") != src_hash:
        return None
    return rec.get("bytes_per_launch")


def progress(msg):
    """One line per finished section on stderr (the JSON line stays alone on stdout)."""
    print("bench: %s" % msg, file=sys.stderr, flush=True)


class Hold:
    """A GPU-side hold: a spin kernel that keeps the stream busy while the host
    queues launches behind it, so that the queued launches then run back to back
    and no host issue time enters their event durations."""

    def __init__(self, stream):
        import torch
        self.stream = stream
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        cycles = 2_000_000
        with torch.cuda.stream(stream):
            torch.cuda._sleep(cycles)  # first call loads the kernel
            torch.cuda.synchronize()
            a.record(stream)
            torch.cuda._sleep(cycles)
            b.record(stream)
        torch.cuda.synchronize()
        self.cycles_per_ms = cycles / max(a.elapsed_time(b), 1e-3)

    def __call__(self, ms):
        import torch
        with torch.cuda.stream(self.stream):
            torch.cuda._sleep(int(self.cycles_per_ms * ms))


def percentiles(per):
    import numpy as np
    p = np.percentile(np.asarray(per, dtype=np.float64), [0, 10, 50, 90, 100])
    return {"min": float(p[0]), "p10": float(p[1]), "p50": float(p[2]), "p90": float(p[3]), "max": float(p[4])}


def time_launches(fn, steps, warmup, stream, hold=None, hold_ms=0.0):
    """Per-launch durations (ms) from HIP events recorded on the launch stream.

    Warm-up launches are queued right before the timed ones (no synchronisation in
    between, so the stream never drains).  With a hold, everything is queued
    behind a GPU-side spin of ``hold_ms`` first.  Returns (per-launch durations,
    host seconds spent queueing, total ms between the first and last event / K)."""
    import torch
    if hold is not None and hold_ms > 0:
        # one untimed call first: a kernel's first launch in the process loads its
        # code, which can take longer on the host than the hold lasts
        fn(0)
    torch.cuda.synchronize()
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    t0 = time.perf_counter()
    if hold is not None and hold_ms > 0:
        hold(hold_ms)
    for i in range(warmup):
        fn(i)
    for i in range(steps):
        starts[i].record(stream)
        fn(warmup + i)
        ends[i].record(stream)
    queued = time.perf_counter() - t0
    torch.cuda.synchronize()
    if hold is not None and hold_ms > 0 and queued * 1e3 > 0.8 * hold_ms:
        # the host took longer to queue than the hold lasted: the GPU may have idled
        # inside a timed launch, so time again behind a longer hold
        return time_launches(fn, steps, warmup, stream, hold, 2.0 * queued * 1e3)
    per = [s.elapsed_time(e) for s, e in zip(starts, ends)]
    span = starts[0].elapsed_time(ends[-1]) / steps
    return per, queued, span


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def gpu_clock():
    """Current shader clock as the SMI tool reports it (best effort, else None)."""
    for cmd in (["amd-smi", "metric", "-c", "--json"], ["rocm-smi", "--showclocks", "--json"]):
        try:
            r = subprocess.run(cmd, capture_output=True, text=True, timeout=20)
        except (OSError, subprocess.SubprocessError):
            continue
        if r.returncode == 0 and r.stdout.strip():
            return r.stdout.strip()[:600]
    return None


def rel(x, r):
    import numpy as np
    x = np.asarray(x, dtype=np.float64)
    r = np.asarray(r, dtype=np.float64)
    return float(np.linalg.norm(x - r) / max(np.linalg.norm(r), 1e-300))


def seq_rel_max(x, r, cu):
    """max over sequences of the per-sequence normwise error (token-major arrays)."""
    import numpy as np
    x = np.asarray(x, dtype=np.float64)
    r = np.asarray(r, dtype=np.float64)
    worst = 0.0
    for n in range(len(cu) - 1):
        a, b = int(cu[n]), int(cu[n + 1])
        if b > a:
            worst = max(worst, float(np.linalg.norm(x[a:b] - r[a:b]) / max(np.linalg.norm(r[a:b]), 1e-300)))
    return worst


def state_rel_max(x, r):
    import numpy as np
    x = np.asarray(x, dtype=np.float64)
    r = np.asarray(r, dtype=np.float64)
    return max(float(np.linalg.norm(x[n] - r[n]) / max(np.linalg.norm(r[n]), 1e-300)) for n in range(r.shape[0]))


COPY_BYTES = 1 << 30  # calibration copy: 1 GiB read + 1 GiB written


def pmc_pass(dev, stream):
    """One launch of each kernel (prefill, decode at B = 256, the short convolution
    and its state update and backward, the backward's six, the chunked form's prefill
    and backward, the preprocessing passes), preceded by a plain device copy of
    COPY_BYTES whose FETCH_SIZE / WRITE_SIZE readings calibrate the counters' units."""
    import torch

    from invariant_linear_attention_amd import gdn, synth
    src = torch.ones(COPY_BYTES // 4, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    dst.copy_(src)
    torch.cuda.synchronize()
    del src, dst
    w = synth.varlen_prefill(1001)
    d = [t.to(dev) for t in (w.q, w.k, w.v, w.g, w.beta, w.h0, w.cu_seqlens)]
    gdn.gdn_fwd_varlen(*d, stream=stream)
    torch.cuda.synchronize()
    B = 256
    dw = synth.make_workload(2000 + B, [1] * B)
    pool = torch.randn((B, 32, 128, 128), device=dev) * 0.1
    gdn.gdn_decode_step(*(t.to(dev) for t in (dw.q, dw.k, dw.v, dw.g, dw.beta)), pool, stream=stream)
    torch.cuda.synchronize()
    del pool
    C, K = 2 * 16 * 128 + 32 * 128, 4   # the short convolution on the batch's q|k|v channels
    gen = torch.Generator().manual_seed(1005)
    xc = torch.randn((w.total_tokens, C), generator=gen).to(torch.bfloat16).to(dev)
    wc = (0.5 * torch.randn((C, K), generator=gen)).to(dev)
    pool_c = torch.zeros((w.n_seqs, C, K - 1), dtype=torch.bfloat16, device=dev)
    gdn.gdn_short_conv(xc, wc, d[6], pool_c, stream=stream)
    torch.cuda.synchronize()
    pool_c.zero_()
    dyc = torch.randn((w.total_tokens, C), generator=torch.Generator().manual_seed(1009)).to(dev)
    bc = torch.zeros((C,), device=dev)
    gdn.gdn_short_conv_backward(xc, wc, d[6], pool_c, dyc, bias=bc, stream=stream)
    torch.cuda.synchronize()
    del xc, pool_c, dyc
    gen = torch.Generator().manual_seed(1006)  # the backward, as in its benchmark line
    dout = torch.randn(tuple(w.v.shape), generator=gen).to(torch.bfloat16).to(dev)
    dhT = torch.randn((w.n_seqs, 32, 128, 128), generator=gen).to(dev)
    gdn.gdn_bwd_varlen(*d, dout, dhT, stream=stream)
    torch.cuda.synchronize()
    # the chunked form (prep + main kernel) and the chunked backward on the same batch
    st_in = gdn.make_chunk_state(w.n_seqs, 16, 32, 128, 128, dev, h0=d[5])
    gdn.gdn_fwd_chunked(*d[:5], d[6], st_in, stream=stream)
    torch.cuda.synchronize()
    del st_in
    gdn.gdn_bwd_chunked(*d, dout, dhT, stream=stream)
    torch.cuda.synchronize()
    del dout, dhT
    # the preprocessing pass and its backward on the raw inputs of the same shape
    rw = synth.make_raw_workload(1001, w.lengths, h0_std=0.1)
    rq, rk, ra, rb = (t.to(dev) for t in (rw.q, rw.k, rw.g, rw.beta))
    pre = gdn.make_preproc(norm_qk=True, eps=1e-6, A_log=rw.meta["A_log"].to(dev), dt_bias=rw.meta["dt_bias"].to(dev))
    gdn.gdn_preprocess(rq, rk, ra, rb, pre=pre, stream=stream)
    genp = torch.Generator().manual_seed(1008)
    dqn = torch.randn(tuple(rw.q.shape), generator=genp).to(dev)
    dkn = torch.randn(tuple(rw.q.shape), generator=genp).to(dev)
    dgp = torch.randn(tuple(rw.g.shape), generator=genp).to(dev)
    dbp = torch.randn(tuple(rw.g.shape), generator=genp).to(dev)
    gdn.gdn_preprocess_backward(rq, rk, ra, rb, dqn, dkn, dgp, dbp, pre=pre, stream=stream)
    torch.cuda.synchronize()
    print("pmc pass: copy %d bytes, prefill %d tokens, decode B=%d, conv %d channels and its backward, backward, "
          "chunked prefill and backward, preprocessing and its backward" % (COPY_BYTES, w.total_tokens, B, C),
          flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--no-workloads", action="store_true", help="skip the long-context and mixed-batch lines")
    ap.add_argument("--cpu-seconds", type=float, default=10.0, help="host time spent on the CPU oracle baseline")
    ap.add_argument("--pmc-pass", action="store_true",
                    help="no timing: one copy of a known size (counter calibration), then one launch each of the "
                         "prefill (the benchmark batch) and of decode at B=256, for rocprofv3 --pmc runs")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py runs on one GPU only: the recurrent forward needs no collective and this "
              "build measures a single MI355X (requested --gpus %d)" % args.gpus, file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    from invariant_linear_attention_amd import gdn, synth
    from oracle import oracle

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream()
    gdn.load_library()
    if args.pmc_pass:
        pmc_pass(dev, stream)
        return
    src_hash = kernel_source_hash()
    hold = Hold(stream)
    checks = []   # (record, name, fn): oracle re-checks run after every GPU line is timed

    w = synth.varlen_prefill(1001)
    T = w.total_tokens
    d = dict(q=w.q.to(dev), k=w.k.to(dev), v=w.v.to(dev), g=w.g.to(dev), beta=w.beta.to(dev),
             h0=w.h0.to(dev), cu=w.cu_seqlens.to(dev))
    out = torch.empty((T, 32, 128), dtype=torch.bfloat16, device=dev)
    hT = torch.empty((w.n_seqs, 32, 128, 128), dtype=torch.float32, device=dev)

    def prefill(_i):
        gdn.gdn_fwd_varlen(d["q"], d["k"], d["v"], d["g"], d["beta"], d["h0"], d["cu"], out=out, hT=hT,
                           stream=stream)

    # ------------------------------------------------------------- decode
    decode = None
    if not args.no_decode:
        decode = {}
        # States from a 512-token prefill of 256 sequences; batch B takes the first B.
        hist = synth.decode_history(1002, batch=256, prefix=512, steps=1)
        cu = hist.cu_seqlens.tolist()
        first = torch.cat([torch.arange(cu[i], cu[i] + 512) for i in range(256)])
        last = torch.tensor([cu[i] + 512 for i in range(256)])
        hd = {n: getattr(hist, n) for n in ("q", "k", "v", "g", "beta")}
        pre = [hd[n][first].contiguous().to(dev) for n in ("q", "k", "v", "g", "beta")]
        cu_pre = torch.arange(0, 256 * 512 + 1, 512, dtype=torch.int32, device=dev)
        _, base = gdn.gdn_fwd_varlen(*pre, None, cu_pre, stream=stream)
        del pre
        tok = [hd[n][last].contiguous().to(dev) for n in ("q", "k", "v", "g", "beta")]
        torch.cuda.synchronize()
        checked = {}
        for B in (1, 8, 64, 256):
            bytes_state = B * 32 * 128 * 128 * 4
            n_pools = max(4, int(np.ceil((1 << 30) / bytes_state)))
            pools = [base[:B].clone() for _ in range(n_pools)]
            dq, dk_, dv_, dg, db = (t[:B].contiguous() for t in tok)
            dout = torch.empty((B, 32, 128), dtype=torch.bfloat16, device=dev)

            def dec(i, B=B):
                gdn.gdn_decode_step(dq, dk_, dv_, dg, db, pools[i % n_pools], out=dout, stream=stream)

            steps = max(args.steps, 2 * n_pools) if B >= 64 else max(args.steps, 100)
            per_d, queued, span = time_launches(dec, steps, max(args.warmup, min(n_pools, 64)), stream, hold=hold,
                                                hold_ms=40.0)
            ms_d = float(np.mean(per_d))
            alg_bytes = B * DECODE_BYTES_PER_SEQ
            # one checked step from the prefill states
            pchk = base[:B].clone()
            ochk = gdn.gdn_decode_step(dq, dk_, dv_, dg, db, pchk, stream=stream)
            torch.cuda.synchronize()
            nb = min(4, B)
            checked[B] = (ochk[:nb].cpu(), pchk[:nb].cpu())
            decode["B%d" % B] = {
                "tokens_per_s": B / (ms_d / 1e3), "launch_ms_mean": ms_d,
                "launch_ms_percentiles": percentiles(per_d), "launch_ms_back_to_back": span,
                "launches": steps, "host_queue_ms": queued * 1e3, "hold_ms": 40.0,
                "roofline": {"bound": "hbm", "achieved": alg_bytes / (ms_d / 1e3) / 1e9, "peak": HBM_PEAK_GBS,
                             "unit": "GB/s", "frac": alg_bytes / (ms_d / 1e3) / 1e9 / HBM_PEAK_GBS,
                             "traffic": traffic_from_profile("decode_B%d" % B, src_hash),
                             "bytes_per_launch": alg_bytes},
                "state_pools": n_pools, "states": "from a 512-token prefill (first B of 256 sequences)"}
            del pools
            progress("decode B=%d mean %.1f us, median %.1f us" % (B, ms_d * 1e3, float(np.median(per_d)) * 1e3))
        del base, tok
        bitwise = all(torch.equal(checked[B][0].view(torch.int16), checked[256][0][:checked[B][0].shape[0]]
                                  .view(torch.int16)) and torch.equal(checked[B][1], checked[256][1][:checked[B][1]
                                                                                                        .shape[0]])
                      for B in (1, 8, 64))
        decode["bitwise_across_batch_sizes"] = bool(bitwise)

        def decode_check():
            four = synth.select(hist, [0, 1, 2, 3])
            ro, rh = oracle.gdn_forward(four.q, four.k, four.v, four.g, four.beta, four.cu_seqlens, None)
            ro_last = ro[[512, 1025, 1538, 2051]]
            res = {}
            for B, (o_, s_) in checked.items():
                nb = o_.shape[0]
                res["B%d" % B] = {"out": seq_rel_max(o_.float().numpy(), ro_last[:nb], list(range(nb + 1))),
                                  "state": state_rel_max(s_.numpy(), rh[:nb])}
            return res
        checks.append((decode, "parity", decode_check))

    # ------------------------------------------------ other prefill workloads
    workloads = None
    late_copies = []  # device -> host copies of checked outputs, run after the benchmark step
    got_g = {}
    if not args.no_workloads:
        workloads = {}

        def prefill_line(name, wl, chunks=1):
            Tw = wl.total_tokens
            dd = [t.to(dev) for t in (wl.q, wl.k, wl.v, wl.g, wl.beta)]
            cu = wl.cu_seqlens.to(dev)
            outw = torch.empty((Tw, 32, 128), dtype=torch.bfloat16, device=dev)
            state = (wl.h0.to(dev) if wl.h0 is not None
                     else torch.zeros((wl.n_seqs, 32, 128, 128), dtype=torch.float32, device=dev))
            if chunks == 1:
                def run(_i):
                    gdn.gdn_fwd_varlen(*dd, state, cu, out=outw, hT=state, stream=stream)
            else:
                # one sequence cut into equal chunks; each launch resumes in place
                assert wl.n_seqs == 1 and Tw % chunks == 0
                step_len = Tw // chunks
                cu_c = torch.tensor([0, step_len], dtype=torch.int32, device=dev)
                views = [[t[c * step_len:(c + 1) * step_len] for t in dd] for c in range(chunks)]
                outs = [outw[c * step_len:(c + 1) * step_len] for c in range(chunks)]

                def run(_i):
                    for c in range(chunks):
                        gdn.gdn_fwd_varlen(*views[c], state, cu_c, out=outs[c], hT=state, stream=stream)
            reps = max(3, min(args.steps, int(200.0 / max(Tw / 2000.0, 1.0))))
            per_w, _, _ = time_launches(run, reps, 3, stream)
            msw = float(np.median(per_w))
            # one checked run from the original initial states (the timed runs carried them on)
            state.copy_(wl.h0.to(dev) if wl.h0 is not None else torch.zeros_like(state))
            run(0)
            torch.cuda.synchronize()
            fl = FLOPS_PER_TOKEN * Tw
            rec = {"tokens": Tw, "n_seqs": wl.n_seqs, "chunks": chunks, "ms_median": msw,
                   "ms_mean": float(np.mean(per_w)), "launch_ms_percentiles": percentiles(per_w),
                   "tokens_per_s": Tw / (msw / 1e3),
                   "roofline_frac": fl / (msw / 1e3) / 1e12 / FP32_VECTOR_PEAK_TFLOPS,
                   "plan": list(gdn.gdn_query_plan(gdn.make_dims(dd[0], dd[2], wl.n_seqs if chunks == 1 else 1,
                                                                 Tw // chunks)))}
            workloads[name] = rec
            got_o, got_s = outw.cpu(), state.cpu()
            del dd, outw, state

            def check(wl=wl, got_o=got_o, got_s=got_s):
                ro, rh = oracle.gdn_forward(wl.q, wl.k, wl.v, wl.g, wl.beta, wl.cu_seqlens, wl.h0)
                return {"all_heads": {"out": seq_rel_max(got_o.float().numpy(), ro, wl.cu_seqlens.tolist()),
                                      "state": state_rel_max(got_s.numpy(), rh)}}
            checks.append((rec, "parity", check))
            progress("%s %.3f ms" % (name, msw))

        # The benchmark batch through the state pool with a snapshot every 256 tokens
        # (prefix caching): 8 source slots, 8 destination slots, one slot per snapshot.
        prefill(0)
        torch.cuda.synchronize()
        ref_out = out.clone()
        N, blk = w.n_seqs, 256
        n_snap = max(w.lengths) // blk
        pool = torch.zeros((2 * N + N * n_snap, 32, 128, 128), dtype=torch.float32, device=dev)
        pool[:N] = d["h0"]
        src = torch.arange(N, dtype=torch.int32, device=dev)
        dst = torch.arange(N, 2 * N, dtype=torch.int32, device=dev)
        snap = torch.arange(2 * N, 2 * N + N * n_snap, dtype=torch.int32, device=dev).view(N, n_snap)
        outp = torch.empty_like(out)

        def pooled(_i):
            gdn.gdn_fwd_varlen_pool(d["q"], d["k"], d["v"], d["g"], d["beta"], d["cu"], pool, src_idx=src,
                                    dst_idx=dst, snap_idx=snap, snap_block=blk, out=outp, stream=stream)

        per_p, _, _ = time_launches(pooled, args.steps, 5, stream)
        msp = float(np.median(per_p))
        torch.cuda.synchronize()
        workloads["varlen_prefill_pool_snapshots_256"] = {
            "tokens": T, "n_seqs": N, "snapshots": int(sum(L // blk for L in w.lengths)), "ms_median": msp,
            "launch_ms_percentiles": percentiles(per_p),
            "tokens_per_s": T / (msp / 1e3), "roofline_frac": FLOPS_PER_TOKEN * T / (msp / 1e3) / 1e12
            / FP32_VECTOR_PEAK_TFLOPS,
            "same_bits_as_plain": bool(torch.equal(outp.view(torch.int16), ref_out.view(torch.int16)))}
        del pool, outp, ref_out
        progress("pool with snapshots %.3f ms" % msp)

        # The benchmark batch's shape on raw inputs with both fused preprocessing steps
        # (in-kernel q/k L2 norm; gate and beta from logits).
        rw = synth.make_raw_workload(1001, w.lengths, h0_std=0.1)
        rd = [t.to(dev) for t in (rw.q, rw.k, rw.v, rw.g, rw.beta, rw.h0, rw.cu_seqlens)]
        A_log, dt_bias = rw.meta["A_log"].to(dev), rw.meta["dt_bias"].to(dev)
        pre_f = gdn.make_preproc(norm_qk=True, eps=1e-6, A_log=A_log, dt_bias=dt_bias)
        outr = torch.empty_like(out)
        hTr = torch.empty_like(hT)

        def fused(_i):
            gdn.gdn_fwd_varlen(*rd, out=outr, hT=hTr, stream=stream, pre=pre_f)

        per_f, _, _ = time_launches(fused, args.steps, 5, stream)
        msf = float(np.median(per_f))
        rec_f = {"tokens": T, "n_seqs": w.n_seqs, "ms_median": msf, "launch_ms_percentiles": percentiles(per_f),
                 "tokens_per_s": T / (msf / 1e3),
                 "roofline_frac": FLOPS_PER_TOKEN * T / (msf / 1e3) / 1e12 / FP32_VECTOR_PEAK_TFLOPS}
        workloads["varlen_prefill_fused_preprocessing"] = rec_f
        got_fo, got_fs = outr.cpu(), hTr.cpu()
        # the preprocessing as a pass of its own and its backward (the fused layer's
        # training path), on the same raw inputs: HBM-bound elementwise passes
        pre_out = gdn.gdn_preprocess(rd[0], rd[1], rd[3], rd[4], pre=pre_f, stream=stream)
        genp = torch.Generator().manual_seed(1008)
        dqn = torch.randn(tuple(rw.q.shape), generator=genp).to(dev)
        dkn = torch.randn(tuple(rw.q.shape), generator=genp).to(dev)
        dgp = torch.randn(tuple(rw.g.shape), generator=genp).to(dev)
        dbp = torch.randn(tuple(rw.g.shape), generator=genp).to(dev)
        pre_g = gdn.gdn_preprocess_backward(rd[0], rd[1], rd[3], rd[4], dqn, dkn, dgp, dbp, pre=pre_f, stream=stream)

        def pre_fwd(_i):
            gdn.gdn_preprocess(rd[0], rd[1], rd[3], rd[4], pre=pre_f, out=pre_out, stream=stream)

        def pre_bwd(_i):
            gdn.gdn_preprocess_backward(rd[0], rd[1], rd[3], rd[4], dqn, dkn, dgp, dbp, pre=pre_f, grads=pre_g,
                                        stream=stream)

        per_pf, _, _ = time_launches(pre_fwd, args.steps, 5, stream)
        per_pb, _, _ = time_launches(pre_bwd, args.steps, 5, stream)
        qk_el, gb_el = 2.0 * rw.q.numel(), 2.0 * rw.g.numel()
        pf_bytes = qk_el * 2 + gb_el * 4 + qk_el * 4 + gb_el * 4  # bf16 q, k and logits in; fp32 out
        # backward: bf16 q, k, fp32 dqn, dkn in and dq, dk out; logits, dg, dbeta in and da, db out
        pb_bytes = qk_el * 2 + qk_el * 4 + qk_el * 4 + gb_el * 4 * 3
        rec_pp = {"tokens": T}
        for name, per_x, nbytes in (("forward", per_pf, pf_bytes), ("backward", per_pb, pb_bytes)):
            msx = float(np.median(per_x))
            rec_pp[name] = {"ms_median": msx, "launch_ms_percentiles": percentiles(per_x),
                            "roofline": {"bound": "hbm", "achieved": nbytes / (msx / 1e3) / 1e9,
                                         "peak": HBM_PEAK_GBS, "unit": "GB/s",
                                         "frac": nbytes / (msx / 1e3) / 1e9 / HBM_PEAK_GBS,
                                         "bytes_per_launch": nbytes,
                                         "traffic": traffic_from_profile("preprocess_%s" % name, src_hash)}}
        workloads["preprocess_passes"] = rec_pp
        pp_got = {k: v[:, 0:1].cpu() for k, v in pre_g.items() if k in ("dq", "dk")}
        pp_got.update({k: pre_g[k].cpu() for k in ("da", "db", "dA_log", "ddt_bias")})
        pp_in = (dqn.cpu(), dkn.cpu(), dgp.cpu(), dbp.cpu())
        del rd, outr, hTr, pre_out, pre_g, dqn, dkn, dgp, dbp

        def pre_check():
            r = oracle.preprocess_backward(rw.q, rw.k, rw.g, rw.beta, *pp_in, A_log=rw.meta["A_log"],
                                           dt_bias=rw.meta["dt_bias"], norm_qk=True)
            out = {k: rel(pp_got[k].numpy(), r[k][:, 0:1]) for k in ("dq", "dk")}
            out.update({k: rel(pp_got[k].numpy(), r[k]) for k in ("da", "db", "dA_log", "ddt_bias")})
            return {"backward": out}
        checks.append((rec_pp, "parity", pre_check))
        progress("preprocessing passes %.3f / %.3f ms" % (rec_pp["forward"]["ms_median"],
                                                         rec_pp["backward"]["ms_median"]))

        def fused_check():
            ro, rh = oracle.gdn_forward_fused(rw.q, rw.k, rw.v, rw.g, rw.beta, rw.cu_seqlens, rw.h0,
                                              A_log=rw.meta["A_log"], dt_bias=rw.meta["dt_bias"])
            return {"all_heads": {"out": seq_rel_max(got_fo.float().numpy(), ro, rw.cu_seqlens.tolist()),
                                  "state": state_rel_max(got_fs.numpy(), rh)}}
        checks.append((rec_f, "parity", fused_check))
        progress("fused preprocessing %.3f ms" % msf)

        # The short convolution on the q|k|v channels of the benchmark batch (HBM-bound:
        # x read once, y written once) and as one decode step at B = 256.
        C, K = 2 * 16 * 128 + 32 * 128, 4
        gen = torch.Generator().manual_seed(1005)
        xc = torch.randn((T, C), generator=gen).to(torch.bfloat16).to(dev)
        wc = (0.5 * torch.randn((C, K), generator=gen)).to(dev)
        bc = (0.1 * torch.randn((C,), generator=gen)).to(dev)
        pool_c = torch.zeros((w.n_seqs, C, K - 1), dtype=torch.bfloat16, device=dev)
        yc = torch.empty_like(xc)

        def conv(_i):
            gdn.gdn_short_conv(xc, wc, d["cu"], pool_c, bias=bc, y=yc, stream=stream)

        per_c, _, _ = time_launches(conv, args.steps, 5, stream)
        msc = float(np.median(per_c))
        cbytes = 2.0 * T * C * 2 + 2.0 * w.n_seqs * C * (K - 1) * 2
        Bd = 256
        xd = xc[:Bd].contiguous()
        cud = torch.arange(Bd + 1, dtype=torch.int32, device=dev)
        pool_d = torch.zeros((Bd, C, K - 1), dtype=torch.bfloat16, device=dev)
        yd = torch.empty_like(xd)

        def conv_dec(_i):
            gdn.gdn_short_conv(xd, wc, cud, pool_d, bias=bc, y=yd, stream=stream)

        per_cd, _, _ = time_launches(conv_dec, max(args.steps, 100), 20, stream, hold=hold, hold_ms=40.0)
        rec_c = {"tokens": T, "channels": C, "taps": K, "ms_median": msc, "tokens_per_s": T / (msc / 1e3),
                 "launch_ms_percentiles": percentiles(per_c),
                 "roofline": {"bound": "hbm", "achieved": cbytes / (msc / 1e3) / 1e9, "peak": HBM_PEAK_GBS,
                              "unit": "GB/s", "frac": cbytes / (msc / 1e3) / 1e9 / HBM_PEAK_GBS,
                              "bytes_per_launch": cbytes, "traffic": traffic_from_profile("short_conv", src_hash)}}
        workloads["short_conv_varlen"] = rec_c
        # one checked run from the zero state, on the first 256 channels
        pool_c.zero_()
        conv(0)
        torch.cuda.synchronize()
        got_y = yc[:, :256].cpu()
        xc256, wc256, bc256 = xc[:, :256].cpu(), wc[:256].cpu(), bc[:256].cpu()
        workloads["short_conv_decode_B256"] = {"latency_us_mean": float(np.mean(per_cd)) * 1e3,
                                               "launch_ms_percentiles": percentiles(per_cd)}
        xc_keep = xc.cpu()
        del xc, yc, pool_c, xd, yd, pool_d

        def conv_check():
            ry, _ = oracle.short_conv(xc256, wc256, w.cu_seqlens, bias=bc256, state=torch.zeros((w.n_seqs, 256, K - 1)))
            return {"y_first256": rel(got_y.float().numpy(), ry)}
        checks.append((rec_c, "parity", conv_check))
        progress("short convolution %.3f ms" % msc)

        # its backward on the same shape (x bf16 read, dy fp32 read, dx fp32 written)
        xc = xc_keep.to(dev)
        pool_c = torch.zeros((w.n_seqs, C, K - 1), dtype=torch.bfloat16, device=dev)
        dyc = torch.randn((T, C), generator=torch.Generator().manual_seed(1009)).to(dev)
        cg = gdn.gdn_short_conv_backward(xc, wc, d["cu"], pool_c, dyc, bias=bc, stream=stream)

        def conv_bwd(_i):
            gdn.gdn_short_conv_backward(xc, wc, d["cu"], pool_c, dyc, bias=bc, grads=cg, stream=stream)

        per_cb, _, _ = time_launches(conv_bwd, args.steps, 5, stream)
        mscb = float(np.median(per_cb))
        cbb = T * C * (2.0 + 4.0 + 4.0)
        rec_cb = {"tokens": T, "channels": C, "taps": K, "ms_median": mscb, "launch_ms_percentiles": percentiles(per_cb),
                  "roofline": {"bound": "hbm", "achieved": cbb / (mscb / 1e3) / 1e9, "peak": HBM_PEAK_GBS,
                               "unit": "GB/s", "frac": cbb / (mscb / 1e3) / 1e9 / HBM_PEAK_GBS,
                               "bytes_per_launch": cbb,
                               "traffic": traffic_from_profile("short_conv_backward", src_hash)}}
        workloads["short_conv_backward"] = rec_cb
        cg_got = {"dx": cg["dx"][:, :256].cpu(), "dw": cg["dw"][:256].cpu(), "dbias": cg["dbias"][:256].cpu(),
                  "dstate": cg["dstate"][:, :256].cpu()}
        dy256 = dyc[:, :256].cpu()
        del xc, pool_c, dyc, cg

        def conv_bwd_check():
            r = oracle.short_conv_backward(xc256, wc256, w.cu_seqlens, dy256, bias=bc256,
                                           state=torch.zeros((w.n_seqs, 256, K - 1)))
            return {"first256": {k: rel(cg_got[k].numpy(), r[k]) for k in cg_got}}
        checks.append((rec_cb, "parity", conv_bwd_check))
        progress("short convolution backward %.3f ms" % mscb)

        lc = synth.long_context(1003)
        prefill_line("long_context_65536", lc)
        prefill_line("long_context_65536_as_8x8192", lc, chunks=8)
        # The chunked form (gdn_fwd_chunked, its automatic waves per tile) on the same
        # sequence, from the zero state: the same 7 dk dv flops per token.
        dl = [t.to(dev) for t in (lc.q, lc.k, lc.v, lc.g, lc.beta)]
        cul = lc.cu_seqlens.to(dev)
        Tl = lc.total_tokens
        ol = torch.empty((Tl, 32, 128), dtype=torch.bfloat16, device=dev)
        ws_l = torch.empty(gdn.gdn_chunked_workspace_size(gdn.make_dims(dl[0], dl[2], 1, Tl)),
                           dtype=torch.uint8, device=dev)

        def chunked_long(_i):
            gdn.gdn_fwd_chunked(*dl, cul, None, out=ol, stream=stream, workspace=ws_l)

        per_cl, _, _ = time_launches(chunked_long, 5, 2, stream)
        mscl = float(np.median(per_cl))
        got_cl = ol.cpu()
        rec_cl = {"tokens": Tl, "n_seqs": 1, "chunk": 16, "ms_median": mscl, "ms_mean": float(np.mean(per_cl)),
                  "launch_ms_percentiles": percentiles(per_cl), "tokens_per_s": Tl / (mscl / 1e3),
                  "roofline_frac": FLOPS_PER_TOKEN * Tl / (mscl / 1e3) / 1e12 / FP32_VECTOR_PEAK_TFLOPS}
        workloads["chunked_long_context_65536"] = rec_cl
        del dl, ol, ws_l

        def chunked_long_check(lc=lc, got=got_cl):
            ro, _ = oracle.gdn_forward(lc.q, lc.k, lc.v, lc.g, lc.beta, lc.cu_seqlens, lc.h0)
            return {"all_heads": {"out": seq_rel_max(got.float().numpy(), ro, lc.cu_seqlens.tolist())}}
        checks.append((rec_cl, "parity", chunked_long_check))
        progress("chunked form, long context %.3f ms" % mscl)
        del lc
        prefill_line("mixed_batch_64", synth.mixed_batch(1004))

        # The chunked form with a replaying decode (gdn_fwd_chunked, matrix cores for the
        # products with the state): the benchmark batch as one prefill from h0, and one
        # in-place decode step at B = 256 from states a chunked prefill left at every
        # position of an open chunk (512 + n % 16 tokens for sequence n); the same
        # 7 dk dv flops per token as the recurrent lines.
        st_in = gdn.make_chunk_state(w.n_seqs, 16, 32, 128, 128, dev, h0=d["h0"])
        st_out = gdn.make_chunk_state(w.n_seqs, 16, 32, 128, 128, dev)
        och = torch.empty((T, 32, 128), dtype=torch.bfloat16, device=dev)
        ws_c = torch.empty(gdn.gdn_chunked_workspace_size(gdn.make_dims(d["q"], d["v"], w.n_seqs, T)),
                           dtype=torch.uint8, device=dev)

        def chunked(_i):
            gdn.gdn_fwd_chunked(d["q"], d["k"], d["v"], d["g"], d["beta"], d["cu"], st_in, st_out, out=och,
                                stream=stream, workspace=ws_c)

        per_ch, _, _ = time_launches(chunked, args.steps, 3, stream)
        msch = float(np.median(per_ch))
        chunked(0)
        torch.cuda.synchronize()
        got_ch = och.cpu()
        Bc = 256
        hl = synth.make_workload(1012, [512 + n % 16 + 1 for n in range(Bc)])
        cuh = hl.cu_seqlens.tolist()
        pre_i = torch.cat([torch.arange(cuh[n], cuh[n + 1] - 1) for n in range(Bc)])
        last_i = torch.tensor([cuh[n + 1] - 1 for n in range(Bc)])
        hp = [getattr(hl, nm)[pre_i].contiguous().to(dev) for nm in ("q", "k", "v", "g", "beta")]
        cu_p = synth.cu_from_lengths([512 + n % 16 for n in range(Bc)]).to(dev)
        _, st_d = gdn.gdn_fwd_chunked(*hp, cu_p, None, stream=stream)
        del hp
        dcd = [getattr(hl, nm)[last_i].contiguous().to(dev) for nm in ("q", "k", "v", "g", "beta")]
        cu_d = torch.arange(Bc + 1, dtype=torch.int32, device=dev)
        ws_d = torch.empty(gdn.gdn_chunked_workspace_size(gdn.make_dims(dcd[0], dcd[2], Bc, Bc)),
                           dtype=torch.uint8, device=dev)
        ocd = torch.empty((Bc, 32, 128), dtype=torch.bfloat16, device=dev)
        cnt_out = torch.empty((Bc,), dtype=torch.int32, device=dev)
        torch.cuda.synchronize()
        # the checked step first (the timed ones then repeat it in place on the same states)
        work = {k_: v_.clone() for k_, v_ in st_d.items()}
        gdn.gdn_fwd_chunked(*dcd, cu_d, work, out=ocd, stream=stream, workspace=ws_d, inplace=True,
                            count_out=cnt_out)
        torch.cuda.synchronize()
        got_cd = ocd[:4].cpu()
        del work

        # the same step without cu_seqlens (one token per sequence: the decode kernel)
        work = {k_: v_.clone() for k_, v_ in st_d.items()}
        ocd2 = torch.empty_like(ocd)
        gdn.gdn_fwd_chunked(*dcd, None, work, out=ocd2, stream=stream, workspace=ws_d, inplace=True,
                            count_out=cnt_out)
        torch.cuda.synchronize()
        no_cu_same_bits = bool(torch.equal(ocd.view(torch.int16), ocd2.view(torch.int16)))
        del work, ocd2

        def chunked_dec(_i):
            gdn.gdn_fwd_chunked(*dcd, None, st_d, out=ocd, stream=stream, workspace=ws_d, inplace=True,
                                count_out=cnt_out)

        def chunked_dec_cu(_i):
            gdn.gdn_fwd_chunked(*dcd, cu_d, st_d, out=ocd, stream=stream, workspace=ws_d, inplace=True,
                                count_out=cnt_out)

        per_cd2, _, _ = time_launches(chunked_dec, max(args.steps, 50), 10, stream, hold=hold, hold_ms=40.0)
        per_cd3, _, _ = time_launches(chunked_dec_cu, max(args.steps, 50), 10, stream, hold=hold, hold_ms=40.0)
        rec_ch = {"tokens": T, "n_seqs": w.n_seqs, "chunk": 16, "ms_median": msch, "tokens_per_s": T / (msch / 1e3),
                  "launch_ms_percentiles": percentiles(per_ch),
                  "roofline_frac": FLOPS_PER_TOKEN * T / (msch / 1e3) / 1e12 / FP32_VECTOR_PEAK_TFLOPS,
                  "decode_B256_inplace_us_mean": float(np.mean(per_cd2)) * 1e3,
                  "decode_B256_launch_ms_percentiles": percentiles(per_cd2),
                  "decode_B256_inplace_with_cu_seqlens_us_mean": float(np.mean(per_cd3)) * 1e3,
                  "decode_without_cu_seqlens_same_bits": no_cu_same_bits,
                  "decode_states": "chunked prefill of 512 + n % 16 tokens (every open-chunk position)"}
        workloads["chunked_prefill_replay"] = rec_ch
        del st_in, st_out, och, st_d, ocd, ws_c, ws_d

        def chunked_check():
            ro, rh = oracle.gdn_forward(w.q, w.k, w.v, w.g, w.beta, w.cu_seqlens, w.h0)
            res = {"all_heads": {"out": seq_rel_max(got_ch.float().numpy(), ro, w.cu_seqlens.tolist())}}
            four = synth.select(hl, [0, 1, 2, 3])
            ro4, _ = oracle.gdn_forward(four.q, four.k, four.v, four.g, four.beta, four.cu_seqlens, None)
            c4 = four.cu_seqlens.tolist()
            ro_last = ro4[[c4[i + 1] - 1 for i in range(4)]]
            res["decode_B256_first4"] = {"out": seq_rel_max(got_cd.float().numpy(), ro_last, list(range(5)))}
            return res
        checks.append((rec_ch, "parity", chunked_check))
        progress("chunked form %.3f ms, decode B=256 %.1f us" % (msch, float(np.mean(per_cd2)) * 1e3))

        # The backward (gdn_bwd_varlen) on the benchmark batch, dL/dout ~ N(0, 1) in
        # bf16 and dL/dhT ~ N(0, 1), against the FP32-VALU roofline on its algorithmic
        # work: 18 flops per state element and token (recompute p and the write: 5;
        # the adjoint D += dO q^T, du = D k, D -= beta du k^T, D *= a: 7; dq = S^T dO,
        # dk = D^T u + S^T w: 6).
        gen = torch.Generator().manual_seed(1006)
        dout_c = torch.randn(tuple(w.v.shape), generator=gen).to(torch.bfloat16)
        dhT_c = torch.randn((w.n_seqs, 32, 128, 128), generator=gen)
        dout_d, dhT_d = dout_c.to(dev), dhT_c.to(dev)
        bdims = gdn.make_dims(d["q"], d["v"], w.n_seqs, T)
        ws = torch.empty(gdn.gdn_bwd_workspace_size(bdims), dtype=torch.uint8, device=dev)
        grads = gdn.gdn_bwd_varlen(d["q"], d["k"], d["v"], d["g"], d["beta"], d["h0"], d["cu"], dout_d, dhT_d,
                                   workspace=ws, stream=stream)

        def bwd(_i):
            gdn.gdn_bwd_varlen(d["q"], d["k"], d["v"], d["g"], d["beta"], d["h0"], d["cu"], dout_d, dhT_d,
                               workspace=ws, grads=grads, stream=stream)

        bflops = 18.0 * 128 * 128 * 32 * T
        ws_b_bytes = int(ws.numel())
        # the chunked backward (gdn_bwd_chunked, matrix cores) on the same inputs
        ws_cb = torch.empty(gdn.gdn_bwd_chunked_workspace_size(bdims), dtype=torch.uint8, device=dev)
        grads_c = gdn.gdn_bwd_chunked(d["q"], d["k"], d["v"], d["g"], d["beta"], d["h0"], d["cu"], dout_d, dhT_d,
                                      workspace=ws_cb, stream=stream)

        def bwd_chunked(_i):
            gdn.gdn_bwd_chunked(d["q"], d["k"], d["v"], d["g"], d["beta"], d["h0"], d["cu"], dout_d, dhT_d,
                                workspace=ws_cb, grads=grads_c, stream=stream)

        per_bc, _, _ = time_launches(bwd_chunked, args.steps, 3, stream)
        msbc = float(np.median(per_bc))
        got_gc = {"dq": grads_c["dq"][:, 0:1].cpu(), "dk": grads_c["dk"][:, 0:1].cpu(),
                  "dv": grads_c["dv"][:, 0:2].cpu(), "dbeta": grads_c["dbeta"][:, 0:2].cpu(),
                  "dg": grads_c["dg"][:, 0:2].cpu(), "dh0": grads_c["dh0"][:, 0:2].cpu()}
        rec_bc = {"tokens": T, "n_seqs": w.n_seqs, "ms_median": msbc, "tokens_per_s": T / (msbc / 1e3),
                  "launch_ms_percentiles": percentiles(per_bc), "launches": 5,
                  "workspace_bytes": int(ws_cb.numel()),
                  "roofline": {"bound": "mfma", "achieved": bflops / (msbc / 1e3) / 1e12,
                               "peak": FP32_MATRIX_PEAK_TFLOPS, "unit": "TFLOP/s",
                               "frac": bflops / (msbc / 1e3) / 1e12 / FP32_MATRIX_PEAK_TFLOPS,
                               "flops_per_launch": bflops,
                               "traffic": traffic_from_profile("backward_chunked", src_hash)}}
        workloads["backward_chunked_prefill"] = rec_bc
        del ws_cb, grads_c

        # The recurrent backward, the training forward (also saves p_t) and the backward
        # fed its p_t are timed last, right before the benchmark step, so that the
        # step's warm-ups start on a chip under load of the same (vector ALU) kind:
        # after even a few idle milliseconds the clock needs tens of milliseconds of
        # load to climb back.  The checked gradients are those of the plain backward,
        # formed and copied only after the step.
        per_b, _, _ = time_launches(bwd, args.steps, 3, stream)
        msb = float(np.median(per_b))
        out_t = torch.empty((T, 32, 128), dtype=torch.bfloat16, device=dev)
        hT_t = torch.empty((w.n_seqs, 32, 128, 128), dtype=torch.float32, device=dev)
        sp_t = torch.empty((T, 32, 128), dtype=torch.float32, device=dev)

        def fwd_train(_i):
            gdn.gdn_fwd_varlen_train(d["q"], d["k"], d["v"], d["g"], d["beta"], d["h0"], d["cu"], out=out_t, hT=hT_t,
                                     saved_p=sp_t, stream=stream)

        per_ft, _, _ = time_launches(fwd_train, args.steps, 3, stream)

        def bwd_saved(_i):
            gdn.gdn_bwd_varlen(d["q"], d["k"], d["v"], d["g"], d["beta"], d["h0"], d["cu"], dout_d, dhT_d,
                               workspace=ws, grads=grads, stream=stream, saved_p=sp_t, hT=hT_t)

        per_bs, _, _ = time_launches(bwd_saved, args.steps, 3, stream)

        def copy_bwd_grads():
            bwd(0)
            torch.cuda.synchronize()
            got_g.update({"dq": grads["dq"][:, 0:1].cpu(), "dk": grads["dk"][:, 0:1].cpu(),
                          "dv": grads["dv"][:, 0:2].cpu(), "dbeta": grads["dbeta"][:, 0:2].cpu(),
                          "dg": grads["dg"][:, 0:2].cpu(), "dh0": grads["dh0"][:, 0:2].cpu()})
        late_copies.append(copy_bwd_grads)
        rec_b = {"tokens": T, "n_seqs": w.n_seqs, "ms_median": msb, "tokens_per_s": T / (msb / 1e3),
                 "launch_ms_percentiles": percentiles(per_b),
                 "launches": 6, "workspace_bytes": ws_b_bytes,
                 "train_forward_ms_median": float(np.median(per_ft)),
                 "ms_median_with_saved_p": float(np.median(per_bs)),
                 "roofline": {"bound": "alu", "achieved": bflops / (msb / 1e3) / 1e12, "peak": FP32_VECTOR_PEAK_TFLOPS,
                              "unit": "TFLOP/s", "frac": bflops / (msb / 1e3) / 1e12 / FP32_VECTOR_PEAK_TFLOPS,
                              "flops_per_launch": bflops}}
        workloads["backward_varlen_prefill"] = rec_b
        bwd_ref = {}

        def bwd_oracle():
            if not bwd_ref:
                s0 = synth.head_slice(w, 0)
                bwd_ref.update(oracle.gdn_backward(s0.q, s0.k, s0.v, s0.g, s0.beta, s0.cu_seqlens,
                                                   dout_c[:, 0:2].contiguous(), h0=s0.h0,
                                                   dhT=dhT_c[:, 0:2].contiguous()))
            return bwd_ref

        def bwd_check():
            rb = bwd_oracle()
            return {"kh0_grads": {k: rel(v.numpy(), rb[k]) for k, v in got_g.items()}}

        def bwd_chunked_check():
            rb = bwd_oracle()
            return {"kh0_grads": {k: rel(v.numpy(), rb[k]) for k, v in got_gc.items()}}
        checks.append((rec_b, "parity", bwd_check))
        checks.append((rec_bc, "parity", bwd_chunked_check))
        progress("backward %.3f ms, chunked backward %.3f ms" % (msb, msbc))

    # ------------------------------------------------ the benchmark step
    # W warm-up launches queued right before the K timed ones; then the timed
    # outputs are re-checked against the oracle on every head.
    per, queued, span = time_launches(prefill, args.steps, args.warmup, stream)
    torch.cuda.synchronize()
    for copy in late_copies:
        copy()
    late_copies.clear()
    clock = gpu_clock()
    ms = float(np.mean(per))
    ms_med = float(np.median(per))
    flops = FLOPS_PER_TOKEN * T
    tokens_per_s = T / (ms / 1e3)
    traffic = traffic_from_profile("prefill", src_hash)
    roofline = {"bound": "alu", "achieved": flops / (ms / 1e3) / 1e12, "peak": FP32_VECTOR_PEAK_TFLOPS,
                "unit": "TFLOP/s", "frac": flops / (ms / 1e3) / 1e12 / FP32_VECTOR_PEAK_TFLOPS,
                "traffic": traffic, "kernel": "gdn_prefill_kernel", "flops_per_launch": flops,
                "launch_ms_mean": ms, "launch_ms_median": ms_med, "launch_ms_percentiles": percentiles(per),
                "launch_ms": [round(x, 5) for x in per], "launch_ms_back_to_back": span}
    got_out, got_hT = out.cpu(), hT.cpu()
    progress("prefill %.3f ms (mean of %d launches after %d warm-ups)" % (ms, args.steps, args.warmup))

    # ------------------------------------------------ oracle re-checks (CPU)
    ro, rh = oracle.gdn_forward(w.q, w.k, w.v, w.g, w.beta, w.cu_seqlens, w.h0)
    parity = {"all_heads": {"out": seq_rel_max(got_out.float().numpy(), ro, w.cu_seqlens.tolist()),
                            "state": state_rel_max(got_hT.numpy(), rh)}}
    del ro, rh
    parity_ok = parity["all_heads"]["out"] <= 2e-3 and parity["all_heads"]["state"] <= 1e-4
    for rec, key, fn in checks:
        rec[key] = fn()
        progress("checked %s" % (list(rec[key].keys()),))

    # ------------------------------------------------------- CPU baseline
    cpu = None
    if not args.no_cpu:
        # The fp64 oracle on every head of the same batch, repeated until about
        # --cpu-seconds of host time have passed (at least one full pass).
        threads = os.cpu_count() or 1
        passes, t0 = 0, time.perf_counter()
        while True:
            oracle.gdn_forward(w.q, w.k, w.v, w.g, w.beta, w.cu_seqlens, w.h0, n_threads=threads)
            passes += 1
            dt = time.perf_counter() - t0
            if dt >= args.cpu_seconds:
                break
        cpu = {"value": passes * T / dt, "unit": "tokens/s", "cores": min(threads, w.n_seqs * 32),
               "kind": "oracle", "cpu_model": cpu_model(),
               "sample": "fp64 oracle, all 32 value heads of the same 8-sequence batch (%d tokens), %d pass(es) "
                         "in %.1f s" % (T, passes, dt),
               "seconds": dt}

    # every line's parity re-check must pass as well
    def grads_ok(gr):  # the backward's gate: 1e-4 normwise for every gradient
        return all(e <= 1e-4 for e in gr.values())

    def line_ok(par):
        ok = True
        for v in par.values():
            if isinstance(v, dict) and ("out" in v or "state" in v):
                ok = ok and v.get("out", 0.0) <= 2e-3 and v.get("state", 0.0) <= 1e-4
            elif isinstance(v, dict):  # gradients
                ok = ok and grads_ok(v)
            else:
                ok = ok and v <= 2e-3
        return ok
    for rec in list((workloads or {}).values()) + ([decode] if decode else []):
        if isinstance(rec, dict) and "parity" in rec:
            parity_ok = parity_ok and line_ok(rec["parity"])
    if decode:
        parity_ok = parity_ok and decode["bitwise_across_batch_sizes"]
    if workloads and "chunked_prefill_replay" in workloads:
        parity_ok = parity_ok and workloads["chunked_prefill_replay"]["decode_without_cu_seqlens_same_bits"]

    line = {
        "metric": METRIC,
        "value": tokens_per_s,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic (seeded; q,k L2-normalised N(0,1), v N(0,1), g=-softplus(N), beta=sigmoid(N))",
        "config": {"workload": w.name, "lengths": w.lengths, "total_tokens": T, "hk": 16, "hv": 32, "dk": 128,
                   "dv": 128, "io": "bf16", "state": "fp32", "seed": 1001},
        "roofline": roofline,
        "cpu_baseline": cpu,
        "decode": decode,
        "workloads": workloads,
        "parity": {"ok": parity_ok, "max_rel_err": parity},
        "kernel_source_hash": src_hash,
        "host_queue_s_timed": queued,
        "gpu_clock_after_timing": clock,
        "device": torch.cuda.get_device_name(0),
    }
    print(json.dumps(line), flush=True)
    if not parity_ok:
        sys.exit(1)


if __name__ == "__main__":
    main()
