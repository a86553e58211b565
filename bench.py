#!/usr/bin/env python3
"""Benchmark of the batch-invariant Gated DeltaNet recurrent forward on one MI355X.

A step is one varlen prefill pass (gdn_fwd_varlen) over the 8-sequence batch with
lengths drawn uniformly from [256, 4096] (16 query/key heads, 32 value heads,
dk = dv = 128, bf16 q/k/v/out, fp32 gates and state, random initial states).
``value`` is that pass's throughput in tokens/s with every input already in HBM.

Also reported on the same line:
  roofline      prefill kernel against the fp32 vector peak (7 dk dv flops per
                token and value head: decay, key read-out, rank-1 write, query
                read-out), from per-launch HIP events on the launch stream;
  decode        one decode step at B = 64 and 256 against the HBM peak (state
                read + written in place), and its latency at B = 1 and 8, rotating
                over state pools of >= 1 GiB so the 256 MB Infinity Cache cannot
                hold them;
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
  parity        the timed outputs re-checked against the oracle (sampled heads).

Usage: python bench.py [--gpus 1] [--steps 20] [--warmup 50] [--no-cpu] [--no-decode] [--no-workloads]
(the warm-up also lets the GPU clock settle: the first ~20 launches run up to 25% slower)
"""
import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

FP32_VECTOR_PEAK_TFLOPS = 157.3   # MI355X: 256 CUs x 2.4 GHz x 256 flop/clk
HBM_PEAK_GBS = 8000.0             # MI355X HBM3E
METRIC = "GDN recurrent fwd tokens/s (prefill, decode) + % HBM/FP32-VALU roofline"


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


def time_launches(fn, steps, warmup, stream):
    """Per-launch durations (ms) from HIP events recorded on the launch stream."""
    import torch
    for _ in range(warmup):
        fn(0)
    torch.cuda.synchronize()
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    t0 = time.perf_counter()
    for i in range(steps):
        starts[i].record(stream)
        fn(i)
        ends[i].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    return [s.elapsed_time(e) for s, e in zip(starts, ends)], wall


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def rel(x, r):
    import numpy as np
    x = np.asarray(x, dtype=np.float64)
    r = np.asarray(r, dtype=np.float64)
    return float(np.linalg.norm(x - r) / max(np.linalg.norm(r), 1e-300))


def head_parity(synth, oracle, wl, out, hT, kh, fused=None):
    """Normwise errors of key head kh's value heads against the fp64 oracle."""
    s = synth.head_slice(wl, kh)
    G = out.shape[1] // wl.q.shape[1]
    vs = slice(G * kh, G * kh + G)
    if fused is None:
        ro, rh = oracle.gdn_forward(s.q, s.k, s.v, s.g, s.beta, s.cu_seqlens, s.h0)
    else:
        ro, rh = oracle.gdn_forward_fused(s.q, s.k, s.v, s.g, s.beta, s.cu_seqlens, s.h0,
                                          A_log=fused[0][vs], dt_bias=fused[1][vs])
    return {"out": rel(out[:, vs].float().cpu().numpy(), ro), "state": rel(hT[:, vs].cpu().numpy(), rh)}


COPY_BYTES = 1 << 30  # calibration copy: 1 GiB read + 1 GiB written


def pmc_pass(dev, stream):
    """One launch of each kernel (prefill, decode at B = 256, the short convolution
    and its state update, the backward's six), preceded by a plain device copy of COPY_BYTES whose
    FETCH_SIZE / WRITE_SIZE readings calibrate the counters' units."""
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
    del xc, pool_c
    gen = torch.Generator().manual_seed(1006)  # the backward, as in its benchmark line
    dout = torch.randn(tuple(w.v.shape), generator=gen).to(torch.bfloat16).to(dev)
    dhT = torch.randn((w.n_seqs, 32, 128, 128), generator=gen).to(dev)
    gdn.gdn_bwd_varlen(*d, dout, dhT, stream=stream)
    torch.cuda.synchronize()
    print("pmc pass: copy %d bytes, prefill %d tokens, decode B=%d, conv %d channels, backward" % (
        COPY_BYTES, w.total_tokens, B, C), flush=True)


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

    # ------------------------------------------------------------ prefill
    w = synth.varlen_prefill(1001)
    T = w.total_tokens
    d = dict(q=w.q.to(dev), k=w.k.to(dev), v=w.v.to(dev), g=w.g.to(dev), beta=w.beta.to(dev),
             h0=w.h0.to(dev), cu=w.cu_seqlens.to(dev))
    out = torch.empty((T, 32, 128), dtype=torch.bfloat16, device=dev)
    hT = torch.empty((w.n_seqs, 32, 128, 128), dtype=torch.float32, device=dev)

    def prefill(_i):
        gdn.gdn_fwd_varlen(d["q"], d["k"], d["v"], d["g"], d["beta"], d["h0"], d["cu"], out=out, hT=hT,
                           stream=stream)

    per, wall = time_launches(prefill, args.steps, args.warmup, stream)
    ms = float(np.mean(per))
    ms_med = float(np.median(per))
    flops = 7.0 * 128 * 128 * 32 * T
    tokens_per_s = T / (ms / 1e3)
    src_hash = kernel_source_hash()
    traffic = traffic_from_profile("prefill", src_hash)
    roofline = {"bound": "alu", "achieved": flops / (ms / 1e3) / 1e12, "peak": FP32_VECTOR_PEAK_TFLOPS,
                "unit": "TFLOP/s", "frac": flops / (ms / 1e3) / 1e12 / FP32_VECTOR_PEAK_TFLOPS,
                "traffic": traffic, "kernel": "gdn_prefill_kernel", "flops_per_launch": flops,
                "launch_ms_mean": ms, "launch_ms_median": ms_med}

    # parity of the timed outputs (sampled key heads; the oracle is test infrastructure)
    parity = {}
    torch.cuda.synchronize()
    for kh in (0, 15):
        s = synth.head_slice(w, kh)
        ro, rh = oracle.gdn_forward(s.q, s.k, s.v, s.g, s.beta, s.cu_seqlens, s.h0)
        vs = slice(2 * kh, 2 * kh + 2)
        parity["kh%d" % kh] = {"out": rel(out[:, vs].float().cpu().numpy(), ro),
                               "state": rel(hT[:, vs].cpu().numpy(), rh)}
    parity_ok = all(p["out"] <= 2e-3 and p["state"] <= 1e-4 for p in parity.values())
    progress("prefill %.3f ms (mean of %d launches), parity %s" % (ms, args.steps, parity_ok))

    # ------------------------------------------------------------- decode
    decode = None
    if not args.no_decode:
        decode = {}
        for B in (1, 8, 64, 256):
            bytes_state = B * 32 * 128 * 128 * 4
            n_pools = max(4, int(np.ceil((1 << 30) / bytes_state)))
            pools = [torch.randn((B, 32, 128, 128), device=dev) * 0.1 for _ in range(n_pools)]
            dw = synth.make_workload(2000 + B, [1] * B)
            dq, dk_, dv_, dg, db = (t.to(dev) for t in (dw.q, dw.k, dw.v, dw.g, dw.beta))
            dout = torch.empty((B, 32, 128), dtype=torch.bfloat16, device=dev)

            def dec(i, B=B):
                gdn.gdn_decode_step(dq, dk_, dv_, dg, db, pools[i % n_pools], out=dout, stream=stream)

            steps = max(args.steps, 2 * n_pools)
            per_d, _ = time_launches(dec, steps, max(args.warmup, n_pools), stream)
            ms_d = float(np.mean(per_d))
            alg_bytes = B * (2 * 32 * 128 * 128 * 4 + 24832)
            # one checked step: rows 0..3 against the oracle from the same states
            nb = min(4, B)
            pchk = pools[0].clone()
            h0c = pchk[:nb].cpu()
            ochk = gdn.gdn_decode_step(dq, dk_, dv_, dg, db, pchk, stream=stream)
            torch.cuda.synchronize()
            ro_d, rh_d = oracle.gdn_forward(dw.q[:nb], dw.k[:nb], dw.v[:nb], dw.g[:nb], dw.beta[:nb],
                                            synth.cu_from_lengths([1] * nb), h0c)
            dpar = {"out": rel(ochk[:nb].float().cpu().numpy(), ro_d), "state": rel(pchk[:nb].cpu().numpy(), rh_d)}
            decode["B%d" % B] = {"tokens_per_s": B / (ms_d / 1e3), "launch_ms_mean": ms_d, "parity": dpar,
                                 "latency_us_median": float(np.median(per_d)) * 1e3,
                                 "launch_ms_median": float(np.median(per_d)),
                                 "roofline": {"bound": "hbm", "achieved": alg_bytes / (ms_d / 1e3) / 1e9,
                                              "peak": HBM_PEAK_GBS, "unit": "GB/s",
                                              "frac": alg_bytes / (ms_d / 1e3) / 1e9 / HBM_PEAK_GBS,
                                              "traffic": traffic_from_profile("decode_B%d" % B, src_hash),
                                              "bytes_per_launch": alg_bytes},
                                 "state_pools": n_pools}
            del pools
            progress("decode B=%d %.1f us" % (B, ms_d * 1e3))

    # ------------------------------------------------ other prefill workloads
    workloads = None
    if not args.no_workloads:
        workloads = {}

        def prefill_line(name, wl, chunks=1, parity_heads=(0,)):
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
            per_w, _ = time_launches(run, reps, 3, stream)
            msw = float(np.median(per_w))
            # one checked run from the original initial states (the timed runs carried them on)
            state.copy_(wl.h0.to(dev) if wl.h0 is not None else torch.zeros_like(state))
            run(0)
            torch.cuda.synchronize()
            par = {"kh%d" % kh: head_parity(synth, oracle, wl, outw, state, kh) for kh in parity_heads}
            fl = 7.0 * 128 * 128 * 32 * Tw
            workloads[name] = {"tokens": Tw, "n_seqs": wl.n_seqs, "chunks": chunks, "ms_median": msw,
                               "tokens_per_s": Tw / (msw / 1e3),
                               "roofline_frac": fl / (msw / 1e3) / 1e12 / FP32_VECTOR_PEAK_TFLOPS,
                               "plan": list(gdn.gdn_query_plan(gdn.make_dims(dd[0], dd[2], wl.n_seqs if chunks == 1 else 1,
                                                                             Tw // chunks))),
                               "parity": par}
            del dd, outw, state
            progress("%s %.3f ms" % (name, msw))

        # The benchmark batch through the state pool with a snapshot every 256 tokens
        # (prefix caching): 8 source slots, 8 destination slots, one slot per snapshot.
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

        per_p, _ = time_launches(pooled, args.steps, 5, stream)
        msp = float(np.median(per_p))
        torch.cuda.synchronize()
        workloads["varlen_prefill_pool_snapshots_256"] = {
            "tokens": T, "n_seqs": N, "snapshots": int(sum(L // blk for L in w.lengths)), "ms_median": msp,
            "tokens_per_s": T / (msp / 1e3), "roofline_frac": flops / (msp / 1e3) / 1e12 / FP32_VECTOR_PEAK_TFLOPS,
            "same_bits_as_plain": bool(torch.equal(outp.view(torch.int16), out.view(torch.int16)))}
        del pool, outp
        progress("pool with snapshots %.3f ms" % msp)

        # The benchmark batch's shape on raw inputs with both fused preprocessing steps
        # (in-kernel q/k L2 norm; gate and beta from logits).
        rw = synth.make_raw_workload(1001, w.lengths, h0_std=0.1)
        rd = [t.to(dev) for t in (rw.q, rw.k, rw.v, rw.g, rw.beta, rw.h0, rw.cu_seqlens)]
        A_log, dt_bias = rw.meta["A_log"].to(dev), rw.meta["dt_bias"].to(dev)
        pre = gdn.make_preproc(norm_qk=True, eps=1e-6, A_log=A_log, dt_bias=dt_bias)
        outr = torch.empty_like(out)
        hTr = torch.empty_like(hT)

        def fused(_i):
            gdn.gdn_fwd_varlen(*rd, out=outr, hT=hTr, stream=stream, pre=pre)

        per_f, _ = time_launches(fused, args.steps, 5, stream)
        msf = float(np.median(per_f))
        workloads["varlen_prefill_fused_preprocessing"] = {
            "tokens": T, "n_seqs": w.n_seqs, "ms_median": msf, "tokens_per_s": T / (msf / 1e3),
            "roofline_frac": flops / (msf / 1e3) / 1e12 / FP32_VECTOR_PEAK_TFLOPS,
            "parity": {"kh0": head_parity(synth, oracle, rw, outr, hTr, 0,
                                          fused=(rw.meta["A_log"], rw.meta["dt_bias"]))}}
        del rd, outr, hTr
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

        per_c, _ = time_launches(conv, args.steps, 5, stream)
        msc = float(np.median(per_c))
        cbytes = 2.0 * T * C * 2 + 2.0 * w.n_seqs * C * (K - 1) * 2
        Bd = 256
        xd = xc[:Bd].contiguous()
        cud = torch.arange(Bd + 1, dtype=torch.int32, device=dev)
        pool_d = torch.zeros((Bd, C, K - 1), dtype=torch.bfloat16, device=dev)
        yd = torch.empty_like(xd)

        def conv_dec(_i):
            gdn.gdn_short_conv(xd, wc, cud, pool_d, bias=bc, y=yd, stream=stream)

        per_cd, _ = time_launches(conv_dec, args.steps, 5, stream)
        workloads["short_conv_varlen"] = {
            "tokens": T, "channels": C, "taps": K, "ms_median": msc, "tokens_per_s": T / (msc / 1e3),
            "roofline": {"bound": "hbm", "achieved": cbytes / (msc / 1e3) / 1e9, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": cbytes / (msc / 1e3) / 1e9 / HBM_PEAK_GBS, "bytes_per_launch": cbytes,
                         "traffic": traffic_from_profile("short_conv", src_hash)}}
        # one checked run from the zero state, on the first 256 channels
        pool_c.zero_()
        conv(0)
        torch.cuda.synchronize()
        ry, _ = oracle.short_conv(xc[:, :256].cpu(), wc[:256].cpu(), w.cu_seqlens, bias=bc[:256].cpu(),
                                  state=torch.zeros((w.n_seqs, 256, K - 1)))
        workloads["short_conv_varlen"]["parity"] = {"y_first256": rel(yc[:, :256].float().cpu().numpy(), ry)}
        workloads["short_conv_decode_B256"] = {"latency_us_median": float(np.median(per_cd)) * 1e3}
        del xc, yc, pool_c, xd, yd, pool_d
        progress("short convolution %.3f ms" % msc)

        lc = synth.long_context(1003)
        prefill_line("long_context_65536", lc)
        prefill_line("long_context_65536_as_8x8192", lc, chunks=8)
        del lc
        prefill_line("mixed_batch_64", synth.mixed_batch(1004), parity_heads=(0, 15))

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

        per_b, _ = time_launches(bwd, args.steps, 3, stream)
        msb = float(np.median(per_b))
        # the training forward (also saves p_t) and the backward fed its p_t
        out_t = torch.empty((T, 32, 128), dtype=torch.bfloat16, device=dev)
        hT_t = torch.empty((w.n_seqs, 32, 128, 128), dtype=torch.float32, device=dev)
        sp_t = torch.empty((T, 32, 128), dtype=torch.float32, device=dev)

        def fwd_train(_i):
            gdn.gdn_fwd_varlen_train(d["q"], d["k"], d["v"], d["g"], d["beta"], d["h0"], d["cu"], out=out_t, hT=hT_t,
                                     saved_p=sp_t, stream=stream)

        per_ft, _ = time_launches(fwd_train, args.steps, 3, stream)

        def bwd_saved(_i):
            gdn.gdn_bwd_varlen(d["q"], d["k"], d["v"], d["g"], d["beta"], d["h0"], d["cu"], dout_d, dhT_d,
                               workspace=ws, grads=grads, stream=stream, saved_p=sp_t, hT=hT_t)

        per_bs, _ = time_launches(bwd_saved, args.steps, 3, stream)
        bflops = 18.0 * 128 * 128 * 32 * T
        s0 = synth.head_slice(w, 0)
        rb = oracle.gdn_backward(s0.q, s0.k, s0.v, s0.g, s0.beta, s0.cu_seqlens, dout_c[:, 0:2].contiguous(),
                                 h0=s0.h0, dhT=dhT_c[:, 0:2].contiguous())
        got = {"dq": grads["dq"][:, 0:1], "dk": grads["dk"][:, 0:1], "dv": grads["dv"][:, 0:2],
               "dbeta": grads["dbeta"][:, 0:2], "dg": grads["dg"][:, 0:2], "dh0": grads["dh0"][:, 0:2]}
        workloads["backward_varlen_prefill"] = {
            "tokens": T, "n_seqs": w.n_seqs, "ms_median": msb, "tokens_per_s": T / (msb / 1e3),
            "launches": 6, "workspace_bytes": int(ws.numel()),
            "train_forward_ms_median": float(np.median(per_ft)),
            "ms_median_with_saved_p": float(np.median(per_bs)),
            "roofline": {"bound": "alu", "achieved": bflops / (msb / 1e3) / 1e12, "peak": FP32_VECTOR_PEAK_TFLOPS,
                         "unit": "TFLOP/s", "frac": bflops / (msb / 1e3) / 1e12 / FP32_VECTOR_PEAK_TFLOPS,
                         "flops_per_launch": bflops},
            "parity": {"kh0_grads": {k: rel(v.cpu().numpy(), rb[k]) for k, v in got.items()}}}
        del dout_d, dhT_d, ws, grads, out_t, hT_t, sp_t
        progress("backward %.3f ms" % msb)

        # The chunked form with a replaying decode (gdn_fwd_chunked): the benchmark
        # batch as one prefill from h0, and one decode step at B = 256 through the
        # chunked state; the same 7 dk dv flops per token as the recurrent lines.
        st_in = gdn.make_chunk_state(w.n_seqs, 16, 32, 128, 128, dev, h0=d["h0"])
        st_out = gdn.make_chunk_state(w.n_seqs, 16, 32, 128, 128, dev)
        och = torch.empty((T, 32, 128), dtype=torch.bfloat16, device=dev)

        def chunked(_i):
            gdn.gdn_fwd_chunked(d["q"], d["k"], d["v"], d["g"], d["beta"], d["cu"], st_in, st_out, out=och,
                                stream=stream)

        per_ch, _ = time_launches(chunked, args.steps, 3, stream)
        msch = float(np.median(per_ch))
        Bc = 256
        dwc = synth.make_workload(2000 + Bc, [1] * Bc)
        dcd = [t.to(dev) for t in (dwc.q, dwc.k, dwc.v, dwc.g, dwc.beta, dwc.cu_seqlens)]
        sts = [gdn.make_chunk_state(Bc, 16, 32, 128, 128, dev) for _ in range(2)]
        for s_ in sts:
            s_["S"].normal_(0.0, 0.1)
            s_["count"].fill_(7)
        ocd = torch.empty((Bc, 32, 128), dtype=torch.bfloat16, device=dev)

        def chunked_dec(_i):
            gdn.gdn_fwd_chunked(*dcd, sts[0], sts[1], out=ocd, stream=stream)

        per_cd2, _ = time_launches(chunked_dec, args.steps, 3, stream)
        chunked(0)
        torch.cuda.synchronize()
        s0 = synth.head_slice(w, 0)
        ro, _ = oracle.gdn_forward(s0.q, s0.k, s0.v, s0.g, s0.beta, s0.cu_seqlens, s0.h0)
        workloads["chunked_prefill_replay"] = {
            "tokens": T, "n_seqs": w.n_seqs, "chunk": 16, "ms_median": msch, "tokens_per_s": T / (msch / 1e3),
            "roofline_frac": flops / (msch / 1e3) / 1e12 / FP32_VECTOR_PEAK_TFLOPS,
            "decode_B256_latency_us_median": float(np.median(per_cd2)) * 1e3,
            "parity": {"kh0": {"out": rel(och[:, 0:2].float().cpu().numpy(), ro)}}}
        del st_in, st_out, och, sts, ocd
        progress("chunked form %.3f ms" % msch)

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
    def grads_ok(gr):  # the backward's gates: 1e-4 normwise, dg 1e-3
        return all(e <= (1e-3 if k == "dg" else 1e-4) for k, e in gr.items())

    def line_ok(par):
        return all((v.get("out", 0.0) <= 2e-3 and v.get("state", 0.0) <= 1e-4 and v.get("y_first256", 0.0) <= 2e-3)
                   if isinstance(v, dict) and "dq" not in v else (grads_ok(v) if isinstance(v, dict) else True)
                   for v in par.values())
    for rec in list((decode or {}).values()) + list((workloads or {}).values()):
        if "parity" in rec:
            par = rec["parity"]
            ok = line_ok(par) if any(isinstance(v, dict) for v in par.values()) else line_ok({"x": par})
            parity_ok = parity_ok and ok

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
        "wall_s_timed": wall,
        "device": torch.cuda.get_device_name(0),
    }
    print(json.dumps(line), flush=True)
    if not parity_ok:
        sys.exit(1)


if __name__ == "__main__":
    main()
