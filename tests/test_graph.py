"""Graph capture and replay of the library's launches.

The serving stacks in the pages replay captured graphs for decode, and require a
graph's results to equal the eager ones, with workspace and state buffers at
stable addresses and states updated in place (summary of "Finish RL Training
Faster: Bitwise-Consistent, High-Performance, Agent-Driven", section
"Consistency has several layers").  The library enqueues plain kernel launches on
the caller's stream and touches no other memory, so a captured prefill plus
decode step must replay with the eager bits, replay after replay, also after
the buffers' contents are replaced in place.
"""
import pytest
import torch

from gpu_helpers import bit_equal, say
from invariant_linear_attention_amd import synth

pytestmark = pytest.mark.gpu
DEV = "cuda"


def test_prefill_then_decode_graph_replays_eager_bits(gpu):
    w = synth.make_workload(301, [300, 17, 1000, 64], h0_std=0.1)          # 16/32 heads, dk = dv = 128, bf16
    dw = synth.make_workload(302, [1] * 4)                                 # one decode token per sequence
    h0 = w.h0.to(DEV)
    x = {n: getattr(w, n).to(DEV) for n in ("q", "k", "v", "g", "beta")}
    cu = w.cu_seqlens.to(DEV)
    y = {n: getattr(dw, n).to(DEV) for n in ("q", "k", "v", "g", "beta")}
    idx = torch.tensor([2, 0, 3, 1], dtype=torch.int32, device=DEV)       # a permuted pool
    out = torch.empty((w.total_tokens, 32, 128), dtype=torch.bfloat16, device=DEV)
    pool = torch.empty((4, 32, 128, 128), dtype=torch.float32, device=DEV)
    dout = torch.empty((4, 32, 128), dtype=torch.bfloat16, device=DEV)

    def step(stream=None):
        # prefill writes the pool's states from h0, then one decode step updates them in place
        gpu.gdn_fwd_varlen(x["q"], x["k"], x["v"], x["g"], x["beta"], h0, cu, out=out, hT=pool, stream=stream)
        gpu.gdn_decode_step(y["q"], y["k"], y["v"], y["g"], y["beta"], pool, state_idx=idx, out=dout,
                            stream=stream)

    def snapshot():
        torch.cuda.synchronize()
        return out.clone(), pool.clone(), dout.clone()

    step()
    eager = snapshot()

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.stream(side):
        with torch.cuda.graph(graph, stream=side):
            step()                       # only the library's two launches are recorded
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()

    for rep in range(3):
        out.fill_(0.0)                   # eager work between replays
        pool.fill_(float("nan"))
        dout.fill_(1.0)
        torch.cuda.synchronize()
        graph.replay()
        got = snapshot()
        assert all(bit_equal(a, b) for a, b in zip(got, eager)), "replay %d differs from eager" % rep

    # replace the inputs' contents in place (same addresses): replay == a new eager run
    h0.mul_(-0.5)
    x["v"].copy_(torch.flip(x["v"], dims=[0]))
    y["beta"].fill_(0.75)
    torch.cuda.synchronize()
    graph.replay()
    got = snapshot()
    step()
    eager2 = snapshot()
    assert all(bit_equal(a, b) for a, b in zip(got, eager2)), "replay after an in-place update differs"
    assert not bit_equal(eager2[0], eager[0])
    say("graph: 4 replays bit-identical to eager (prefill %d tokens + decode B=4)" % w.total_tokens)
