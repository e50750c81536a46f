"""Decode steps captured in a HIP graph (torch.cuda.CUDAGraph on the current
stream) and replayed: every replay must give the eager result bit for bit.
The library makes no allocation, synchronisation or memset at call time, so
a whole per-loop decode step (decode kernels, split merges, BF16 tail) can be
replayed without host launches.  Replays are interleaved with eager work that
overwrites the outputs, and each replay is checked."""
import numpy as np
import pytest
import torch

import synth
from rq_testutil import Case

pytestmark = pytest.mark.gpu


def _anchor_w():
    return synth.Workload("g", n_loops=4, batch=2, heads=4, d=128, g=16, n_ctx=0, bits=[2, 2, 2],
                          c=[0.8, 0.85, 0.9], sigma=[0.15, 0.12, 0.1], rotate=1, seed=91, ref_bits=4,
                          ref_group=32, extra={"tail": 8})


def test_graph_replay_matches_eager():
    import decode_attention_rq_amd as rq
    w = _anchor_w()
    n, T = 1500, 8
    case = Case(w, n, cap=n)
    tl = synth.draw_tail(w, 5, batch=case.B, n=T, device="cuda")
    tail = rq.Tail([tl["k"][l].contiguous() for l in range(w.n_loops)],
                   [tl["v"][l].contiguous() for l in range(w.n_loops)], T)
    scale = 1.0 / np.sqrt(w.d)
    out = torch.empty(w.n_loops, case.B, w.heads, w.d, device="cuda")
    ws = rq.workspace_for(case.lay, n, 3)

    def step():
        for l in range(w.n_loops):                      # per-loop calls, 3 splits + tail merge
            rq.rq_decode_attn_tail(case.lay, case.k, case.v, tail, case.q, 1 << l, n, scale, out, ws, 3)

    step()
    torch.cuda.synchronize()
    eager = out.clone()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):                           # warm up on the capture stream
        step()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for r in range(4):
        out.fill_(float("nan"))
        ws.fill_(0xFF)                                   # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, eager), f"replay {r}"
        step()                                           # and eager calls still agree
        torch.cuda.synchronize()
        assert torch.equal(out, eager)


def test_graph_replay_bf16_baseline_matches_eager():
    import decode_attention_rq_amd as rq
    L, B, H, d, n = 4, 2, 4, 128, 1100
    lay = rq.Layout(L, B, H, d, 32, n, 1, [2, 2, 2])
    gen = torch.Generator(device="cuda").manual_seed(3)
    ks = [torch.randn(B, H, n, d, generator=gen, device="cuda").to(torch.bfloat16) for _ in range(L)]
    vs = [torch.randn(B, H, n, d, generator=gen, device="cuda").to(torch.bfloat16) for _ in range(L)]
    q = torch.randn(L, B, H, d, generator=gen, device="cuda").to(torch.bfloat16)
    out = torch.empty(L, B, H, d, device="cuda")
    ws = rq.workspace_for(lay, n, 2)

    def step():
        for l in range(L):
            rq.rq_bf16_decode_attn(lay, ks, vs, q, 1 << l, n, 0.09, out, ws, 2)

    step()
    torch.cuda.synchronize()
    eager = out.clone()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        step()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for r in range(3):
        out.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, eager), f"replay {r}"
