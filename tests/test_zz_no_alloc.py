"""The no-allocation decode entry point against the one with a caller
workspace: same kernels, same split choice, so the outputs must be
identical, over two calls in a row (the second smaller, so the scratch holds
the first call's records when it starts), with split records, with and
without a BF16 tail, and under every workgroup shape."""
import numpy as np
import pytest
import torch

import synth
from rq_testutil import Case


def _tail(w, B, T):
    tl = synth.draw_tail(w, seed=w.seed + 77, batch=B, n=T)
    return ([tl["k"][l].cuda().contiguous() for l in range(w.n_loops)],
            [tl["v"][l].cuda().contiguous() for l in range(w.n_loops)])


def _both(case, w, mask, n_ctx, splits, T):
    import decode_attention_rq_amd as rq
    scale = 1.0 / np.sqrt(w.d)
    tail = None
    if T:
        kt, vt = _tail(w, case.B, T)
        tail = rq.Tail(kt, vt, T)
    shape = (w.n_loops, case.B, w.heads, w.d)
    want = torch.full(shape, float("nan"), device="cuda")
    got = torch.full(shape, float("nan"), device="cuda")
    ws = rq.workspace_for(case.lay, n_ctx, splits)
    rq.rq_decode_attn_tail(case.lay, case.k, case.v, tail, case.q, mask, n_ctx, scale, want, ws, splits)
    rq.rq_decode_attn_tail_noalloc(case.lay, case.k, case.v, tail, case.q, mask, n_ctx, scale, got, splits)
    torch.cuda.synchronize()
    return want.cpu().numpy(), got.cpu().numpy()


@pytest.mark.gpu
@pytest.mark.parametrize("splits", [0, 5])
def test_noalloc_matches_the_workspace_entry_point(waves, splits):
    w1 = synth.Workload("noalloc-a", n_loops=4, batch=2, heads=4, d=128, g=32, n_ctx=3000, bits=[4, 2, 2],
                        c=[0.8, 0.85, 0.9], sigma=[0.15, 0.12, 0.1], rotate=1, seed=31)
    w2 = synth.Workload("noalloc-b", n_loops=4, batch=1, heads=2, d=128, g=16, n_ctx=700, bits=[2, 2, 2],
                        c=[0.8, 0.85, 0.9], sigma=[0.15, 0.12, 0.1], rotate=1, seed=32, ref_bits=4,
                        ref_group=32)
    for w, n_ctx, T, mask in ((w1, 3000, 24, 0b1111), (w2, 650, 0, 0b0101)):
        print(f"noalloc case {w.name}: n_ctx {n_ctx}, tail {T}, mask {mask:#x}, splits {splits}", flush=True)
        case = Case(w, w.n_ctx, cap=w.n_ctx)
        want, got = _both(case, w, mask, n_ctx, splits, T)
        rows = [l for l in range(w.n_loops) if (mask >> l) & 1]
        assert np.isfinite(want[rows]).all()
        assert np.array_equal(want[rows], got[rows])
        assert np.isnan(got[[l for l in range(w.n_loops) if l not in rows]]).all()
