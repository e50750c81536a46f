"""Parity at the workloads' full sizes, in the launch configuration bench.py
times (automatic token splits), on sampled (batch, head) pairs: the encoded
bytes of every sampled pair are compared with the oracle's encode of the same
inputs, and every loop's attention row with the oracle's FP64 decode.

Inputs are drawn on the GPU by torch's seeded generator (the CPU copies of the
sampled pairs go to the oracle); nothing the oracle sees comes from the
library's kernels."""
import numpy as np
import pytest
import torch

import synth
from rq_testutil import Case, plane_bits, tol_rel_row

pytestmark = pytest.mark.gpu


def _check_pairs(oracle, case, pairs, n_ctx, mask=None, t_hi=None):
    import decode_attention_rq_amd as rq
    w = case.w
    mask = mask if mask is not None else (1 << w.n_loops) - 1
    t_hi = t_hi or case.n
    lay, kp, vp, qb = case.oracle_planes(oracle, pairs)
    for side, planes in (("k", kp), ("v", vp)):
        gc = getattr(case, side)
        for l in range(w.n_loops - 1):
            for name in ("codes", "meta", "alpha"):
                full = getattr(gc, name)[l]
                for i, (b, h) in enumerate(pairs):
                    got = plane_bits(full[b, h, :t_hi])
                    want = getattr(planes, name)[l][i, 0, :t_hi]
                    assert np.array_equal(got, want), (side, l, name, b, h)
    out = torch.full((w.n_loops, case.B, w.heads, w.d), float("nan"), device="cuda")
    splits = rq.rq_decode_splits(case.lay, n_ctx)
    ws = rq.workspace_for(case.lay, n_ctx, splits)
    scale = 1.0 / np.sqrt(w.d)
    rq.rq_decode_attn(case.lay, case.k, case.v, case.q, mask, n_ctx, scale, out, ws, splits)
    torch.cuda.synchronize()
    got = out.cpu().double().numpy()
    worst = 0.0
    for l in range(w.n_loops):
        if not (mask >> l) & 1:
            continue
        for i, (b, h) in enumerate(pairs):
            want = oracle.decode_row(lay, kp, vp, qb, l, i, 0, n_ctx, scale)
            rel = float(tol_rel_row(got[l, b, h], want))
            worst = max(worst, rel)
            assert rel <= 2e-3, (l, b, h, rel)
    return worst


def test_tiny_workload(oracle):
    w = synth.WORKLOADS["tiny"]
    case = Case(w, w.n_ctx)
    _check_pairs(oracle, case, [(0, 0)], w.n_ctx)


def test_int2_8k_full(oracle):
    w = synth.WORKLOADS["int2-8k"]
    case = Case(w, w.n_ctx, gen_device="cuda")
    _check_pairs(oracle, case, [(0, 0), (7, 11), (15, 15)], w.n_ctx)


def test_mixed_8k_prefill_then_appends(oracle):
    """Prefill 8192 tokens, then one-token appends: each appended token's
    reference slot is written, rq_encode(t0 = n, n = 1), then decode over n+1
    tokens (the append-decode loop of the workload, 4 of its 64 steps)."""
    import decode_attention_rq_amd as rq
    w = synth.WORKLOADS["mixed-8k-append"]
    steps = 4
    n0 = w.n_ctx
    case = Case(w, n0 + steps, cap=n0 + w.steps, gen_device="cuda", t_chunks=[(0, n0)])
    kin = case.data["k_loops"]
    vin = case.data["v_loops"]
    out = torch.empty(w.n_loops, case.B, w.heads, w.d, device="cuda")
    scale = 1.0 / np.sqrt(w.d)
    for s in range(steps):
        t = n0 + s
        rq.rq_encode(case.lay, case.k, case.v, kin[:, :, :, t:t + 1].contiguous(),
                     vin[:, :, :, t:t + 1].contiguous(), t, 1)
        ws = rq.workspace_for(case.lay, t + 1)
        rq.rq_decode_attn(case.lay, case.k, case.v, case.q, 0b1111, t + 1, scale, out, ws)
    torch.cuda.synchronize()
    _check_pairs(oracle, case, [(0, 3), (63, 15)], n0 + steps)


def test_int2_32k_one_layer(oracle):
    w = synth.WORKLOADS["int2-32k-24l"]
    case = Case(w, w.n_ctx, gen_device="cuda")
    _check_pairs(oracle, case, [(5, 9)], w.n_ctx)


def test_peak_batch_one_layer(oracle):
    """The largest batch of the peak-batch workload (97 at 8k context under a
    250 GB KV budget over 24 layers), one layer."""
    w = synth.WORKLOADS["peak-batch-8k"]
    case = Case(w, w.n_ctx, batch=97, gen_device="cuda")
    _check_pairs(oracle, case, [(96, 15)], w.n_ctx)


def test_encode_empty_range_touches_nothing():
    import decode_attention_rq_amd as rq
    w = synth.WORKLOADS["tiny"]
    case = Case(w, 16, cap=32)
    planes = [t for t in case.k.codes + case.k.meta + case.k.alpha if t is not None]
    before = [plane_bits(t).copy() for t in planes]
    # n = 0 at the end of the cache: valid, enqueues nothing (any aligned
    # pointer stands in for the empty inputs)
    rq.rq_encode(case.lay, case.k, case.v, case.k.ref, case.v.ref, 32, 0)
    torch.cuda.synchronize()
    after = [plane_bits(t) for t in planes]
    assert all(np.array_equal(a, b) for a, b in zip(before, after))
