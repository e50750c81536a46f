"""Parity at the workloads' full sizes, in the launch configuration bench.py
times (automatic token splits): the encoded bytes of the checked (batch,
head) pairs are compared with the oracle's encode of the same inputs, and
every loop's attention row with the oracle's FP64 decode.  The metric's
workload (int2-8k) is checked on every one of its 256 pairs; the larger ones
on whole batch rows of heads plus a pair at the far corner.

Inputs are drawn on the GPU by torch's seeded generator (the CPU copies of the
sampled pairs go to the oracle); nothing the oracle sees comes from the
library's kernels."""
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import pytest
import torch

import synth
from rq_testutil import Case, plane_bits, tol_rel_row

pytestmark = pytest.mark.gpu


def _oracle_by_chunk(oracle, case, pairs, chunk=16):
    """The oracle's encode of the given (batch, head) pairs, in chunks of
    `chunk` pairs encoded on parallel host threads (the oracle is C called
    through ctypes, which releases the GIL).  Returns [(pairs, (layout,
    k_planes, v_planes, q_bits))] per chunk."""
    chunks = [pairs[i:i + chunk] for i in range(0, len(pairs), chunk)]
    with ThreadPoolExecutor(max_workers=min(16, len(chunks))) as ex:
        return list(zip(chunks, ex.map(lambda c: case.oracle_planes(oracle, c), chunks)))


def _check_pairs(oracle, case, pairs, n_ctx, mask=None, t_hi=None):
    """Encoded bytes of every listed pair against the oracle's, then every
    loop's decode row of those pairs against the oracle's FP64 decode (rows
    on parallel host threads)."""
    import decode_attention_rq_amd as rq
    w = case.w
    mask = mask if mask is not None else (1 << w.n_loops) - 1
    t_hi = t_hi or case.n
    per_chunk = _oracle_by_chunk(oracle, case, pairs)
    for side in ("k", "v"):
        gc = getattr(case, side)
        for l in range(w.n_loops - 1):
            for name in ("codes", "meta", "alpha"):
                full = plane_bits(getattr(gc, name)[l][:, :, :t_hi])
                for chunk, (lay, kp, vp, qb) in per_chunk:
                    planes = kp if side == "k" else vp
                    want = getattr(planes, name)[l][:, 0, :t_hi]
                    got = full[[b for b, _ in chunk], [h for _, h in chunk]]
                    assert np.array_equal(got, want), (side, l, name, chunk)
    out = torch.full((w.n_loops, case.B, w.heads, w.d), float("nan"), device="cuda")
    splits = rq.rq_decode_splits(case.lay, n_ctx)
    ws = rq.workspace_for(case.lay, n_ctx, splits)
    scale = 1.0 / np.sqrt(w.d)
    rq.rq_decode_attn(case.lay, case.k, case.v, case.q, mask, n_ctx, scale, out, ws, splits)
    torch.cuda.synchronize()
    got = out.cpu().double().numpy()
    rows = [(l, i, b, h, chunk_planes) for chunk, chunk_planes in per_chunk
            for i, (b, h) in enumerate(chunk) for l in range(w.n_loops) if (mask >> l) & 1]

    def row_error(row):
        l, i, b, h, (lay, kp, vp, qb) = row
        want = oracle.decode_row(lay, kp, vp, qb, l, i, 0, n_ctx, scale)
        return l, b, h, float(tol_rel_row(got[l, b, h], want))

    with ThreadPoolExecutor(max_workers=16) as ex:
        errors = list(ex.map(row_error, rows))
    worst = max(e for *_, e in errors)
    bad = [(l, b, h, e) for l, b, h, e in errors if not e <= 2e-3]
    assert not bad, bad[:8]
    return worst


def test_tiny_workload(oracle):
    w = synth.WORKLOADS["tiny"]
    case = Case(w, w.n_ctx)
    _check_pairs(oracle, case, [(0, 0)], w.n_ctx)


def test_int2_8k_full(oracle):
    """Every (batch, head) pair of the metric's workload: all encoded bytes
    and all 1024 attention rows."""
    w = synth.WORKLOADS["int2-8k"]
    case = Case(w, w.n_ctx, gen_device="cuda")
    pairs = [(b, h) for b in range(w.batch) for h in range(w.heads)]
    _check_pairs(oracle, case, pairs, w.n_ctx)


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
    _check_pairs(oracle, case, [(0, h) for h in range(w.heads)] + [(63, 15)], n0 + steps)


def test_int2_32k_one_layer(oracle):
    w = synth.WORKLOADS["int2-32k-24l"]
    case = Case(w, w.n_ctx, gen_device="cuda")
    _check_pairs(oracle, case, [(5, h) for h in range(w.heads)] + [(7, 15)], w.n_ctx)


def test_peak_batch_one_layer(oracle):
    """The largest batch of the peak-batch workload (97 at 8k context under a
    250 GB KV budget over 24 layers), one layer."""
    w = synth.WORKLOADS["peak-batch-8k"]
    case = Case(w, w.n_ctx, batch=97, gen_device="cuda")
    _check_pairs(oracle, case, [(96, h) for h in range(w.heads)] + [(0, 0)], w.n_ctx)


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
