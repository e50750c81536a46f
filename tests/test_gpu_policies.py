"""Scaling-coefficient variants and the First-loop reference policy: parity
of the HIP path with the oracle.

ResidualQuant page, Table 9: residual variants with no scaling (alpha = 1),
the norm ratio ||x||/||y|| and least squares; Table 1 and Table 9: the
First-loop reference policy against Last-loop.  Bars as everywhere: encoded
planes byte-identical to the oracle, attention rows within 2e-3 of the FP64
oracle, reconstruction within 1e-3 of the vector's largest group scale."""
import numpy as np
import pytest
import torch

import synth
from rq_testutil import Case, plane_bits, tol_rel_row

pytestmark = pytest.mark.gpu


def _w(alpha_mode=0, ref_first=0, ref_bits=0, group_loops=0, L=4, g=32, seed=71, d=128):
    bits = [2, 4, 2, 2, 2, 4, 2][:L - 1]
    if ref_first:
        bits = [0] + bits                          # loop 0 is the reference
    if group_loops:
        bits = [0 if (l % group_loops == (0 if ref_first else group_loops - 1)) else 2 for l in range(L)]
    return synth.Workload("p", n_loops=L, batch=2, heads=2, d=d, g=g, n_ctx=0, bits=bits,
                          c=[0.85] * (L - 1), sigma=[0.12] * (L - 1), rotate=1, seed=seed,
                          ref_bits=ref_bits, ref_group=32 if ref_bits else 0, group_loops=group_loops,
                          ref_first=ref_first, alpha_mode=alpha_mode)


CASES = {
    "alpha-one-bf16": _w(alpha_mode=1),
    "norm-ratio-bf16": _w(alpha_mode=2),
    "norm-ratio-anchor": _w(alpha_mode=2, ref_bits=4),
    "first-loop-bf16": _w(ref_first=1),
    "first-loop-anchor": _w(ref_first=1, ref_bits=4, g=16),
    "first-loop-groups": _w(ref_first=1, ref_bits=4, group_loops=4, L=8),
    "first-loop-norm-ratio-alpha-one": _w(ref_first=1, alpha_mode=1, ref_bits=2),
}


@pytest.mark.parametrize("name", list(CASES))
def test_policy_parity(oracle, name):
    import decode_attention_rq_amd as rq
    w = CASES[name]
    n = 333
    case = Case(w, n, cap=340, t_chunks=[(0, 200), (200, 133)])
    lay, kp, vp, qb = case.oracle_planes(oracle)
    for side, planes in (("k", kp), ("v", vp)):
        gc = getattr(case, side)
        for l in range(w.n_loops):
            for nm in ("codes", "meta", "alpha"):
                want = getattr(planes, nm)[l]
                got = getattr(gc, nm)[l]
                assert (want is None) == (got is None), (side, l, nm)
                if want is not None:
                    assert np.array_equal(plane_bits(got)[:, :, :n], want[:, :, :n]), (side, l, nm)
    for l in range(w.n_loops):
        if case.lay.is_anchor(l) and not w.ref_bits:
            continue
        out = torch.empty(case.B, w.heads, 50, w.d, dtype=torch.float32, device="cuda")
        rq.rq_reconstruct(case.lay, case.k, l, 11, 50, out)
        torch.cuda.synchronize()
        want = oracle.reconstruct(lay, kp, l, 11, 50)
        scales = [plane_bits(case.k.meta[l])[:, :, 11:61, :, 0]]
        if w.ref_bits:
            an = oracle.anchor_loop(lay, l)
            scales.append(plane_bits(case.k.meta[an])[:, :, 11:61, :, 0])
        s = np.max([x.view(np.float16).astype(np.float64).max(-1) for x in scales], axis=0)
        err = np.abs(out.cpu().double().numpy() - want).max(-1)
        assert np.all(err <= 1e-3 * s), l
    full = (1 << w.n_loops) - 1
    scale = 1.0 / np.sqrt(w.d)
    for mask, splits in ((full, 0), (full, 2), (1 << (w.n_loops - 1), 1), (0b1, 0)):
        out = torch.full((w.n_loops, case.B, w.heads, w.d), float("nan"), device="cuda")
        ws = rq.workspace_for(case.lay, n, splits)
        rq.rq_decode_attn(case.lay, case.k, case.v, case.q, mask, n, scale, out, ws, splits)
        torch.cuda.synchronize()
        got = out.cpu().double().numpy()
        want = oracle.decode(lay, kp, vp, qb, mask, n, scale)
        for l in range(w.n_loops):
            if (mask >> l) & 1:
                assert tol_rel_row(got[l], want[l]).max() <= 2e-3, (mask, l)
            else:
                assert np.isnan(got[l]).all()


# --------------------------------------------------------------------------
# chained references (Table 9 "Next-loop", "Previous-loop")
# --------------------------------------------------------------------------

def _wc(ref_first=0, ref_bits=0, group_loops=0, L=4, seed=81, d=128, g=16, alpha_mode=0):
    w = _w(ref_first=ref_first, ref_bits=ref_bits, group_loops=group_loops, L=L, g=g, seed=seed, d=d,
           alpha_mode=alpha_mode)
    w.ref_chain = 1
    return w


CHAIN_CASES = {
    "next-loop-bf16": _wc(),
    "next-loop-anchor": _wc(ref_bits=4),
    "previous-loop-anchor": _wc(ref_first=1, ref_bits=4),
    "previous-loop-bf16": _wc(ref_first=1),
    "next-loop-groups": _wc(ref_bits=4, group_loops=4, L=8),
    "next-loop-anchor-d64": _wc(ref_bits=4, d=64),
    "previous-loop-bf16-d256-g32": _wc(ref_first=1, d=256, g=32),
    "next-loop-two-links": _wc(ref_bits=4, L=3),
    "next-loop-norm-ratio": _wc(ref_bits=4, alpha_mode=2),
    "previous-loop-alpha-one": _wc(ref_first=1, alpha_mode=1),
}


@pytest.mark.parametrize("name", list(CHAIN_CASES))
def test_chain_parity(oracle, name, waves):
    import decode_attention_rq_amd as rq
    w = CHAIN_CASES[name]
    n = 301
    case = Case(w, n, cap=310, t_chunks=[(0, 150), (150, 151)])
    lay, kp, vp, qb = case.oracle_planes(oracle)
    for side, planes in (("k", kp), ("v", vp)):
        gc = getattr(case, side)
        for l in range(w.n_loops):
            for nm in ("codes", "meta", "alpha"):
                want = getattr(planes, nm)[l]
                if want is not None:
                    assert np.array_equal(plane_bits(getattr(gc, nm)[l])[:, :, :n], want[:, :, :n]), (side, l, nm)
    for l in range(w.n_loops):
        if case.lay.is_anchor(l) and not w.ref_bits:
            continue
        out = torch.empty(case.B, w.heads, 40, w.d, dtype=torch.float32, device="cuda")
        rq.rq_reconstruct(case.lay, case.k, l, 5, 40, out)
        torch.cuda.synchronize()
        want = oracle.reconstruct(lay, kp, l, 5, 40)
        g0, root, order = oracle.chain_order(lay, l)
        links = [m for m in [root] + order if m != root or w.ref_bits]
        s = np.max([plane_bits(case.k.meta[m])[:, :, 5:45, :, 0].view(np.float16).astype(np.float64).max(-1)
                    for m in links], axis=0)
        err = np.abs(out.cpu().double().numpy() - want).max(-1)
        assert np.all(err <= 1e-3 * s), l
    scale = 1.0 / np.sqrt(w.d)
    tl = synth.draw_tail(w, 4, batch=case.B, n=3, device="cuda")
    tail = rq.Tail([tl["k"][l].contiguous() for l in range(w.n_loops)],
                   [tl["v"][l].contiguous() for l in range(w.n_loops)], 3)
    tkb = np.stack([synth.bf16_bits(tl["k"][l]) for l in range(w.n_loops)])
    tvb = np.stack([synth.bf16_bits(tl["v"][l]) for l in range(w.n_loops)])
    masks = [((1 << w.n_loops) - 1, 0, None), ((1 << w.n_loops) - 1, 2, "tail")]
    masks += [(1 << l, s, None) for l, s in zip(range(w.n_loops), [0, 1, 3, 0, 2, 1, 0, 1])]
    # one loop with a tail whose other loops' planes are absent (NULL): a
    # call for one loop along the chain must touch only that loop's tail
    masks += [(1 << l, s, "own-tail") for l, s in zip(range(w.n_loops), [1, 2, 0, 1, 2, 0, 1, 2])]
    for mask, splits, tailed in masks:
        out = torch.full((w.n_loops, case.B, w.heads, w.d), float("nan"), device="cuda")
        ws = rq.workspace_for(case.lay, n, splits)
        if tailed:
            tl_call = tail
            if tailed == "own-tail":
                tl_call = rq.Tail([t if (mask >> l) & 1 else None for l, t in enumerate(tail.k)],
                                  [t if (mask >> l) & 1 else None for l, t in enumerate(tail.v)], tail.n)
            rq.rq_decode_attn_tail(case.lay, case.k, case.v, tl_call, case.q, mask, n, scale, out, ws, splits)
            want = oracle.decode(lay, kp, vp, qb, mask, n, scale, tkb, tvb)
        else:
            rq.rq_decode_attn(case.lay, case.k, case.v, case.q, mask, n, scale, out, ws, splits)
            want = oracle.decode(lay, kp, vp, qb, mask, n, scale)
        torch.cuda.synchronize()
        got = out.cpu().double().numpy()
        for l in range(w.n_loops):
            if (mask >> l) & 1:
                assert tol_rel_row(got[l], want[l]).max() <= 2e-3, (mask, l)
            else:
                assert np.isnan(got[l]).all(), (mask, l)
