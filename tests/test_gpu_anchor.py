"""Quantized anchor and BF16 tail: parity of the HIP path with the oracle.

The pages' final configuration stores the final loop itself at INT4 ("Ascending
[2,2,2,4]", ResidualQuant page Fig. 3 caption; INT4 anchor at g=32 with INT2
residuals at g=16, Fig. 6 caption) and keeps recent tokens in BF16 (Table 10).
Bars as everywhere: encoded planes (the anchor's and the residuals') byte-
identical to the oracle; reconstruction within 1e-3 x the vector's largest
group scale; attention rows within 2e-3 of the FP64 oracle (max |o - o64| /
max |o64| per row).  Decode is checked loop by loop (one loop per call, as a
looped model runs) and fused, with and without a tail, over split counts."""
import numpy as np
import pytest
import torch

import synth
from rq_testutil import Case, plane_bits, tol_rel_row
from synth import bf16_bits

pytestmark = pytest.mark.gpu

ATT_TOL = 2e-3
REC_TOL = 1e-3


def _w(d=128, g=16, ga=32, abits=4, bits=(2, 2, 2), rotate=1, B=2, H=3, seed=41):
    nres = len(bits)
    return synth.Workload("a", n_loops=nres + 1, batch=B, heads=H, d=d, g=g, n_ctx=0, bits=list(bits),
                          c=[0.8, 0.85, 0.9, 0.9][:nres], sigma=[0.15, 0.12, 0.1, 0.1][:nres],
                          rotate=rotate, seed=seed, ref_bits=abits, ref_group=ga)


ENCODE_CASES = {
    "d128-g16-a4g32-rot": _w(),
    "d128-g32-a4g32-norot": _w(g=32, rotate=0),
    "d64-g16-a2g16-rot-mixed": _w(d=64, ga=16, abits=2, bits=(4, 2)),
    "d256-g32-a4g16-rot": _w(d=256, g=32, ga=16, bits=(2,)),
    "d128-g16-a4g32-rot-int4res": _w(bits=(4, 4, 2)),
}


@pytest.mark.parametrize("name", list(ENCODE_CASES))
def test_anchored_encode_is_byte_exact(oracle, name):
    w = ENCODE_CASES[name]
    n = 77                                   # ragged against the tokens per wave
    case = Case(w, n, cap=80, t_chunks=[(0, 40), (40, 1), (41, 36)])
    _, kp, vp, _ = case.oracle_planes(oracle)
    for side, planes in (("k", kp), ("v", vp)):
        gc = getattr(case, side)
        for l in range(w.n_loops):
            names = ("codes", "meta") + (("alpha",) if l < w.n_loops - 1 else ())
            for nm in names:
                got = plane_bits(getattr(gc, nm)[l])[:, :, :n]
                want = getattr(planes, nm)[l][:, :, :n]
                assert np.array_equal(got, want), (side, l, nm)


@pytest.mark.parametrize("name", ["d128-g16-a4g32-rot", "d128-g32-a4g32-norot", "d64-g16-a2g16-rot-mixed"])
def test_anchored_reconstruct(oracle, name):
    import decode_attention_rq_amd as rq
    w = ENCODE_CASES[name]
    n, t0, cnt = 90, 13, 70
    case = Case(w, n, cap=96)
    lay, kp, _, _ = case.oracle_planes(oracle)
    for l in range(w.n_loops):                # the anchor loop too
        out = torch.empty(case.B, w.heads, cnt, w.d, dtype=torch.float32, device="cuda")
        rq.rq_reconstruct(case.lay, case.k, l, t0, cnt, out)
        torch.cuda.synchronize()
        want = oracle.reconstruct(lay, kp, l, t0, cnt)
        s = plane_bits(case.k.meta[l])[:, :, t0:t0 + cnt, :, 0].view(np.float16).astype(np.float64)
        if l < w.n_loops - 1:
            # the anchor's error enters a residual loop scaled by alpha
            sa = plane_bits(case.k.meta[-1])[:, :, t0:t0 + cnt, :, 0].view(np.float16).astype(np.float64)
            s = np.maximum(s.max(-1), sa.max(-1))
        else:
            s = s.max(-1)
        err = np.abs(out.cpu().double().numpy() - want).max(-1)
        assert np.all(err <= REC_TOL * s), (l, float((err / np.maximum(REC_TOL * s, 1e-30)).max()))


@pytest.mark.parametrize("chain", [0, 1])
def test_zero_signs_of_rebuilt_references(oracle, chain):
    """References rebuilt from codes (the dequantized, rotated INT4 anchor; a
    chain link) with exact zeros: a one-hot anchor row rotates to a constant
    group, which dequantizes to its offset, which rebuilds to one non-zero
    entry and zeros.  Loops of signed zeros against it make every product of
    alpha's numerator a zero whose sign depends on those zeros, so the stored
    alpha (FP16 +0 or -0) shows whether the rebuilt reference's zeros match
    the oracle's, bit for bit."""
    import decode_attention_rq_amd as rq
    from rq_testutil import encoder_input
    w = _w(B=1, H=2, bits=(2, 2, 2))
    if chain:
        w = synth.Workload(w.name, n_loops=w.n_loops, batch=1, heads=2, d=w.d, g=w.g, n_ctx=0, bits=w.bits,
                           c=w.c, sigma=w.sigma, rotate=1, seed=w.seed, ref_bits=4, ref_group=32, ref_chain=1)
    n = 12
    case = Case(w, n, cap=n)
    for side in ("k", "v"):
        ref, loops = case.data[side + "_ref"], case.data[side + "_loops"]
        for t, (dim, val, zero) in enumerate([(0, 1.0, -0.0), (5, -1.0, 0.0), (64, 2.0, -0.0), (127, 0.5, 0.0)]):
            ref[:, :, t] = 0.0                 # one-hot: rebuilds to one non-zero entry and zeros
            ref[:, :, t, dim] = val
            loops[:, :, :, t] = zero           # every product of alpha's numerator a signed zero
        ref[:, :, 4] = 0.0                     # an all-zero anchor row (alpha's denominator 0)
        loops[:, :, :, 4] = -0.0
        loops[:, :, 1, 5] = -0.0               # one loop of -0 against a random anchor row
    kin = encoder_input(w, case.data["k_loops"], case.data["k_ref"]).cuda().contiguous()
    vin = encoder_input(w, case.data["v_loops"], case.data["v_ref"]).cuda().contiguous()
    rq.rq_encode(case.lay, case.k, case.v, kin, vin, 0, n)
    torch.cuda.synchronize()
    _, kp, vp, _ = case.oracle_planes(oracle)
    for side, planes in (("k", kp), ("v", vp)):
        gc = getattr(case, side)
        for l in range(w.n_loops):
            names = ("codes", "meta") + (("alpha",) if l < w.n_loops - 1 else ())
            for nm in names:
                got = plane_bits(getattr(gc, nm)[l])[:, :, :n]
                want = getattr(planes, nm)[l][:, :, :n]
                assert np.array_equal(got, want), (side, l, nm)
        # the case is not vacuous: some stored alpha is a negative zero
        if not chain:
            assert (plane_bits(gc.alpha[0])[:, :, 0] == 0x8000).any()


def _tail(w, B, T, seed=3):
    if T == 0:
        return None, None
    t = synth.draw_tail(w, seed, batch=B, n=T)
    return t["k"], t["v"]


def _run(case, mask, n_ctx, tk, tv, T, splits=0, scale=None):
    import decode_attention_rq_amd as rq
    w = case.w
    scale = scale if scale is not None else 1.0 / np.sqrt(w.d)
    out = torch.full((w.n_loops, case.B, w.heads, w.d), float("nan"), device="cuda")
    ws = rq.workspace_for(case.lay, n_ctx, splits)
    if tk is None:
        rq.rq_decode_attn(case.lay, case.k, case.v, case.q, mask, n_ctx, scale, out, ws, splits)
    else:
        # tail planes with spare capacity, rows [0, T) filled
        cap = T + 3
        kt = [torch.zeros(case.B, w.heads, cap, w.d, dtype=torch.bfloat16, device="cuda") for _ in range(w.n_loops)]
        vt = [torch.zeros_like(kt[0]) for _ in range(w.n_loops)]
        for l in range(w.n_loops):
            kt[l][:, :, :T] = tk[l].cuda()
            vt[l][:, :, :T] = tv[l].cuda()
        tail = rq.Tail(kt, vt, T)
        rq.rq_decode_attn_tail(case.lay, case.k, case.v, tail, case.q, mask, n_ctx, scale, out, ws, splits)
    torch.cuda.synchronize()
    return out.cpu().double().numpy()


def _check(oracle, case, got, mask, n_ctx, tk, tv, scale=None):
    w = case.w
    scale = scale if scale is not None else 1.0 / np.sqrt(w.d)
    lay, kp, vp, qb = case.oracle_planes(oracle)
    tkb = None if tk is None else bf16_bits(tk)
    tvb = None if tv is None else bf16_bits(tv)
    want = oracle.decode(lay, kp, vp, qb, mask, n_ctx, scale, tkb, tvb)
    worst = 0.0
    for l in range(w.n_loops):
        if (mask >> l) & 1:
            rel = tol_rel_row(got[l], want[l])
            worst = max(worst, float(rel.max()))
            assert rel.max() <= ATT_TOL, (l, float(rel.max()))
        else:
            assert np.isnan(got[l]).all(), f"loop {l} not in the mask was written"
    return worst


DECODE_CASES = {
    # name: (workload, n (cached tokens), mask, tail tokens, split counts)
    "perloop-res-a4": (_w(), 600, 0b0001, 0, [0, 1, 3]),
    "perloop-res-a4-tail": (_w(), 600, 0b0010, 17, [0, 1, 2]),
    "perloop-anchor-tail": (_w(), 513, 0b1000, 64, [0, 1, 5]),
    "fused-a4-tail": (_w(), 700, 0b1111, 9, [0, 1, 4]),
    "fused-a4-notail": (_w(), 700, 0b1111, 0, [0, 2]),
    "norot-g32-a4-tail": (_w(g=32, rotate=0), 300, 0b1011, 5, [0, 1]),
    "d64-a2g16-mixed": (_w(d=64, ga=16, abits=2, bits=(4, 2)), 333, 0b111, 3, [0, 2]),
    "d256-a4g16": (_w(d=256, g=32, ga=16, bits=(2,)), 260, 0b11, 2, [0, 1]),
    # a tail longer than one batch of tail loads of every workgroup shape
    # (8 waves x 4 rows x 2 groups = 64 rows), ragged, per loop and fused
    "long-tail-perloop": (_w(), 400, 0b0100, 150, [0, 1, 2, 3]),
    "long-tail-fused": (_w(), 400, 0b1111, 139, [0, 1, 2]),
}


@pytest.mark.parametrize("name", list(DECODE_CASES))
def test_anchored_decode(oracle, name, waves):
    w, n, mask, T, splits = DECODE_CASES[name]
    case = Case(w, n, cap=n + 8)
    tk, tv = _tail(w, case.B, T)
    for s in splits:
        got = _run(case, mask, n, tk, tv, T, splits=s)
        _check(oracle, case, got, mask, n, tk, tv)


@pytest.mark.parametrize("anchored", [False, True])
def test_tail_alone(oracle, anchored):
    """No cached token yet: the tail is the whole context."""
    w = _w() if anchored else synth.Workload("b", n_loops=4, batch=2, heads=3, d=128, g=32, n_ctx=0,
                                             bits=[2, 2, 2], c=[0.8, 0.85, 0.9],
                                             sigma=[0.15, 0.12, 0.1], rotate=1, seed=43)
    case = Case(w, 8, cap=16)
    tk, tv = _tail(w, case.B, 6)
    got = _run(case, 0b1111, 0, tk, tv, 6)
    _check(oracle, case, got, 0b1111, 0, tk, tv)


@pytest.mark.parametrize("T,mask", [(1, 0b0111), (97, 0b1111), (97, 0b0010)])
def test_bf16_reference_with_tail(oracle, waves, T, mask):
    """The tail works with the BF16 reference too: a one-token tail (the
    current token of a looped model's earlier loops), and a ragged tail longer
    than one batch of tail loads, fused and per loop."""
    w = synth.Workload("b", n_loops=4, batch=2, heads=3, d=128, g=32, n_ctx=0, bits=[2, 4, 2],
                       c=[0.8, 0.85, 0.9], sigma=[0.15, 0.12, 0.1], rotate=1, seed=44)
    case = Case(w, 500, cap=512)
    tk, tv = _tail(w, case.B, T)
    for s in (0, 1, 2, 3):
        got = _run(case, mask, 500, tk, tv, T, splits=s)
        _check(oracle, case, got, mask, 500, tk, tv)


@pytest.mark.parametrize("anchored", [False, True])
def test_tail_shared_over_many_splits(oracle, waves, anchored):
    """Each split attends an equal share of the tail rows: tails shorter than
    the split count (the last splits have none), one row per split, and a
    ragged last share; fused and per loop, under every workgroup shape."""
    w = _w() if anchored else synth.Workload("b", n_loops=4, batch=2, heads=3, d=128, g=32, n_ctx=0,
                                             bits=[2, 4, 2], c=[0.8, 0.85, 0.9],
                                             sigma=[0.15, 0.12, 0.1], rotate=1, seed=45)
    n = 900
    case = Case(w, n, cap=n + 4)
    for T, s in ((1, 7), (5, 13), (13, 13), (70, 24)):
        tk, tv = _tail(w, case.B, T, seed=T)
        for mask in (0b1111, 0b0010):
            got = _run(case, mask, n, tk, tv, T, splits=s)
            _check(oracle, case, got, mask, n, tk, tv)


def test_tail_of_zero_tokens_is_plain_decode():
    import decode_attention_rq_amd as rq
    w = _w()
    case = Case(w, 300, cap=300)
    tk, tv = _tail(w, case.B, 4)
    a = _run(case, 0b1111, 300, None, None, 0, splits=1)
    out = torch.full((w.n_loops, case.B, w.heads, w.d), float("nan"), device="cuda")
    ws = rq.workspace_for(case.lay, 300, 1)
    kt = [t.cuda().contiguous() for t in tk]
    vt = [t.cuda().contiguous() for t in tv]
    rq.rq_decode_attn_tail(case.lay, case.k, case.v, rq.Tail(kt, vt, 0), case.q, 0b1111, 300,
                           1.0 / np.sqrt(w.d), out, ws, 1)
    torch.cuda.synchronize()
    assert np.array_equal(a, out.cpu().double().numpy())


@pytest.mark.parametrize("wname", ["anchor-8k-perloop", "chain-8k-perloop", "grid-g16-2k-batch512"])
def test_anchor_perloop_full_size(oracle, wname):
    """The per-loop workloads at full size (batch 16, 16 heads, 8192 cached
    tokens + 64 BF16 tail tokens, INT4 anchor g=32, INT2 residuals g=16; Last-
    loop references, or Next-loop chains), and the decode grid's largest
    launch (batch 512 at 2k context: the most the 250 GB budget holds, 8192
    batch*heads), in the launch configuration the benchmark uses, on one whole
    batch row of heads and two corner pairs: bytes of those pairs, then every
    loop's row, one loop per call."""
    import dataclasses
    import decode_attention_rq_amd as rq
    if wname == "grid-g16-2k-batch512":
        w = dataclasses.replace(synth.WORKLOADS["grid-g16"], name=wname, batch=512, n_ctx=2048)
    else:
        w = synth.WORKLOADS[wname]
    T = w.extra["tail"]
    n = w.n_ctx
    case = Case(w, n, gen_device="cuda")
    mid = w.batch // 2 + 1
    pairs = [(mid, h) for h in range(w.heads)] + [(0, 0), (w.batch - 1, w.heads - 1)]
    lay, kp, vp, qb = case.oracle_planes(oracle, pairs)
    for side, planes in (("k", kp), ("v", vp)):
        gc = getattr(case, side)
        for l in range(w.n_loops):
            names = ("codes", "meta") + (("alpha",) if l < w.n_loops - 1 else ())
            for nm in names:
                full = getattr(gc, nm)[l]
                for i, (b, h) in enumerate(pairs):
                    assert np.array_equal(plane_bits(full[b, h, :n]), getattr(planes, nm)[l][i, 0, :n]), \
                        (side, l, nm, b, h)
    tail = synth.draw_tail(w, 99, batch=case.B, n=T, device="cuda")
    kt = [tail["k"][l].contiguous() for l in range(w.n_loops)]
    vt = [tail["v"][l].contiguous() for l in range(w.n_loops)]
    out = torch.full((w.n_loops, case.B, w.heads, w.d), float("nan"), device="cuda")
    scale = 1.0 / np.sqrt(w.d)
    for l in range(w.n_loops):
        splits = rq.rq_decode_splits(case.lay, n)
        ws = rq.workspace_for(case.lay, n, splits)
        rq.rq_decode_attn_tail(case.lay, case.k, case.v, rq.Tail(kt, vt, T), case.q, 1 << l, n, scale,
                               out, ws, splits)
    torch.cuda.synchronize()
    got = out.cpu().double().numpy()
    for l in range(w.n_loops):
        for i, (b, h) in enumerate(pairs):
            want = oracle.decode_row(lay, kp, vp, qb, l, i, 0, n, scale,
                                     bf16_bits(tail["k"][l, b, h]), bf16_bits(tail["v"][l, b, h]))
            rel = float(tol_rel_row(got[l, b, h], want))
            assert rel <= ATT_TOL, (l, b, h, rel)


# --------------------------------------------------------------------------
# several anchor groups (Table 8: one INT4 anchor per group of loops)
# --------------------------------------------------------------------------

def _wg(L, G, bits, g=16, B=2, H=2, seed=61):
    return synth.Workload("grp", n_loops=L, batch=B, heads=H, d=128, g=g, n_ctx=0, bits=list(bits),
                          c=[0.85] * (L - 1), sigma=[0.12] * (L - 1), rotate=1, seed=seed, ref_bits=4,
                          ref_group=32, group_loops=G)


GROUP_CASES = {
    "2x[2,4,2,4]": _wg(8, 4, [2, 4, 2, 0, 2, 2, 4]),
    "2x[2^7,4]": _wg(16, 8, [2, 2, 2, 2, 2, 2, 2, 0, 2, 2, 2, 2, 2, 2, 2], g=32),
}


@pytest.mark.parametrize("name", list(GROUP_CASES))
def test_anchor_groups_encode_reconstruct_decode(oracle, name):
    import decode_attention_rq_amd as rq
    w = GROUP_CASES[name]
    n = 150
    case = Case(w, n, cap=160, t_chunks=[(0, 99), (99, 51)])
    lay, kp, vp, qb = case.oracle_planes(oracle)
    for side, planes in (("k", kp), ("v", vp)):
        gc = getattr(case, side)
        for l in range(w.n_loops):
            assert np.array_equal(plane_bits(gc.codes[l])[:, :, :n], planes.codes[l][:, :, :n]), (side, l)
            assert np.array_equal(plane_bits(gc.meta[l])[:, :, :n], planes.meta[l][:, :, :n]), (side, l)
            if planes.alpha[l] is not None:
                assert np.array_equal(plane_bits(gc.alpha[l])[:, :, :n], planes.alpha[l][:, :, :n]), (side, l)
    for l in (0, w.group_loops - 1, w.group_loops, w.n_loops - 1):
        out = torch.empty(case.B, w.heads, 40, w.d, dtype=torch.float32, device="cuda")
        rq.rq_reconstruct(case.lay, case.k, l, 7, 40, out)
        torch.cuda.synchronize()
        want = oracle.reconstruct(lay, kp, l, 7, 40)
        an = (l // w.group_loops + 1) * w.group_loops - 1
        sa = plane_bits(case.k.meta[an])[:, :, 7:47, :, 0].view(np.float16).astype(np.float64).max(-1)
        sr = plane_bits(case.k.meta[l])[:, :, 7:47, :, 0].view(np.float16).astype(np.float64).max(-1)
        err = np.abs(out.cpu().double().numpy() - want).max(-1)
        assert np.all(err <= REC_TOL * np.maximum(sa, sr)), l
    tk, tv = _tail(w, case.B, 4)
    full = (1 << w.n_loops) - 1
    for mask, splits in ((full, 0), (full, 3), (0b1 | (1 << (w.n_loops - 1)), 1)):
        got = _run(case, mask, n, tk, tv, 4, splits=splits)
        _check(oracle, case, got, mask, n, tk, tv)
