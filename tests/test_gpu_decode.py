"""Reconstruction and decode-attention parity against the oracle.

Bars: reconstruction within 1e-3 x (largest group scale of the vector) of the
oracle's FP64 reconstruction; attention rows within 2e-3 of the FP64 oracle,
measured as max |o - o64| / max |o64| per (loop, batch, head) row.  Covers
folded rotation vs the oracle's explicit un-rotation, split counts, loop
masks (including multi-pass masks with more than three residual loops),
ragged contexts, one-token contexts and run-to-run determinism."""
import numpy as np
import pytest
import torch

import synth
from rq_testutil import Case, plane_bits, tol_rel_row

pytestmark = pytest.mark.gpu

ATT_TOL = 2e-3
REC_TOL = 1e-3


def _w(d=128, g=32, bits=(2, 2, 2), rotate=1, B=2, H=3, seed=11):
    nres = len(bits)
    c = [0.8, 0.85, 0.9, 0.9, 0.95, 0.95][:nres]
    s = [0.15, 0.12, 0.1, 0.1, 0.08, 0.08][:nres]
    return synth.Workload("t", n_loops=nres + 1, batch=B, heads=H, d=d, g=g, n_ctx=0,
                          bits=list(bits), c=c, sigma=s, rotate=rotate, seed=seed)


@pytest.mark.parametrize("d,g,bits,rotate", [(128, 32, (2, 4, 2), 1), (64, 16, (4,), 0),
                                             (256, 32, (2,), 1), (128, 16, (2, 2), 0)])
def test_reconstruct(oracle, d, g, bits, rotate):
    import decode_attention_rq_amd as rq
    w = _w(d=d, g=g, bits=bits, rotate=rotate)
    n, t0, cnt = 90, 13, 70
    case = Case(w, n, cap=96)
    lay, kp, vp, _ = case.oracle_planes(oracle)
    for l in range(w.n_loops - 1):
        out = torch.empty(case.B, w.heads, cnt, d, dtype=torch.float32, device="cuda")
        rq.rq_reconstruct(case.lay, case.k, l, t0, cnt, out)
        torch.cuda.synchronize()
        want = oracle.reconstruct(lay, kp, l, t0, cnt)
        s = plane_bits(case.k.meta[l])[:, :, t0:t0 + cnt, :, 0].view(np.float16).astype(np.float64)
        bound = REC_TOL * s.max(-1)
        err = np.abs(out.cpu().double().numpy() - want).max(-1)
        assert np.all(err <= bound), float((err / np.maximum(bound, 1e-30)).max())


def _decode_gpu(case, mask, n_ctx, splits=0, scale=None, out=None):
    import decode_attention_rq_amd as rq
    w = case.w
    scale = scale if scale is not None else 1.0 / np.sqrt(w.d)
    if out is None:
        out = torch.full((w.n_loops, case.B, w.heads, w.d), float("nan"), device="cuda")
    ws = rq.workspace_for(case.lay, n_ctx, splits)
    rq.rq_decode_attn(case.lay, case.k, case.v, case.q, mask, n_ctx, scale, out, ws, splits)
    torch.cuda.synchronize()
    return out.cpu().double().numpy()


def _check_rows(oracle, case, got, mask, n_ctx, scale=None):
    w = case.w
    scale = scale if scale is not None else 1.0 / np.sqrt(w.d)
    lay, kp, vp, qb = case.oracle_planes(oracle)
    want = oracle.decode(lay, kp, vp, qb, mask, n_ctx, scale)
    for l in range(w.n_loops):
        if (mask >> l) & 1:
            rel = tol_rel_row(got[l], want[l])
            assert rel.max() <= ATT_TOL, (l, float(rel.max()))
        else:
            assert np.isnan(got[l]).all(), f"loop {l} not in the mask was written"


DECODE_CASES = {
    "tiny-d64-int2-norot": (_w(d=64, bits=(2,), rotate=0, B=1, H=1, seed=0), 128, 128, 0b11, [0, 1, 3]),
    "d128-int2x3": (_w(), 1000, 1024, 0b1111, [0, 1, 2, 7]),
    "d128-mixed-ragged": (_w(bits=(4, 2, 2)), 517, 600, 0b1111, [0, 2, 3]),
    "d128-residual-only": (_w(), 300, 300, 0b0101, [0, 5]),
    "d128-reference-only": (_w(), 300, 300, 0b1000, [0]),
    "d128-g16-norot": (_w(g=16, rotate=0), 257, 260, 0b1011, [0]),
    "d64-g32": (_w(d=64, bits=(2, 4)), 333, 333, 0b111, [0, 2]),
    "d256": (_w(d=256, bits=(2, 2), B=1, H=2), 190, 200, 0b111, [0, 2, 4]),
    "multipass-6-loops": (_w(bits=(2, 4, 2, 2, 4), B=1, H=2), 150, 150, 0b111111, [0, 2, 3]),
    "multipass-sparse-mask": (_w(bits=(2, 4, 2, 2, 4), B=1, H=2), 150, 150, 0b101110, [0]),
}


@pytest.mark.parametrize("name", list(DECODE_CASES))
def test_decode(oracle, name, waves):
    w, n, cap, mask, splits_list = DECODE_CASES[name]
    case = Case(w, n, cap=cap)
    for splits in splits_list:
        got = _decode_gpu(case, mask, n, splits)
        _check_rows(oracle, case, got, mask, n)


def test_decode_partial_context_and_scale(oracle):
    """Attend over a prefix of the encoded tokens with a non-default scale."""
    w = _w()
    case = Case(w, 400, cap=512)
    for n_ctx in (1, 2, 9, 63, 250):
        got = _decode_gpu(case, 0b1111, n_ctx, 0, scale=0.3)
        _check_rows(oracle, case, got, 0b1111, n_ctx, scale=0.3)


def test_decode_one_token_is_the_value(oracle):
    """n_ctx = 1: every loop's output is that loop's reconstructed first value."""
    import decode_attention_rq_amd as rq
    w = _w(bits=(2, 4, 2))
    case = Case(w, 8, cap=8)
    got = _decode_gpu(case, 0b1111, 1)
    for l in range(3):
        v = torch.empty(case.B, w.heads, 1, w.d, device="cuda")
        rq.rq_reconstruct(case.lay, case.v, l, 0, 1, v)
        torch.cuda.synchronize()
        assert np.allclose(got[l], v[:, :, 0].cpu().double().numpy(), rtol=1e-5, atol=1e-5)
    assert np.allclose(got[3], case.data["v_ref"][:, :, 0].double().numpy(), rtol=1e-6, atol=1e-6)


def test_decode_deterministic():
    w = _w()
    case = Case(w, 700, cap=700)
    a = _decode_gpu(case, 0b1111, 700, 0)
    b = _decode_gpu(case, 0b1111, 700, 0)
    assert np.array_equal(a, b)


def test_decode_split_invariance(monkeypatch):
    """Split counts and workgroup shapes (4 or 8 waves per split; two splits
    without a tail as one 8-wave workgroup per (batch, head)) agree to FP32
    reordering, also with a ragged context."""
    w = _w()
    for n in (640, 653):
        case = Case(w, n, cap=n)
        outs = []
        for wv in ("4", "8", ""):
            monkeypatch.setenv("RQ_DECODE_WAVES", wv)
            outs += [_decode_gpu(case, 0b1111, n, s) for s in (1, 2, 3, 5, 16, 40)]
        for o in outs[1:]:
            assert tol_rel_row(o, outs[0]).max() <= 1e-5
