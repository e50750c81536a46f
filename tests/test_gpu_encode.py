"""Encoder parity: the HIP encoder's codes, scales/zeros and LS coefficients
are byte-identical to the oracle's (bit-exact FP32 contract, round half to
even), over head dims, group sizes, bit widths, rotation on/off, ragged token
counts, chunked appends and degenerate vectors."""
import numpy as np
import pytest
import torch

import synth
from rq_testutil import Case, plane_bits
from synth import bf16_bits

pytestmark = pytest.mark.gpu


def _w(d=128, g=32, bits=(2, 2, 2), rotate=1, B=2, H=3, seed=7):
    nres = len(bits)
    c = [0.8, 0.85, 0.9, 0.9, 0.95, 0.95][:nres]
    s = [0.15, 0.12, 0.1, 0.1, 0.08, 0.08][:nres]
    return synth.Workload("t", n_loops=nres + 1, batch=B, heads=H, d=d, g=g, n_ctx=0,
                          bits=list(bits), c=c, sigma=s, rotate=rotate, seed=seed)


def _compare(case, oracle, t_lo, t_hi):
    lay, kp, vp, _ = case.oracle_planes(oracle)
    for side, planes in (("k", kp), ("v", vp)):
        gc = getattr(case, side)
        for l in range(case.w.n_loops - 1):
            for name in ("codes", "meta", "alpha"):
                got = plane_bits(getattr(gc, name)[l])[:, :, t_lo:t_hi]
                want = getattr(planes, name)[l][:, :, t_lo:t_hi]
                if not np.array_equal(got, want):
                    bad = np.argwhere(got != want)
                    raise AssertionError(f"{side} loop {l} {name}: {len(bad)} mismatches, first at {bad[0]}")
                if t_hi < case.cap:     # slots past the encoded range untouched
                    assert not plane_bits(getattr(gc, name)[l])[:, :, t_hi:].any()


CASES = {
    "tiny-d64-int2-norot": dict(w=_w(d=64, bits=(2,), rotate=0, B=1, H=1, seed=0), n=128),
    "tiny-d64-int2-rot": dict(w=_w(d=64, bits=(2,), rotate=1, B=1, H=1, seed=0), n=128),
    "d128-int2x3-ragged": dict(w=_w(), n=203, cap=256),
    "d128-mixed-4-2-2": dict(w=_w(bits=(4, 2, 2)), n=77),
    "d128-g16": dict(w=_w(g=16, bits=(2, 4, 2)), n=64),
    "d256-int2-int4": dict(w=_w(d=256, bits=(2, 4), B=1, H=2), n=41),
    "d64-g16-int4-norot": dict(w=_w(d=64, g=16, bits=(4,), rotate=0, B=3, H=1), n=33),
    "d128-many-loops": dict(w=_w(bits=(2, 4, 2, 2, 4), B=1, H=2), n=19),
    "one-token": dict(w=_w(B=1, H=1), n=1),
}


@pytest.mark.parametrize("name", list(CASES))
def test_encode_bit_exact(oracle, name):
    cfg = CASES[name]
    case = Case(cfg["w"], cfg["n"], cap=cfg.get("cap", 0))
    _compare(case, oracle, 0, cfg["n"])


def test_encode_chunked_appends(oracle):
    """Prefill in uneven chunks then single-token appends: same bytes as the
    oracle's one-shot encode (the encoder has no cross-token state)."""
    w = _w(bits=(4, 2, 2))
    n = 70
    chunks = [(0, 33), (33, 20)] + [(t, 1) for t in range(53, 70)]
    case = Case(w, n, cap=80, t_chunks=chunks)
    _compare(case, oracle, 0, n)


def test_encode_degenerate_vectors(oracle):
    """Zero reference (alpha = 0), exact multiples (zero residual, zero scale),
    constant vectors, huge and tiny magnitudes (saturation, subnormal FP16,
    group ranges beyond 2^120, FP32-subnormal ranges)."""
    w = _w(bits=(2, 4), B=1, H=1)
    case = Case(w, 16, cap=16)
    import decode_attention_rq_amd as rq
    g = torch.Generator().manual_seed(3)
    kref = torch.randn(1, 1, 16, 128, generator=g)
    kin = torch.randn(2, 1, 1, 16, 128, generator=g)
    kref[..., 0, :] = 0.0                                  # zero reference
    kin[:, :, :, 1] = kref[..., 1, :] * 0.75               # exact multiple (before bf16 rounding)
    kref[..., 2, :] = torch.round(kref[..., 2, :] * 8) / 8
    kin[:, :, :, 2] = kref[..., 2, :] * 0.5                # exact in bf16 too
    kin[:, :, :, 3] = 1.5                                  # constant loop vector
    kin[:, :, :, 4] *= 3e4                                 # scales near the FP16 limit
    kin[:, :, :, 5] *= 1e6                                 # saturating scale/zero
    kin[:, :, :, 6] *= 1e-6                                # subnormal FP16 scales
    kref[..., 7, :] *= 1e-20                               # tiny reference: huge alpha, saturated
    kin[:, :, :, 8] *= 1e36                                # group ranges past 2^120: the scale's quotient
                                                           # is taken on a clamped range (still finite)
    kin[:, :, :, 9] *= 1e-39                               # BF16 subnormal inputs: FP32-subnormal ranges
    kref, kin = kref.to(torch.bfloat16), kin.to(torch.bfloat16)
    case.data["k_ref"], case.data["k_loops"] = kref, kin
    case.data["v_ref"], case.data["v_loops"] = kref.clone(), kin.clone()
    for side in (case.k, case.v):
        side.ref.copy_(kref.cuda())
    rq.rq_encode(case.lay, case.k, case.v, kin.cuda().contiguous(), kin.cuda().contiguous(), 0, 16)
    torch.cuda.synchronize()
    _compare(case, oracle, 0, 16)
    # the exact-multiple token really has a zero residual on the oracle side too
    lay, kp, vp, _ = case.oracle_planes(oracle)
    assert not kp.codes[0][0, 0, 2].any() and not kp.meta[0][0, 0, 2].any()
