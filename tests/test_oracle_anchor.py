"""Pins of the oracle's quantized anchor and BF16 tail.

ResidualQuant page ("ResidualQuant: KV Cache Quantization for Looped
Transformers with 2-Bit Residuals"): the final configuration stores the final
loop itself at INT4 ("Ascending [2,2,2,4]", Fig. 3 caption; one INT4 anchor
per loop group, Table 8 caption; INT4 anchors at g=32 with INT2 residuals at
g=16, Fig. 6 caption), and recent tokens stay in BF16 (Table 10, "Recent 64").
Readings pinned here: the anchor goes through the same rotation and group
quantizer as a residual (no LS coefficient); residuals are taken against the
dequantized anchor; tail tokens are attended as plain BF16 keys and values
after the cached ones.
"""
import numpy as np
import pytest
import torch

import synth
from synth import bf16_bits


def _bf16(x):
    return bf16_bits(torch.from_numpy(np.asarray(x, dtype=np.float32)).to(torch.bfloat16))


def _f32(bits):
    return (np.asarray(bits, dtype=np.uint32) << 16).view(np.float32)


def _f16_bits(x):
    return np.asarray(x, dtype=np.float16).view(np.uint16)


def _grid_anchor(rng, d, g, bits):
    """A vector that lies exactly on an INT`bits` grid in every group: offset z
    (a few-bit FP16 value), step s = 2^e, codes with 0 and the top code present
    so that min and max give back exactly s and z.  Every value is exact in
    BF16.  Returns (y_bits, codes, s[G], z[G])."""
    top = (1 << bits) - 1
    G = d // g
    codes = rng.integers(0, top + 1, size=d)
    s = 2.0 ** rng.integers(-5, -2, size=G)
    z = -rng.integers(0, 32, size=G) / 16.0
    for k in range(G):
        idx = rng.permutation(g)[:2] + k * g
        codes[idx[0]], codes[idx[1]] = 0, top
    y = z[np.arange(d) // g] + s[np.arange(d) // g] * codes
    yb = _bf16(y)
    assert np.array_equal(_f32(yb).astype(np.float64), y)        # exact in BF16
    return yb, codes.astype(np.uint8), s, z


@pytest.mark.parametrize("bits,g", [(4, 32), (2, 16), (4, 16)])
def test_anchor_worked_example_on_its_grid(oracle, bits, g):
    """Without rotation a vector already on a grid is quantized to that grid:
    the codes, FP16 scale and offset come back as constructed, and the
    dequantized anchor equals the input exactly."""
    rng = np.random.default_rng(bits * 100 + g)
    d = 128
    yb, codes, s, z = _grid_anchor(rng, d, g, bits)
    packed, meta, yhat = oracle.anchor_vector(yb, g, bits, rotate=False)
    assert np.array_equal(oracle.unpack(packed, d, bits), codes)
    assert np.array_equal(meta.reshape(-1, 2)[:, 0], _f16_bits(s))
    assert np.array_equal(meta.reshape(-1, 2)[:, 1], _f16_bits(z))
    assert np.array_equal(yhat, _f32(yb))
    assert np.array_equal(oracle.dequant_f64(packed, meta, d, g, bits, False), _f32(yb).astype(np.float64))


def _layouts(L=4, B=2, H=2, d=128, g=16, n=24, rotate=0, bits=(2, 2, 2), ref_bits=4, ref_group=32):
    common = dict(n_loops=L, batch=B, heads=H, d=d, g=g, cap=n, rotate=rotate, bits=list(bits))
    return dict(common), dict(common, ref_bits=ref_bits, ref_group=ref_group)


def test_exact_anchor_reduces_to_the_bf16_reference(oracle):
    """When the anchor is exactly representable on its grid, its dequantized
    value IS the BF16 reference, so encoding against the anchor gives the very
    bytes that encoding against the BF16 reference gives."""
    rng = np.random.default_rng(7)
    L, B, H, d, g, n = 4, 2, 2, 128, 16, 24
    lay_bf, lay_an = _layouts(L, B, H, d, g, n)
    ref = np.zeros((B, H, n, d), dtype=np.uint16)
    for b in range(B):
        for h in range(H):
            for t in range(n):
                ref[b, h, t] = _grid_anchor(rng, d, 32, 4)[0]
    yf = _f32(ref)
    x = np.stack([_bf16(c * yf + 0.1 * rng.standard_normal(yf.shape)) for c in (0.8, 0.85, 0.9)])
    p_bf = oracle.Planes(L, B, H, d, g, n, [2, 2, 2])
    p_bf.ref[:] = ref
    oracle.encode(lay_bf, p_bf, x, 0, n)
    p_an = oracle.Planes(L, B, H, d, g, n, [2, 2, 2], ref_bits=4, ref_group=32)
    oracle.encode(lay_an, p_an, np.concatenate([x, ref[None]]), 0, n)
    for l in range(L - 1):
        assert np.array_equal(p_bf.codes[l], p_an.codes[l])
        assert np.array_equal(p_bf.meta[l], p_an.meta[l])
        assert np.array_equal(p_bf.alpha[l], p_an.alpha[l])
    assert np.array_equal(oracle.reconstruct(lay_an, p_an, L - 1, 0, n), yf.astype(np.float64))


@pytest.mark.parametrize("rotate", [0, 1])
@pytest.mark.parametrize("bits,g", [(4, 32), (2, 32)])
def test_anchor_round_trip_is_within_the_grid(oracle, rotate, bits, g):
    """|u_i - (z + s q_i)| <= s/2 in the rotated domain, and the normalized
    Hadamard matrix is orthonormal, so ||y - y_hat||_2 <= sqrt(sum_k g (s_k/2)^2)."""
    rng = np.random.default_rng(31 + rotate + bits)
    d = 128
    for _ in range(20):
        yb = _bf16(rng.standard_normal(d) * np.exp(0.5 * rng.standard_normal(d)))
        packed, meta, yhat32 = oracle.anchor_vector(yb, g, bits, rotate=bool(rotate))
        y = _f32(yb).astype(np.float64)
        yhat = oracle.dequant_f64(packed, meta, d, g, bits, bool(rotate))
        s = oracle.f16_bits_to_f32(meta.reshape(-1, 2)[:, 0]).astype(np.float64)
        grid = np.sqrt((g * (s / 2) ** 2).sum())
        assert np.linalg.norm(y - yhat) <= grid * (1 + 1e-3) + 1e-6 * np.linalg.norm(y)
        # the FP32 value the encoder subtracts is the FP64 one to FP32 rounding
        assert np.abs(yhat32 - yhat).max() <= 1e-5 * np.abs(yhat).max()


@pytest.mark.parametrize("rotate", [0, 1])
def test_residual_is_taken_against_the_dequantized_anchor(oracle, rotate):
    """A loop equal to the dequantized anchor (rounded to BF16) is
    reconstructed to within its own tiny residual grid -- far closer than the
    anchor's quantization error, which a residual taken against the BF16 input
    would leave uncorrected."""
    rng = np.random.default_rng(5 + rotate)
    d, g, ga = 128, 16, 32
    lay = dict(n_loops=2, batch=1, heads=1, d=d, g=g, cap=16, rotate=rotate, bits=[2],
               ref_bits=4, ref_group=ga)
    y = _bf16(rng.standard_normal((16, d)) * np.exp(0.5 * rng.standard_normal(d)))
    yhat32 = np.stack([oracle.anchor_vector(v, ga, 4, bool(rotate))[2] for v in y])
    x = _bf16(yhat32)
    p = oracle.Planes(2, 1, 1, d, g, 16, [2], ref_bits=4, ref_group=ga)
    oracle.encode(lay, p, np.stack([x, y])[:, None, None], 0, 16)
    xh = oracle.reconstruct(lay, p, 0, 0, 16)[0, 0]
    yh = oracle.reconstruct(lay, p, 1, 0, 16)[0, 0]
    xf, yf = _f32(x).astype(np.float64), _f32(y).astype(np.float64)
    alpha = oracle.f16_bits_to_f32(p.alpha[0].ravel())
    assert np.all(np.abs(alpha - 1.0) <= 2.0 ** -9)
    err = np.abs(xh - xf).max(1)
    anchor_err = np.abs(yh - yf).max(1)
    assert np.all(err <= 2.0 ** -8 * np.abs(xf).max(1))
    assert np.all(err < 0.1 * anchor_err)


@pytest.mark.parametrize("seed", range(4))
def test_anchored_alpha_is_the_least_squares_minimiser(oracle, seed):
    """Brute-force scan of ||x - a*y_hat||^2 (FP64, y_hat the FP32 dequantized
    anchor) finds the stored coefficient's unrounded value."""
    rng = np.random.default_rng(50 + seed)
    d = 128
    y = _bf16(rng.standard_normal(d) * np.exp(0.5 * rng.standard_normal(d)))
    _, _, yhat = oracle.anchor_vector(y, 32, 4, True)
    x = _bf16(_f32(y) * rng.uniform(0.5, 1.2) + 0.2 * rng.standard_normal(d))
    a32 = float(oracle.lib().rqo_alpha_f32_y(x, yhat, d))
    xf, yf = _f32(x).astype(np.float64), yhat.astype(np.float64)
    grid = a32 + np.arange(-0.5, 0.5, 1e-5)
    f = ((xf[None, :] - grid[:, None] * yf[None, :]) ** 2).sum(1)
    assert abs(grid[np.argmin(f)] - a32) <= 1.5e-5
    _, _, a16 = oracle.encode_vector_y(x, yhat, 16, 2, True)
    assert a16 == oracle.f32_to_f16_bits(np.array([a32]))[0]


@pytest.mark.parametrize("rotate", [0, 1])
def test_anchored_reconstruction_error_bound(oracle, rotate):
    """x - x_hat = r - r_hat + a (y_hat32 - y_hat64): within the residual grid
    error plus the FP32 rounding of the dequantized anchor."""
    w = synth.Workload("a", n_loops=4, batch=2, heads=2, d=128, g=16, n_ctx=40, bits=[2, 2, 2],
                       c=[0.8, 0.85, 0.9], sigma=[0.15, 0.12, 0.1], rotate=rotate, seed=9)
    data = synth.draw_layer(w)
    lay = dict(n_loops=4, batch=2, heads=2, d=128, g=16, cap=40, rotate=rotate, bits=[2, 2, 2],
               ref_bits=4, ref_group=32)
    p = oracle.Planes(4, 2, 2, 128, 16, 40, [2, 2, 2], ref_bits=4, ref_group=32)
    xin = np.concatenate([bf16_bits(data["k_loops"]), bf16_bits(data["k_ref"])[None]])
    oracle.encode(lay, p, xin, 0, 40)
    for l in range(3):
        xh = oracle.reconstruct(lay, p, l, 0, 40)
        x = data["k_loops"][l].double().numpy()
        s = oracle.f16_bits_to_f32(p.meta[l][..., 0].ravel()).reshape(p.meta[l].shape[:-1])
        grid = np.sqrt((16 * (s.astype(np.float64) / 2) ** 2).sum(-1))
        err = np.linalg.norm(x - xh, axis=-1)
        assert np.all(err <= grid * (1 + 1e-3) + 1e-5 * np.linalg.norm(x, axis=-1))


def _sdpa(q, k, v, scale):
    q = torch.from_numpy(q).double()[None, None, None]
    k = torch.from_numpy(k).double()[None, None]
    v = torch.from_numpy(v).double()[None, None]
    return torch.nn.functional.scaled_dot_product_attention(q, k, v, scale=scale)[0, 0, 0].numpy()


@pytest.mark.parametrize("anchor", [False, True])
def test_tail_is_attended_after_the_cache(oracle, anchor):
    """Reference loop with a BF16 tail = library attention over the cached
    reference rows followed by the tail rows.  With an anchor on its grid the
    cached rows are the BF16 input itself."""
    rng = np.random.default_rng(77 + anchor)
    L, d, g, n, T = 2, 128, 16, 20, 5
    ref = np.stack([_grid_anchor(rng, d, 32, 4)[0] for _ in range(n)])[None, None]
    vref = np.stack([_grid_anchor(rng, d, 32, 4)[0] for _ in range(n)])[None, None]
    lay = dict(n_loops=L, batch=1, heads=1, d=d, g=g, cap=n, rotate=0, bits=[2])
    if anchor:
        lay.update(ref_bits=4, ref_group=32)
    kp = oracle.Planes(L, 1, 1, d, g, n, [2], **({"ref_bits": 4, "ref_group": 32} if anchor else {}))
    vp = oracle.Planes(L, 1, 1, d, g, n, [2], **({"ref_bits": 4, "ref_group": 32} if anchor else {}))
    xk = _bf16(0.9 * _f32(ref) + 0.1 * rng.standard_normal(ref.shape))[None]
    xv = _bf16(0.9 * _f32(vref) + 0.1 * rng.standard_normal(ref.shape))[None]
    if anchor:
        oracle.encode(lay, kp, np.concatenate([xk, ref[None]]), 0, n)
        oracle.encode(lay, vp, np.concatenate([xv, vref[None]]), 0, n)
    else:
        kp.ref[:], vp.ref[:] = ref, vref
        oracle.encode(lay, kp, xk, 0, n)
        oracle.encode(lay, vp, xv, 0, n)
    q = _bf16(rng.standard_normal((L, 1, 1, d)))
    tk = _bf16(rng.standard_normal((T, d)))
    tv = _bf16(rng.standard_normal((T, d)))
    got = oracle.decode_row(lay, kp, vp, q, L - 1, 0, 0, n, 0.2, tk, tv)
    k = np.concatenate([_f32(ref[0, 0]), _f32(tk)]).astype(np.float64)
    v = np.concatenate([_f32(vref[0, 0]), _f32(tv)]).astype(np.float64)
    want = _sdpa(_f32(q[L - 1, 0, 0]).astype(np.float64), k, v, 0.2)
    assert np.allclose(got, want, rtol=1e-12, atol=1e-12)
    # tail only: no cached tokens at all
    got0 = oracle.decode_row(lay, kp, vp, q, L - 1, 0, 0, 0, 0.2, tk, tv)
    want0 = _sdpa(_f32(q[L - 1, 0, 0]).astype(np.float64), _f32(tk).astype(np.float64),
                  _f32(tv).astype(np.float64), 0.2)
    assert np.allclose(got0, want0, rtol=1e-12, atol=1e-12)
    # a residual loop's row with a tail = attention over its reconstruction + tail
    kh = oracle.reconstruct(lay, kp, 0, 0, n)[0, 0]
    vh = oracle.reconstruct(lay, vp, 0, 0, n)[0, 0]
    got1 = oracle.decode_row(lay, kp, vp, q, 0, 0, 0, n, 0.2, tk, tv)
    want1 = _sdpa(_f32(q[0, 0, 0]).astype(np.float64), np.concatenate([kh, _f32(tk)]),
                  np.concatenate([vh, _f32(tv)]), 0.2)
    assert np.allclose(got1, want1, rtol=1e-12, atol=1e-12)


def test_anchor_groups_are_independent_schedules(oracle):
    """Table 8 caption: with several anchor groups each group of loops ends in
    its own INT4 anchor.  An 8-loop 2 x [2,2,2,4] layout encodes, reconstructs
    and decodes exactly as its two 4-loop halves do on their own."""
    rng = np.random.default_rng(88)
    L, G, B, H, d, g, n = 8, 4, 1, 2, 64, 16, 12
    bits = [2, 4, 2, 0, 2, 2, 4, 0]
    lay = dict(n_loops=L, batch=B, heads=H, d=d, g=g, cap=n, rotate=1, bits=bits, ref_bits=4,
               ref_group=32, group_loops=G)
    x = _bf16(rng.standard_normal((L, B, H, n, d)))
    whole = oracle.Planes(L, B, H, d, g, n, bits, 4, 32, group_loops=G)
    oracle.encode(lay, whole, x, 0, n)
    q = _bf16(rng.standard_normal((L, B, H, d)))
    tk = _bf16(rng.standard_normal((L, B, H, 3, d)))
    tv = _bf16(rng.standard_normal((L, B, H, 3, d)))
    for g0 in (0, G):
        sub = dict(lay, n_loops=G, bits=bits[g0:g0 + G], group_loops=0)
        part = oracle.Planes(G, B, H, d, g, n, bits[g0:g0 + G], 4, 32)
        oracle.encode(sub, part, x[g0:g0 + G], 0, n)
        for l in range(G):
            assert np.array_equal(whole.codes[g0 + l], part.codes[l])
            assert np.array_equal(whole.meta[g0 + l], part.meta[l])
            if l < G - 1:
                assert np.array_equal(whole.alpha[g0 + l], part.alpha[l])
            assert np.array_equal(oracle.reconstruct(lay, whole, g0 + l, 0, n),
                                  oracle.reconstruct(sub, part, l, 0, n))
            got = oracle.decode_row(lay, whole, whole, q, g0 + l, 0, 1, n, 0.3, tk[g0 + l, 0, 1], tv[g0 + l, 0, 1])
            want = oracle.decode_row(sub, part, part, q[g0:g0 + G], l, 0, 1, n, 0.3, tk[g0 + l, 0, 1],
                                     tv[g0 + l, 0, 1])
            assert np.array_equal(got, want)


# --------------------------------------------------------------------------
# chained references (Table 9 "Previous-loop" / "Next-loop")
# --------------------------------------------------------------------------

def _chain_layout(L, ref_first, anchored, n, d=64, g=16):
    lay = dict(n_loops=L, batch=1, heads=2, d=d, g=g, cap=n, rotate=1, bits=[2] * L, ref_chain=1,
               ref_first=ref_first)
    if anchored:
        lay.update(ref_bits=4, ref_group=32)
    return lay


@pytest.mark.parametrize("ref_first", [0, 1])
def test_chain_references_the_neighbour(oracle, ref_first):
    """Loops that halve along the chain: with the neighbour as reference every
    stored alpha is 0.5 (the Last-loop policy would store 0.5, 0.25, 0.125)."""
    rng = np.random.default_rng(17)
    L, n, d = 4, 6, 64
    lay = _chain_layout(L, ref_first, False, n, d=d)
    root = 0 if ref_first else L - 1
    y = _bf16(rng.standard_normal((1, 2, n, d)))
    yf = _f32(y)
    loops = {}
    for k, l in enumerate(oracle.chain_order(lay, 0)[2]):
        loops[l] = _bf16(yf * 0.5 ** (k + 1))            # exact in BF16
    x = np.stack([loops[l] for l in range(L) if l != root])
    p = oracle.Planes(L, 1, 2, d, 16, n, lay["bits"], ref_first=ref_first)
    p.ref[:] = y
    oracle.encode(lay, p, x, 0, n)
    for l in range(L):
        if l != root:
            assert np.all(p.alpha[l] == 0x3800), l          # FP16 0.5
            # and the chain rebuilds each loop exactly (zero residuals)
            assert np.array_equal(oracle.reconstruct(lay, p, l, 0, n), _f32(loops[l]).astype(np.float64))


@pytest.mark.parametrize("anchored", [False, True])
@pytest.mark.parametrize("ref_first", [0, 1])
def test_chain_error_does_not_accumulate(oracle, anchored, ref_first):
    """Closed loop along the chain: each loop is rebuilt to within its own
    grid error, however far from the root (an open chain would add up the
    errors of every loop in between)."""
    w = synth.Workload("c", n_loops=4, batch=1, heads=2, d=64, g=16, n_ctx=30, bits=[2, 2, 2],
                       c=[0.8, 0.85, 0.9], sigma=[0.15, 0.12, 0.1], rotate=1, seed=23)
    data = synth.draw_layer(w)
    lay = _chain_layout(4, ref_first, anchored, 30)
    root = 0 if ref_first else 3
    loops = [bf16_bits(data["k_loops"][i]) for i in range(3)]
    refb = bf16_bits(data["k_ref"])
    seq = [refb] + loops if ref_first else loops + [refb]      # loop order
    p = oracle.Planes(4, 1, 2, 64, 16, 30, lay["bits"], 4 if anchored else 0, 32 if anchored else None,
                      ref_first=ref_first)
    if anchored:
        oracle.encode(lay, p, np.stack(seq), 0, 30)
    else:
        p.ref[:] = refb
        oracle.encode(lay, p, np.stack([seq[l] for l in range(4) if l != root]), 0, 30)
    for l in range(4):
        if l == root:
            continue
        xh = oracle.reconstruct(lay, p, l, 0, 30)
        x = _f32(seq[l]).astype(np.float64)
        s = oracle.f16_bits_to_f32(p.meta[l][..., 0].ravel()).reshape(p.meta[l].shape[:-1]).astype(np.float64)
        grid = np.sqrt((16 * (s / 2) ** 2).sum(-1))
        err = np.linalg.norm(x - xh, axis=-1)
        assert np.all(err <= grid * (1 + 1e-3) + 1e-5 * np.linalg.norm(x, axis=-1)), l
        # decode over the chain's reconstruction is plain attention over it
        q = _bf16(np.random.default_rng(l).standard_normal((4, 1, 2, 64)))
        got = oracle.decode_row(lay, p, p, q, l, 0, 1, 30, 0.3)
        want = _sdpa(_f32(q[l, 0, 1]).astype(np.float64), xh[0, 1], xh[0, 1], 0.3)
        assert np.allclose(got, want, rtol=1e-12, atol=1e-12)


def test_chain_of_one_residual_is_the_plain_policy(oracle):
    """With a single residual loop its neighbour is the root: the chain policy
    gives the Last-loop bytes."""
    rng = np.random.default_rng(3)
    y = _bf16(rng.standard_normal((1, 2, 9, 64)))
    x = _bf16(0.9 * _f32(y) + 0.1 * rng.standard_normal((1, 1, 2, 9, 64)))
    base = dict(n_loops=2, batch=1, heads=2, d=64, g=16, cap=9, rotate=1, bits=[2])
    pa = oracle.Planes(2, 1, 2, 64, 16, 9, [2])
    pb = oracle.Planes(2, 1, 2, 64, 16, 9, [2])
    pa.ref[:], pb.ref[:] = y, y
    oracle.encode(base, pa, x, 0, 9)
    oracle.encode(dict(base, ref_chain=1), pb, x, 0, 9)
    assert np.array_equal(pa.codes[0], pb.codes[0]) and np.array_equal(pa.meta[0], pb.meta[0])
    assert np.array_equal(pa.alpha[0], pb.alpha[0])
