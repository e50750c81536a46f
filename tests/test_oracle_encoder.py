"""Pins of the oracle's encoder steps against what the pages and mathematics fix.

ResidualQuant page ("ResidualQuant: KV Cache Quantization for Looped
Transformers with 2-Bit Residuals"):
  * least-square scaling (Abstract; Fig. 1 step 3; Fig. 2 residual K2 - a2*K1;
    Fig. 3 right: LS against alpha = 1),
  * rotation of the residual (Abstract; Fig. 1 step 4),
  * group-wise INT2/INT4 quantization with scales and offsets (Fig. 1, Table 5,
    Table 8 caption).
Each pin is chosen so that a plausible slip (dropped term, wrong sign or index,
transposed operand, wrong rounding) fails it.
"""
import numpy as np
import pytest
import scipy.linalg

from synth import bf16_bits


def _bf16(x):
    import torch
    return bf16_bits(torch.from_numpy(np.asarray(x, dtype=np.float32)).to(torch.bfloat16))


def _f32(bits):
    return (np.asarray(bits, dtype=np.uint32) << 16).view(np.float32)


# --------------------------------------------------------------------------
# least-square coefficient
# --------------------------------------------------------------------------

@pytest.mark.parametrize("seed", range(6))
def test_alpha_is_the_least_squares_minimiser(oracle, seed):
    """Brute-force scan of f(a) = ||x - a*y||^2 in FP64 finds the closed form."""
    rng = np.random.default_rng(seed)
    d = 128
    y = _bf16(rng.standard_normal(d) * np.exp(0.5 * rng.standard_normal(d)))
    x = _bf16(_f32(y) * rng.uniform(0.5, 1.2) + 0.2 * rng.standard_normal(d))
    a32 = oracle.alpha_f32(x, y)
    xf, yf = _f32(x).astype(np.float64), _f32(y).astype(np.float64)
    grid = a32 + np.arange(-0.5, 0.5, 1e-5)
    f = ((xf[None, :] - grid[:, None] * yf[None, :]) ** 2).sum(1)
    assert abs(grid[np.argmin(f)] - a32) <= 1.5e-5
    # and agrees with the exact ratio to FP32 rounding of two tree sums
    exact = float(np.dot(xf, yf) / np.dot(yf, yf))
    assert abs(a32 - exact) <= 1e-5 * abs(exact) + 1e-7


@pytest.mark.parametrize("seed", range(6))
def test_ls_never_worse_than_alpha_one(oracle, seed):
    """Fig. 3 right: removing LS scaling (alpha = 1) only adds error.  The stored
    FP16 coefficient is the half nearest the optimum and 1.0 is a half, so the
    stored value is at least as good as 1."""
    rng = np.random.default_rng(100 + seed)
    d = 64
    y = _bf16(rng.standard_normal(d))
    x = _bf16(_f32(y) * rng.uniform(0.3, 1.7) + 0.3 * rng.standard_normal(d))
    a = oracle.f16_bits_to_f32(np.array([oracle.alpha_bits(x, y)], dtype=np.uint16))[0]
    xf, yf = _f32(x).astype(np.float64), _f32(y).astype(np.float64)
    err = lambda al: float(((xf - al * yf) ** 2).sum())
    assert err(a) <= err(1.0) * (1 + 1e-12)


def test_alpha_exact_multiple_gives_zero_residual(oracle):
    """x = c*y exactly -> alpha = c and the residual vanishes: every code is 0,
    every scale and offset is +0."""
    rng = np.random.default_rng(5)
    y = _bf16(np.round(rng.standard_normal(128) * 16) / 16)
    x = _bf16(_f32(y) * 0.75)
    assert np.array_equal(_f32(x), _f32(y) * np.float32(0.75))
    assert oracle.alpha_f32(x, y) == 0.75
    packed, meta, a = oracle.encode_vector(x, y, g=32, bits=2, rotate=True)
    assert a == 0x3a00  # 0.75 in binary16
    assert not packed.any() and not meta.any()


def test_alpha_zero_reference(oracle):
    """Reading: a zero reference vector gives alpha = 0 (no prediction)."""
    x = _bf16(np.linspace(-1, 1, 64))
    y = np.zeros(64, dtype=np.uint16)
    assert oracle.alpha_f32(x, y) == 0.0
    packed, meta, a = oracle.encode_vector(x, y, g=32, bits=2, rotate=False)
    assert a == 0


def test_tree_sum_order_worked_example(oracle):
    """The pairwise-halving order, worked by hand: [2^24, 1, -2^24, 1] ->
    (2^24 + -2^24, 1 + 1) = (0, 2) -> 2.  Left-to-right float summation gives 1."""
    a = np.array([2.0 ** 24, 1.0, -(2.0 ** 24), 1.0], dtype=np.float32)
    assert oracle.tree_sum(a) == 2.0
    seq = np.float32(0)
    for v in a:
        seq = np.float32(seq + v)
    assert seq == 1.0


def test_dot_sum_order_worked_example(oracle):
    """The dot-product order (blocks of 8 by halving, then over blocks), worked
    by hand on 16 terms with a = 2^24 at 0, 1 at 1 and 4, -2^24 at 8:
    block 0: (2^24 + 1, 1, 0, 0) -> (2^24, 1) -> 2^24 (each 2^24 + 1 rounds to
    the even 2^24); block 1: -2^24; total 0.  Plain halving over all 16 terms
    pairs 2^24 with -2^24 first and gives the exact 2."""
    a = np.zeros(16, dtype=np.float32)
    a[0], a[1], a[4], a[8] = 2.0 ** 24, 1.0, 1.0, -(2.0 ** 24)
    assert oracle.dot_sum(a) == 0.0
    assert oracle.tree_sum(a) == 2.0


def test_tree_sum_exact_and_bounded(oracle):
    rng = np.random.default_rng(3)
    ints = rng.integers(-1000, 1000, size=256).astype(np.float32)
    assert oracle.tree_sum(ints) == float(ints.sum(dtype=np.float64))
    assert oracle.dot_sum(ints) == float(ints.sum(dtype=np.float64))
    for d in (64, 128, 256):
        a = (rng.standard_normal(d) * 10).astype(np.float32)
        gamma = np.log2(d) * 2.0 ** -24 / (1 - np.log2(d) * 2.0 ** -24)
        for f in (oracle.tree_sum, oracle.dot_sum):
            err = abs(f(a) - float(np.sum(a.astype(np.float64))))
            assert err <= gamma * float(np.abs(a).sum())


# --------------------------------------------------------------------------
# rotation
# --------------------------------------------------------------------------

@pytest.mark.parametrize("d", [64, 128, 256])
def test_fwht_columns_are_sylvester_hadamard(oracle, d):
    """The oracle's transform of e_j is column j of H_d / sqrt(d) with H_d
    Sylvester-ordered (scipy.linalg.hadamard), sign for sign."""
    H = scipy.linalg.hadamard(d)
    c = np.float32(1.0 / np.sqrt(d))
    for j in (0, 1, 2, d // 2 - 1, d // 2, d - 1, 37 % d):
        e = np.zeros(d, dtype=np.float32)
        e[j] = 1.0
        assert np.array_equal(oracle.fwht_f32(e), (H[:, j] * c).astype(np.float32))


@pytest.mark.parametrize("d", [64, 128, 256])
def test_fwht_matches_library_hadamard(oracle, d):
    rng = np.random.default_rng(d)
    H = scipy.linalg.hadamard(d).astype(np.float64)
    assert np.array_equal(H @ H.T, d * np.eye(d))          # H H^T = d I, exactly
    for _ in range(20):
        r = (rng.standard_normal(d) * np.exp(rng.standard_normal(d))).astype(np.float32)
        got = oracle.fwht_f32(r).astype(np.float64)
        want = H @ r.astype(np.float64) / np.sqrt(d)
        bound = (np.log2(d) + 2) * 2.0 ** -24 * np.abs(r).sum() / np.sqrt(d) * 2
        assert np.max(np.abs(got - want)) <= bound
        # orthonormal: norm preserved; applying it twice is the identity
        assert abs(np.linalg.norm(got) - np.linalg.norm(r)) <= 1e-5 * np.linalg.norm(r)
        twice = oracle.fwht_f32(oracle.fwht_f32(r)).astype(np.float64)
        assert np.max(np.abs(twice - r)) <= 1e-5 * np.abs(r).max() * 4


# --------------------------------------------------------------------------
# group quantization and packing
# --------------------------------------------------------------------------

@pytest.mark.parametrize("bits", [2, 4])
@pytest.mark.parametrize("seed", range(5))
def test_quantizer_round_trip_and_nearest_level(oracle, bits, seed):
    rng = np.random.default_rng(seed * 7 + bits)
    for g in (16, 32):
        u = (rng.standard_normal(g) * rng.uniform(0.01, 3)).astype(np.float32)
        codes, s16, z16 = oracle.quantize_group(u, bits)
        s, z = oracle.f16_bits_to_f32(np.array([s16, z16], dtype=np.uint16)).astype(np.float64)
        levels = 2 ** bits - 1
        assert codes.max() <= levels
        # the stored scale and offset are the FP16 roundings of (max-min)/levels and min
        assert s16 == np.float32((u.max() - u.min()) / np.float32(levels)).astype(np.float16).view(np.uint16)
        assert z16 == np.float16(u.min()).view(np.uint16)
        deq = z + s * codes
        lo, hi = z, z + levels * s
        inside = (u >= lo) & (u <= hi)
        assert np.all(np.abs(u[inside] - deq[inside]) <= s / 2 + 2.0 ** -16 * s)
        # outside the grid only because of FP16 rounding of s and z
        edge = max(abs(u.min() - lo), abs(u.max() - hi))
        assert np.all(np.abs(u - deq) <= s / 2 + edge + 2.0 ** -16 * s)
        # brute force: the code is a nearest level (away from exact ties)
        dist = np.abs(u[:, None].astype(np.float64) - (z + s * np.arange(levels + 1))[None, :])
        best = dist.min(1)
        mine = dist[np.arange(g), codes]
        assert np.all((mine - best) <= 4 * 2.0 ** -24 * (np.abs(u) + abs(z) + s * levels))


def test_quantizer_constant_group(oracle):
    u = np.full(32, 0.3, dtype=np.float32)
    codes, s16, z16 = oracle.quantize_group(u, 2)
    assert s16 == 0 and not codes.any()
    assert z16 == np.float16(0.3).view(np.uint16)


def test_quantizer_ties_round_to_even(oracle):
    """u = z + (k + 1/2) s exactly: round-half-even picks the even code."""
    u = np.array([0.0, 0.5, 1.5, 2.5, 3.0] + [0.0] * 27, dtype=np.float32)  # s = 1, z = 0
    codes, s16, z16 = oracle.quantize_group(u, 2)
    assert s16 == 0x3c00 and z16 == 0
    assert list(codes[:5]) == [0, 0, 2, 2, 3]


def test_packing_worked_example(oracle):
    """LSB-first packing, worked by hand."""
    c2 = np.array([0, 1, 2, 3, 3, 2, 1, 0], dtype=np.uint8)
    assert list(oracle.pack(c2, 2)) == [0b11100100, 0b00011011]
    c4 = np.array([1, 15, 7, 8], dtype=np.uint8)
    assert list(oracle.pack(c4, 4)) == [0xF1, 0x87]
    rng = np.random.default_rng(0)
    for bits in (2, 4):
        c = rng.integers(0, 2 ** bits, size=128).astype(np.uint8)
        assert np.array_equal(oracle.unpack(oracle.pack(c, bits), 128, bits), c)


def test_groups_are_contiguous_dims(oracle):
    """Group k covers dims [k*g, (k+1)*g): a residual that is constant on dims
    32..63 only gives a zero scale in group 1 only (no rotation)."""
    rng = np.random.default_rng(9)
    r = rng.standard_normal(128).astype(np.float32)
    r[32:64] = 0.5
    x = _bf16(r)
    y0 = np.zeros(128, dtype=np.uint16)  # zero reference -> alpha = 0, residual = x
    packed, meta, a = oracle.encode_vector(x, y0, g=32, bits=2, rotate=False)
    scales = meta[0::2]
    assert scales[1] == 0 and all(scales[k] != 0 for k in (0, 2, 3))
    assert meta[3] == np.float16(_f32(x)[32]).view(np.uint16)


# --------------------------------------------------------------------------
# scaling-coefficient variants (Table 9 columns "Residual", "Norm-ratio",
# "LS scaling"; Fig. 3 right: alpha = 1 without LS)
# --------------------------------------------------------------------------

@pytest.mark.parametrize("seed", range(4))
def test_alpha_modes_closed_forms(oracle, seed):
    rng = np.random.default_rng(300 + seed)
    d = 128
    y = _bf16(rng.standard_normal(d) * np.exp(0.5 * rng.standard_normal(d)))
    x = _bf16(_f32(y) * rng.uniform(0.5, 1.2) + 0.3 * rng.standard_normal(d))
    yf = _f32(y)
    xd, yd = _f32(x).astype(np.float64), yf.astype(np.float64)
    # no scaling: exactly one
    assert oracle.alpha_mode_f32(x, yf, 1) == 1.0
    # norm ratio: ||x|| / ||y|| to FP32 rounding of the sums
    nr = oracle.alpha_mode_f32(x, yf, 2)
    assert abs(nr - np.linalg.norm(xd) / np.linalg.norm(yd)) <= 1e-6 * nr
    # least squares is the default mode and minimises the residual energy
    ls = oracle.alpha_mode_f32(x, yf, 0)
    assert ls == oracle.alpha_f32(x, y)
    e = lambda a: float(((xd - a * yd) ** 2).sum())
    assert e(ls) <= e(nr) and e(ls) <= e(1.0)


def test_norm_ratio_ignores_sign_least_squares_does_not(oracle):
    """x = -2 y: least squares finds -2 exactly, the norm ratio +2."""
    rng = np.random.default_rng(9)
    y = _bf16(rng.standard_normal(64))
    x = _bf16(-2.0 * _f32(y))
    yf = _f32(y)
    assert oracle.alpha_mode_f32(x, yf, 0) == -2.0
    assert oracle.alpha_mode_f32(x, yf, 2) == 2.0
    # and a zero reference gives 0 for both
    z = np.zeros(64, dtype=np.float32)
    assert oracle.alpha_mode_f32(x, z, 0) == 0.0 and oracle.alpha_mode_f32(x, z, 2) == 0.0


@pytest.mark.parametrize("anchored", [False, True])
def test_first_loop_policy_is_a_relabelling(oracle, anchored):
    """Table 1 / Table 9: the First-loop policy references loop 1 instead of the
    last.  Encoding loops [r, a, b, c] with the first as reference gives, loop
    for loop, the planes of encoding [a, b, c, r] with the last as reference."""
    import synth
    rng = np.random.default_rng(5)
    L, B, H, d, g, n = 4, 1, 2, 64, 16, 10
    ref = _bf16(rng.standard_normal((B, H, n, d)))
    loops = _bf16(0.9 * _f32(ref)[None] + 0.1 * rng.standard_normal((L - 1, B, H, n, d)))
    extra = dict(ref_bits=4, ref_group=32) if anchored else {}
    base = dict(n_loops=L, batch=B, heads=H, d=d, g=g, cap=n, rotate=1, **extra)
    first = dict(base, bits=[0, 2, 4, 2], ref_first=1)
    last = dict(base, bits=[2, 4, 2, 0])
    pf = oracle.Planes(L, B, H, d, g, n, first["bits"], extra.get("ref_bits", 0), extra.get("ref_group"),
                       ref_first=1)
    pl = oracle.Planes(L, B, H, d, g, n, last["bits"], extra.get("ref_bits", 0), extra.get("ref_group"))
    if anchored:
        oracle.encode(first, pf, np.concatenate([ref[None], loops]), 0, n)
        oracle.encode(last, pl, np.concatenate([loops, ref[None]]), 0, n)
    else:
        pf.ref[:], pl.ref[:] = ref, ref
        oracle.encode(first, pf, loops, 0, n)
        oracle.encode(last, pl, loops, 0, n)
    perm = [3, 0, 1, 2]             # loop of `first` -> loop of `last`
    for lf, ll in enumerate(perm):
        for name in ("codes", "meta", "alpha"):
            a, b = getattr(pf, name)[lf], getattr(pl, name)[ll]
            assert (a is None) == (b is None)
            if a is not None:
                assert np.array_equal(a, b), (lf, name)
    q = _bf16(rng.standard_normal((L, B, H, d)))
    qp = q[[1, 2, 3, 0]]           # the same queries in `last`'s loop order
    for lf, ll in enumerate(perm):
        if anchored or lf != 0:
            assert np.array_equal(oracle.reconstruct(first, pf, lf, 0, n), oracle.reconstruct(last, pl, ll, 0, n))
        assert np.array_equal(oracle.decode_row(first, pf, pf, q, lf, 0, 1, n, 0.2),
                              oracle.decode_row(last, pl, pl, qp, ll, 0, 1, n, 0.2))
