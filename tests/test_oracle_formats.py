"""Pins of the oracle's number-format conversions against numpy / torch.

The bit-exact encoder stores scales, offsets and LS coefficients as FP16
(ResidualQuant page, Table 8 caption: b_eff counts scales, offsets and LS
coefficients), so the oracle's own FP16 rounding is checked against numpy's
IEEE binary16 conversion (a library routine) on random and edge-case values.
"""
import numpy as np
import torch


def _edge_values():
    two = np.float32(2.0)
    vals = [0.0, -0.0, 1.0, -1.0, 65504.0, -65504.0, 65519.996, 65520.0, 65536.0, 1e10,
            2.0 ** -14, 2.0 ** -24, 2.0 ** -25, 3 * 2.0 ** -26, 2.0 ** -26, 1.5 * 2.0 ** -24,
            2.5 * 2.0 ** -24, 1e-10, np.inf, -np.inf,
            1.0 + 2.0 ** -11, 1.0 + 3 * 2.0 ** -11, 1.0 + 2.0 ** -11 + 2.0 ** -20,
            2048.0 + 1.0, 2048.0 + 3.0, 0.1, 1.0 / 3.0, 6.1e-5, 6.0e-5]
    out = [np.float32(v) for v in vals]
    # ties between every pair of neighbouring halves in a few binades
    for e in (-20, -14, -3, 0, 7, 15):
        base = two ** e
        for m in (0, 1, 2, 511, 1022):
            lo = np.float32(base * (1 + m / 1024))
            out.append(np.float32(base * (1 + (m + 0.5) / 1024)))
            out.append(np.nextafter(out[-1], np.float32(np.inf)))
            out.append(np.nextafter(out[-2], np.float32(-np.inf)))
            out.append(lo)
    return np.array(out, dtype=np.float32)


def test_f32_to_f16_matches_numpy_random(oracle):
    rng = np.random.default_rng(11)
    # wide magnitude spread: random bit patterns restricted to finite floats
    bits = rng.integers(0, 2 ** 32, size=200_000, dtype=np.uint64).astype(np.uint32)
    x = bits.view(np.float32)
    x = x[np.isfinite(x)]
    # plus values concentrated around the FP16 range
    y = (rng.standard_normal(200_000) * np.exp(rng.uniform(-20, 12, 200_000))).astype(np.float32)
    for arr in (x, y):
        got = oracle.f32_to_f16_bits(arr)
        want = arr.astype(np.float16).view(np.uint16)
        assert np.array_equal(got, want)


def test_f32_to_f16_matches_numpy_edges(oracle):
    x = _edge_values()
    got = oracle.f32_to_f16_bits(x)
    want = x.astype(np.float16).view(np.uint16)
    assert np.array_equal(got, want), list(zip(x[got != want], got[got != want], want[got != want]))


def test_f16_to_f32_all_patterns(oracle):
    h = np.arange(65536, dtype=np.uint16)
    got = oracle.f16_bits_to_f32(h)
    want = h.view(np.float16).astype(np.float32)
    nan = np.isnan(want)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan].view(np.uint32), want[~nan].view(np.uint32))


def test_bf16_to_f32_matches_torch(oracle):
    h = np.arange(0, 65536, 7, dtype=np.uint16)
    got = oracle.bf16_bits_to_f32(h)
    want = torch.from_numpy(h.view(np.int16).copy()).view(torch.bfloat16).float().numpy()
    nan = np.isnan(want)
    assert np.array_equal(got[~nan].view(np.uint32), want[~nan].view(np.uint32))


def test_saturating_store(oracle):
    lib = oracle.lib()
    assert lib.rqo_f32_to_f16_sat(1e6) == 0x7bff
    assert lib.rqo_f32_to_f16_sat(-1e6) == 0xfbff
    assert lib.rqo_f32_to_f16_sat(65519.0) == 0x7bff
    assert lib.rqo_f32_to_f16_sat(1.0) == 0x3c00
    assert lib.rqo_f32_to_f16_sat(float("inf")) == 0x7bff
