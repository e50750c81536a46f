"""Pins of the oracle's reconstruction and attention.

ResidualQuant page ("ResidualQuant: KV Cache Quantization for Looped
Transformers with 2-Bit Residuals"), Abstract: earlier loops are stored as
low-precision residuals against the final loop and reconstructed cheaply; the
decode step attends over every loop's cache.  The attention of the final loop
is plain softmax attention over the BF16 reference and is pinned against
torch's scaled_dot_product_attention in float64 on the CPU (a library
routine); the special cases below follow from the definition of softmax.
"""
import numpy as np
import pytest
import torch

import synth
from synth import bf16_bits


def _layout(w, cap=None):
    return dict(n_loops=w.n_loops, batch=w.batch, heads=w.heads, d=w.d, g=w.g,
                cap=cap or w.n_ctx, rotate=w.rotate, bits=list(w.bits))


def _encoded(oracle, w, n=None, seed=None, cap=None):
    n = n or w.n_ctx
    data = synth.draw_layer(w, seed=seed, n=n)
    lay = _layout(w, cap or n)
    kp = oracle.Planes(w.n_loops, w.batch, w.heads, w.d, w.g, lay["cap"], w.bits)
    vp = oracle.Planes(w.n_loops, w.batch, w.heads, w.d, w.g, lay["cap"], w.bits)
    kp.ref[:, :, :n] = bf16_bits(data["k_ref"])
    vp.ref[:, :, :n] = bf16_bits(data["v_ref"])
    oracle.encode(lay, kp, bf16_bits(data["k_loops"]), 0, n)
    oracle.encode(lay, vp, bf16_bits(data["v_loops"]), 0, n)
    return lay, kp, vp, data


def _small(rotate=1, bits=(2, 2, 2), d=128, g=32, n=96, B=2, H=2):
    return synth.Workload("t", n_loops=len(bits) + 1, batch=B, heads=H, d=d, g=g, n_ctx=n,
                          bits=list(bits), c=[0.8, 0.85, 0.9][:len(bits)],
                          sigma=[0.15, 0.12, 0.1][:len(bits)], rotate=rotate, seed=21)


@pytest.mark.parametrize("rotate", [0, 1])
@pytest.mark.parametrize("bits", [(2, 2, 2), (4, 2, 2)])
def test_reconstruction_error_is_the_quantization_error(oracle, rotate, bits):
    """x - x_hat = H_n (u - u_hat) up to FP32 rounding, and H_n is orthonormal,
    so ||x - x_hat||_2 is at most the grid error sqrt(sum_k g (s_k/2)^2)."""
    w = _small(rotate=rotate, bits=bits)
    lay, kp, vp, data = _encoded(oracle, w)
    for l in range(w.n_loops - 1):
        xh = oracle.reconstruct(lay, kp, l, 0, w.n_ctx)
        x = data["k_loops"][l].float().double().numpy()
        s = oracle.f16_bits_to_f32(kp.meta[l][..., 0].ravel()).reshape(kp.meta[l].shape[:-1])
        grid = np.sqrt((w.g * (s.astype(np.float64) / 2) ** 2).sum(-1))
        err = np.linalg.norm(x - xh, axis=-1)
        xnorm = np.linalg.norm(x, axis=-1)
        assert np.all(err <= grid * (1 + 1e-3) + 1e-5 * xnorm)
        # and the residual coding really helps: error far below the signal
        assert np.median(err / xnorm) < 0.2


def test_reconstruct_without_rotation_is_dequantize_plus_alpha_ref(oracle):
    w = _small(rotate=0)
    lay, kp, vp, data = _encoded(oracle, w, n=8)
    xh = oracle.reconstruct(lay, kp, 1, 0, 8)
    b, h, t = 1, 0, 5
    codes = oracle.unpack(kp.codes[1][b, h, t], w.d, 2)
    meta = oracle.f16_bits_to_f32(kp.meta[1][b, h, t].ravel()).astype(np.float64).reshape(-1, 2)
    a = float(oracle.f16_bits_to_f32(np.array([kp.alpha[1][b, h, t]], dtype=np.uint16))[0])
    y = data["k_ref"][b, h, t].double().numpy()
    want = a * y + meta[np.arange(w.d) // w.g, 1] + meta[np.arange(w.d) // w.g, 0] * codes
    assert np.allclose(xh[b, h, t], want, rtol=0, atol=1e-12)


def test_append_equals_prefill(oracle):
    """Encoding [0, n) at once gives the same bytes as n one-token encodes."""
    w = _small(n=40)
    data = synth.draw_layer(w, n=40)
    lay = _layout(w, 48)
    whole = oracle.Planes(w.n_loops, w.batch, w.heads, w.d, w.g, 48, w.bits)
    step = oracle.Planes(w.n_loops, w.batch, w.heads, w.d, w.g, 48, w.bits)
    for p in (whole, step):
        p.ref[:, :, :40] = bf16_bits(data["k_ref"])
    x = bf16_bits(data["k_loops"])
    oracle.encode(lay, whole, x, 0, 40)
    for t in range(40):
        oracle.encode(lay, step, np.ascontiguousarray(x[:, :, :, t:t + 1]), t, 1)
    for l in range(w.n_loops - 1):
        assert np.array_equal(whole.codes[l], step.codes[l])
        assert np.array_equal(whole.meta[l], step.meta[l])
        assert np.array_equal(whole.alpha[l], step.alpha[l])


def test_reference_loop_matches_torch_sdpa(oracle):
    w = _small(n=200)
    lay, kp, vp, data = _encoded(oracle, w)
    L = w.n_loops
    out = oracle.decode(lay, kp, vp, bf16_bits(data["q"]), 1 << (L - 1), w.n_ctx, 1 / np.sqrt(w.d))
    q = data["q"][L - 1].double()[:, :, None, :]              # [B, H, 1, d]
    k = data["k_ref"].double()
    v = data["v_ref"].double()
    want = torch.nn.functional.scaled_dot_product_attention(q, k, v)[:, :, 0].numpy()
    assert np.allclose(out[L - 1], want, rtol=1e-12, atol=1e-12)


def test_residual_loop_matches_sdpa_over_reconstruction(oracle):
    w = _small(n=64)
    lay, kp, vp, data = _encoded(oracle, w)
    out = oracle.decode(lay, kp, vp, bf16_bits(data["q"]), 0b0110, 50, 0.3)
    for l in (1, 2):
        kh = torch.from_numpy(oracle.reconstruct(lay, kp, l, 0, 50))
        vh = torch.from_numpy(oracle.reconstruct(lay, vp, l, 0, 50))
        q = data["q"][l].double()[:, :, None, :]
        want = torch.nn.functional.scaled_dot_product_attention(q, kh, vh, scale=0.3)[:, :, 0]
        assert np.allclose(out[l], want.numpy(), rtol=1e-12, atol=1e-12)
    assert np.isnan(out[0]).all() and np.isnan(out[3]).all()


def test_attention_special_cases(oracle):
    rng = np.random.default_rng(4)
    d, n = 64, 37
    k = rng.standard_normal((n, d))
    v = rng.standard_normal((n, d))
    q = rng.standard_normal(d)
    # one token: the output is that token's value
    assert np.allclose(oracle.attention(q, k[:1], v[:1], 0.125), v[0], atol=1e-15)
    # zero query: uniform weights, the output is the mean value
    assert np.allclose(oracle.attention(np.zeros(d), k, v, 0.125), v.mean(0), atol=1e-13)
    # identical values: the output is that value whatever the weights
    vv = np.tile(v[3], (n, 1))
    assert np.allclose(oracle.attention(q, k, vv, 0.125), v[3], atol=1e-13)
    # permuting tokens changes nothing
    perm = rng.permutation(n)
    assert np.allclose(oracle.attention(q, k[perm], v[perm], 0.125),
                       oracle.attention(q, k, v, 0.125), atol=1e-13)
    # a dominant key selects its value
    kk = k.copy()
    kk[11] = q * 50
    assert np.allclose(oracle.attention(q, kk, v, 1.0), v[11], atol=1e-10)


def test_rotation_folds_into_the_query():
    """The identity a decode kernel may use instead of un-rotating every key:
    q . (H_n u) = (H_n q) . u and sum_t p_t H_n u_t = H_n sum_t p_t u_t, because
    the Sylvester Hadamard matrix is symmetric (checked in FP64)."""
    import scipy.linalg
    rng = np.random.default_rng(1)
    d = 128
    Hn = scipy.linalg.hadamard(d) / np.sqrt(d)
    assert np.array_equal(Hn, Hn.T)
    q, u = rng.standard_normal(d), rng.standard_normal((50, d))
    assert np.allclose(u @ Hn @ q, (Hn @ u.T).T @ q, atol=1e-12)
    p = rng.random(50)
    assert np.allclose(p @ (u @ Hn.T), Hn @ (p @ u), atol=1e-12)
