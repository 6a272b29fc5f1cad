"""Pins for the oracle's 32-point random Hadamard transform and the combine:
H32 H32^T = 32 I (library Sylvester matrix), the fp32 butterfly against an
explicit product, one-hot columns, Parseval, the round trip, and the combine
against an independent fp64 matrix form."""
import numpy as np
import scipy.linalg

import oracle
from precision_moe_numerics_amd import synth

H32 = scipy.linalg.hadamard(32).astype(np.int64)


def signs(seed):
    w = oracle.rht32_signs(seed)
    return np.array([-1 if (w >> j) & 1 else 1 for j in range(32)], np.int64)


def test_hadamard_orthogonal():
    assert np.array_equal(H32 @ H32.T, 32 * np.eye(32, dtype=np.int64))
    Hn = H32 / np.sqrt(32.0)
    assert np.abs(Hn @ Hn.T - np.eye(32)).max() < 1e-15
    i, j = np.meshgrid(np.arange(32), np.arange(32), indexing="ij")
    pc = np.vectorize(lambda v: bin(v).count("1"))(i & j)
    assert np.array_equal(H32, np.where(pc % 2, -1, 1))


def test_sign_word_from_philox():
    w = oracle.philox4x32_10([0, 0, 4, 0], [7, 0])[0]
    assert oracle.rht32_signs(7) == w


def test_butterfly_matches_matrix_on_integers():
    """Small integers keep every fp32 add exact, so the butterfly equals the
    integer product H32 (s .* x) exactly before the final scaling."""
    g = np.random.default_rng(2)
    xi = g.integers(-64, 64, (50, 32))
    x = synth.to_bf16_bits(xi.astype(np.float64))
    for seed in (0, 1, 12345):
        z = oracle.rht32_forward(x, seed)
        s = signs(seed)
        want = (xi * s) @ H32.T
        c32 = np.float32(1.0 / np.sqrt(32.0))
        assert np.array_equal(z, (want.astype(np.float32) * c32).astype(np.float32))


def test_one_hot_columns():
    s = signs(3)
    x = np.zeros((32, 32))
    x[np.arange(32), np.arange(32)] = 1.0
    z = oracle.rht32_forward(synth.to_bf16_bits(x), 3)
    c32 = np.float32(1.0 / np.sqrt(32.0))
    for j in range(32):
        assert np.array_equal(z[j], (s[j] * H32[:, j]).astype(np.float32) * c32)


def test_parseval_and_round_trip():
    x = synth.normal_bf16((64, 128), 1.0, 94, 0)
    xf = oracle.bf16_to_f32(x).astype(np.float64).reshape(-1, 32)
    z = oracle.rht32_forward(x, 5).astype(np.float64).reshape(-1, 32)
    assert np.allclose((z ** 2).sum(axis=1), (xf ** 2).sum(axis=1), rtol=1e-5)
    s = signs(5)
    back = s * (z @ H32) / np.sqrt(32.0)  # H32 symmetric: inverse is H32/sqrt32 then signs
    assert np.abs(back - xf).max() <= 1e-5 * np.abs(xf).max()


def test_combine_against_matrix_form():
    T, k, C = 6, 8, 64
    y = synth.normal_bf16((T * k, C), 1.0, 94, 1)
    w = np.random.default_rng(4).dirichlet(np.ones(k), size=T).astype(np.float32)
    z = oracle.rht32_forward(y, 11)
    codes, scales, D = oracle.nvfp4_quantize(z)
    zd = oracle.nvfp4_dequantize(codes, scales, D).astype(np.float64)  # fp32 rounding of q*s*D
    out = oracle.rht32_combine(codes, scales, D, T, k, 11, w)
    s = signs(11)
    inv = (zd.reshape(-1, 32) @ H32.T / np.sqrt(32.0)) * s
    inv = inv.reshape(T, k, C)
    ref = np.einsum("tk,tkc->tc", w.astype(np.float64), inv)
    assert np.allclose(out, ref, rtol=1e-6, atol=1e-6 * np.abs(ref).max())
    # without the quantizer the combine is the weighted sum of the inputs
    yf = oracle.bf16_to_f32(y).astype(np.float64).reshape(T, k, C)
    approx = np.einsum("tk,tkc->tc", w.astype(np.float64), yf)
    rel = np.linalg.norm(out - approx) / np.linalg.norm(approx)
    assert rel < 0.15  # 4-bit quantization error, not a structural mismatch
    zz = oracle.rht32_forward(y, 12)  # a different sign vector is not interchangeable
    c2, s2, D2 = oracle.nvfp4_quantize(zz)
    bad = oracle.rht32_combine(c2, s2, D2, T, k, 11, w)
    assert np.linalg.norm(bad - approx) / np.linalg.norm(approx) > 0.5
