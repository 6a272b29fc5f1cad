"""Pins of the oracle's NVFP4 backward (page "Thinking Machines Details
End-to-End 4-Bit Training for Inkling 2 Small", section "Developer quick
start": FP4 backward passes are the next step): the exact grouped GEMMs
against Fraction brute force and float64 matmul on the decoded integers, and
the transposed, segment-padded quantizer of the wgrad operands against what
the layout and the transform must satisfy (the 32-point transform of each
token chunk cancels in a product per segment; weights per expert equal the
batched quantization of the transposed matrices)."""
from fractions import Fraction

import numpy as np
import scipy.linalg

import oracle
from precision_moe_numerics_amd import synth


def _deq_int_frac(codes, scales):
    """Exact decoded values (before the tensor scale) as Fractions."""
    n = codes.shape[-1] * 2
    out = []
    for row_c, row_s in zip(codes.reshape(-1, codes.shape[-1]), scales.reshape(-1, scales.shape[-1])):
        vals = []
        for i in range(n):
            q = (int(row_c[i // 2]) >> (4 * (i & 1))) & 0xF
            vals.append(Fraction(oracle.e2m1_decode(q)) * Fraction(oracle.e4m3_decode(int(row_s[i // 16]))))
        out.append(vals)
    return out


def _deq_f64(codes, scales):
    """Decoded values before the tensor scale, exact in fp64."""
    return oracle.nvfp4_dequantize(codes, scales, 1.0).astype(np.float64)


def test_dgrad_fraction_brute_force():
    g = np.random.default_rng(601)
    E, N, K, rows = 2, 3, 32, 7
    a = oracle.nvfp4_quantize(synth.to_bf16_bits(g.standard_normal((rows, K))))
    b = oracle.nvfp4_quantize_batched(synth.to_bf16_bits(g.standard_normal((E, N, K)) * 0.3))
    offsets = np.array([0, 3, 7], np.int32)
    gather = np.array([6, 0, 2, 5, 1, 3, 4], np.int32)
    out = oracle.nvfp4_gemm_dgrad(a, b, offsets, a_gather=gather)
    A = _deq_int_frac(a[0], a[1])
    for r in range(rows):
        e = 0 if r < 3 else 1
        B = _deq_int_frac(b[0][e], b[1][e])
        for n in range(N):
            exact = sum(x * y for x, y in zip(A[gather[r]], B[n])) * Fraction(float(a[2])) * Fraction(float(b[2][e]))
            assert out[r, n] == float(exact), (r, n)


def test_dgrad_equals_matmul_of_decoded_integers():
    g = np.random.default_rng(602)
    E, N, K, R = 3, 40, 256, 50
    a = oracle.nvfp4_quantize(synth.to_bf16_bits(g.standard_t(3, (R, K))))
    b = oracle.nvfp4_quantize_batched(synth.to_bf16_bits(g.standard_normal((E, N, K)) * 0.02))
    offsets = np.array([0, 20, 20, R], np.int32)
    out = oracle.nvfp4_gemm_dgrad(a, b, offsets)
    A = _deq_f64(a[0], a[1])
    for e in range(E):
        r0, r1 = offsets[e], offsets[e + 1]
        ref = (A[r0:r1] @ _deq_f64(b[0][e], b[1][e]).T) * (np.float64(a[2]) * np.float64(b[2][e]))
        assert np.array_equal(out[r0:r1], ref)   # every partial sum is exact in fp64: one rounding each


def test_wgrad_fraction_brute_force_and_matmul():
    g = np.random.default_rng(603)
    M, N = 3, 2
    seg = np.array([0, 5, 5, 37], np.int32)          # ragged, one empty segment
    ya = synth.to_bf16_bits(g.standard_normal((37, M)))
    yb = synth.to_bf16_bits(g.standard_normal((37, N)))
    qa = oracle.nvfp4_quantize_axis1(ya, seg_offsets=seg)
    qb = oracle.nvfp4_quantize_axis1(yb, seg_offsets=seg)
    pad = oracle.pad_offsets(seg)
    out = oracle.nvfp4_gemm_wgrad(qa, qb, pad)
    A, B = _deq_int_frac(qa[0], qa[1]), _deq_int_frac(qb[0], qb[1])
    for e in range(3):
        for m in range(M):
            for n in range(N):
                exact = sum(A[m][k] * B[n][k] for k in range(pad[e], pad[e + 1]))
                exact *= Fraction(float(qa[2][0])) * Fraction(float(qb[2][0]))
                assert out[e, m, n] == float(exact)
    assert not out[1].any()
    # larger: float64 matmul of the decoded integers
    R, M, N = 300, 24, 40
    seg = np.array([0, 100, 101, 300], np.int32)
    qa = oracle.nvfp4_quantize_axis1(synth.to_bf16_bits(g.standard_normal((R, M))), seg_offsets=seg, rht_seed=5)
    qb = oracle.nvfp4_quantize_axis1(synth.to_bf16_bits(g.standard_normal((R, N))), seg_offsets=seg, rht_seed=5)
    pad = oracle.pad_offsets(seg)
    out = oracle.nvfp4_gemm_wgrad(qa, qb, pad)
    A, B = _deq_f64(qa[0], qa[1]), _deq_f64(qb[0], qb[1])
    for e in range(3):
        ref = A[:, pad[e]:pad[e + 1]] @ B[:, pad[e]:pad[e + 1]].T * (np.float64(qa[2][0]) * np.float64(qb[2][0]))
        assert np.array_equal(out[e], ref)


def test_token_axis_transform_cancels_per_segment():
    """Per segment, the transformed operands' products over the segment's padded
    columns equal the original products over its rows (the transform is
    orthogonal and every 32-column chunk holds rows of one segment only); a
    chunk that mixed two segments would break this at O(1)."""
    g = np.random.default_rng(604)
    R, Ca, Cb = 230, 5, 7
    seg = np.array([0, 31, 31, 96, 97, 230], np.int32)
    gather = g.permutation(R).astype(np.int32)
    xa = synth.to_bf16_bits(g.standard_normal((R, Ca)))
    xb = synth.to_bf16_bits(g.standard_normal((R, Cb)))
    signs = oracle.rht32_signs(9)
    s = np.array([-1.0 if (signs >> j) & 1 else 1.0 for j in range(32)])
    H = scipy.linalg.hadamard(32) / np.sqrt(32.0)
    pad = oracle.pad_offsets(seg)
    ld = oracle.nvfp4_axis1_ld(R, len(seg) - 1)

    def transformed(x):
        # fp64 transform of the padded transposed layout, built row by row
        xt = np.zeros((x.shape[1], ld))
        for si in range(len(seg) - 1):
            for j, r in enumerate(range(seg[si], seg[si + 1])):
                xt[:, pad[si] + j] = oracle.bf16_to_f32(x[gather[r]])
        chunks = xt.reshape(x.shape[1], ld // 32, 32)
        return (chunks * s) @ H.T

    za, zb = transformed(xa), transformed(xb)
    fa = oracle.bf16_to_f32(xa).astype(np.float64)[gather]
    fb = oracle.bf16_to_f32(xb).astype(np.float64)[gather]
    for si in range(len(seg) - 1):
        c0, c1 = pad[si] // 32, pad[si + 1] // 32
        got = np.einsum("aij,bij->ab", za[:, c0:c1], zb[:, c0:c1])
        ref = fa[seg[si]:seg[si + 1]].T @ fb[seg[si]:seg[si + 1]]
        assert np.allclose(got, ref, rtol=1e-12, atol=1e-12)
    # the oracle's fp32 transform of the same layout agrees with the fp64 one
    q = oracle.nvfp4_quantize_axis1(xa, row_gather=gather, seg_offsets=seg, rht_seed=9)
    xt = np.zeros((Ca, ld), np.uint16)
    for si in range(len(seg) - 1):
        xt[:, pad[si]:pad[si] + seg[si + 1] - seg[si]] = xa[gather[seg[si]:seg[si + 1]]].T
    z32 = oracle.rht32_forward(xt.ravel(), 9).reshape(Ca, ld).astype(np.float64)
    assert np.allclose(z32, za.reshape(Ca, ld), rtol=0, atol=1e-6 * np.abs(za).max())
    assert np.array_equal(q[0], oracle.nvfp4_quantize(z32.astype(np.float32))[0])


def test_quantized_wgrad_approximates_the_product():
    """The whole chain (transpose, transform, NVFP4 with one scale per operand,
    exact GEMM) approximates dY_e^T H_e; with the signs of one operand from
    another seed the transform no longer cancels."""
    g = np.random.default_rng(605)
    R, M, N = 512, 64, 48
    seg = np.array([0, 200, 512], np.int32)
    dy = synth.to_bf16_bits(g.standard_normal((R, M)) * 1e-3)
    h = synth.to_bf16_bits(g.standard_normal((R, N)))
    pad = oracle.pad_offsets(seg)
    qa = oracle.nvfp4_quantize_axis1(dy, mode=1, stream=3, seg_offsets=seg, rht_seed=0)
    qb = oracle.nvfp4_quantize_axis1(h, seg_offsets=seg, rht_seed=0)
    out = oracle.nvfp4_gemm_wgrad(qa, qb, pad)
    fa = oracle.bf16_to_f32(dy).astype(np.float64)
    fb = oracle.bf16_to_f32(h).astype(np.float64)
    for e in range(2):
        ref = fa[seg[e]:seg[e + 1]].T @ fb[seg[e]:seg[e + 1]]
        rel = np.linalg.norm(out[e] - ref) / np.linalg.norm(ref)
        assert rel < 0.3, rel          # NVFP4 noise on random data: about 0.15-0.2, independent of K
    qb_other = oracle.nvfp4_quantize_axis1(h, seg_offsets=seg, rht_seed=1)
    bad = oracle.nvfp4_gemm_wgrad(qa, qb_other, pad)
    ref = fa[:200].T @ fb[:200]
    assert np.linalg.norm(bad[0] - ref) / np.linalg.norm(ref) > 0.5


def test_per_expert_weight_scales_equal_batched_transposed_quantization():
    g = np.random.default_rng(606)
    E, R, C = 3, 64, 48                                  # W_e [R, C]; B_e = W_e^T, blocks along R
    w = synth.to_bf16_bits(g.standard_normal((E, R, C)) * 0.02 * np.array([1.0, 7.0, 0.1])[:, None, None])
    seg = (np.arange(E + 1) * R).astype(np.int32)
    codes, scales, D = oracle.nvfp4_quantize_axis1(w.reshape(E * R, C), seg_offsets=seg, ld=E * R, per_segment=True)
    bc, bs, bd = oracle.nvfp4_quantize_batched(np.ascontiguousarray(w.transpose(0, 2, 1)))
    for e in range(E):
        assert np.array_equal(codes[:, e * R // 2:(e + 1) * R // 2], bc[e])
        assert np.array_equal(scales[:, e * R // 16:(e + 1) * R // 16], bs[e])
    assert np.array_equal(D, bd)
