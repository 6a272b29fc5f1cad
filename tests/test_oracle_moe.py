"""Pins for the oracle's routing, exact NVFP4 expert GEMMs, SwiGLU and the
exact MXFP8 GEMMs: stable sort by a library sort, Fraction-exact tiny GEMMs,
the E=1, k=1 case against torch.matmul in float64, and SwiGLU forward and
backward against torch's silu and autograd in float64."""
from fractions import Fraction

import numpy as np
import torch

import oracle
from precision_moe_numerics_amd import synth

E4M3 = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).double().numpy()
E2M1 = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0, -0.0, -0.5, -1.0, -1.5, -2.0, -3.0, -4.0, -6.0])


def deq_nvfp4_exact(codes, scales):
    """codes * scales as float64 (exact), D not applied."""
    c = codes.reshape(codes.shape[:-1] + (-1,))
    q = np.empty(c.shape[:-1] + (c.shape[-1] * 2,), np.uint8)
    q[..., 0::2] = c & 0xF
    q[..., 1::2] = c >> 4
    return E2M1[q] * np.repeat(E4M3[scales], 16, axis=-1)


def test_route_stable_vs_sorted():
    g = np.random.default_rng(1)
    T, k, E = 300, 4, 9
    ids = np.stack([g.permutation(E)[:k] for _ in range(T)]).astype(np.int32)
    ids[5] = [1, 2, 3, 4]
    offsets, s2a = oracle.route(ids, E)
    flat = ids.reshape(-1)
    want = sorted(range(flat.size), key=lambda a: (flat[a], a))
    assert list(s2a) == want
    assert list(np.diff(offsets)) == [int((flat == e).sum()) for e in range(E)]


def test_route_drops_out_of_range_ids():
    ids = np.array([[0, 5], [7, 1], [-1, 1]], np.int32)
    offsets, s2a = oracle.route(ids, 6)
    assert offsets[-1] == 4 and list(s2a[:4]) == [0, 3, 5, 1]


def _tiny_case(T=6, d=32, E=2, k=2, d_ff=16, seed=3):
    c = synth.moe_shapes(T, d, E, k, d_ff, seed=seed, wid=95)
    xq = oracle.nvfp4_quantize(c["x"])
    w1q = oracle.nvfp4_quantize_batched(c["w1"])
    w2q = oracle.nvfp4_quantize_batched(c["w2"])
    offsets, s2a = oracle.route(c["topk_ids"], E)
    return c, xq, w1q, w2q, offsets, s2a


def test_fc1_fraction_exact():
    c, xq, w1q, w2q, offsets, s2a = _tiny_case()
    G = oracle.moe_fc1(xq, offsets, s2a, c["k"], w1q)
    X = deq_nvfp4_exact(xq[0], xq[1])
    W = deq_nvfp4_exact(w1q[0], w1q[1])
    E = c["E"]
    for r in range(offsets[E]):
        e = int(np.searchsorted(offsets, r, side="right") - 1)
        t = s2a[r] // c["k"]
        for n in range(0, W.shape[1], 3):
            exact = sum(Fraction(float(a)) * Fraction(float(b)) for a, b in zip(X[t], W[e, n]))
            exact *= Fraction(float(xq[2])) * Fraction(float(w1q[2][e]))
            assert G[r, n] == float(exact)  # the exact value rounded once to fp64


def test_single_expert_reduces_to_matmul():
    T, d, d_ff = 24, 64, 32
    c = synth.moe_shapes(T, d, 1, 1, d_ff, seed=4, wid=95)
    xq = oracle.nvfp4_quantize(c["x"])
    w1q = oracle.nvfp4_quantize_batched(c["w1"])
    w2q = oracle.nvfp4_quantize_batched(c["w2"])
    out = oracle.moe_forward(c["x"], c["topk_ids"], w1q, w2q)
    X = torch.from_numpy(deq_nvfp4_exact(xq[0], xq[1]) * float(xq[2]))
    W1 = torch.from_numpy(deq_nvfp4_exact(w1q[0][0], w1q[1][0]) * float(w1q[2][0]))
    G = X @ W1.T
    assert np.allclose(out["G"], G.numpy(), rtol=1e-12, atol=0)
    h = torch.nn.functional.silu(G[:, :d_ff]) * G[:, d_ff:]
    assert np.allclose(out["H"], h.numpy(), rtol=1e-12, atol=1e-300)
    Hd = torch.from_numpy(deq_nvfp4_exact(out["hq"][0], out["hq"][1]) * float(out["hq"][2]))
    W2 = torch.from_numpy(deq_nvfp4_exact(w2q[0][0], w2q[1][0]) * float(w2q[2][0]))
    assert np.allclose(out["y"][:, 0, :], (Hd @ W2.T).numpy(), rtol=1e-12, atol=1e-300)


def test_identity_weights_reproduce_input():
    """W1 with identity gate and a constant up row: G's gate half is deq(Xq)."""
    d = 32
    x = synth.normal_bf16((4, d), 1.0, 95, 7)
    xq = oracle.nvfp4_quantize(x)
    w = np.zeros((1, 2 * d, d))
    w[0, :d, :] = np.eye(d)
    w[0, d:, :] = np.eye(d)
    w1q = oracle.nvfp4_quantize_batched(synth.to_bf16_bits(w))
    offsets, s2a = oracle.route(np.zeros((4, 1), np.int32), 1)
    G = oracle.moe_fc1(xq, offsets, s2a, 1, w1q)
    # the identity quantizes to code 6 with scale 448 and D_w = fl(1/2688)
    assert np.array_equal(w1q[1][0], np.full((2 * d, d // 16), 0x7E, np.uint8) * (np.arange(d // 16)[None, :] == (np.arange(2 * d)[:, None] % d) // 16))
    X = deq_nvfp4_exact(xq[0], xq[1]) * float(xq[2])
    assert np.allclose(G[:, :d], X * (2688.0 * float(w1q[2][0])), rtol=1e-15, atol=0)
    assert np.allclose(G[:, d:], G[:, :d], rtol=0, atol=0)


def test_fc2_rows_subset_matches_full():
    c, xq, w1q, w2q, offsets, s2a = _tiny_case(T=20, E=3, k=2)
    full = oracle.moe_forward(c["x"], c["topk_ids"], w1q, w2q)
    rows = np.array([0, 7, int(offsets[3]) - 1], np.int32)
    Ys = oracle.moe_fc2(full["hq"], offsets, w2q, rows=rows)
    assert np.array_equal(Ys, full["Y_sorted"][rows])
    G = oracle.moe_fc1(xq, offsets, s2a, c["k"], w1q, rows=rows)
    assert np.array_equal(G, full["G"][rows])


def test_swiglu_bwd_vs_autograd():
    g = np.random.default_rng(8)
    n, d_ff = 16, 24
    gu = synth.to_bf16_bits(g.standard_normal((n, 2 * d_ff)) * 3)
    dH = (g.standard_normal((n, d_ff))).astype(np.float32)
    dA = oracle.swiglu_bwd(dH, gu)
    t = torch.from_numpy(oracle.bf16_to_f32(gu).astype(np.float64)).requires_grad_(True)
    h = torch.nn.functional.silu(t[:, :d_ff]) * t[:, d_ff:]
    h.backward(torch.from_numpy(dH.astype(np.float64)))
    assert np.allclose(dA, t.grad.numpy(), rtol=1e-13, atol=1e-300)


def _e4m3_int(b):
    return Fraction(float(E4M3[b]))


def test_mxfp8_dgrad_fraction_exact_and_matmul():
    g = np.random.default_rng(9)
    R, K, N, E = 10, 64, 5, 2
    offsets = np.array([0, 4, 10], np.int32)
    a = oracle.mxfp8_quantize(synth.to_bf16_bits(g.standard_normal((R, K))), axis=0)
    b_src = synth.to_bf16_bits(g.standard_normal((E * N, K)) * 0.02)
    be, bs = oracle.mxfp8_quantize(b_src, axis=0)
    b = (be.reshape(E, N, K), bs.reshape(E, N, K // 32))
    out = oracle.mxfp8_gemm_dgrad(a, b, offsets)
    for r in (0, 3, 4, 9):
        e = 0 if r < 4 else 1
        for n in range(N):
            tot = Fraction(0)
            for k in range(K):
                sa = Fraction(2) ** (int(a[1][r, k // 32]) - 127)
                sb = Fraction(2) ** (int(b[1][e, n, k // 32]) - 127)
                tot += _e4m3_int(a[0][r, k]) * sa * _e4m3_int(b[0][e, n, k]) * sb
            assert abs(out[r, n] - float(tot)) <= abs(float(tot)) * 2 ** -50 + 1e-300
    A = torch.from_numpy(E4M3[a[0]] * np.repeat(2.0 ** (a[1] - 127.0), 32, axis=1))
    B = torch.from_numpy(E4M3[b[0]] * np.repeat(2.0 ** (b[1] - 127.0), 32, axis=2))
    ref = torch.cat([A[0:4] @ B[0].T, A[4:10] @ B[1].T]).numpy()
    assert np.allclose(out, ref, rtol=1e-12)


def test_mxfp8_wgrad_vs_matmul():
    g = np.random.default_rng(10)
    R, M, N = 70, 8, 6
    seg = np.array([0, 30, 30, 70], np.int32)
    dy = synth.to_bf16_bits(g.standard_normal((R, M)))
    h = synth.to_bf16_bits(g.standard_normal((R, N)))
    a = oracle.mxfp8_quantize(dy, axis=1, seg_offsets=seg)
    b = oracle.mxfp8_quantize(h, axis=1, seg_offsets=seg)
    po = oracle.pad_offsets(seg)
    out = oracle.mxfp8_gemm_wgrad(a, b, po)
    A = E4M3[a[0]] * np.repeat(2.0 ** (a[1] - 127.0), 32, axis=1)
    B = E4M3[b[0]] * np.repeat(2.0 ** (b[1] - 127.0), 32, axis=1)
    for e in range(3):
        ref = A[:, po[e]:po[e + 1]] @ B[:, po[e]:po[e + 1]].T
        assert np.allclose(out[e], ref, rtol=1e-12, atol=1e-300)
    assert not out[1].any()
