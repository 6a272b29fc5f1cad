"""GPU parity of the NVFP4 backward (page "Thinking Machines Details End-to-End
4-Bit Training for Inkling 2 Small", section "Developer quick start": FP4
backward passes are the next step) against the oracle:

  * the transposed, segment-padded quantizer (with and without the token-axis
    RHT, nearest even and stochastic, gathered rows, empty and ragged
    segments, one scale or one per expert): codes, scale bytes and tensor
    scales bit-exact;
  * the grouped dgrad and wgrad GEMMs on identical operands: plain relative
    Frobenius error <= 2e-5 against the exact (int64) oracle;
  * the moe_layer fc2 and fc1 backward at full size on sampled rows and
    experts."""
import numpy as np
import pytest
import torch

import oracle
import precision_moe_numerics_amd as nvq
from precision_moe_numerics_amd import synth
from gpu_util import host, require_gpu, to_dev, to_dev_u16

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _gpu():
    require_gpu()


def _rel_frob(got, ref):
    ref = np.asarray(ref, np.float64)
    return float(np.linalg.norm(np.asarray(got, np.float64) - ref) / max(np.linalg.norm(ref), 1e-300))


def _eq(g, o, what):
    for part, gi, oi in zip(("codes", "scales", "tscale"), g, o):
        gh = host(gi)
        assert gh.shape == np.asarray(oi).shape, (what, part, gh.shape, np.asarray(oi).shape)
        bad = gh != oi
        assert not bad.any(), f"{what}: {part} differ at {np.argwhere(bad)[:5].tolist()}"


def _segs(R, nseg, g, empty=True):
    cuts = np.sort(g.choice(np.arange(1, R), size=nseg - 1, replace=False)) if nseg > 1 else np.array([], int)
    seg = np.concatenate([[0], cuts, [R]]).astype(np.int32)
    if empty and nseg > 2:
        seg[2] = seg[1]                                  # one empty segment
    return seg


@pytest.mark.parametrize("case", [
    dict(R=300, C=96, nseg=3, gather=False, rht=True, mode=0),
    dict(R=300, C=96, nseg=4, gather=True, rht=True, mode=1),
    dict(R=1000, C=200, nseg=7, gather=False, rht=False, mode=1),
    dict(R=77, C=64, nseg=1, gather=False, rht=True, mode=0),
    dict(R=513, C=128, nseg=9, gather=True, rht=False, mode=0),
    dict(R=64, C=130, nseg=1, gather=False, rht=False, mode=1),
])
def test_axis1_quantizer_exact(case):
    g = np.random.default_rng(700 + case["R"] + case["C"])
    R, C, nseg = case["R"], case["C"], case["nseg"]
    src = synth.to_bf16_bits(g.standard_t(3, (R // 2 + 3 if case["gather"] else R, C)) * 0.3)
    gather = g.integers(0, src.shape[0] * 2, R).astype(np.int32) if case["gather"] else None
    gdiv = 2 if case["gather"] else 1
    seg = _segs(R, nseg, g) if nseg > 1 else None
    rs = 11 if case["rht"] else None
    o = oracle.nvfp4_quantize_axis1(src, mode=case["mode"], seed=3, stream=4, row_gather=gather, gather_div=gdiv,
                                    seg_offsets=seg, rht_seed=rs)
    q = nvq.nvfp4_quantize_axis1(to_dev_u16(src), round_mode=case["mode"], seed=3, stream_id=4,
                                 row_gather=None if gather is None else to_dev(gather), gather_div=gdiv,
                                 seg_offsets=None if seg is None else to_dev(seg), R=R,
                                 rht=case["rht"], sign_seed=11)
    _eq(q, o, str(case))


# segmentations the chunk-row table must resolve like a search over the padded
# starts: empty segments first, in runs and last; exactly 32 rows (a chunk
# boundary on a segment boundary); one-row segments
EDGE_SEGS = [[0, 0, 0, 5, 5, 37, 37, 69, 70, 70, 70],
             [0, 32, 64, 65, 97, 97],
             [0, 1, 2, 3, 35, 100, 100]]


@pytest.mark.parametrize("seg", EDGE_SEGS)
@pytest.mark.parametrize("rht,mode", [(True, 1), (False, 0)])
def test_axis1_quantizer_edge_segments(seg, rht, mode):
    seg = np.asarray(seg, dtype=np.int32)
    R, C = int(seg[-1]), 64
    g = np.random.default_rng(710 + R + len(seg))
    src = synth.to_bf16_bits(g.standard_t(3, (R, C)) * 0.3)
    rs = 11 if rht else None
    o = oracle.nvfp4_quantize_axis1(src, mode=mode, seed=3, stream=4, seg_offsets=seg, rht_seed=rs)
    q = nvq.nvfp4_quantize_axis1(to_dev_u16(src), round_mode=mode, seed=3, stream_id=4, seg_offsets=to_dev(seg),
                                 R=R, rht=rht, sign_seed=11)
    _eq(q, o, f"seg={seg.tolist()} rht={rht} mode={mode}")


def test_axis1_quantizer_per_expert_weights_and_zero():
    g = np.random.default_rng(710)
    E, Re, C = 5, 64, 160
    w = synth.to_bf16_bits(g.standard_normal((E * Re, C)) * 0.02)
    w[Re:2 * Re] = 0                                    # an all-zero expert: scale 1, zero bytes
    seg = (np.arange(E + 1) * Re).astype(np.int32)
    o = oracle.nvfp4_quantize_axis1(w, seg_offsets=seg, ld=E * Re, per_segment=True)
    q = nvq.nvfp4_quantize_axis1(to_dev_u16(w), nseg=E, per_segment=True)
    _eq(q, o, "per-expert weights")
    z = np.zeros((40, 64), np.uint16)
    o = oracle.nvfp4_quantize_axis1(z, rht_seed=0)
    q = nvq.nvfp4_quantize_axis1(to_dev_u16(z), rht=True, sign_seed=0)
    _eq(q, o, "zero tensor")


@pytest.mark.parametrize("R,E,N,K,gather", [(300, 3, 128, 256, False), (700, 5, 256, 128, True),
                                            (64, 2, 128, 1024, True), (1000, 4, 384, 512, False)])
def test_dgrad(R, E, N, K, gather):
    """out[r] = deq(A[arow]) . deq(B_e)^T, A rows quantized as nvfp4_quantize
    writes them (stochastic, as the gradients are), B the per-expert transposed
    weights."""
    g = np.random.default_rng(720 + R)
    seg = _segs(R, E, g)
    a_src = synth.to_bf16_bits(g.standard_normal((R + 5, K)) * 1e-3)
    w = synth.to_bf16_bits(g.standard_normal((E * K, N)) * 0.02)     # E stacked [K, N] weights
    a_o = oracle.nvfp4_quantize(a_src, mode=1, stream=1)
    a_g = nvq.nvfp4_quantize(to_dev_u16(a_src), round_mode=nvq.SR, stream_id=1)
    assert np.array_equal(host(a_g[0]), a_o[0]) and np.array_equal(host(a_g[1]), a_o[1])
    b_o = oracle.nvfp4_quantize_axis1(w, seg_offsets=(np.arange(E + 1) * K).astype(np.int32), ld=E * K,
                                      per_segment=True)
    b_g = nvq.nvfp4_quantize_axis1(to_dev_u16(w), nseg=E, per_segment=True)
    _eq(b_g, b_o, "transposed weights")
    gat = g.permutation(R + 5)[:R].astype(np.int32) if gather else None
    out = nvq.moe_grouped_gemm_nvfp4_bwd(nvq.DGRAD, a_g, b_g, to_dev(seg), M=R, N=N, K=K,
                                         a_gather=None if gat is None else to_dev(gat))
    b3 = (np.stack([b_o[0][:, e * K // 2:(e + 1) * K // 2] for e in range(E)]),
          np.stack([b_o[1][:, e * K // 16:(e + 1) * K // 16] for e in range(E)]), b_o[2])
    ref = oracle.nvfp4_gemm_dgrad((a_o[0], a_o[1], a_o[2]), b3, seg, a_gather=gat)
    err = _rel_frob(host(out)[:seg[-1]], ref)
    print(f"dgrad R={R} E={E} N={N} K={K}: rel Frobenius {err:.2e}")
    assert err <= 2e-5


@pytest.mark.parametrize("R,E,M,N,gather", [(300, 3, 128, 128, False), (777, 6, 256, 128, True),
                                            (1500, 7, 384, 256, False), (40, 3, 128, 256, True)])
def test_wgrad(R, E, M, N, gather):
    """out[e] = deq(A)[:, seg e] . deq(B)[:, seg e]^T with both operands the
    token-axis RHT + NVFP4 of the segment rows (A stochastic, B nearest even)."""
    g = np.random.default_rng(730 + R)
    seg = _segs(R, E, g)
    dy = synth.to_bf16_bits(g.standard_normal((R, M)) * 1e-3)
    h_src = synth.to_bf16_bits(g.standard_normal((R // 2 + 1 if gather else R, N)))
    gat = g.integers(0, h_src.shape[0] * 2, R).astype(np.int32) if gather else None
    a_o = oracle.nvfp4_quantize_axis1(dy, mode=1, stream=3, seg_offsets=seg, rht_seed=0)
    b_o = oracle.nvfp4_quantize_axis1(h_src, row_gather=gat, gather_div=2, seg_offsets=seg, rht_seed=0)
    a_g = nvq.nvfp4_quantize_axis1(to_dev_u16(dy), round_mode=nvq.SR, stream_id=3, seg_offsets=to_dev(seg),
                                   rht=True, sign_seed=0)
    b_g = nvq.nvfp4_quantize_axis1(to_dev_u16(h_src), row_gather=None if gat is None else to_dev(gat), gather_div=2,
                                   seg_offsets=to_dev(seg), R=R, rht=True, sign_seed=0)
    _eq(a_g, a_o, "dY^T")
    _eq(b_g, b_o, "H^T")
    out = nvq.moe_grouped_gemm_nvfp4_bwd(nvq.WGRAD, a_g, b_g, to_dev(seg), M=M, N=N, K=R)
    ref = oracle.nvfp4_gemm_wgrad(a_o, b_o, oracle.pad_offsets(seg))
    err = _rel_frob(host(out), ref)
    print(f"wgrad R={R} E={E} M={M} N={N}: rel Frobenius {err:.2e}")
    assert err <= 2e-5
    empty = np.flatnonzero(np.diff(seg) == 0)
    assert not host(out)[empty].any()


def test_rejects_bad_arguments():
    L = nvq.lib()
    import ctypes as C
    buf = torch.zeros(1 << 20, dtype=torch.uint8, device="cuda")
    p = C.c_void_p(buf.data_ptr())
    ws = C.c_void_p(buf.data_ptr())
    # dgrad: K not a multiple of 128; N not a multiple of 128; bad mode
    assert L.moe_grouped_gemm_nvfp4_bwd(0, p, p, p, None, p, p, p, p, 96, 192, 2, 64, 128, 96, p, ws, 4096, None) == -2
    assert L.moe_grouped_gemm_nvfp4_bwd(0, p, p, p, None, p, p, p, p, 128, 256, 2, 64, 100, 128, p, ws, 4096,
                                        None) == -2
    assert L.moe_grouped_gemm_nvfp4_bwd(5, p, p, p, None, p, p, p, p, 128, 256, 2, 64, 128, 128, p, ws, 4096,
                                        None) == -5
    # wgrad: ld too short for the segments' padding
    assert L.moe_grouped_gemm_nvfp4_bwd(1, p, p, p, None, p, p, p, p, 128, 128, 4, 128, 128, 300, p, ws, 4096,
                                        None) == -2
    # quantizer: per-expert scales with a transform; NULL input
    assert L.nvfp4_quantize_axis1(p, 64, 64, None, 1, None, 2, 64, 1, 0, 1, 0, 0, 1, p, p, p, ws, 1 << 16,
                                  None) == -5
    assert L.nvfp4_quantize_axis1(None, 64, 64, None, 1, None, 1, 256, 0, 0, 0, 0, 0, 1, p, p, p, ws, 1 << 16,
                                  None) == -1


def test_moe_layer_fc2_backward_full_size():
    """The fc2 backward at the full moe_layer size (A = 131072 assignments of
    16384 tokens, top-8 of 384 experts, d = 4096, d_ff = 1024), launched as the
    benchmark launches it. dgrad dH = dY_e . W2_e on sampled rows of four
    experts (the largest, the smallest, a median one and the last non-empty
    one, >= 256): dY's stochastic codes under the tensor scale of all of dY,
    W2's transposed bytes per expert, and dH within 2e-5 of the exact product.
    wgrad dW2_e = dY_e^T H_e for three small experts: the token-axis RHT of the
    whole transposed dY (and H) is computed by the oracle for the tensor
    scales, the experts' columns are compared byte for byte (stochastic for
    dY), and dW2_e is within 2e-5 of the exact product."""
    dev = torch.device("cuda")
    T, d, E, k, d_ff = 16384, 4096, 384, 8, 1024
    A = T * k
    ids, _ = synth.moe_layer_routing()
    offs, s2a, _ = nvq.moe_route(to_dev(ids), E)
    o_offs, o_s2a = oracle.route(ids, E)
    dy = synth.device_normal_bf16((A, d), 1e-3, 1, dev, workload_id=4)
    w2 = synth.device_normal_bf16((E, d, d_ff), 0.02, 3, dev)
    hin = synth.device_normal_bf16((A, d_ff), 1.0, 4, dev, workload_id=4)   # H-shaped rows in expert order
    dy0 = nvq.nvfp4_quantize(dy, round_mode=nvq.SR, stream_id=1)
    w2t = nvq.nvfp4_quantize_axis1(w2.view(E * d, d_ff), nseg=E, per_segment=True)
    dH = nvq.moe_grouped_gemm_nvfp4_bwd(nvq.DGRAD, dy0, w2t, offs, M=A, N=d_ff, K=d, a_gather=s2a)
    dyT = nvq.nvfp4_quantize_axis1(dy, round_mode=nvq.SR, stream_id=3, row_gather=s2a, seg_offsets=offs, rht=True)
    hT = nvq.nvfp4_quantize_axis1(hin, seg_offsets=offs, rht=True)
    dW2 = nvq.moe_grouped_gemm_nvfp4_bwd(nvq.WGRAD, dyT, hT, offs, M=d, N=d_ff, K=A)
    torch.cuda.synchronize()
    print("full-size NVFP4 fc2 backward done on the GPU", flush=True)
    bits = lambda t: t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
    n_e = np.diff(o_offs)
    nz = np.flatnonzero(n_e)
    order = nz[np.argsort(n_e[nz], kind="stable")]

    # ---- dgrad
    dyb = bits(dy)
    dyf = oracle.bf16_to_f32(dyb)
    amax = oracle.amax_f32(dyf)
    experts = list(dict.fromkeys([int(order[-1]), int(order[0]), int(order[len(order) // 2]), int(nz[-1])]))
    assert max(experts) >= 256
    rng = np.random.default_rng(14)
    rows, counts = [], []
    for e in experts:
        seg = np.arange(o_offs[e], o_offs[e + 1])
        pick = np.unique(np.concatenate([seg[:3], seg[-3:], rng.choice(seg, size=min(len(seg), 8), replace=False)]))
        rows.append(pick)
        counts.append(len(pick))
    rows = np.concatenate(rows)
    sub_offs = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    gc, gs, gD = host(dy0[0]), host(dy0[1]), host(dy0[2])[0]
    a_c, a_s = [], []
    for r in rows:
        a = int(o_s2a[r])
        oc, os_, oD = oracle.nvfp4_quantize_slice(dyf[a], amax, a * d, mode=1, seed=0, stream=1)
        assert np.array_equal(gc[a], oc) and np.array_equal(gs[a], os_), f"dY row {a}"
        assert gD == oD
        a_c.append(oc)
        a_s.append(os_)
    del dyf
    b_c, b_s, b_D = [], [], []
    wc, wsc, wD = host(w2t[0]), host(w2t[1]), host(w2t[2])
    for e in experts:
        oc, os_, oD = oracle.nvfp4_quantize(np.ascontiguousarray(bits(w2[e]).T))   # W2_e^T [d_ff, d]
        assert np.array_equal(wc[:, e * d // 2:(e + 1) * d // 2], oc) and wD[e] == oD, f"W2^T of expert {e}"
        assert np.array_equal(wsc[:, e * d // 16:(e + 1) * d // 16], os_)
        b_c.append(oc)
        b_s.append(os_)
        b_D.append(oD)
    ref = oracle.nvfp4_gemm_dgrad((np.stack(a_c), np.stack(a_s), gD), (np.stack(b_c), np.stack(b_s), np.array(b_D)),
                                  sub_offs)
    err = _rel_frob(host(dH[torch.from_numpy(rows.astype(np.int64)).to(dev)]), ref)
    print(f"dgrad fc2: {len(rows)} rows of experts {experts} ({n_e[experts].tolist()} rows), rel Frobenius "
          f"{err:.2e}", flush=True)
    assert err <= 2e-5

    # ---- wgrad: the transposed, padded tensors through the RHT, for the tensor scales
    ld = nvq.nvfp4_axis1_ld(A, E)
    pad = oracle.pad_offsets(o_offs)
    e_of_row = np.repeat(np.arange(E), n_e)
    col_of_row = pad[e_of_row] + (np.arange(A) - o_offs[e_of_row])
    used = int(pad[-1])

    def transformed(src_rows, C):
        xt = np.zeros((C, used), np.uint16)
        xt[:, col_of_row] = src_rows.T
        return oracle.rht32_forward(xt.ravel(), 0).reshape(C, used)

    zy = transformed(dyb[o_s2a], d)
    del dyb
    amax_y = oracle.amax_f32(zy)
    zh = transformed(bits(hin), d_ff)
    amax_h = oracle.amax_f32(zh)
    print("oracle transforms of the whole transposed dY and H done", flush=True)
    yc, ys, yD = host(dyT[0]), host(dyT[1]), host(dyT[2])[0]
    hc, hs, hD = host(hT[0]), host(hT[1]), host(hT[2])[0]
    hi = [int(e) for e in order if e >= 256]
    for e in list(dict.fromkeys([int(order[0]), hi[0], int(order[len(order) // 2])])):
        w = int(pad[e + 1] - pad[e])
        blocks = []
        for (z, am, gc_, gs_, gD_, mode, stream) in ((zy, amax_y, yc, ys, yD, 1, 3), (zh, amax_h, hc, hs, hD, 0, 1)):
            oc = np.empty((z.shape[0], w // 2), np.uint8)
            os_ = np.empty((z.shape[0], w // 16), np.uint8)
            for c in range(z.shape[0]):
                oc[c], os_[c], oD = oracle.nvfp4_quantize_slice(z[c, pad[e]:pad[e] + w], am, c * ld + int(pad[e]),
                                                                mode=mode, seed=0, stream=stream)
            assert gD_ == oD, f"tensor scale, expert {e}"
            assert np.array_equal(gc_[:, pad[e] // 2:(pad[e] + w) // 2], oc), f"codes of expert {e}"
            assert np.array_equal(gs_[:, pad[e] // 16:(pad[e] + w) // 16], os_), f"scales of expert {e}"
            blocks.append((oc, os_, oD))
        ref = oracle.nvfp4_gemm_wgrad(blocks[0], blocks[1], np.array([0, w], np.int32))[0]
        err = _rel_frob(host(dW2[e]), ref)
        print(f"wgrad fc2 expert {e} ({n_e[e]} rows): operands exact, rel Frobenius {err:.2e}", flush=True)
        assert err <= 2e-5


def test_moe_layer_fc1_backward_full_size():
    """The fc1 backward at the full moe_layer size, launched as the benchmark
    launches it (dA in expert order, X gathered from token rows). dgrad
    dX = dA_e . W1_e on sampled rows of four experts (the largest, the
    smallest, a median one and the last non-empty one, >= 256): dA's
    stochastic codes under the tensor scale of all of dA, the bytes of W1's
    transposed operand (4096 x 384*2048 values, code offsets past 2^31) for
    those experts, and dX within 2e-5 of the exact product. wgrad
    dW1_e = dA_e^T X_e for three experts (the smallest, the smallest >= 256,
    a median one): the token-axis RHT of the whole transposed dA and gathered
    X is computed by the oracle for the tensor scales, the experts' columns
    are compared byte for byte (stochastic for dA), and dW1_e is within 2e-5
    of the exact product. dA is a synthetic N(0, 1e-3) input."""
    dev = torch.device("cuda")
    T, d, E, k, d_ff = 16384, 4096, 384, 8, 1024
    A, F2 = T * k, 2 * d_ff
    ids, _ = synth.moe_layer_routing()
    offs, s2a, _ = nvq.moe_route(to_dev(ids), E)
    o_offs, o_s2a = oracle.route(ids, E)
    x = synth.device_normal_bf16((T, d), 1.0, 1, dev)
    w1 = synth.device_normal_bf16((E, F2, d), 0.02, 2, dev)
    dA = synth.device_normal_bf16((A, F2), 1e-3, 5, dev, workload_id=4)
    da0 = nvq.nvfp4_quantize(dA, round_mode=nvq.SR, stream_id=1)
    w1t = nvq.nvfp4_quantize_axis1(w1.view(E * F2, d), nseg=E, per_segment=True)
    dX = nvq.moe_grouped_gemm_nvfp4_bwd(nvq.DGRAD, da0, w1t, offs, M=A, N=d, K=F2)
    daT = nvq.nvfp4_quantize_axis1(dA, round_mode=nvq.SR, stream_id=3, seg_offsets=offs, rht=True)
    xT = nvq.nvfp4_quantize_axis1(x, row_gather=s2a, gather_div=k, seg_offsets=offs, rht=True)
    dW1 = nvq.moe_grouped_gemm_nvfp4_bwd(nvq.WGRAD, daT, xT, offs, M=F2, N=d, K=A)
    torch.cuda.synchronize()
    print("full-size NVFP4 fc1 backward done on the GPU", flush=True)
    bits = lambda t: t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
    n_e = np.diff(o_offs)
    nz = np.flatnonzero(n_e)
    order = nz[np.argsort(n_e[nz], kind="stable")]

    # ---- dgrad: dA rows are the sorted rows themselves (no gather)
    dab = bits(dA)
    daf = oracle.bf16_to_f32(dab)
    amax = oracle.amax_f32(daf)
    experts = list(dict.fromkeys([int(order[-1]), int(order[0]), int(order[len(order) // 2]), int(nz[-1])]))
    assert max(experts) >= 256
    rng = np.random.default_rng(15)
    rows, counts = [], []
    for e in experts:
        seg = np.arange(o_offs[e], o_offs[e + 1])
        pick = np.unique(np.concatenate([seg[:3], seg[-3:], rng.choice(seg, size=min(len(seg), 8), replace=False)]))
        rows.append(pick)
        counts.append(len(pick))
    rows = np.concatenate(rows)
    sub_offs = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    rows_d = torch.from_numpy(rows.astype(np.int64)).to(dev)
    gc, gs, gD = host(da0[0][rows_d]), host(da0[1][rows_d]), host(da0[2])[0]
    a_c, a_s = [], []
    for i, r in enumerate(rows):
        oc, os_, oD = oracle.nvfp4_quantize_slice(daf[r], amax, int(r) * F2, mode=1, seed=0, stream=1)
        assert np.array_equal(gc[i], oc) and np.array_equal(gs[i], os_), f"dA row {r}"
        assert gD == oD
        a_c.append(oc)
        a_s.append(os_)
    del daf
    b_c, b_s, b_D = [], [], []
    wD = host(w1t[2])
    for e in experts:
        oc, os_, oD = oracle.nvfp4_quantize(np.ascontiguousarray(bits(w1[e]).T))   # W1_e^T [d, 2 d_ff]
        gcw = host(w1t[0][:, e * F2 // 2:(e + 1) * F2 // 2])
        gsw = host(w1t[1][:, e * F2 // 16:(e + 1) * F2 // 16])
        assert np.array_equal(gcw, oc) and wD[e] == oD, f"W1^T of expert {e}"
        assert np.array_equal(gsw, os_), f"W1^T scales of expert {e}"
        b_c.append(oc)
        b_s.append(os_)
        b_D.append(oD)
    ref = oracle.nvfp4_gemm_dgrad((np.stack(a_c), np.stack(a_s), gD), (np.stack(b_c), np.stack(b_s), np.array(b_D)),
                                  sub_offs)
    err = _rel_frob(host(dX[rows_d]), ref)
    print(f"dgrad fc1: {len(rows)} rows of experts {experts} ({n_e[experts].tolist()} rows), rel Frobenius "
          f"{err:.2e}", flush=True)
    assert err <= 2e-5

    # ---- wgrad: the transposed, padded tensors through the RHT, for the tensor scales
    ld = nvq.nvfp4_axis1_ld(A, E)
    pad = oracle.pad_offsets(o_offs)
    e_of_row = np.repeat(np.arange(E), n_e)
    col_of_row = pad[e_of_row] + (np.arange(A) - o_offs[e_of_row])
    used = int(pad[-1])

    def transformed(src_rows, C):
        xt = np.zeros((C, used), np.uint16)
        xt[:, col_of_row] = src_rows.T
        return oracle.rht32_forward(xt.ravel(), 0).reshape(C, used)

    za = transformed(dab, F2)
    del dab
    amax_a = oracle.amax_f32(za)
    zx = transformed(bits(x)[o_s2a // k], d)
    amax_x = oracle.amax_f32(zx)
    print("oracle transforms of the whole transposed dA and gathered X done", flush=True)
    yD, xD = host(daT[2])[0], host(xT[2])[0]
    hi = [int(e) for e in order if e >= 256]
    for e in list(dict.fromkeys([int(order[0]), hi[0], int(order[len(order) // 2])])):
        w = int(pad[e + 1] - pad[e])
        blocks = []
        for (z, am, q, gD_, mode, stream) in ((za, amax_a, daT, yD, 1, 3), (zx, amax_x, xT, xD, 0, 1)):
            oc = np.empty((z.shape[0], w // 2), np.uint8)
            os_ = np.empty((z.shape[0], w // 16), np.uint8)
            for c in range(z.shape[0]):
                oc[c], os_[c], oD = oracle.nvfp4_quantize_slice(z[c, pad[e]:pad[e] + w], am, c * ld + int(pad[e]),
                                                                mode=mode, seed=0, stream=stream)
            assert gD_ == oD, f"tensor scale, expert {e}"
            assert np.array_equal(host(q[0][:, pad[e] // 2:(pad[e] + w) // 2]), oc), f"codes of expert {e}"
            assert np.array_equal(host(q[1][:, pad[e] // 16:(pad[e] + w) // 16]), os_), f"scales of expert {e}"
            blocks.append((oc, os_, oD))
        ref = oracle.nvfp4_gemm_wgrad(blocks[0], blocks[1], np.array([0, w], np.int32))[0]
        err = _rel_frob(host(dW1[e]), ref)
        print(f"wgrad fc1 expert {e} ({n_e[e]} rows): operands exact, rel Frobenius {err:.2e}", flush=True)
        assert err <= 2e-5
