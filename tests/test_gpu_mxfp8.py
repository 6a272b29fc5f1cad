"""GPU parity of the MXFP8 backward: requantization on both axes (elements and
E8M0 bytes exact, nearest-even and Philox stochastic rounding, row gathers,
per-segment restarts and padding), the E8M0-scaled FP8 grouped GEMMs (relative
Frobenius error <= 2e-5 against the oracle's exact-block fp64 result on
identical operands) and the SwiGLU backward (1 bf16 ulp)."""
import numpy as np
import pytest
import torch

import oracle
import precision_moe_numerics_amd as nvq
from precision_moe_numerics_amd import synth
from gpu_util import check_bf16_close, host, require_gpu, to_dev, to_dev_u16

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _gpu():
    require_gpu()


def _seg(R, nseg, seed, empty=True):
    g = synth.rng(60, seed)
    cuts = np.sort(g.integers(0, R + 1, nseg - 1))
    seg = np.concatenate([[0], cuts, [R]]).astype(np.int32)
    return seg


@pytest.mark.parametrize("R,C", [(1, 32), (5, 96), (300, 4096), (1031, 160)])
@pytest.mark.parametrize("mode", [0, 1])
def test_axis0(R, C, mode):
    x = synth.normal_bf16((R, C), 1e-3, 61, R)
    x[0, :32] = 0
    ge, gs = nvq.mxfp8_requant_sr(to_dev_u16(x), 0, round_mode=mode, seed=7, stream_id=2)
    oe, os_ = oracle.mxfp8_quantize(x, 0, mode=mode, seed=7, stream=2)
    assert np.array_equal(host(gs), os_)
    assert np.array_equal(host(ge), oe), np.argwhere(host(ge) != oe)[:5]


def test_axis0_gather():
    x = synth.normal_bf16((50, 64), 1.0, 62, 0)
    gather = synth.rng(62, 1).integers(0, 50 * 3, 77).astype(np.int32)
    ge, gs = nvq.mxfp8_requant_sr(to_dev_u16(x), 0, round_mode=1, seed=2, row_gather=to_dev(gather), gather_div=3)
    oe, os_ = oracle.mxfp8_quantize(x, 0, mode=1, seed=2, stream=2, row_gather=gather, gather_div=3)
    assert np.array_equal(host(ge), oe) and np.array_equal(host(gs), os_)


@pytest.mark.parametrize("R,C,nseg", [(1, 2, 1), (70, 64, 3), (500, 256, 9), (1200, 130, 40), (333, 200, 5),
                                      (1200, 136, 40)])
@pytest.mark.parametrize("mode", [0, 1])
def test_axis1_segments(R, C, nseg, mode):
    """Nearest even with C % 8 == 0 takes the tiled kernel (128 rows x 128 columns
    per workgroup; C = 200 and 136 end in a partial column tile), other cases the
    per-column kernel."""
    x = synth.normal_bf16((R, C), 1e-3, 63, R)
    seg = _seg(R, nseg, R)
    ge, gs = nvq.mxfp8_requant_sr(to_dev_u16(x), 1, round_mode=mode, seed=11, stream_id=3,
                                  seg_offsets=to_dev(seg) if nseg > 1 else None)
    oe, os_ = oracle.mxfp8_quantize(x, 1, mode=mode, seed=11, stream=3, seg_offsets=seg if nseg > 1 else None,
                                    ld=ge.shape[1])
    assert np.array_equal(host(gs), os_)
    assert np.array_equal(host(ge), oe), np.argwhere(host(ge) != oe)[:5]


@pytest.mark.parametrize("seg", [[0, 0, 0, 5, 5, 37, 37, 69, 70, 70, 70], [0, 32, 64, 65, 97, 97],
                                 [0, 1, 2, 3, 35, 100, 100]])
@pytest.mark.parametrize("mode,C", [(1, 136), (0, 136), (1, 34)])
def test_axis1_edge_segments(seg, mode, C):
    """Segmentations the block-row table must resolve like a search over the
    padded starts: empty segments first, in runs and last; exactly 32 rows;
    one-row segments (C = 136: the tiled kernel for SR, the per-column one for
    nearest even without 128-multiple strides; C = 34: the per-column SR path)."""
    seg = np.asarray(seg, dtype=np.int32)
    R = int(seg[-1])
    x = synth.normal_bf16((R, C), 1e-3, 69, R + C)
    ge, gs = nvq.mxfp8_requant_sr(to_dev_u16(x), 1, round_mode=mode, seed=13, stream_id=3, seg_offsets=to_dev(seg))
    oe, os_ = oracle.mxfp8_quantize(x, 1, mode=mode, seed=13, stream=3, seg_offsets=seg, ld=ge.shape[1])
    assert np.array_equal(host(gs), os_)
    assert np.array_equal(host(ge), oe), np.argwhere(host(ge) != oe)[:5]


def test_axis1_gather_segments():
    x = synth.normal_bf16((40, 96), 1.0, 64, 0)
    gather = synth.rng(64, 1).integers(0, 40 * 8, 150).astype(np.int32)
    seg = np.array([0, 0, 33, 34, 100, 150], np.int32)
    ge, gs = nvq.mxfp8_requant_sr(to_dev_u16(x), 1, round_mode=1, seed=3, row_gather=to_dev(gather), gather_div=8,
                                  seg_offsets=to_dev(seg))
    oe, os_ = oracle.mxfp8_quantize(x, 1, mode=1, seed=3, stream=3, row_gather=gather, gather_div=8,
                                    seg_offsets=seg, ld=ge.shape[1])
    assert np.array_equal(host(ge), oe) and np.array_equal(host(gs), os_)


@pytest.mark.parametrize("mode", [0, 1])
def test_negative_zero_blocks(mode):
    """A 32-value block holding only -0 has scale byte 0 and zero bytes on both
    axes; a -0 inside a non-zero block keeps its sign bit."""
    x = synth.normal_bf16((96, 64), 1.0, 65, mode)
    x[0:32, 3] = 0x8000      # an all -0 column block (axis 1)
    x[40, 0:32] = 0x8000     # an all -0 row block (axis 0)
    x[70, 5] = 0x8000        # a lone -0 among normal values
    for axis in (0, 1):
        ge, gs = nvq.mxfp8_requant_sr(to_dev_u16(x), axis, round_mode=mode, seed=5, stream_id=2)
        oe, os_ = oracle.mxfp8_quantize(x, axis, mode=mode, seed=5, stream=2, ld=ge.shape[1] if axis else None)
        assert np.array_equal(host(gs), os_), axis
        assert np.array_equal(host(ge), oe), (axis, np.argwhere(host(ge) != oe)[:5])


def _rel_frob(got, ref):
    ref = np.asarray(ref, np.float64)
    return np.linalg.norm(got.astype(np.float64) - ref) / max(np.linalg.norm(ref), 1e-300)


def _ld128(R, nseg):
    return (oracle.mxfp8_ld(R, nseg) + 127) // 128 * 128


@pytest.mark.parametrize("R,E,N,K,aligned", [(300, 3, 128, 256, False), (700, 5, 256, 96, False),
                                             (64, 2, 128, 4096, False), (300, 3, 128, 256, True),
                                             (900, 4, 256, 384, True), (600, 3, 128, 512, True),
                                             (1100, 5, 256, 1024, True)])
def test_dgrad(R, E, N, K, aligned):
    """out[r] = A[r] . B_e^T with A row-quantized and B the axis-1 quantized stack
    (aligned: 128-multiple row strides, the whole-cache-line path; with K a
    multiple of 512 also the path that loads scale words four steps at a time,
    here with B scale rows that are not 16-byte aligned)."""
    seg = _seg(R, E, K)
    a_src = synth.normal_bf16((R, K), 1e-3, 65, 0)
    w = synth.normal_bf16((E * K, N), 0.02, 65, 1)           # E stacked [K, N] weights
    a = oracle.mxfp8_quantize(a_src, 0)
    wseg = (np.arange(E + 1) * K).astype(np.int32)
    be, bs = oracle.mxfp8_quantize(w, 1, seg_offsets=wseg,   # [N, ld], expert e at columns e*K
                                   ld=_ld128(E * K, E) if aligned else None)
    out = nvq.moe_grouped_gemm_mxfp8(nvq.DGRAD, (to_dev(a[0]), to_dev(a[1])), (to_dev(be), to_dev(bs)),
                                     to_dev(seg), N=N, K=K)
    b3 = (np.stack([be[:, e * K:(e + 1) * K] for e in range(E)]),
          np.stack([bs[:, e * K // 32:(e + 1) * K // 32] for e in range(E)]))
    ref = oracle.mxfp8_gemm_dgrad(a, b3, seg)
    err = _rel_frob(host(out)[:seg[-1]], ref)
    print(f"dgrad R={R} E={E} N={N} K={K}: rel Frobenius {err:.2e}")
    assert err <= 2e-5


@pytest.mark.parametrize("R,E,M,N,aligned", [(300, 3, 128, 128, False), (777, 6, 256, 128, False),
                                             (300, 3, 128, 128, True), (1500, 7, 384, 256, True)])
def test_wgrad(R, E, M, N, aligned):
    """aligned: 128-multiple row strides, where K steps start on whole cache
    lines below each segment and the head is masked."""
    seg = _seg(R, E, M + N)
    dy = synth.normal_bf16((R, M), 1e-3, 66, 0)
    h = synth.normal_bf16((R, N), 1.0, 66, 1)
    ld = _ld128(R, E) if aligned else None
    a = oracle.mxfp8_quantize(dy, 1, mode=1, seg_offsets=seg, stream=3, ld=ld)
    b = oracle.mxfp8_quantize(h, 1, seg_offsets=seg, stream=3, ld=ld)
    out = nvq.moe_grouped_gemm_mxfp8(nvq.WGRAD, (to_dev(a[0]), to_dev(a[1])), (to_dev(b[0]), to_dev(b[1])),
                                     to_dev(seg), M=M, N=N)
    ref = oracle.mxfp8_gemm_wgrad(a, b, oracle.pad_offsets(seg))
    err = _rel_frob(host(out), ref)
    print(f"wgrad R={R} E={E} M={M} N={N}: rel Frobenius {err:.2e}")
    assert err <= 2e-5
    empty = np.flatnonzero(np.diff(seg) == 0)
    assert not host(out)[empty].any()


@pytest.mark.parametrize("n,d_ff", [(333, 192), (77, 100)])  # eight columns per lane / one per thread
def test_swiglu_bwd(n, d_ff):
    g = synth.rng(67, 0)
    gu = synth.to_bf16_bits(g.standard_normal((n, 2 * d_ff)) * 3)
    dH = (g.standard_normal((n, d_ff)) * 1e-3).astype(np.float32)
    out = nvq.swiglu_bwd(to_dev(dH), to_dev_u16(gu))
    ref = oracle.swiglu_bwd(dH, gu)
    nf, mx = check_bf16_close(host(out), ref, "swiglu_bwd")
    print(f"swiglu_bwd: {nf} on the floor, max {mx:.3f} ulp")


def test_dy_full_size_sr_sampled():
    """dY [131072, 4096] N(0, 1e-3) of the backward workload as the benchmark
    quantizes it: stochastic rounding with the rows gathered into expert order,
    axis 0 (stream 2) on sampled rows and axis 1 (stream 3, per-expert
    segments) on sampled experts. The oracle encodes each sample on its own at
    its logical row offset, so its draws are the full tensor's."""
    dev = torch.device("cuda")
    T, d, E, k = 16384, 4096, 384, 8
    A = T * k
    ids, _ = synth.moe_layer_routing()
    offs, s2a, _ = nvq.moe_route(to_dev(ids), E)
    o_offs, o_s2a = oracle.route(ids, E)
    dy = synth.device_normal_bf16((A, d), 1e-3, 1, dev, workload_id=4)
    ge, gs = nvq.mxfp8_requant_sr(dy, 0, round_mode=1, seed=0, stream_id=2, row_gather=s2a)
    he, hs = nvq.mxfp8_requant_sr(dy, 1, round_mode=1, seed=0, stream_id=3, row_gather=s2a, seg_offsets=offs)
    torch.cuda.synchronize()
    bits = lambda t: t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
    rows = np.sort(synth.rng(4, 5).choice(A, size=48, replace=False))
    for r in rows:
        src = bits(dy[int(o_s2a[r])]).reshape(1, d)
        oe, os_ = oracle.mxfp8_quantize(src, 0, mode=1, stream=2, row0=int(r))
        assert np.array_equal(host(ge[int(r)]), oe[0]) and np.array_equal(host(gs[int(r)]), os_[0]), f"row {r}"
    n_e = np.diff(o_offs)
    nz = np.flatnonzero(n_e)
    order = nz[np.argsort(n_e[nz], kind="stable")]
    pad = oracle.pad_offsets(o_offs)
    for e in (int(order[0]), int(order[len(order) // 2]), int(nz[-1])):
        r0, r1 = int(o_offs[e]), int(o_offs[e + 1])
        src = bits(dy[torch.from_numpy(o_s2a[r0:r1].astype(np.int64)).to(dev)])
        oe, os_ = oracle.mxfp8_quantize(src, 1, mode=1, stream=3, row0=r0)
        w = int(pad[e + 1] - pad[e])
        assert np.array_equal(host(he[:, pad[e]:pad[e] + w]), oe[:, :w]), f"expert {e} elements"
        assert np.array_equal(host(hs[:, pad[e] // 32:(pad[e] + w) // 32]), os_[:, :w // 32]), f"expert {e} scales"
        print(f"axis-1 SR of expert {e} ({r1 - r0} rows) exact", flush=True)


def test_moe_layer_fc1_backward_full_size_sampled():
    """The fc1 backward GEMMs at the full moe_layer size, launched as the
    benchmark launches them: dgrad dX = dA . W1_e on sampled rows of four
    experts (the largest, the smallest, a median one and the last non-empty
    one, >= 256), with the bytes of W1's transposed operand checked for those
    experts; wgrad dW1_e = dA_e^T X_e in full for the smallest expert, the
    non-empty expert >= 256 with the fewest rows, and a median one. Nearest-even
    operands, so the oracle can quantize the samples alone; dA is a synthetic
    N(0, 1e-3) input in expert order."""
    dev = torch.device("cuda")
    T, d, E, k, d_ff = 16384, 4096, 384, 8, 1024
    A = T * k
    ids, _ = synth.moe_layer_routing()
    offs, s2a, _ = nvq.moe_route(to_dev(ids), E)
    o_offs, o_s2a = oracle.route(ids, E)
    x = synth.device_normal_bf16((T, d), 1.0, 1, dev)
    w1 = synth.device_normal_bf16((E, 2 * d_ff, d), 0.02, 2, dev)
    dA = synth.device_normal_bf16((A, 2 * d_ff), 1e-3, 5, dev, workload_id=4)
    e_w1 = torch.arange(E + 1, dtype=torch.int32, device=dev) * (2 * d_ff)
    w1t = nvq.mxfp8_requant_sr(w1.view(E * 2 * d_ff, d), 1, round_mode=0, seg_offsets=e_w1)
    da0 = nvq.mxfp8_requant_sr(dA, 0, round_mode=0)
    dX = nvq.moe_grouped_gemm_mxfp8(nvq.DGRAD, da0, w1t, offs, N=d, K=2 * d_ff)
    da1 = nvq.mxfp8_requant_sr(dA, 1, round_mode=0, seg_offsets=offs)
    x1 = nvq.mxfp8_requant_sr(x, 1, round_mode=0, row_gather=s2a, gather_div=k, seg_offsets=offs)
    dW1 = nvq.moe_grouped_gemm_mxfp8(nvq.WGRAD, da1, x1, offs, M=2 * d_ff, N=d)
    torch.cuda.synchronize()
    print("full-size fc1 dgrad and wgrad done on the GPU", flush=True)
    bits = lambda t: t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
    n_e = np.diff(o_offs)
    nz = np.flatnonzero(n_e)
    order = nz[np.argsort(n_e[nz], kind="stable")]
    pad = oracle.pad_offsets(o_offs)

    experts = list(dict.fromkeys([int(order[-1]), int(order[0]), int(order[len(order) // 2]), int(nz[-1])]))
    assert experts[-1] >= 256
    rng = np.random.default_rng(13)
    rows, counts, b_e, b_s = [], [], [], []
    for e in experts:
        seg = np.arange(o_offs[e], o_offs[e + 1])
        pick = np.unique(np.concatenate([seg[:3], seg[-3:], rng.choice(seg, size=min(len(seg), 8), replace=False)]))
        rows.append(pick)
        counts.append(len(pick))
        be, bs = oracle.mxfp8_quantize(bits(w1[e]), 1)                 # [d, >= 2 d_ff], one segment
        assert np.array_equal(host(w1t[0][:, e * 2 * d_ff:(e + 1) * 2 * d_ff]), be[:, :2 * d_ff]), f"W1t {e}"
        assert np.array_equal(host(w1t[1][:, e * 2 * d_ff // 32:(e + 1) * 2 * d_ff // 32]),
                              bs[:, :2 * d_ff // 32]), f"W1t scales {e}"
        b_e.append(be[:, :2 * d_ff])
        b_s.append(bs[:, :2 * d_ff // 32])
    rows = np.concatenate(rows)
    sub_offs = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    rows_t = torch.from_numpy(rows.astype(np.int64)).to(dev)
    a = oracle.mxfp8_quantize(bits(dA[rows_t]), 0)
    assert np.array_equal(host(da0[0][rows_t]), a[0]) and np.array_equal(host(da0[1][rows_t]), a[1])
    ref = oracle.mxfp8_gemm_dgrad(a, (np.stack(b_e), np.stack(b_s)), sub_offs)
    err = _rel_frob(host(dX[rows_t]), ref)
    print(f"dgrad fc1: {len(rows)} rows of experts {experts} ({n_e[experts].tolist()} rows), rel Frobenius "
          f"{err:.2e}", flush=True)
    assert err <= 2e-5

    hi = [int(e) for e in order if e >= 256]
    for e in list(dict.fromkeys([int(order[0]), hi[0], int(order[len(order) // 2])])):
        seg = np.arange(o_offs[e], o_offs[e + 1])
        so = np.array([0, len(seg)], np.int32)
        ya = oracle.mxfp8_quantize(bits(dA[int(o_offs[e]):int(o_offs[e + 1])]), 1, seg_offsets=so)
        xb = oracle.mxfp8_quantize(bits(x[torch.from_numpy(o_s2a[seg] // k).to(dev)]), 1, seg_offsets=so)
        w = int(pad[e + 1] - pad[e])
        for g, o in ((da1, ya), (x1, xb)):
            assert np.array_equal(host(g[0][:, pad[e]:pad[e] + w]), o[0][:, :w])
            assert np.array_equal(host(g[1][:, pad[e] // 32:(pad[e] + w) // 32]), o[1][:, :w // 32])
        ref = oracle.mxfp8_gemm_wgrad(ya, xb, oracle.pad_offsets(so))[0]
        err = _rel_frob(host(dW1[e]), ref)
        print(f"wgrad fc1 expert {e} ({len(seg)} rows): rel Frobenius {err:.2e}", flush=True)
        assert err <= 2e-5


def test_moe_layer_gemms_full_size_sampled():
    """The fc2 backward GEMMs at the full moe_layer size (A = 131072 assignments
    of 16384 tokens, top-8 of 384 experts, d = 4096, d_ff = 1024), launched as
    the benchmark launches them: dgrad dH = dY_e . W2_e on sampled rows of three
    experts, wgrad dW2_e = dY_e^T H_e in full for the smallest, the median and
    the 75th-percentile expert. Operands are quantized with nearest-even so the
    oracle can quantize the sampled rows (axis-0 blocks are per row) and the
    sampled experts (axis-1 blocks restart at each segment) on their own; every
    GPU operand byte used is compared."""
    dev = torch.device("cuda")
    T, d, E, k, d_ff = 16384, 4096, 384, 8, 1024
    A = T * k
    ids, _ = synth.moe_layer_routing()
    offs, s2a, _ = nvq.moe_route(to_dev(ids), E)
    o_offs, o_s2a = oracle.route(ids, E)
    dy = synth.device_normal_bf16((A, d), 1e-3, 1, dev, workload_id=4)
    w2 = synth.device_normal_bf16((E, d, d_ff), 0.02, 3, dev)
    hin = synth.device_normal_bf16((A, d_ff), 1.0, 4, dev, workload_id=4)
    e_w2 = torch.arange(E + 1, dtype=torch.int32, device=dev) * d
    dy0 = nvq.mxfp8_requant_sr(dy, 0, round_mode=0, row_gather=s2a)
    w2t = nvq.mxfp8_requant_sr(w2.view(E * d, d_ff), 1, round_mode=0, seg_offsets=e_w2)
    dH = nvq.moe_grouped_gemm_mxfp8(nvq.DGRAD, dy0, w2t, offs, N=d_ff, K=d)
    dy1 = nvq.mxfp8_requant_sr(dy, 1, round_mode=0, row_gather=s2a, seg_offsets=offs)
    h1 = nvq.mxfp8_requant_sr(hin, 1, round_mode=0, seg_offsets=offs)
    dW2 = nvq.moe_grouped_gemm_mxfp8(nvq.WGRAD, dy1, h1, offs, M=d, N=d_ff)
    torch.cuda.synchronize()
    print("full-size dgrad and wgrad done on the GPU", flush=True)

    n_e = np.diff(o_offs)
    nz = np.flatnonzero(n_e)
    order = nz[np.argsort(n_e[nz], kind="stable")]
    pad = oracle.pad_offsets(o_offs)
    bits = lambda t: t.view(torch.int16).cpu().numpy().view(np.uint16)

    # dgrad: sampled rows of the largest, the smallest and a middle expert
    rng = np.random.default_rng(12)
    experts = [int(order[-1]), int(order[0]), int(order[len(order) // 2])]
    rows, counts = [], []
    for e in experts:
        seg = np.arange(o_offs[e], o_offs[e + 1])
        pick = np.unique(np.concatenate([seg[:3], seg[-3:], rng.choice(seg, size=min(len(seg), 8), replace=False)]))
        rows.append(pick)
        counts.append(len(pick))
    rows = np.concatenate(rows)
    sub_offs = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    x_rows = bits(dy[torch.from_numpy(o_s2a[rows].astype(np.int64)).to(dev)])
    a = oracle.mxfp8_quantize(x_rows, 0)
    rows_t = torch.from_numpy(rows.astype(np.int64)).to(dev)
    assert np.array_equal(host(dy0[0][rows_t]), a[0]) and np.array_equal(host(dy0[1][rows_t]), a[1])
    b_e, b_s = [], []
    for e in experts:
        be, bs = oracle.mxfp8_quantize(bits(w2[e]), 1)             # [d_ff, >= d], one segment of d rows
        assert np.array_equal(host(w2t[0][:, e * d:(e + 1) * d]), be[:, :d])
        assert np.array_equal(host(w2t[1][:, e * d // 32:(e + 1) * d // 32]), bs[:, :d // 32])
        b_e.append(be[:, :d]); b_s.append(bs[:, :d // 32])
    ref = oracle.mxfp8_gemm_dgrad(a, (np.stack(b_e), np.stack(b_s)), sub_offs)
    err = _rel_frob(host(dH[rows_t]), ref)
    print(f"dgrad: {len(rows)} rows of experts {experts} ({n_e[experts].tolist()} rows), rel Frobenius {err:.2e}",
          flush=True)
    assert err <= 2e-5

    # wgrad: the whole dW2 of the smallest, the median and the 75th-percentile expert
    for e in (int(order[0]), int(order[len(order) // 2]), int(order[3 * len(order) // 4])):
        seg = np.arange(o_offs[e], o_offs[e + 1])
        so = np.array([0, len(seg)], np.int32)
        ya = oracle.mxfp8_quantize(bits(dy[torch.from_numpy(o_s2a[seg].astype(np.int64)).to(dev)]), 1, seg_offsets=so)
        hb = oracle.mxfp8_quantize(bits(hin[int(o_offs[e]):int(o_offs[e + 1])]), 1, seg_offsets=so)
        w = pad[e + 1] - pad[e]
        for g, o in ((dy1, ya), (h1, hb)):
            assert np.array_equal(host(g[0][:, pad[e]:pad[e] + w]), o[0][:, :w])
            assert np.array_equal(host(g[1][:, pad[e] // 32:(pad[e] + w) // 32]), o[1][:, :w // 32])
        ref = oracle.mxfp8_gemm_wgrad(ya, hb, oracle.pad_offsets(so))[0]
        err = _rel_frob(host(dW2[e]), ref)
        print(f"wgrad expert {e} ({len(seg)} rows): rel Frobenius {err:.2e}", flush=True)
        assert err <= 2e-5


@pytest.mark.parametrize("axis,mode,gather,C", [(0, 0, False, 96), (0, 1, True, 64), (1, 0, False, 64),
                                                (1, 1, True, 48), (1, 0, True, 40)])
def test_no_saturation_scale_rule(axis, mode, gather, C):
    """scale_rule = 1 (ceil(log2(amax / 448))) bit-exact against the oracle on
    every kernel path (rows, the tiled and the general transposed kernels, SR
    with and without gathers), with block maxima on and around 1.75 * 2^k."""
    g = np.random.default_rng(900 + 10 * axis + mode + C)
    R = 300
    x = g.standard_normal((R + 7, C)) * 2.0 ** g.integers(-10, 10, (R + 7, 1))
    m = np.array([1.0, 1.75, 1.7578125, 1.875, 1.5])
    x[::3, ::5] = (m[g.integers(0, 5, x[::3, ::5].shape)] * 2.0 ** g.integers(-4, 8, x[::3, ::5].shape)
                   * np.where(g.random(x[::3, ::5].shape) < 0.5, -1.0, 1.0))
    xb = synth.to_bf16_bits(x)
    gat = g.integers(0, 2 * (R + 7), R).astype(np.int32) if gather else None
    seg = np.array([0, 37, 37, 160, R], np.int32) if axis == 1 else None
    ld = nvq.mxfp8_axis1_ld(R, 4) if axis == 1 else None
    o = oracle.mxfp8_quantize(xb, axis, mode=mode, row_gather=gat, gather_div=2, seg_offsets=seg, R=R,
                              stream=2 + axis, rule=1, ld=ld)
    q = nvq.mxfp8_requant_sr(to_dev_u16(xb), axis, round_mode=mode, row_gather=None if gat is None else to_dev(gat),
                             gather_div=2, seg_offsets=None if seg is None else to_dev(seg), R=R, scale_rule=1)
    assert host(q[1]).shape == o[1].shape and np.array_equal(host(q[1]), o[1]), "scale bytes differ"
    assert np.array_equal(host(q[0]), o[0]), "elements differ"
    o0 = oracle.mxfp8_quantize(xb, axis, mode=mode, row_gather=gat, gather_div=2, seg_offsets=seg, R=R,
                               stream=2 + axis, rule=0, ld=ld)
    assert not np.array_equal(o0[1], o[1])     # the two rules part on this input
