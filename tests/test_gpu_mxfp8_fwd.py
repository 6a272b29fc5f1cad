"""GPU parity of the MXFP8 expert forward (the comparison precision for the
NVFP4 forward), staged as the chain requires, each stage on identical
operands: X rows gathered into expert order and quantized, and the weights
quantized, byte for byte; fc1 (expert-major weight operand) within 2e-5
Frobenius error of the oracle's exact-block fp64 GEMM; SwiGLU within
1 bf16 ulp; H quantized byte for byte; fc2 within 2e-5 (both GEMMs measured
against the magnitude of the products they sum); and the fused call
equal, bit for bit, to the staged chain's rows scattered to (token, slot)."""
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


def _rel_frob(got, ref):
    ref = np.asarray(ref, np.float64)
    return float(np.linalg.norm(np.asarray(got, np.float64) - ref) / max(np.linalg.norm(ref), 1e-300))


def _q_equal(gpu, ref, what):
    for g, r, part in zip(gpu, ref, ("elements", "scales")):
        assert np.array_equal(host(g), r), f"{what}: {part} differ"


def _abs_q(q):
    """|operand|: E4M3 with the sign bit cleared (E8M0 scales are positive)."""
    return q[0] & np.uint8(0x7F), q[1]


def _check_gemm(got, ref, a_o, b_o, offsets, what):
    """Error of a scaled-FP8 MFMA product on identical operands. The hardware
    rounds relative to the magnitudes it accumulates (about 2^-16 of them), so
    the bound is 2e-5 of ||(|A| |B|)||_F; on operands whose products cancel
    (fc2 on the SwiGLU output) the plain relative error can exceed that while
    this one does not. Both are printed."""
    ref_abs = oracle.mxfp8_gemm_dgrad(_abs_q(a_o), tuple(_abs_q(b_o)), offsets)
    diff = np.linalg.norm(np.asarray(got, np.float64) - ref)
    print(f"  {what}: rel Frobenius {diff / max(np.linalg.norm(ref), 1e-300):.2e}, "
          f"rel to |A||B| {diff / max(np.linalg.norm(ref_abs), 1e-300):.2e}")
    assert diff <= 2e-5 * np.linalg.norm(ref_abs)


def _expert_major(q, E):
    e, s = q
    return e.reshape(E, -1, e.shape[1]), s.reshape(E, -1, s.shape[1])


@pytest.mark.parametrize("case", [
    dict(T=64, d=256, E=4, k=2, d_ff=256, skew=False),     # single K steps, ragged segments
    dict(T=300, d=384, E=5, k=2, d_ff=128, skew=True),     # skewed load, K not a multiple of 512
    dict(T=96, d=512, E=3, k=2, d_ff=512, skew=True),      # scale words four K steps at a time (both GEMMs)
    dict(T=40, d=128, E=6, k=3, d_ff=256, skew=True),      # empty experts likely
])
def test_mxfp8_forward_staged(case):
    T, d, E, k, d_ff = case["T"], case["d"], case["E"], case["k"], case["d_ff"]
    c = synth.moe_shapes(T, d, E, k, d_ff, seed=9, skew=case["skew"])
    print(f"[mxfp8 fwd] {case}", flush=True)
    A = T * k
    offsets, s2a = oracle.route(c["topk_ids"], E)
    offs_d, s2a_d = to_dev(offsets), to_dev(s2a)
    w1 = c["w1"].reshape(E * 2 * d_ff, d)
    w2 = c["w2"].reshape(E * d, d_ff)

    # operands: quantized bytes identical to the oracle's
    xq = nvq.mxfp8_requant_sr(to_dev_u16(c["x"]), 0, nvq.RTN, row_gather=s2a_d, gather_div=k)
    xq_o = oracle.mxfp8_quantize(c["x"], 0, row_gather=s2a, gather_div=k)
    _q_equal(xq, xq_o, "Xq")
    w1q = nvq.mxfp8_requant_sr(to_dev_u16(w1), 0, nvq.RTN)
    w1q_o = oracle.mxfp8_quantize(w1, 0)
    _q_equal(w1q, w1q_o, "W1q")
    w2q = nvq.mxfp8_requant_sr(to_dev_u16(w2), 0, nvq.RTN)
    w2q_o = oracle.mxfp8_quantize(w2, 0)
    _q_equal(w2q, w2q_o, "W2q")

    # fc1 with the expert-major weight operand
    G = nvq.moe_grouped_gemm_mxfp8(nvq.FWD, xq, w1q, offs_d, N=2 * d_ff, K=d)
    G_ref = oracle.mxfp8_gemm_dgrad(xq_o, _expert_major(w1q_o, E), offsets)
    Gh = host(G)[:A]
    _check_gemm(Gh, G_ref, xq_o, _expert_major(w1q_o, E), offsets, "fc1")

    # SwiGLU on the GPU's G
    H = nvq.swiglu_fwd(G)
    H_ref = oracle.swiglu(Gh.astype(np.float64))
    check_bf16_close(host(H)[:A], H_ref, "swiglu_fwd")

    # H quantized byte for byte, then fc2 on identical operands
    Hbits = host(H.view(torch.int16)).view(np.uint16)
    hq = nvq.mxfp8_requant_sr(H, 0, nvq.RTN)
    hq_o = oracle.mxfp8_quantize(Hbits, 0)
    _q_equal(hq, hq_o, "Hq")
    Y = nvq.moe_grouped_gemm_mxfp8(nvq.FWD, hq, w2q, offs_d, N=d, K=d_ff)
    Y_ref = oracle.mxfp8_gemm_dgrad(hq_o, _expert_major(w2q_o, E), offsets)
    _check_gemm(host(Y)[:A], Y_ref, hq_o, _expert_major(w2q_o, E), offsets, "fc2")

    # the fused call: the staged rows, rounded to bf16 and scattered
    y = nvq.moe_expert_fwd_mxfp8(to_dev_u16(c["x"]).view(torch.bfloat16), to_dev(c["topk_ids"]), w1q, w2q)
    chain = torch.zeros((A, d), dtype=torch.bfloat16, device=y.device)
    chain[s2a_d.long()] = Y[:A].to(torch.bfloat16)
    assert torch.equal(y.view(A, d), chain), "fused forward differs from the staged chain"


def test_mxfp8_forward_dropped_ids_leave_rows_untouched():
    """Assignments with an out-of-range expert id get no rows; their y rows keep
    what the caller had there, and every other row matches a run without them."""
    T, d, E, k, d_ff = 48, 128, 4, 2, 128
    c = synth.moe_shapes(T, d, E, k, d_ff, seed=3)
    ids = c["topk_ids"].copy()
    ids[5, 1] = E + 2
    ids[17, 0] = -1
    w1q = nvq.mxfp8_requant_sr(to_dev_u16(c["w1"].reshape(E * 2 * d_ff, d)), 0, nvq.RTN)
    w2q = nvq.mxfp8_requant_sr(to_dev_u16(c["w2"].reshape(E * d, d_ff)), 0, nvq.RTN)
    x = to_dev_u16(c["x"]).view(torch.bfloat16)
    sentinel = torch.full((T, k, d), 7.0, dtype=torch.bfloat16, device=x.device)
    y = nvq.moe_expert_fwd_mxfp8(x, to_dev(ids), w1q, w2q, y=sentinel.clone())
    assert torch.all(y[5, 1] == 7.0) and torch.all(y[17, 0] == 7.0)
    y_full = nvq.moe_expert_fwd_mxfp8(x, to_dev(c["topk_ids"]), w1q, w2q)
    keep = torch.ones((T, k), dtype=torch.bool, device=x.device)
    keep[5, 1] = False
    keep[17, 0] = False
    # the same expert rows in the same order give the same bits, except that
    # dropping two assignments changes nothing else (per-row quantization)
    assert torch.equal(y[keep], y_full[keep])


def test_mxfp8_forward_rejects_bad_arguments():
    L = nvq.lib()
    fake = [torch.empty(4096, dtype=torch.uint8, device="cuda") for _ in range(7)]
    p = [f.data_ptr() for f in fake]
    ws = torch.empty(1 << 20, dtype=torch.uint8, device="cuda")
    import ctypes as C
    v = [C.c_void_p(q) for q in p]
    call = lambda d, d_ff, k, E: L.moe_expert_fwd_mxfp8(v[0], 8, d, v[1], k, E, d_ff, v[2], v[3], v[4], v[5], v[6],
                                                       C.c_void_p(ws.data_ptr()), ws.numel(), None)
    assert call(200, 128, 2, 4) == -2    # d not a multiple of 128
    assert call(128, 100, 2, 4) == -2    # d_ff not a multiple of 128
    assert call(128, 128, 5, 4) == -2    # k > E
    assert L.moe_expert_fwd_mxfp8(None, 8, 128, v[1], 2, 4, 128, v[2], v[3], v[4], v[5], v[6],
                                  C.c_void_p(ws.data_ptr()), ws.numel(), None) == -1
