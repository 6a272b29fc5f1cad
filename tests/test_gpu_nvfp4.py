"""GPU parity of NVFP4 quantize/dequantize against the CPU oracle: codes,
scale bytes and tensor-scale bits must match exactly (nearest-even and Philox
stochastic rounding), dequantized values bit for bit."""
import numpy as np
import pytest
import torch

import oracle
import precision_moe_numerics_amd as nvq
from precision_moe_numerics_amd import synth
from gpu_util import host, require_gpu, to_dev_u16

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _gpu():
    require_gpu()


def _check_quant(x_bits, mode=0, seed=0, stream=1):
    xg = to_dev_u16(x_bits)
    c, s, t = nvq.nvfp4_quantize(xg, round_mode=mode, seed=seed, stream_id=stream)
    torch.cuda.synchronize()
    oc, os_, od = oracle.nvfp4_quantize(x_bits, mode=mode, seed=seed, stream=stream)
    assert np.array_equal(host(s), os_), f"scale bytes differ at {np.argwhere(host(s) != os_)[:5].tolist()}"
    assert np.array_equal(host(c), oc), f"codes differ at {np.argwhere(host(c) != oc)[:5].tolist()}"
    assert host(t)[0].view(np.uint32) == np.float32(od).view(np.uint32)
    return c, s, t, (oc, os_, od)


@pytest.mark.parametrize("shape", [(1, 16), (3, 48), (5, 80), (37, 272), (129, 1040), (1024, 4096)])
@pytest.mark.parametrize("mode", [0, 1])
def test_quantize_shapes(shape, mode):
    x = synth.student_t_outliers(*shape, workload_id=80 + shape[0] % 7)
    _check_quant(x, mode=mode, seed=3, stream=1)


def test_quantize_quant_8192_rtn_and_sr():
    """The full 8192x8192 quantize workload (Student-t(3) x 0.1, 0.1% x100)."""
    x = synth.student_t_outliers(8192, 8192)
    print("quant_8192 rtn", flush=True)
    c, s, t, _ = _check_quant(x, mode=0)
    print("quant_8192 sr", flush=True)
    _check_quant(x, mode=1, seed=0, stream=1)
    print("quant_8192 dequant", flush=True)
    d32 = nvq.nvfp4_dequantize(c, s, t, torch.float32)
    ref = oracle.nvfp4_dequantize(host(c), host(s), host(t)[0])
    assert np.array_equal(host(d32).view(np.uint32), ref.view(np.uint32))
    d16 = nvq.nvfp4_dequantize(c, s, t, torch.bfloat16)
    ref16 = synth.to_bf16_bits(ref)  # torch's fp32 -> bf16 nearest-even
    assert np.array_equal(host(d16), ref16)


def test_quantize_beyond_2_28_units():
    """262208 x 8192 bf16 values (4.3 GB; 2^28 + 8192 units of 8 values): past
    2^28 units the encode pass addresses with 64-bit offsets. Rows at both
    ends, on both sides of the 2^31-byte boundary (row 131072) and past 2^28
    units (the last 64 rows), nearest even and stochastic (element indices
    past 2^31 in the draws), against the oracle's slice quantization under
    the tensor maximum (taken by torch over the whole tensor)."""
    R, C = 262208, 8192
    x = synth.device_normal_bf16((R, C), 1.0, 9, "cuda", workload_id=88)
    amax_bits = int((x.view(torch.int16) & 0x7FFF).max().item())
    amax = float(np.array([amax_bits << 16], np.uint32).view(np.float32)[0])
    rows = [0, 1, 131071, 131072, R - 64, R - 2, R - 1]
    for mode in (0, 1):
        print(f"beyond 2^28 units, mode {mode}", flush=True)
        c, s, t = nvq.nvfp4_quantize(x, round_mode=mode, seed=3, stream_id=1)
        torch.cuda.synchronize()
        for r in rows:
            f = oracle.bf16_to_f32(host(x[r:r + 1]))
            oc, os_, od = oracle.nvfp4_quantize_slice(f, amax, r * C, mode=mode, seed=3, stream=1)
            assert np.array_equal(host(s[r:r + 1]), os_), (mode, r)
            assert np.array_equal(host(c[r:r + 1]), oc), (mode, r)
        assert host(t)[0].view(np.uint32) == np.float32(od).view(np.uint32)
        del c, s, t


def test_batched_tensor_scales():
    """One tensor scale per batch entry; 3*5*48/16 = 45 scale bytes per entry is
    not a multiple of 4, so entries 1 and 2 start unaligned."""
    x = synth.normal_bf16((3, 5, 48), 1.0, 81, 0)
    x[1] = synth.to_bf16_bits(oracle.bf16_to_f32(x[1]) * 1000.0)
    xg = to_dev_u16(x)
    c, s, t = nvq.nvfp4_quantize(xg, batched=True)
    for b in range(3):
        oc, os_, od = oracle.nvfp4_quantize(x[b])
        assert np.array_equal(host(c)[b], oc) and np.array_equal(host(s)[b], os_)
        assert host(t)[b] == od


def test_tensor_max_at_every_position():
    """The tensor maximum is found wherever it sits: each of the 8 values of
    a 16-byte load, in the first, a middle and the last unit of a tensor
    that spans several workgroup chunks, with either sign."""
    base = synth.normal_bf16((64, 4096), 1.0, 82, 0)
    n = base.size
    for unit in (0, n // 16 + 3, n // 8 - 1):
        for p in range(8):
            for sign in (1.0, -1.0):
                x = base.copy().reshape(-1)
                x[8 * unit + p] = synth.to_bf16_bits(np.array([sign * 77.0]))[0]
                x = x.reshape(base.shape)
                c, s, t = nvq.nvfp4_quantize(to_dev_u16(x))
                oc, os_, od = oracle.nvfp4_quantize(x)
                assert host(t)[0] == od, (unit, p, sign)
                assert np.array_equal(host(s), os_) and np.array_equal(host(c), oc)


def test_zero_and_tiny_tensors():
    z = np.zeros((4, 64), np.uint16)
    z[2, 5] = 0x8000  # negative zero
    _check_quant(z)
    tiny = np.zeros((2, 32), np.uint16)
    tiny[0, 3] = 0x0001
    tiny[1, 20] = 0x8003
    tiny[1, 21] = 0x0080  # smallest normal
    _check_quant(tiny)
    _check_quant(tiny, mode=1, seed=1)


def test_tiny_blocks_under_large_and_small_tensor_scales():
    """Block maxima from bf16 subnormals up to 2^-124 under tensor maxima 1
    and 2^-88 (S just under 2^100: the encoders' FMA quotient by 6) and 2^-89
    (S just over it: the IEEE division)."""
    for top in (0x3F80, 0x1380, 0x1300):  # 1.0, 2^-88, 2^-89
        x = np.zeros((3, 96), np.uint16)
        x[0, 0] = top
        x[0, 16:32] = np.arange(1, 17)                  # subnormal block
        x[0, 32:48] = 0x0080 | np.arange(16)            # block max near 2^-126
        x[1, 0:16] = 0x0100 | (np.arange(16) * 7)       # near 2^-125 (the quotient's exactness bound)
        x[1, 16:32] = 0x0180 | (np.arange(16) * 5)      # near 2^-124
        x[1, 48:64] = 0x8D80 | np.arange(16)            # -2^-100 and neighbours
        x[2, :] = (0x0380 + np.arange(96) * 37) & 0x7FFF  # a spread of small magnitudes
        _check_quant(x)
        _check_quant(x, mode=1, seed=5)


def test_sr_draws_depend_on_seed_and_stream():
    x = synth.normal_bf16((64, 256), 1.0, 82, 0)
    a, _, _, _ = _check_quant(x, mode=1, seed=1, stream=1)
    b, _, _, _ = _check_quant(x, mode=1, seed=2, stream=1)
    c, _, _, _ = _check_quant(x, mode=1, seed=1, stream=7)
    assert not torch.equal(a, b) and not torch.equal(a, c)


def test_bad_arguments_rejected():
    x = torch.zeros((4, 24), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(nvq.NvqError, match="status -2"):
        nvq.nvfp4_quantize(x)
    x = torch.zeros((4, 32), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(nvq.NvqError, match="status -5"):
        nvq.nvfp4_quantize(x, round_mode=7)
