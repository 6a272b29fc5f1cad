"""nvfp4_quantize_noalloc, the quantize entry point for callers that cannot
allocate device memory, against nvfp4_quantize through the C ABI: identical
code bytes, scale bytes and tensor-scale bits on consecutive calls, each
later one smaller than the one before (the shared partial-maximum array
keeps the previous call's contents), in both rounding modes."""
import ctypes as C

import pytest
import torch

import precision_moe_numerics_amd as nvq
from precision_moe_numerics_amd import synth
from gpu_util import require_gpu

pytestmark = pytest.mark.gpu


def _vp(t):
    return C.c_void_p(t.data_ptr()) if t is not None else None


def _noalloc(x, mode, seed):
    B, R, Cc = x.shape
    codes = torch.full((B, R, Cc // 2), 0xAA, dtype=torch.uint8, device=x.device)
    scales = torch.full((B, R, Cc // 16), 0xAA, dtype=torch.uint8, device=x.device)
    ts = torch.full((B,), -1.0, dtype=torch.float32, device=x.device)
    rc = nvq.lib().nvfp4_quantize_noalloc(_vp(x), B, R, Cc, _vp(codes), _vp(scales), _vp(ts), mode, seed, 1,
                                          C.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert rc == 0, nvq.lib().nvq_status_string(rc)
    return codes, scales, ts


@pytest.mark.parametrize("mode", [nvq.RTN, nvq.SR])
def test_noalloc_equals_quantize_on_consecutive_calls(mode):
    require_gpu()
    dev = torch.device("cuda")
    # large first (2048 partial maxima), then smaller ones: batched, ragged, tiny
    shapes = [(1, 4096, 4096), (3, 1000, 96), (2, 7, 32), (1, 1, 16)]
    for i, (B, R, Cc) in enumerate(shapes):
        x = synth.device_normal_bf16((B, R, Cc), 0.5 / (i + 1), 10 + i, dev, workload_id=9)
        ref = nvq.nvfp4_quantize(x, round_mode=mode, seed=11, batched=True)
        got = _noalloc(x, mode, 11)
        torch.cuda.synchronize()
        assert torch.equal(got[0], ref[0]), (B, R, Cc, "codes")
        assert torch.equal(got[1], ref[1]), (B, R, Cc, "scales")
        assert torch.equal(got[2].view(torch.int32), ref[2].view(torch.int32)), (B, R, Cc, "tscale")


def test_noalloc_argument_errors():
    require_gpu()
    L = nvq.lib()
    x = torch.zeros((1, 4, 32), dtype=torch.bfloat16, device="cuda")
    o = torch.zeros(4096, dtype=torch.uint8, device="cuda")
    f = torch.zeros(4, dtype=torch.float32, device="cuda")
    call = lambda xx, B, R, Cc, mode: L.nvfp4_quantize_noalloc(xx, B, R, Cc, _vp(o), _vp(o), _vp(f), mode, 0, 1,
                                                               None)
    assert call(None, 1, 4, 32, 0) == -1
    assert call(_vp(x), 0, 4, 32, 0) == -2
    assert call(_vp(x), 1, 4, 24, 0) == -2
    assert call(_vp(x), 1, 4, 32, 7) == -5
