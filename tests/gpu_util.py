"""Helpers shared by the GPU parity tests (no method arithmetic here)."""
import numpy as np
import pytest
import torch


def require_gpu():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    import precision_moe_numerics_amd as nvq
    nvq.lib()  # fails loudly if libnvq.so is missing


def to_dev_u16(bits):
    """numpy uint16 bf16 bits -> CUDA bf16 tensor."""
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).cuda().view(torch.bfloat16)


def to_dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def host(t):
    t = t.detach().cpu()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


def bf16_bits_to_f64(bits):
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def ulp_bf16(v):
    """Spacing of bf16 at |v| (2^(e-7) for |v| in [2^e, 2^e+1))."""
    a = np.maximum(np.abs(v), 2.0 ** -126)
    return 2.0 ** (np.floor(np.log2(a)) - 7)


def check_bf16_close(got_bits, ref, what, floor_frac=2.0 ** -6):
    """|got - ref| <= 1 bf16 ulp of max(|ref|, floor_frac * rms(ref)), elementwise.
    Returns (number of elements that used the floor, max error in ulps)."""
    got = bf16_bits_to_f64(got_bits)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (what, got.shape, ref.shape)
    rms = np.sqrt(np.mean(ref ** 2)) if ref.size else 0.0
    mag = np.maximum(np.abs(ref), floor_frac * rms)
    tol = ulp_bf16(mag)
    err = np.abs(got - ref)
    bad = ~(err <= tol)
    if bad.any():
        idx = np.argwhere(bad)[:5]
        raise AssertionError(f"{what}: {int(bad.sum())} of {bad.size} elements beyond 1 bf16 ulp; "
                             f"first {idx.tolist()} got {got[bad][:5]} ref {ref[bad][:5]}")
    used_floor = int((np.abs(ref) < floor_frac * rms).sum())
    return used_floor, float((err / tol).max()) if err.size else 0.0
