"""Where the MXFP8 GEMMs' error comes from: exact-sum operands through the
library's E8M0-scaled FP8 grouped GEMM (gfx950 v_mfma_scale_f32_32x32x64_
f8f6f4), compared with the oracle's exact-block fp64 GEMM.

What these tests pin (the error model the design notes state):
  * sums whose every partial and total is exact in fp32 come back bit for bit
    equal to the oracle, with block scales differing from block to block, so
    scale application, masking, tile seams and the epilogue add no error;
  * inside one 32-value block the instruction drops a product 2^-14 below the
    block's largest product (1 + 2^-14 comes back as 1, although it is an
    fp32 value), while one 2^-12 below is kept;
  * the same small product in a block of its own (scaled by its E8M0 byte) is
    kept exactly: block sums meet each other and the accumulator in fp32.
So the GEMMs' error on real data is the instruction's in-block alignment,
about 2^-14 of each block's largest product, not the kernel's.

MXFP8 is the backward format of page "Thinking Machines Details End-to-End
4-Bit Training for Inkling 2 Small" (section "Key Takeaways")."""
import numpy as np
import pytest

import oracle
import precision_moe_numerics_amd as nvq
from gpu_util import host, require_gpu, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _gpu():
    require_gpu()


def _e4m3_bytes(vals):
    """E4M3 bytes of values that are exactly representable (checked)."""
    v = np.asarray(vals, dtype=np.float32)
    b = np.array([oracle.e4m3_rne_sat(x) for x in v.ravel()], dtype=np.uint8).reshape(v.shape)
    back = np.array([oracle.e4m3_decode(x) for x in b.ravel()], dtype=np.float32).reshape(v.shape)
    assert np.array_equal(back, v), "test values must be E4M3 values"
    return b


def _gemm(a, b, R, N, K, mode):
    """One expert: out[r][n] = sum_k A[r][k] B[n][k] (FWD: B rows [N, K];
    DGRAD: B as the axis-1 layout [N, >= K])."""
    seg = np.array([0, R], np.int32)
    out = nvq.moe_grouped_gemm_mxfp8(mode, (to_dev(a[0]), to_dev(a[1])), (to_dev(b[0]), to_dev(b[1])), to_dev(seg),
                                     N=N, K=K)
    return host(out)[:R]


@pytest.mark.parametrize("mode", [nvq.FWD, nvq.DGRAD])
@pytest.mark.parametrize("R,N,K", [(256, 128, 256), (300, 256, 512), (40, 128, 96), (512, 128, 4096)])
def test_exact_sums_are_bit_exact(mode, R, N, K):
    """Integer elements |v| <= 15 and block scales 2^0..2^3 (2^0..2^2 for the
    longest K): every product is an integer and the sum of all |products|
    stays below 2^24, so every partial sum in any order is an fp32 integer and
    the GPU must equal the oracle bit for bit."""
    rng = np.random.default_rng(R * 7 + K)
    ints = np.arange(-15, 16)
    smax = 3 if K <= 512 else 2
    a_el = _e4m3_bytes(rng.choice(ints, (R, K)))
    b_el = _e4m3_bytes(rng.choice(ints, (N, K)))
    a_sc = rng.integers(127, 128 + smax, (R, K // 32)).astype(np.uint8)
    b_sc = rng.integers(127, 128 + smax, (N, K // 32)).astype(np.uint8)
    seg = np.array([0, R], np.int32)
    ref = oracle.mxfp8_gemm_dgrad((a_el, a_sc), (b_el[None], b_sc[None]), seg)
    mag = oracle.mxfp8_gemm_dgrad((a_el & np.uint8(0x7F), a_sc), (b_el[None] & np.uint8(0x7F), b_sc[None]), seg)
    assert mag.max() < 2.0 ** 24 and np.array_equal(np.round(ref), ref)
    got = _gemm((a_el, a_sc), (b_el, b_sc), R, N, K, mode)
    bad = got != ref.astype(np.float32)
    assert not bad.any(), f"{int(bad.sum())} outputs differ; first {np.argwhere(bad)[:4].tolist()}"


def test_in_block_window():
    """Inside one 32-value block: 1 + 2^-12 exact, 1 + 2^-14 comes back as 1.
    (Both are fp32 values, so an fp32 accumulation would keep them.)"""
    R, N, K = 64, 128, 64
    a_val = np.zeros((R, K), np.float32)
    b_val = np.zeros((N, K), np.float32)
    a_val[:, 0] = 1.0
    b_val[:, 0] = 1.0
    b_val[:, 1] = 2.0 ** -7                       # E4M3 subnormal 0x04
    j = np.array([0, 1, 2, 3, 4, 5, 6, 7])[np.arange(R) % 8]
    a_val[:, 1] = 2.0 ** -j.astype(np.float64)    # product 2^-(7+j)
    a_sc = np.full((R, 2), 127, np.uint8)
    b_sc = np.full((N, 2), 127, np.uint8)
    a_el, b_el = _e4m3_bytes(a_val), _e4m3_bytes(b_val)
    got = _gemm((a_el, a_sc), (b_el, b_sc), R, N, K, nvq.FWD)
    ref = oracle.mxfp8_gemm_dgrad((a_el, a_sc), (b_el[None], b_sc[None]), np.array([0, R], np.int32))
    exact = 1.0 + 2.0 ** -(7.0 + j)
    assert np.array_equal(ref[:, 0], exact) and np.all(exact.astype(np.float32) == exact)
    for jj in range(8):
        rows = j == jj
        g = np.unique(got[rows])
        print(f"  1 + 2^-{7 + jj} inside one block -> {g.tolist()} (exact {1 + 2.0 ** -(7 + jj)!r})")
        assert len(g) == 1
    kept = 7 + j <= 12
    assert np.all(got[kept] == ref[kept].astype(np.float32)), "products within 2^-12 of the block max are exact"
    dropped = 7 + j >= 14
    assert np.all(got[dropped] == 1.0), "a product 2^-14 below the block max is dropped inside the block"


def test_cross_block_sum_is_fp32():
    """The same small products in a 32-block of their own (E8M0 scale 2^-m):
    1 + 2^-m comes back exactly for every m up to 23, as fp32 accumulation of
    exact block sums gives."""
    R, N, K = 64, 128, 64
    a_val = np.zeros((R, K), np.float32)
    b_val = np.zeros((N, K), np.float32)
    a_val[:, 0] = 1.0
    b_val[:, 0] = 1.0
    a_val[:, 32] = 1.0
    b_val[:, 32] = 1.0
    m = np.arange(R) % 24                          # 0..23
    a_sc = np.full((R, 2), 127, np.uint8)
    a_sc[:, 1] = (127 - m).astype(np.uint8)
    b_sc = np.full((N, 2), 127, np.uint8)
    a_el, b_el = _e4m3_bytes(a_val), _e4m3_bytes(b_val)
    got = _gemm((a_el, a_sc), (b_el, b_sc), R, N, K, nvq.FWD)
    exact = (1.0 + 2.0 ** -m.astype(np.float64))
    assert np.all(exact.astype(np.float32) == exact)
    assert np.all(got == exact.astype(np.float32)[:, None])
