"""GPU parity of the RHT32 + NVFP4 combine-path quantizer (codes, scale bytes
and tensor-scale bits exact against the oracle's fp32 butterfly + encoder)
and of the dequantize + inverse transform + top-k combine (within 1 bf16 ulp
of the oracle's fp64 combine on identical codes)."""
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


def _y(R, C, wid=70, outlier_rows=0.01):
    y = synth.normal_bf16((R, C), 1.0, wid, 0)
    n = max(1, int(round(outlier_rows * R)))
    rows = synth.rng(wid, 1).choice(R, size=n, replace=False)
    y[rows] = synth.to_bf16_bits(oracle.bf16_to_f32(y[rows]).astype(np.float64) * 20.0)
    return y


@pytest.mark.parametrize("shape,seed", [((1, 32), 0), ((3, 64), 5), ((97, 4096), 0), ((1000, 96), 123456789)])
def test_rht_quant_exact(shape, seed):
    y = _y(*shape)
    q = nvq.rht32_blockquant(to_dev_u16(y), sign_seed=seed)
    z = oracle.rht32_forward(y, seed)
    oc, os_, od = oracle.nvfp4_quantize(z)
    assert np.array_equal(host(q[1]), os_), np.argwhere(host(q[1]) != os_)[:5]
    assert np.array_equal(host(q[0]), oc), np.argwhere(host(q[0]) != oc)[:5]
    assert host(q[2])[0] == od


@pytest.mark.parametrize("shape", [(1, 32), (1, 64), (3, 96), (5, 4096 + 32 * 7)])
@pytest.mark.parametrize("seed", [0, 1, 2, 3, 4, 5])
def test_rht_quant_tail_maximum(shape, seed):
    """Chunk counts that leave lanes of the last wave idle, with the tensor's
    largest values in its last 8 elements and zeros in the rest of that chunk:
    idle lanes see copies of the last 8 values, whose transform can exceed the
    real maximum, so they must not enter the tensor scale."""
    R, C = shape
    x = synth.rng(72, seed).standard_normal((R, C)) * 0.01
    x[-1, -32:] = 0.0
    x[-1, -8:] = synth.rng(72, 100 + seed).standard_normal(8) * 3.0
    y = synth.to_bf16_bits(x)
    q = nvq.rht32_blockquant(to_dev_u16(y), sign_seed=seed)
    z = oracle.rht32_forward(y, seed)
    oc, os_, od = oracle.nvfp4_quantize(z)
    assert host(q[2])[0] == od, (host(q[2])[0], od)
    assert np.array_equal(host(q[1]), os_)
    assert np.array_equal(host(q[0]), oc)


@pytest.mark.parametrize("T,k,C", [(4, 8, 32), (33, 8, 4096), (50, 3, 96)])
def test_combine_matches_oracle(T, k, C):
    y = _y(T * k, C, wid=71)
    z = oracle.rht32_forward(y, 9)
    codes, scales, D = oracle.nvfp4_quantize(z)
    w = synth.rng(71, 2).dirichlet(np.ones(k), size=T).astype(np.float32)
    out = nvq.rht32_dequant_combine((to_dev(codes), to_dev(scales), to_dev(np.atleast_1d(D))), T, k, to_dev(w),
                                    sign_seed=9)
    ref = oracle.rht32_combine(codes, scales, D, T, k, 9, w)
    nf, mx = check_bf16_close(host(out), ref, "combine")
    print(f"combine T={T} k={k} C={C}: {nf} on the rms floor, max {mx:.3f} ulp")


def test_combine_rht_full_size_sampled():
    """The full combine workload: Y [131072, 4096] N(0,1) with 1% of rows x20,
    signs from seed 0, top-8 weights of the moe_layer routing. The tensor scale
    needs all of z, so the oracle transforms every row and encodes sampled rows."""
    R, C, T, k = 131072, 4096, 16384, 8
    dev = torch.device("cuda")
    yd = synth.device_normal_bf16((R, C), 1.0, 1, dev, workload_id=5)
    synth.rows_scaled(yd, 0.01, 20.0, 2)
    q = nvq.rht32_blockquant(yd, sign_seed=0)
    torch.cuda.synchronize()
    print("full-size rht quant done", flush=True)
    y = host(yd)
    z = oracle.rht32_forward(y, 0)
    amax = oracle.amax_f32(z)
    del y
    assert host(q[2])[0] == np.float32(amax / np.float32(2688.0))
    rows = np.sort(synth.rng(5, 3).choice(R, size=48, replace=False))
    gc, gs = host(q[0]), host(q[1])
    for r in rows:
        oc, os_, _ = oracle.nvfp4_quantize_slice(z[r:r + 1], amax, int(r) * C)
        assert np.array_equal(gc[r:r + 1], oc) and np.array_equal(gs[r:r + 1], os_), r
    del z
    print("sampled rows exact", flush=True)
    _, w = synth.moe_layer_routing()
    out = nvq.rht32_dequant_combine(q, T, k, to_dev(w), sign_seed=0)
    ts = np.sort(synth.rng(5, 4).choice(T, size=16, replace=False))
    sel = (ts[:, None] * k + np.arange(k)[None, :]).reshape(-1)
    ref = oracle.rht32_combine(gc[sel], gs[sel], host(q[2])[0], len(ts), k, 0, w[ts])
    check_bf16_close(host(out)[ts], ref, "combine full size")
