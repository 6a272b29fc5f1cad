"""GPU parity of the sigmoid top-k router against the oracle: ids equal (the
choice is made on fp64 keys on both sides), weights within the fp32 rounding
of the oracle's fp64 values."""
import numpy as np
import pytest
import torch

import oracle
import precision_moe_numerics_amd as nvq
from gpu_util import host, require_gpu, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _gpu():
    require_gpu()


def _check(logits, bias, k, what):
    ids, w = nvq.moe_router_sigmoid_topk(to_dev(logits), to_dev(bias), k)
    ids_o, w_o = oracle.router_sigmoid_topk(logits, bias, k)
    assert np.array_equal(host(ids), ids_o), f"{what}: ids differ"
    assert np.allclose(host(w).astype(np.float64), w_o, rtol=2.0 ** -23, atol=0), f"{what}: weights differ"


@pytest.mark.parametrize("T,E,k,bias_std", [(100, 8, 2, 0.3), (333, 384, 8, 0.3), (64, 1024, 64, 0.3),
                                            (50, 17, 17, 0.3), (7, 100, 1, 0.3), (200, 384, 8, 3.0),
                                            (65, 65, 6, 0.0)])
def test_router(T, E, k, bias_std):
    """Ragged expert counts (not multiples of 64), k = E, k = 64, E = 1024, a
    bias that dominates the choice, and no bias."""
    g = np.random.default_rng(400 + T)
    logits = g.standard_normal((T, E)).astype(np.float32)
    bias = (bias_std * g.standard_normal(E)).astype(np.float32)
    _check(logits, bias, k, f"T={T} E={E} k={k}")


def test_router_ties_pick_the_lower_index():
    ids, w = nvq.moe_router_sigmoid_topk(torch.zeros((9, 70), device="cuda"), torch.zeros(70, device="cuda"), 5)
    assert np.array_equal(host(ids), np.tile(np.arange(5, dtype=np.int32), (9, 1)))
    assert np.allclose(host(w), 0.2)


def test_router_full_size():
    """The moe_layer router shape: 16384 tokens, 384 experts, top-8."""
    g = np.random.default_rng(404)
    logits = g.standard_normal((16384, 384)).astype(np.float32)
    bias = g.standard_normal(384).astype(np.float32)
    _check(logits, bias, 8, "full size")


def test_router_rejects_bad_arguments():
    L = nvq.lib()
    import ctypes as C
    x = torch.zeros(4096, device="cuda")
    p = C.c_void_p(x.data_ptr())
    assert L.moe_router_sigmoid_topk(p, 4, 8, p, 9, p, p, None) == -2        # k > E
    assert L.moe_router_sigmoid_topk(p, 4, 2048, p, 8, p, p, None) == -2     # E > 1024
    assert L.moe_router_sigmoid_topk(p, 4, 128, p, 65, p, p, None) == -2     # k > 64
    assert L.moe_router_sigmoid_topk(None, 4, 8, p, 2, p, p, None) == -1
