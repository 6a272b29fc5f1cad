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


# ---------------------------------------------------------------- softmax router (the configs' reading)
from precision_moe_numerics_amd import synth


def _ulp32(v):
    return np.spacing(np.abs(np.asarray(v, np.float32))).astype(np.float64)


def _check_softmax(logits, bias, k, what):
    ids, w = nvq.moe_router_softmax_topk(to_dev(logits), None if bias is None else to_dev(bias), k)
    ids_o, w_o = oracle.router_softmax_topk(logits, bias, k)
    assert np.array_equal(host(ids), ids_o), f"{what}: ids differ"
    err = np.abs(host(w).astype(np.float64) - w_o)
    assert np.all(err <= _ulp32(w_o)), f"{what}: weights beyond 1 fp32 ulp, max {(err / _ulp32(w_o)).max():.2f}"


@pytest.mark.parametrize("T,E,k,bias_std", [(256, 8, 2, None), (333, 384, 8, 1.0), (100, 100, 5, 0.3),
                                            (50, 1024, 8, 1.0), (64, 300, 20, 1.0), (17, 64, 64, 0.5),
                                            (9, 513, 16, 0.0), (7, 33, 1, 2.0), (1, 16, 16, None)])
def test_softmax_router(T, E, k, bias_std):
    """Both lane-group sizes (16 lanes per token for k <= 16 and E <= 512, 64
    otherwise), ragged expert counts, k = E, k = 1, no bias and a zero bias."""
    g = np.random.default_rng(500 + T + E)
    logits = g.standard_normal((T, E)).astype(np.float32)
    bias = None if bias_std is None else (bias_std * g.standard_normal(E)).astype(np.float32)
    _check_softmax(logits, bias, k, f"T={T} E={E} k={k}")


def test_softmax_router_ties_and_signed_zero():
    """Equal keys pick the lower index; -0 and +0 are equal keys."""
    logits = np.zeros((6, 70), np.float32)
    logits[:, 1::2] = -0.0
    ids, w = nvq.moe_router_softmax_topk(to_dev(logits), None, 5)
    assert np.array_equal(host(ids), np.tile(np.arange(5, dtype=np.int32), (6, 1)))
    assert np.all(host(w) == np.float32(0.2))


def test_softmax_router_tiny_moe_ids():
    """The tiny_moe draw (256 tokens, 8 experts, top-2, no bias): the GPU's ids
    are the input generator's."""
    c = synth.tiny_moe()
    ids, w = nvq.moe_router_softmax_topk(to_dev(c["logits"]), None, c["k"])
    assert np.array_equal(host(ids), c["topk_ids"])
    _check_softmax(c["logits"], None, c["k"], "tiny_moe")


def test_softmax_router_moe_layer_full_size_and_route():
    """The moe_layer router (16384 tokens, 384 experts, top-8, per-expert bias
    N(0,1)) with the routing sort in the same call: ids bit-identical to the
    oracle and to the input generator's routing, weights within 1 fp32 ulp,
    offsets and sorted2assign equal to the oracle's routing of those ids."""
    logits, bias = synth.moe_layer_router_inputs()
    ids, w, (offs, s2a, tiles) = nvq.moe_router_softmax_topk(to_dev(logits), to_dev(bias), 8, route=True)
    ids_o, w_o = oracle.router_softmax_topk(logits, bias, 8)
    assert np.array_equal(host(ids), ids_o)
    assert np.array_equal(host(ids), synth.moe_layer_routing()[0])
    err = np.abs(host(w).astype(np.float64) - w_o)
    assert np.all(err <= _ulp32(w_o))
    o_offs, o_s2a = oracle.route(ids_o, 384)
    assert np.array_equal(host(offs), o_offs)
    assert np.array_equal(host(s2a), o_s2a)
    n = np.diff(o_offs)
    assert np.array_equal(host(tiles), np.concatenate([[0], np.cumsum((n + 255) // 256)]).astype(np.int32))
    print(f"moe_layer routing: hottest expert {n.max()} rows, mean {n.mean():.0f}, {int((n == 0).sum())} empty")


def test_softmax_router_rejects_bad_arguments():
    L = nvq.lib()
    import ctypes as C
    x = torch.zeros(1 << 16, device="cuda")
    p = C.c_void_p(x.data_ptr())
    assert L.moe_router_softmax_topk(p, 4, 8, p, 9, p, p, None, None, None, None, 0, None) == -2     # k > E
    assert L.moe_router_softmax_topk(p, 4, 2048, p, 8, p, p, None, None, None, None, 0, None) == -2  # E > 1024
    assert L.moe_router_softmax_topk(p, 4, 128, p, 65, p, p, None, None, None, None, 0, None) == -2  # k > 64
    assert L.moe_router_softmax_topk(None, 4, 8, p, 2, p, p, None, None, None, None, 0, None) == -1
    assert L.moe_router_softmax_topk(p, 4, 8, p, 2, p, p, p, None, None, p, 1 << 16, None) == -1     # no s2a
    assert L.moe_router_softmax_topk(p, 4, 8, p, 2, p, p, p, p, None, p, 4, None) == -3              # ws small
