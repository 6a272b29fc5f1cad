"""The routed NVFP4 expert forward (softmax top-k router + fused expert call)
captured once in a HIP graph and replayed: every replay must equal, byte for
byte, the eager calls on the same inputs.

The entry points enqueue only kernels on the caller's stream (zeroing is a
fill kernel, never a memset node) and allocate nothing once the caller passes
its outputs and workspace, so the sequence is capturable. The replays run on
alternating input sets copied into the captured buffers, with the outputs
cleared and eager work and a synchronisation between replays, so a replay
that reused stale results or skipped a node shows up as a mismatch."""
import numpy as np
import pytest
import torch

import precision_moe_numerics_amd as nvq
from precision_moe_numerics_amd import synth
from gpu_util import host, require_gpu, to_dev, to_dev_u16

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _gpu():
    require_gpu()


def _eager(logits, x, k, w1q, w2q, E):
    T, d = x.shape
    d_ff = w2q[0].shape[-1] * 2
    ids = torch.empty((T, k), dtype=torch.int32, device=x.device)
    w = torch.empty((T, k), dtype=torch.float32, device=x.device)
    nvq.moe_router_softmax_topk(logits, None, k, ids=ids, w=w)
    ws = torch.empty(nvq.moe_expert_fwd_workspace_bytes(T, d, k, E, d_ff), dtype=torch.uint8, device=x.device)
    y = nvq.moe_expert_fwd_nvfp4(x, ids, w1q, w2q, ws=ws)
    torch.cuda.synchronize()
    return host(ids), host(w), host(y)


def test_router_and_expert_forward_graph_replays_match_eager():
    c0, c1 = synth.tiny_moe(seed=0), synth.tiny_moe(seed=1)
    T, d, E, k, d_ff = c0["T"], c0["d"], c0["E"], c0["k"], c0["d_ff"]
    print(f"[graph] tiny MoE T={T} d={d} E={E} k={k} d_ff={d_ff}", flush=True)
    w1q = nvq.nvfp4_quantize(to_dev_u16(c0["w1"]), batched=True)
    w2q = nvq.nvfp4_quantize(to_dev_u16(c0["w2"]), batched=True)
    inputs = [(to_dev(c["logits"]), to_dev_u16(c["x"])) for c in (c0, c1)]
    expect = [_eager(lg, xx, k, w1q, w2q, E) for lg, xx in inputs]
    assert not np.array_equal(expect[0][2], expect[1][2])

    dev = inputs[0][1].device
    logits = torch.empty_like(inputs[0][0])
    x = torch.empty_like(inputs[0][1])
    ids = torch.empty((T, k), dtype=torch.int32, device=dev)
    w = torch.empty((T, k), dtype=torch.float32, device=dev)
    y = torch.empty((T, k, d), dtype=torch.bfloat16, device=dev)
    ws = torch.empty(nvq.moe_expert_fwd_workspace_bytes(T, d, k, E, d_ff), dtype=torch.uint8, device=dev)

    def step():
        nvq.moe_router_softmax_topk(logits, None, k, ids=ids, w=w)
        nvq.moe_expert_fwd_nvfp4(x, ids, w1q, w2q, y=y, ws=ws)

    logits.copy_(inputs[0][0])
    x.copy_(inputs[0][1])
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    torch.cuda.synchronize()

    for r, sel in enumerate((1, 0, 1, 1, 0)):
        logits.copy_(inputs[sel][0])
        x.copy_(inputs[sel][1])
        ids.fill_(-1)
        w.zero_()
        y.zero_()
        ws.zero_()
        # eager work of the program between replays
        other = _eager(inputs[1 - sel][0], inputs[1 - sel][1], k, w1q, w2q, E)
        assert np.array_equal(other[2], expect[1 - sel][2])
        g.replay()
        torch.cuda.synchronize()
        print(f"[graph] replay {r} on input set {sel}", flush=True)
        e_ids, e_w, e_y = expect[sel]
        assert np.array_equal(host(ids), e_ids), f"replay {r}: ids"
        assert np.array_equal(host(w).view(np.uint32), e_w.view(np.uint32)), f"replay {r}: weights"
        assert np.array_equal(host(y), e_y), f"replay {r}: y"
