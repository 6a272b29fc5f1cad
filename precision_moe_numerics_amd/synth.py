"""Seeded synthetic inputs for the five workloads of the NVFP4 MoE expert path.

This module draws random tensors and nothing else: it holds none of the
quantization, GEMM or transform arithmetic. Both the CPU oracle (in the tests)
and the GPU path are fed from here.

Workloads (sizes as the harness names them):
  tiny_moe        T=256 d=256 E=8 k=2 d_ff=512, logits N(0,1), X N(0,1), W N(0,0.02)
  quant_8192      8192x8192, 0.1 * Student-t(3), 0.1% of elements x100
  moe_layer       T=16384 d=4096 E=384 k=8 d_ff=1024, logits N(0,1) + bias_e N(0,1)
  mxfp8_bwd       dY N(0, 1e-3) [T*k, d] over moe_layer's routing
  combine_rht     Y N(0,1) [131072, 4096], 1% of rows x20, weights from moe_layer's routing
Top-k of 384 experts per token follows the page "AI模型库 · 今日一模 Inkling 2 Small"
(10100.com), "01 PART" (8 of 384). Router: top-k by logit + bias, ties to the
lower expert id; weights = softmax over the k selected raw logits in fp64, then
fp32.

Small tensors are drawn with numpy on the host: Generator(PCG64(SeedSequence(
[seed, workload_id, tensor_id]))), fp64 draws rounded to bf16 by torch. Tensors
too large to draw on the host in seconds (the moe_layer weights and the
backward/combine activations) are drawn on the device with torch's seeded
generator.
"""
import numpy as np
import torch

WORKLOADS = {
    "tiny_moe": dict(id=1, T=256, d=256, E=8, k=2, d_ff=512),
    "quant_8192": dict(id=2, R=8192, C=8192),
    "moe_layer": dict(id=3, T=16384, d=4096, E=384, k=8, d_ff=1024),
    "mxfp8_bwd": dict(id=4, T=16384, d=4096, E=384, k=8, d_ff=1024),
    "combine_rht": dict(id=5, R=131072, C=4096, T=16384, k=8),
}


def rng(workload_id, tensor_id, seed=0):
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, workload_id, tensor_id])))


def to_bf16_bits(a):
    """fp64/fp32 numpy array -> bf16 bit patterns (uint16), rounded by torch."""
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def bf16_bits_to_tensor(bits, device="cpu"):
    t = torch.from_numpy(np.ascontiguousarray(bits, dtype=np.uint16).view(np.int16))
    return t.view(torch.bfloat16).to(device)


def normal_bf16(shape, std, workload_id, tensor_id, seed=0):
    return to_bf16_bits(rng(workload_id, tensor_id, seed).standard_normal(shape) * std)


def router(logits, k, bias=None):
    """Top-k by logit (+ bias) in fp64 from fp32 inputs, ties to the lower id;
    softmax over the selected raw logits (fp64) -> fp32 weights.
    Returns (topk_ids int32 [T,k], w fp32 [T,k])."""
    logits = np.asarray(logits, dtype=np.float32)
    score = logits.astype(np.float64)
    if bias is not None:
        score = score + np.asarray(bias, dtype=np.float32).astype(np.float64)[None, :]
    # stable argsort on -score keeps the lower id first among equal scores
    order = np.argsort(-score, axis=1, kind="stable")[:, :k]
    sel = np.take_along_axis(logits, order, axis=1).astype(np.float64)
    sel = sel - sel.max(axis=1, keepdims=True)
    w = np.exp(sel)
    w = w / w.sum(axis=1, keepdims=True)
    return order.astype(np.int32), w.astype(np.float32)


def logits_f32(workload_id, tensor_id, shape, seed=0):
    """Router logits N(0,1), drawn in fp64 and rounded to fp32 (the router's input type)."""
    return rng(workload_id, tensor_id, seed).standard_normal(shape).astype(np.float32)


def tiny_moe(seed=0):
    c = WORKLOADS["tiny_moe"]
    T, d, E, k, d_ff, wid = c["T"], c["d"], c["E"], c["k"], c["d_ff"], c["id"]
    logits = logits_f32(wid, 0, (T, E), seed)
    topk_ids, w = router(logits, k)
    return dict(logits=logits,
        x=normal_bf16((T, d), 1.0, wid, 1, seed),
        w1=normal_bf16((E, 2 * d_ff, d), 0.02, wid, 2, seed),
        w2=normal_bf16((E, d, d_ff), 0.02, wid, 3, seed),
        topk_ids=topk_ids, weights=w, T=T, d=d, E=E, k=k, d_ff=d_ff)


def moe_shapes(T, d, E, k, d_ff, seed=0, wid=90, skew=False, x_std=1.0, w_std=0.02):
    """A MoE case of any size drawn on the host (for parity cases)."""
    logits = logits_f32(wid, 0, (T, E), seed)
    bias = logits_f32(wid, 4, E, seed) if skew else None
    topk_ids, w = router(logits, k, bias)
    return dict(
        x=normal_bf16((T, d), x_std, wid, 1, seed),
        w1=normal_bf16((E, 2 * d_ff, d), w_std, wid, 2, seed),
        w2=normal_bf16((E, d, d_ff), w_std, wid, 3, seed),
        topk_ids=topk_ids, weights=w, T=T, d=d, E=E, k=k, d_ff=d_ff)


def student_t_outliers(R, C, workload_id=2, seed=0):
    """0.1 * Student-t(3) with a random 0.1% of elements scaled by 100."""
    g = rng(workload_id, 0, seed)
    x = 0.1 * g.standard_t(3, size=(R, C))
    n_out = int(round(0.001 * R * C))
    idx = g.choice(R * C, size=n_out, replace=False)
    x.reshape(-1)[idx] *= 100.0
    return to_bf16_bits(x)


def moe_layer_router_inputs(seed=0):
    """Router inputs of the moe_layer workload: logits N(0,1) [T, E] and a
    per-expert bias N(0,1) [E] (skewed load), both fp32."""
    c = WORKLOADS["moe_layer"]
    return logits_f32(c["id"], 0, (c["T"], c["E"]), seed), logits_f32(c["id"], 4, c["E"], seed)


def moe_layer_routing(seed=0):
    """Skewed routing of the moe_layer workload: logits N(0,1) + bias_e N(0,1)."""
    logits, bias = moe_layer_router_inputs(seed)
    return router(logits, WORKLOADS["moe_layer"]["k"], bias)


def device_normal_bf16(shape, std, tensor_id, device, seed=0, workload_id=3):
    """Large normal tensors drawn on the device by torch's seeded generator."""
    gen = torch.Generator(device=device)
    gen.manual_seed(int(np.random.SeedSequence([seed, workload_id, tensor_id]).generate_state(1)[0]))
    t = torch.empty(shape, dtype=torch.float32, device=device)
    t.normal_(0.0, std, generator=gen)
    return t.to(torch.bfloat16)


def rows_scaled(x_bf16, frac, factor, tensor_id, seed=0, workload_id=5):
    """Scale a random `frac` of the rows of a device bf16 tensor by `factor` (in place)."""
    R = x_bf16.shape[0]
    n = int(round(frac * R))
    idx = rng(workload_id, tensor_id, seed).choice(R, size=n, replace=False)
    ii = torch.from_numpy(np.sort(idx)).to(x_bf16.device)
    x_bf16[ii] = (x_bf16[ii].float() * factor).to(torch.bfloat16)
    return x_bf16
