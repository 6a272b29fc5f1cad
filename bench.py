"""Benchmark of the NVFP4 MoE expert path on one MI355X.

One step is one NVFP4 forward through an MoE expert layer of the moe_layer
workload (T=16384 tokens, d=4096, 384 experts, top-8, SwiGLU d_ff=1024):
router (top-8 of logit + bias, softmax weights) -> quantize X -> route ->
fc1 + SwiGLU -> re-quantize H -> fc2. Weights are
quantized to NVFP4 once before the timed region (timed separately below).
`value` is the step's algorithmic TFLOP/s (2*A*(2*d_ff)*d + 2*A*d*d_ff,
A = T*k). The JSON line also carries the dominant kernel's roofline, the CPU
oracle's rate on a bounded sample, and the companion measurements (quantize
GB/s on the 8192x8192 workload, weight quantization, the RHT combine, the
MXFP8 backward, and the same forward with MXFP8 operands for comparison).

    python bench.py [--steps K] [--warmup W] [--no-cpu-baseline]
"""
import argparse
import json
import os
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import precision_moe_numerics_amd as nvq  # noqa: E402
from precision_moe_numerics_amd import synth  # noqa: E402

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
MFMA_F16_PEAK_TFLOPS = 2500.0  # MI355X dense fp16/bf16 MFMA
MFMA_F8_PEAK_TFLOPS = 5000.0   # MI355X dense fp8 MFMA
CALIB_BYTES = 1 << 30          # plain copy used to scale the HBM byte counters
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "fc1_gemm_traffic.md")
TRAFFIC_SOURCES = ("precision_moe_numerics_amd/csrc/nvq_moe.hip", "precision_moe_numerics_amd/csrc/nvq_device.hpp")
# HBM bytes of the streaming legs (quantize, dequantize, RHT, combine, MXFP8 requant)
STREAM_TRAFFIC_FILE = os.path.join(ROOT, "profiles", "streaming_kernels_hbm_traffic.md")
STREAM_SOURCES = ("precision_moe_numerics_amd/csrc/nvq_quant.hip", "precision_moe_numerics_amd/csrc/nvq_rht.hip",
                  "precision_moe_numerics_amd/csrc/nvq_mxfp8.hip", "precision_moe_numerics_amd/csrc/nvq_device.hpp")


def log(msg):
    print(msg, file=sys.stderr, flush=True)


class Timer:
    """HIP events on torch's current stream (the stream libnvq launches on)."""

    def __init__(self):
        self.a = torch.cuda.Event(enable_timing=True)
        self.b = torch.cuda.Event(enable_timing=True)

    def start(self):
        self.a.record()

    def stop_ms(self):
        self.b.record()
        self.b.synchronize()
        return self.a.elapsed_time(self.b)


def kernel_source_digest(sources=TRAFFIC_SOURCES):
    """Digest of kernel code with comments and whitespace removed (so a
    comment edit keeps the counters; any code change invalidates them)."""
    import hashlib
    import re
    h = hashlib.sha256()
    for rel in sources:
        with open(os.path.join(ROOT, rel)) as f:
            src = f.read()
        src = re.sub(r"/\*.*?\*/", " ", src, flags=re.S)
        src = re.sub(r"//[^\n]*", " ", src)
        h.update(" ".join(src.split()).encode())
    return h.hexdigest()[:16]


def counted_traffic():
    """HBM bytes per fc1 launch from the committed counter summary (FETCH_SIZE +
    WRITE_SIZE, each scaled by the same counter on a plain copy of known size),
    or None when the summary is missing or the GEMM source changed since."""
    try:
        fields = {}
        with open(TRAFFIC_FILE) as f:
            for line in f:
                if line.startswith("- ") and ": " in line:
                    k, v = line[2:].split(": ", 1)
                    fields[k.strip()] = v.strip().strip("`")
        if fields.get("source_digest") != kernel_source_digest():
            return None
        return int(fields["traffic_bytes_per_launch"])
    except (OSError, KeyError, ValueError):
        return None


def counted_leg_bytes():
    """HBM bytes (FETCH_SIZE + WRITE_SIZE, copy-calibrated) of each streaming
    bench leg from the committed counter summary, {} when it is missing or
    the kernels' source changed since it was taken."""
    try:
        fields = {}
        with open(STREAM_TRAFFIC_FILE) as f:
            for line in f:
                if line.startswith("- ") and ": " in line:
                    k, v = line[2:].split(": ", 1)
                    fields[k.strip()] = v.strip().strip("`")
        if fields.get("source_digest") != kernel_source_digest(STREAM_SOURCES):
            return {}
        return {k[4:]: int(v) for k, v in fields.items() if k.startswith("leg.")}
    except (OSError, ValueError):
        return {}


def counter_rates(leg_ms):
    """Counter bytes of each leg divided by its time measured in this run."""
    out = {}
    for leg, nbytes in counted_leg_bytes().items():
        ms = leg_ms.get(leg)
        if ms:
            gbps = nbytes / ms / 1e6
            out[leg] = dict(bytes=nbytes, ms=round(ms, 4), gbps=round(gbps, 1), frac_hbm=round(gbps / HBM_PEAK_GBS, 4))
    return out


def calibration_copy(dev, reps=5):
    """A plain elementwise copy of CALIB_BYTES (read once, written once): the
    counter runs read FETCH_SIZE / WRITE_SIZE of its first dispatch to scale
    the kernels' counts to bytes. Its median rate over `reps` further runs is
    the HBM rate a plain vendor elementwise kernel reaches here (context for
    the streaming kernels' fractions of the published peak)."""
    src = torch.ones(CALIB_BYTES // 4, dtype=torch.int32, device=dev)
    dst = torch.empty_like(src)
    torch.neg(src, out=dst)
    torch.cuda.synchronize()
    tm = Timer()
    ts = []
    for _ in range(reps):
        tm.start()
        torch.neg(src, out=dst)
        ts.append(tm.stop_ms())
    del src, dst
    return 2 * CALIB_BYTES / float(np.median(ts)) / 1e6


def vendor_fp16_gemm(dev, M, N, K, reps=5):
    """torch.matmul (hipBLASLt) on dense fp16 operands of fc1's shape: the MFMA
    rate the vendor library reaches here on random data (context for the
    grouped GEMM's fraction of the published peak; not a parity reference)."""
    g = torch.Generator(device=dev)
    g.manual_seed(7)
    a = torch.randn((M, K), generator=g, device=dev, dtype=torch.float16)
    b = torch.randn((K, N), generator=g, device=dev, dtype=torch.float16)
    c = a @ b
    torch.cuda.synchronize()
    tm = Timer()
    ts = []
    for _ in range(reps):
        tm.start()
        torch.matmul(a, b, out=c)
        ts.append(tm.stop_ms())
    del a, b, c
    return 2.0 * M * N * K / float(np.median(ts)) / 1e9


def vendor_mxfp8_gemm(dev, M, N, K, reps=5):
    """torch._scaled_mm (hipBLASLt) on dense MXFP8 operands (E4M3 elements, one
    E8M0 scale per 32 along K, bf16 out) of a dgrad GEMM's shape: the rate the
    vendor library reaches here for the format the grouped MXFP8 GEMMs
    contract (context; not a parity reference). None where this torch build
    has no block-scaled path."""
    try:
        g = torch.Generator(device=dev)
        g.manual_seed(8)
        a = torch.randn((M, K), generator=g, device=dev).to(torch.float8_e4m3fn)
        b = torch.randn((N, K), generator=g, device=dev).to(torch.float8_e4m3fn)
        sa = torch.full((M, K // 32), 127, dtype=torch.uint8, device=dev).view(torch.float8_e8m0fnu)
        sb = torch.full((N, K // 32), 127, dtype=torch.uint8, device=dev).view(torch.float8_e8m0fnu)
        run = lambda: torch._scaled_mm(a, b.t(), scale_a=sa, scale_b=sb, out_dtype=torch.bfloat16)
        run()
        torch.cuda.synchronize()
        tm = Timer()
        ts = []
        for _ in range(reps):
            tm.start()
            run()
            ts.append(tm.stop_ms())
        del a, b, sa, sb
        return round(2.0 * M * N * K / float(np.median(ts)) / 1e9, 1)
    except (RuntimeError, AttributeError, TypeError) as e:
        log(f"[bench] vendor MXFP8 GEMM unavailable: {e}")
        return None


def flush_mall(buf):
    # A 512 MiB read evicts the 256 MB Infinity Cache and, unlike a write,
    # leaves no dirty lines whose write-back would be billed to the next kernel.
    buf.max()


def moe_layer_inputs(dev):
    """X, and the router inputs (fp32 logits N(0,1) [T, E], per-expert bias N(0,1)
    [E]); the ids come from the library's router, checked once against the
    input generator's routing (bit-identical)."""
    c = synth.WORKLOADS["moe_layer"]
    T, d, E, k, d_ff = c["T"], c["d"], c["E"], c["k"], c["d_ff"]
    logits, bias = synth.moe_layer_router_inputs()
    logits_d, bias_d = torch.from_numpy(logits).to(dev), torch.from_numpy(bias).to(dev)
    ids, weights = nvq.moe_router_softmax_topk(logits_d, bias_d, k)
    ids_ref, _ = synth.moe_layer_routing()
    if not np.array_equal(ids.cpu().numpy(), ids_ref):
        raise RuntimeError("the library router's ids differ from the input generator's routing")
    x = synth.device_normal_bf16((T, d), 1.0, 1, dev)
    return dict(T=T, d=d, E=E, k=k, d_ff=d_ff, ids=ids, weights=weights.cpu().numpy(), x=x, ids_np=ids_ref,
                logits=logits_d, bias=bias_d, rweights=weights)


def bench_weight_quant(dev, E, d, d_ff, flush):
    """Quantize W1 [E, 2 d_ff, d] and W2 [E, d, d_ff] (one scale per expert matrix)."""
    w1 = synth.device_normal_bf16((E, 2 * d_ff, d), 0.02, 2, dev)
    w2 = synth.device_normal_bf16((E, d, d_ff), 0.02, 3, dev)
    tm = Timer()
    w1q = nvq.nvfp4_quantize(w1, batched=True)  # warm-up
    w2q = nvq.nvfp4_quantize(w2, batched=True)
    torch.cuda.synchronize()
    flush_mall(flush)
    tm.start()
    w1q = nvq.nvfp4_quantize(w1, batched=True)
    w2q = nvq.nvfp4_quantize(w2, batched=True)
    ms = tm.stop_ms()
    n = w1.numel() + w2.numel()
    # algorithmic bytes of the two-pass quantizer: read 2 B (amax) + read 2 B,
    # write 0.5 + 1/16 B (encode) per value
    return w1q, w2q, (w1, w2), dict(ms=ms, gbps=n * (2 + 2 + 0.5625) / ms / 1e6, values=n)


def bench_quant_8192(dev, flush, reps=10):
    x = synth.bf16_bits_to_tensor(synth.student_t_outliers(8192, 8192), dev)
    n = x.numel()
    ws = torch.empty(nvq.lib().nvfp4_quantize_workspace_size(1, 8192, 8192), dtype=torch.uint8, device=dev)
    out = {}
    for mode, name in ((nvq.RTN, "rtn"), (nvq.SR, "sr")):
        nvq.nvfp4_quantize(x, round_mode=mode, ws=ws)
        times = []
        tm = Timer()
        for _ in range(reps):
            flush_mall(flush)
            tm.start()
            q = nvq.nvfp4_quantize(x, round_mode=mode, ws=ws)
            times.append(tm.stop_ms())
        ms = float(np.median(times))
        out[name] = dict(ms=ms, gbps=n * (2 + 2 + 0.5625) / ms / 1e6)
    c, s, t = q
    times = []
    for _ in range(reps):
        flush_mall(flush)
        tm.start()
        nvq.nvfp4_dequantize(c, s, t, torch.bfloat16)
        times.append(tm.stop_ms())
    ms = float(np.median(times))
    out["dequant_bf16"] = dict(ms=ms, gbps=n * (0.5625 + 2) / ms / 1e6)
    return out


def bench_combine_rht(dev, flush, reps=5):
    """Combine workload: Y [131072, 4096] bf16 N(0,1), 1% of rows x20; RHT32 +
    NVFP4 (two passes), then dequantize + inverse RHT + top-8 combine."""
    R, C, T, k = 131072, 4096, 16384, 8
    y = synth.device_normal_bf16((R, C), 1.0, 1, dev, workload_id=5)
    synth.rows_scaled(y, 0.01, 20.0, 2)
    _, w = synth.moe_layer_routing()
    w = torch.from_numpy(w).to(dev)
    ws = torch.empty(4096, dtype=torch.uint8, device=dev)
    q = nvq.rht32_blockquant(y, ws=ws)
    out = nvq.rht32_dequant_combine(q, T, k, w)
    tm = Timer()
    tq, tc = [], []
    for _ in range(reps):
        flush_mall(flush)
        tm.start()
        q = nvq.rht32_blockquant(y, ws=ws)
        tq.append(tm.stop_ms())
        flush_mall(flush)
        tm.start()
        nvq.rht32_dequant_combine(q, T, k, w, out=out)
        tc.append(tm.stop_ms())
    n = R * C
    mq, mc = float(np.median(tq)), float(np.median(tc))
    return dict(quant_ms=round(mq, 4), quant_gbps=round(n * (2 + 2 + 0.5625) / mq / 1e6, 1),
                combine_ms=round(mc, 4), combine_gbps=round((n * 0.5625 + T * k * 4 + T * C * 2) / mc / 1e6, 1))


def bench_mxfp8_bwd(dev, inp, it, wbf16, flush, reps=3):
    """MXFP8 backward of the moe_layer workload: requantize dY (both axes, SR),
    the weights (transposed axis), H and the gathered X (transposed axis, RTN),
    dA (both axes, SR); dgrad fc2, SwiGLU backward, dgrad fc1, wgrad fc2,
    wgrad fc1 on the E8M0-scaled FP8 MFMA."""
    T, d, E, k, d_ff = inp["T"], inp["d"], inp["E"], inp["k"], inp["d_ff"]
    A = T * k
    w1, w2 = wbf16
    offs, s2a = it["offsets"], it["sorted2assign"]
    dy = synth.device_normal_bf16((A, d), 1e-3, 1, dev, workload_id=4)
    ws = torch.empty(1 << 20, dtype=torch.uint8, device=dev)
    e_w1 = torch.arange(E + 1, dtype=torch.int32, device=dev) * (2 * d_ff)
    e_w2 = torch.arange(E + 1, dtype=torch.int32, device=dev) * d
    w1v, w2v = w1.view(E * 2 * d_ff, d), w2.view(E * d, d_ff)
    outs = {}

    def step():
        t = {}
        ev = []

        def mark(name):
            e = torch.cuda.Event(enable_timing=True)
            e.record()
            ev.append((name, e))
        mark("start")
        dy0 = nvq.mxfp8_requant_sr(dy, 0, nvq.SR, seed=0, stream_id=2, row_gather=s2a, ws=ws)
        dy1 = nvq.mxfp8_requant_sr(dy, 1, nvq.SR, seed=0, stream_id=3, row_gather=s2a, seg_offsets=offs, ws=ws)
        w2t = nvq.mxfp8_requant_sr(w2v, 1, nvq.RTN, seg_offsets=e_w2, ws=ws)
        w1t = nvq.mxfp8_requant_sr(w1v, 1, nvq.RTN, seg_offsets=e_w1, ws=ws)
        h1 = nvq.mxfp8_requant_sr(it["h"], 1, nvq.RTN, seg_offsets=offs, ws=ws)
        x1 = nvq.mxfp8_requant_sr(inp["x"], 1, nvq.RTN, row_gather=s2a, gather_div=k, seg_offsets=offs, ws=ws)
        mark("requant_in")
        dH = nvq.moe_grouped_gemm_mxfp8(nvq.DGRAD, dy0, w2t, offs, N=d_ff, K=d, ws=ws)
        mark("dgrad_fc2")
        dA = nvq.swiglu_bwd(dH, it["gu"])
        mark("swiglu_bwd")
        da0 = nvq.mxfp8_requant_sr(dA, 0, nvq.SR, seed=0, stream_id=2, ws=ws)
        da1 = nvq.mxfp8_requant_sr(dA, 1, nvq.SR, seed=0, stream_id=3, seg_offsets=offs, ws=ws)
        mark("requant_dA")
        dX = nvq.moe_grouped_gemm_mxfp8(nvq.DGRAD, da0, w1t, offs, N=d, K=2 * d_ff, ws=ws)
        mark("dgrad_fc1")
        dW2 = nvq.moe_grouped_gemm_mxfp8(nvq.WGRAD, dy1, h1, offs, M=d, N=d_ff, ws=ws)
        mark("wgrad_fc2")
        dW1 = nvq.moe_grouped_gemm_mxfp8(nvq.WGRAD, da1, x1, offs, M=2 * d_ff, N=d, ws=ws)
        mark("wgrad_fc1")
        torch.cuda.synchronize()
        for (n0, e0), (n1, e1) in zip(ev[:-1], ev[1:]):
            t[n1] = e0.elapsed_time(e1)
        t["total"] = ev[0][1].elapsed_time(ev[-1][1])
        return t
    step()
    runs = []
    for _ in range(reps):
        flush_mall(flush)
        runs.append(step())
    med = {key: float(np.median([r[key] for r in runs])) for key in runs[0]}
    flop = {"dgrad_fc2": 2.0 * A * d * d_ff, "dgrad_fc1": 2.0 * A * 2 * d_ff * d,
            "wgrad_fc2": 2.0 * A * d * d_ff, "wgrad_fc1": 2.0 * A * 2 * d_ff * d}
    gemm_ms = sum(med[kk] for kk in flop)
    req_vals = 2 * A * d + E * 2 * d_ff * d + E * d * d_ff + A * d_ff + A * d + 2 * A * 2 * d_ff
    res = {kk: round(v, 4) for kk, v in med.items()}
    res.update({f"{kk}_tflops": round(flop[kk] / med[kk] / 1e9, 1) for kk in flop})
    res["gemm_tflops"] = round(sum(flop.values()) / gemm_ms / 1e9, 1)
    res["gemm_frac_fp8_peak"] = round(sum(flop.values()) / gemm_ms / 1e9 / MFMA_F8_PEAK_TFLOPS, 4)
    req_ms = med["requant_in"] + med["requant_dA"]
    res["requant_gbps"] = round(req_vals * (2 + 1 + 1 / 32) / req_ms / 1e6, 1)
    return res


def bench_nvfp4_bwd(dev, inp, it, wbf16, flush, reps=3):
    """The same backward with NVFP4 operands: dY and dA quantized along their
    rows with stochastic rounding for dgrad, the weights transposed (one
    scale per expert, nearest even), and for wgrad dY, dA (stochastic), H and
    the gathered X (nearest even) transposed into expert token segments
    through the token-axis RHT32; GEMMs on exactly dequantized fp16 operands."""
    T, d, E, k, d_ff = inp["T"], inp["d"], inp["E"], inp["k"], inp["d_ff"]
    A = T * k
    w1, w2 = wbf16
    offs, s2a = it["offsets"], it["sorted2assign"]
    dy = synth.device_normal_bf16((A, d), 1e-3, 1, dev, workload_id=4)
    ws = torch.empty(1 << 20, dtype=torch.uint8, device=dev)
    w1v, w2v = w1.view(E * 2 * d_ff, d), w2.view(E * d, d_ff)

    def step():
        ev = []

        def mark(name):
            e = torch.cuda.Event(enable_timing=True)
            e.record()
            ev.append((name, e))
        mark("start")
        dy0 = nvq.nvfp4_quantize(dy, round_mode=nvq.SR, stream_id=1, ws=ws)
        dyT = nvq.nvfp4_quantize_axis1(dy, round_mode=nvq.SR, stream_id=3, row_gather=s2a, seg_offsets=offs,
                                       rht=True, ws=ws)
        w2t = nvq.nvfp4_quantize_axis1(w2v, nseg=E, per_segment=True, ws=ws)
        w1t = nvq.nvfp4_quantize_axis1(w1v, nseg=E, per_segment=True, ws=ws)
        hT = nvq.nvfp4_quantize_axis1(it["h"], seg_offsets=offs, rht=True, ws=ws)
        xT = nvq.nvfp4_quantize_axis1(inp["x"], row_gather=s2a, gather_div=k, seg_offsets=offs, rht=True, ws=ws)
        mark("requant_in")
        dH = nvq.moe_grouped_gemm_nvfp4_bwd(nvq.DGRAD, dy0, w2t, offs, M=A, N=d_ff, K=d, a_gather=s2a, ws=ws)
        mark("dgrad_fc2")
        dA = nvq.swiglu_bwd(dH, it["gu"])
        mark("swiglu_bwd")
        da0 = nvq.nvfp4_quantize(dA, round_mode=nvq.SR, stream_id=1, ws=ws)
        daT = nvq.nvfp4_quantize_axis1(dA, round_mode=nvq.SR, stream_id=3, seg_offsets=offs, rht=True, ws=ws)
        mark("requant_dA")
        dX = nvq.moe_grouped_gemm_nvfp4_bwd(nvq.DGRAD, da0, w1t, offs, M=A, N=d, K=2 * d_ff, ws=ws)
        mark("dgrad_fc1")
        dW2 = nvq.moe_grouped_gemm_nvfp4_bwd(nvq.WGRAD, dyT, hT, offs, M=d, N=d_ff, K=A, ws=ws)
        mark("wgrad_fc2")
        dW1 = nvq.moe_grouped_gemm_nvfp4_bwd(nvq.WGRAD, daT, xT, offs, M=2 * d_ff, N=d, K=A, ws=ws)
        mark("wgrad_fc1")
        torch.cuda.synchronize()
        t = {n1: e0.elapsed_time(e1) for (n0, e0), (n1, e1) in zip(ev[:-1], ev[1:])}
        t["total"] = ev[0][1].elapsed_time(ev[-1][1])
        del dX, dW1, dW2
        return t
    step()
    runs = []
    for _ in range(reps):
        flush_mall(flush)
        runs.append(step())
    med = {key: float(np.median([r[key] for r in runs])) for key in runs[0]}
    flop = {"dgrad_fc2": 2.0 * A * d * d_ff, "dgrad_fc1": 2.0 * A * 2 * d_ff * d,
            "wgrad_fc2": 2.0 * A * d * d_ff, "wgrad_fc1": 2.0 * A * 2 * d_ff * d}
    gemm_ms = sum(med[kk] for kk in flop)
    res = {kk: round(v, 4) for kk, v in med.items()}
    res.update({f"{kk}_tflops": round(flop[kk] / med[kk] / 1e9, 1) for kk in flop})
    res["gemm_tflops"] = round(sum(flop.values()) / gemm_ms / 1e9, 1)
    res["gemm_frac_fp16_peak"] = round(sum(flop.values()) / gemm_ms / 1e9 / MFMA_F16_PEAK_TFLOPS, 4)
    return res


def bench_mxfp8_fwd(dev, inp, wbf16, steps, warmup, nvfp4_ms):
    """The same expert forward with MXFP8 operands (the precision the NVFP4
    forward is compared against): weights quantized once (axis 0, nearest
    even) outside the timed region; the whole forward timed as the NVFP4 step
    is; its fc1 + SwiGLU alone (exact bf16 operands, bf16 MFMA) against the
    2.5 PF dense bf16 peak; and, for comparison, fc1 on the FP8 matrix pipe
    (E8M0-scaled FP8 MFMA, fp32 out, not exact) against the 5 PF fp8 peak."""
    T, d, E, k, d_ff = inp["T"], inp["d"], inp["E"], inp["k"], inp["d_ff"]
    A = T * k
    w1, w2 = wbf16
    w1m = nvq.mxfp8_requant_sr(w1.view(E * 2 * d_ff, d), 0, nvq.RTN)
    w2m = nvq.mxfp8_requant_sr(w2.view(E * d, d_ff), 0, nvq.RTN)
    y = torch.empty((T, k, d), dtype=torch.bfloat16, device=dev)
    ws = torch.empty(nvq.lib().moe_expert_fwd_mxfp8_workspace_size(T, d, k, E, d_ff), dtype=torch.uint8, device=dev)
    for _ in range(warmup):
        nvq.moe_expert_fwd_mxfp8(inp["x"], inp["ids"], w1m, w2m, y=y, ws=ws)
    torch.cuda.synchronize()
    tm = Timer()
    tm.start()
    for _ in range(steps):
        nvq.moe_expert_fwd_mxfp8(inp["x"], inp["ids"], w1m, w2m, y=y, ws=ws)
    ms = tm.stop_ms() / steps
    flops_fc1 = 2.0 * A * (2 * d_ff) * d
    flops = flops_fc1 + 2.0 * A * d * d_ff
    offs, s2a, _ = nvq.moe_route(inp["ids"], E)
    xq = nvq.mxfp8_requant_sr(inp["x"], 0, nvq.RTN)
    h = torch.empty((A, d_ff), dtype=torch.bfloat16, device=dev)
    gws = torch.empty(1 << 24, dtype=torch.uint8, device=dev)

    def timed(fn):
        for _ in range(2):
            fn()
        torch.cuda.synchronize()
        tm.start()
        for _ in range(steps):
            fn()
        return tm.stop_ms() / steps
    fc1_ms = timed(lambda: nvq.moe_fc1_swiglu_mxfp8(xq, offs, s2a, k, w1m, d_ff, h=h, ws=gws))
    xg = nvq.mxfp8_requant_sr(inp["x"], 0, nvq.RTN, row_gather=s2a, gather_div=k)
    G = torch.empty((A, 2 * d_ff), dtype=torch.float32, device=dev)
    fp8_ms = timed(lambda: nvq.moe_grouped_gemm_mxfp8(nvq.FWD, xg, w1m, offs, N=2 * d_ff, K=d, out=G, ws=gws))
    del w1m, w2m, ws, G, xq, xg, h
    return {"ms_per_step": round(ms, 4), "tflops": round(flops / ms / 1e9, 2),
            "nvfp4_speedup": round(ms / nvfp4_ms, 4),
            "fc1_ms": round(fc1_ms, 4), "fc1_tflops": round(flops_fc1 / fc1_ms / 1e9, 2),
            "fc1_frac_bf16_peak": round(flops_fc1 / fc1_ms / 1e9 / MFMA_F16_PEAK_TFLOPS, 4),
            "fc1_fp8_pipe_ms": round(fp8_ms, 4),
            "fc1_fp8_pipe_frac_fp8_peak": round(flops_fc1 / fp8_ms / 1e9 / MFMA_F8_PEAK_TFLOPS, 4)}


def bench_router(inp, steps):
    """The softmax top-k router at the moe_layer shape with the routing sort in
    the same call, and the sigmoid router (the other model's reading) for
    reference. Bytes: logits and bias read, ids and weights written."""
    T, E, k = inp["T"], inp["E"], inp["k"]
    logits, bias = inp["logits"], inp["bias"]
    ws = torch.empty(nvq.lib().moe_router_softmax_topk_workspace_size(T, E, k), dtype=torch.uint8,
                     device=logits.device)
    res = {}
    for name, fn in (("softmax_topk", lambda: nvq.moe_router_softmax_topk(logits, bias, k)),
                     ("softmax_topk_and_route", lambda: nvq.moe_router_softmax_topk(logits, bias, k, route=True,
                                                                                    ws=ws)),
                     ("sigmoid_topk", lambda: nvq.moe_router_sigmoid_topk(logits, bias, k))):
        for _ in range(3):
            fn()
        torch.cuda.synchronize()
        tm = Timer()
        tm.start()
        for _ in range(steps):
            fn()
        ms = tm.stop_ms() / steps
        nbytes = T * E * 4 + E * 4 + T * k * 8
        res[name] = {"us": round(ms * 1000, 2), "gbps": round(nbytes / ms / 1e6, 1)}
    return res


def _cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def bench_tiny(dev, reps=200):
    """The tiny MoE forward (256 tokens, d_model 256, 8 experts, top-2, d_ff 512):
    the softmax router and the whole NVFP4 expert forward, timed per call over
    `reps` back-to-back calls (latency-bound: a few small launches), both as
    eager calls and as replays of one HIP graph holding the same launches."""
    c = synth.tiny_moe()
    T, d, E, k, d_ff = c["T"], c["d"], c["E"], c["k"], c["d_ff"]

    def bits(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(dev).view(torch.bfloat16)
    w1q = nvq.nvfp4_quantize(bits(c["w1"]), batched=True)
    w2q = nvq.nvfp4_quantize(bits(c["w2"]), batched=True)
    logits, x = torch.from_numpy(c["logits"]).to(dev), bits(c["x"])
    ws = torch.empty(nvq.moe_expert_fwd_workspace_bytes(T, d, k, E, d_ff), dtype=torch.uint8, device=dev)
    y = torch.empty((T, k, d), dtype=torch.bfloat16, device=dev)
    ids = torch.empty((T, k), dtype=torch.int32, device=dev)
    w = torch.empty((T, k), dtype=torch.float32, device=dev)

    def step():
        nvq.moe_router_softmax_topk(logits, None, k, ids=ids, w=w)
        nvq.moe_expert_fwd_nvfp4(x, ids, w1q, w2q, y=y, ws=ws)
    for _ in range(10):
        step()
    torch.cuda.synchronize()
    if not np.array_equal(ids.cpu().numpy(), c["topk_ids"]):
        raise RuntimeError("the library router's ids differ from the input generator's routing (tiny MoE)")
    tm = Timer()
    tm.start()
    for _ in range(reps):
        step()
    ms = tm.stop_ms() / reps
    y_eager = y.clone()
    # the same step captured once in a HIP graph and replayed (the entry points
    # enqueue only kernels and allocate nothing once outputs and workspace are
    # given); the last replay's y must equal the eager result byte for byte
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    y.zero_()
    for _ in range(10):
        g.replay()
    tm.start()
    for _ in range(reps):
        g.replay()
    ms_g = tm.stop_ms() / reps
    if not torch.equal(y.view(torch.int16), y_eager.view(torch.int16)):
        raise RuntimeError("graph replay of the tiny MoE step differs from the eager calls")
    flop = 2.0 * T * k * (2 * d_ff) * d + 2.0 * T * k * d * d_ff
    return {"us": round(ms * 1e3, 2), "tflops": round(flop / ms / 1e9, 3),
            "graph_us": round(ms_g * 1e3, 2), "graph_tflops": round(flop / ms_g / 1e9, 3)}


def _oracle_threads():
    """Host threads for the oracle: the cores this process may use, capped by
    OMP_NUM_THREADS when it is set (the box gives each GPU a share of its CPUs)."""
    n = len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else (os.cpu_count() or 1)
    cap = os.environ.get("OMP_NUM_THREADS")
    return max(1, min(n, int(cap))) if cap and cap.isdigit() else max(1, n)


def _timed_median(fn, threads, reps=3):
    """Median wall time of fn(pool) over reps runs; the oracle's C calls
    release the GIL, so row chunks handed to a thread pool run in parallel."""
    from concurrent.futures import ThreadPoolExecutor
    ts = []
    with ThreadPoolExecutor(max_workers=threads) as pool:
        for _ in range(reps):
            t0 = time.perf_counter()
            fn(pool, threads)
            ts.append(time.perf_counter() - t0)
    return float(np.median(ts))


def _chunks(n, parts):
    b = np.linspace(0, n, parts + 1).astype(np.int64)
    return [(int(b[i]), int(b[i + 1])) for i in range(parts) if b[i + 1] > b[i]]


def cpu_baseline(inp, w1q, w2q, it, w2_e, fc_rows=512, q_rows=512, rht_rows=1024, combine_tokens=128,
                 mx_rows=512):
    """The CPU oracle (plain C) on every configuration, whole (tiny MoE) or on a
    bounded sample, each timed on one core and on all the host cores this
    process may use (row chunks over a thread pool; median of three runs):
      tiny_moe: the whole tiny forward (softmax router, X quantize, routing,
        fc1, SwiGLU, H quantize, fc2);
      moe_layer: fc1 + SwiGLU + fc2 for `fc_rows` expert-sorted rows of the
        most loaded expert (int64-exact GEMMs);
      mxfp8_bwd: SR requantization of `mx_rows` rows of dY N(0, 1e-3) along the
        rows, and dgrad fc2 (dH = dY W2) of those rows against one expert's
        W2 requantized along d (outside the timed region);
      quant_8192: amax + NVFP4 nearest-even encode of `q_rows` rows of the
        8192 x 8192 Student-t tensor (the tensor scale from the sample);
      combine_rht: RHT32 + amax + NVFP4 of `rht_rows` rows of 4096, and the
        dequantize + inverse RHT + top-8 combine of `combine_tokens` tokens."""
    import oracle
    threads = _oracle_threads()
    offs = it["offsets"].cpu().numpy()
    s2a = it["sorted2assign"].cpu().numpy()
    xq = tuple(t.cpu().numpy() for t in (it["xq_codes"], it["xq_scales"])) + (it["xq_tscale"].cpu().numpy()[0],)
    hq = tuple(t.cpu().numpy() for t in (it["hq_codes"], it["hq_scales"])) + (it["hq_tscale"].cpu().numpy()[0],)
    n = np.diff(offs)
    e = int(np.argmax(n))
    rows = np.arange(offs[e], offs[e] + min(fc_rows, n[e]), dtype=np.int32)
    R = len(rows)
    w1 = tuple(t[e:e + 1].cpu().numpy() for t in w1q)
    w2 = tuple(t[e:e + 1].cpu().numpy() for t in w2q)
    local_offs = np.array([0, R], np.int32)
    local_s2a = s2a[rows]
    hq_rows = (hq[0][rows], hq[1][rows], hq[2])
    d, d_ff, k = inp["d"], inp["d_ff"], inp["k"]

    def fc_chain(pool, parts):
        def run(a, b):
            sub = np.arange(a, b, dtype=np.int32)
            oracle.swiglu(oracle.moe_fc1(xq, local_offs, local_s2a, k, w1, rows=sub))
            oracle.moe_fc2(hq_rows, local_offs, w2, rows=sub)
        list(pool.map(lambda ab: run(*ab), _chunks(R, parts)))

    xs = synth.student_t_outliers(8192, 8192)[:q_rows]

    def quant(pool, parts):
        f = oracle.bf16_to_f32(xs)
        ch = _chunks(len(f), parts)
        am = max(pool.map(lambda ab: oracle.amax_f32(f[ab[0]:ab[1]]), ch))
        list(pool.map(lambda ab: oracle.nvfp4_quantize_slice(f[ab[0]:ab[1]], am, ab[0] * f.shape[1]), ch))

    g = np.random.default_rng(5)
    yr = synth.to_bf16_bits(g.standard_normal((rht_rows, 4096)))

    def rht(pool, parts):
        ch = _chunks(rht_rows, parts)
        zs = list(pool.map(lambda ab: oracle.rht32_forward(yr[ab[0]:ab[1]], 0), ch))
        am = max(pool.map(oracle.amax_f32, zs))
        list(pool.map(lambda iz: oracle.nvfp4_quantize_slice(iz[1], am, ch[iz[0]][0] * 4096), enumerate(zs)))

    cq = oracle.nvfp4_quantize(oracle.rht32_forward(yr[:combine_tokens * 8], 0))
    wk = g.random((combine_tokens, 8)).astype(np.float32)

    def combine(pool, parts):
        ch = _chunks(combine_tokens, parts)
        list(pool.map(lambda ab: oracle.rht32_combine(cq[0][ab[0] * 8:ab[1] * 8], cq[1][ab[0] * 8:ab[1] * 8], cq[2],
                                                      ab[1] - ab[0], 8, 0, wk[ab[0]:ab[1]]), ch))

    c1 = synth.tiny_moe()
    t1_T, t1_E, t1_k = c1["T"], c1["E"], c1["k"]
    t1_w1 = oracle.nvfp4_quantize_batched(c1["w1"])
    t1_w2 = oracle.nvfp4_quantize_batched(c1["w2"])

    def tiny(pool, parts):
        ids, _ = oracle.router_softmax_topk(c1["logits"], None, t1_k)
        xq1 = oracle.nvfp4_quantize(c1["x"])
        o1, a1 = oracle.route(ids, t1_E)
        n1 = int(o1[t1_E])
        G = np.concatenate(list(pool.map(lambda ab: oracle.moe_fc1(xq1, o1, a1, t1_k, t1_w1, rows=np.arange(
            ab[0], ab[1], dtype=np.int32)), _chunks(n1, parts))))
        hq1 = oracle.nvfp4_quantize(oracle.f64_to_bf16_fast(oracle.swiglu(G)))
        list(pool.map(lambda ab: oracle.moe_fc2(hq1, o1, t1_w2, rows=np.arange(ab[0], ab[1], dtype=np.int32)),
                      _chunks(n1, parts)))

    dy = synth.to_bf16_bits(synth.rng(4, 7).standard_normal((mx_rows, d)) * 1e-3)
    w2t = oracle.mxfp8_quantize(np.ascontiguousarray(w2_e.T), 0)         # W2 of expert e, [d_ff, d] along d
    w2t = (w2t[0][None], w2t[1][None])
    mx_offs = np.array([0, mx_rows], np.int32)
    dyq = oracle.mxfp8_quantize(dy, 0, mode=1, seed=0, stream=2)

    def mx_requant(pool, parts):
        list(pool.map(lambda ab: oracle.mxfp8_quantize(dy[ab[0]:ab[1]], 0, mode=1, seed=0, stream=2, row0=ab[0]),
                      _chunks(mx_rows, parts)))

    def mx_dgrad(pool, parts):
        list(pool.map(lambda ab: oracle.mxfp8_gemm_dgrad(dyq, w2t, mx_offs, rows=np.arange(ab[0], ab[1],
                                                                                            dtype=np.int32)),
                      _chunks(mx_rows, parts)))

    t1_flops = 2.0 * t1_T * t1_k * (2 * c1["d_ff"]) * c1["d"] + 2.0 * t1_T * t1_k * c1["d"] * c1["d_ff"]
    mx_bytes = dy.size * (2 + 1 + 1 / 32)
    mx_flops = 2.0 * mx_rows * d * d_ff
    fc_flops = 2.0 * R * (2 * d_ff) * d + 2.0 * R * d * d_ff
    q_bytes = xs.size * (2 + 2 + 0.5625)           # the GPU leg's algorithmic bytes for the same values
    rht_bytes = yr.size * (2 + 2 + 0.5625)
    comb_bytes = combine_tokens * 8 * 4096 * 0.5625 + combine_tokens * 4096 * 2
    res = {}
    for name, fn, work, unit, scale in (("tiny_moe_fwd", tiny, t1_flops, "TFLOP/s", 1e12),
                                         ("moe_layer_fc1_swiglu_fc2", fc_chain, fc_flops, "TFLOP/s", 1e12),
                                         ("mxfp8_requant_sr_rows", mx_requant, mx_bytes, "GB/s", 1e9),
                                         ("mxfp8_dgrad_fc2", mx_dgrad, mx_flops, "TFLOP/s", 1e12),
                                         ("quant_8192_rtn", quant, q_bytes, "GB/s", 1e9),
                                         ("combine_rht_quant", rht, rht_bytes, "GB/s", 1e9),
                                         ("combine_rht_combine", combine, comb_bytes, "GB/s", 1e9)):
        t1 = _timed_median(fn, 1)
        tn = _timed_median(fn, threads) if threads > 1 else t1
        res[name] = dict(unit=unit, one_core=work / t1 / scale, all_cores=work / tn / scale,
                         seconds_one_core=round(t1, 3), seconds_all_cores=round(tn, 3))
    main = res["moe_layer_fc1_swiglu_fc2"]
    return dict(value=main["all_cores"], unit="TFLOP/s", cores=threads, kind="oracle",
                sample=f"{R} expert-sorted rows of expert {e} (fc1+SwiGLU+fc2, int64-exact), median of 3, "
                       f"{threads} threads ({main['seconds_all_cores']} s) and 1 thread "
                       f"({main['seconds_one_core']} s)",
                one_core_value=main["one_core"], cpu_model=_cpu_model(), host_cpus=os.cpu_count(),
                configs=res)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path (the expert-parallel "
              "all-to-all is out of scope); run with --gpus 1", file=sys.stderr)
        sys.exit(2)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    flush = torch.zeros(512 << 20, dtype=torch.uint8, device=dev)

    log("[bench] moe_layer inputs")
    inp = moe_layer_inputs(dev)
    T, d, E, k, d_ff = inp["T"], inp["d"], inp["E"], inp["k"], inp["d_ff"]
    A = T * k
    log("[bench] weight quantization")
    w1q, w2q, wbf16, wq = bench_weight_quant(dev, E, d, d_ff, flush)
    log(f"[bench] weights: {wq['ms']:.2f} ms, {wq['gbps']:.0f} GB/s")

    ws = torch.empty(nvq.moe_expert_fwd_workspace_bytes(T, d, k, E, d_ff), dtype=torch.uint8, device=dev)
    y = torch.empty((T, k, d), dtype=torch.bfloat16, device=dev)
    _, it = nvq.moe_expert_fwd_nvfp4(inp["x"], inp["ids"], w1q, w2q, export=True, save_gu=True)
    torch.cuda.synchronize()
    ids_buf, w_buf = torch.empty_like(inp["ids"]), torch.empty_like(inp["rweights"])

    def fwd_step():
        nvq.moe_router_softmax_topk(inp["logits"], inp["bias"], k, ids=ids_buf, w=w_buf)
        nvq.moe_expert_fwd_nvfp4(inp["x"], ids_buf, w1q, w2q, y=y, ws=ws)

    for _ in range(args.warmup):
        fwd_step()
    torch.cuda.synchronize()
    log(f"[bench] timing {args.steps} forward steps (router + expert forward)")
    tm = Timer()
    tm.start()
    for _ in range(args.steps):
        fwd_step()
    ms = tm.stop_ms() / args.steps
    if not torch.equal(ids_buf, inp["ids"]):
        raise RuntimeError("router ids changed between calls")
    flops_fc1 = 2.0 * A * (2 * d_ff) * d
    flops_fc2 = 2.0 * A * d * d_ff
    tflops = (flops_fc1 + flops_fc2) / ms / 1e9
    log(f"[bench] forward {ms:.3f} ms/step, {tflops:.1f} TFLOP/s")

    copy_gbps = calibration_copy(dev)
    # dominant kernel: the fc1 grouped GEMM (+SwiGLU epilogue), timed alone
    xq = (it["xq_codes"], it["xq_scales"], it["xq_tscale"])
    h = torch.empty((A, d_ff), dtype=torch.bfloat16, device=dev)
    fc1_ws = torch.empty(max(nvq.lib().moe_fc1_workspace_size(A, E), nvq.lib().moe_fc2_workspace_size(A, E)),
                         dtype=torch.uint8, device=dev)
    for _ in range(2):
        nvq.moe_fc1_swiglu_nvfp4(xq, it["offsets"], it["sorted2assign"], k, w1q, h=h, ws=fc1_ws)
    torch.cuda.synchronize()
    tm.start()
    for _ in range(args.steps):
        nvq.moe_fc1_swiglu_nvfp4(xq, it["offsets"], it["sorted2assign"], k, w1q, h=h, ws=fc1_ws)
    fc1_ms = tm.stop_ms() / args.steps
    hq = (it["hq_codes"], it["hq_scales"], it["hq_tscale"])
    tm.start()
    for _ in range(args.steps):
        nvq.moe_fc2_nvfp4(hq, it["offsets"], it["sorted2assign"], w2q, y=y.view(A, d), ws=fc1_ws)
    fc2_ms = tm.stop_ms() / args.steps
    fc1_tflops = flops_fc1 / fc1_ms / 1e9
    log(f"[bench] fc1 {fc1_ms:.3f} ms ({fc1_tflops:.1f} TFLOP/s), fc2 {fc2_ms:.3f} ms "
        f"({flops_fc2 / fc2_ms / 1e9:.1f} TFLOP/s)")

    log("[bench] quant_8192")
    q8 = bench_quant_8192(dev, flush)
    log(f"[bench] quant_8192 {q8}")

    log("[bench] combine_rht")
    cr = bench_combine_rht(dev, flush)
    log(f"[bench] combine_rht {cr}")
    log("[bench] mxfp8_bwd")
    bw = bench_mxfp8_bwd(dev, inp, it, wbf16, flush, reps=max(2, min(args.steps, 5)))
    log(f"[bench] mxfp8_bwd {bw}")
    log("[bench] nvfp4_bwd")
    nb = bench_nvfp4_bwd(dev, inp, it, wbf16, flush, reps=max(2, min(args.steps, 5)))
    log(f"[bench] nvfp4_bwd {nb}")
    rt = bench_router(inp, args.steps)
    log(f"[bench] router {rt}")
    log("[bench] mxfp8_fwd")
    mf = bench_mxfp8_fwd(dev, inp, wbf16, args.steps, args.warmup, ms)
    log(f"[bench] mxfp8_fwd {mf}")
    tn = bench_tiny(dev)
    log(f"[bench] tiny_moe {tn}")
    e_max = int(np.argmax(np.diff(it["offsets"].cpu().numpy())))
    w2_host = wbf16[1][e_max].cpu().view(torch.int16).numpy().view(np.uint16)     # the expert the CPU samples
    del wbf16
    vendor_tflops = vendor_fp16_gemm(dev, A, 2 * d_ff, d)
    log(f"[bench] vendor dense fp16 GEMM of fc1's shape: {vendor_tflops:.1f} TFLOP/s; plain copy {copy_gbps:.0f} GB/s")
    vendor_mx = {"dgrad_fc1_shape": vendor_mxfp8_gemm(dev, A, d, 2 * d_ff),
                 "dgrad_fc2_shape": vendor_mxfp8_gemm(dev, A, d_ff, d)}
    log(f"[bench] vendor dense MXFP8 GEMM (TFLOP/s): {vendor_mx}")

    n_e = np.diff(it["offsets"].cpu().numpy())
    wave_rows = int(((n_e + 31) // 32 * 32).sum())  # rows the MFMAs run on (32-row block granularity)
    traffic = counted_traffic()
    result = {
        "metric": "NVFP4 MoE expert fwd TFLOPS + quantize GB/s, as fraction of MI355X peak",
        "value": round(tflops, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp16",
        "data": "synthetic",
        "config": {"workload": "moe_layer: NVFP4 expert forward, T=16384 d=4096 E=384 top-8 SwiGLU d_ff=1024, "
                               "logits N(0,1)+bias N(0,1) through the library router, X N(0,1), W N(0,0.02)",
                   "tokens": T, "d_model": d, "experts": E, "top_k": k, "d_ff": d_ff,
                   "assignments": A, "mfma_rows": wave_rows,
                   "contraction": "NVFP4 operands dequantized exactly to fp16 in LDS, fp16 MFMA, fp32 accumulate"},
        "roofline": {"bound": "mfma", "kernel": "nvq::k_grouped_gemm_dq<0, 0, 4, 4, false> (NVFP4 operands, fc1 with SwiGLU epilogue)",
                     "achieved": round(fc1_tflops, 2), "peak": MFMA_F16_PEAK_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(fc1_tflops / MFMA_F16_PEAK_TFLOPS, 4), "traffic": traffic,
                     "traffic_unit": "HBM bytes per launch (rocprofv3 FETCH_SIZE + WRITE_SIZE, copy-calibrated)",
                     "avg_launch_ms": round(fc1_ms, 4), "flops_per_launch": flops_fc1},
        "extra": {
            "fc2_ms": round(fc2_ms, 4), "fc2_tflops": round(flops_fc2 / fc2_ms / 1e9, 2),
            "quant_8192_rtn_gbps": round(q8["rtn"]["gbps"], 1), "quant_8192_sr_gbps": round(q8["sr"]["gbps"], 1),
            "quant_8192_rtn_frac_hbm": round(q8["rtn"]["gbps"] / HBM_PEAK_GBS, 4),
            "dequant_8192_bf16_gbps": round(q8["dequant_bf16"]["gbps"], 1),
            "weight_quant_gbps": round(wq["gbps"], 1), "weight_quant_ms": round(wq["ms"], 3),
            "combine_rht": cr,
            "mxfp8_bwd": bw,
            "nvfp4_bwd": nb,
            "mxfp8_fwd": mf,
            "router": rt,
            "tiny_moe": tn,
            "hbm_counters": counter_rates({
                "quant_8192_rtn": q8["rtn"]["ms"], "quant_8192_sr": q8["sr"]["ms"],
                "dequant_8192_bf16": q8["dequant_bf16"]["ms"], "weight_quant": wq["ms"],
                "rht32_blockquant": cr["quant_ms"], "rht32_dequant_combine": cr["combine_ms"],
                "mxfp8_requant_in": bw["requant_in"], "mxfp8_requant_dA": bw["requant_dA"]}),
            "context": {"vendor_fp16_gemm_fc1_shape_tflops": round(vendor_tflops, 1),
                        "vendor_mxfp8_gemm_tflops": vendor_mx,
                        "plain_copy_gbps": round(copy_gbps, 1)},
            "expert_load_max": int(n_e.max()), "expert_load_mean": float(n_e.mean()),
            "empty_experts": int((n_e == 0).sum()),
        },
    }
    if not args.no_cpu_baseline:
        log("[bench] cpu baseline (oracle)")
        result["cpu_baseline"] = cpu_baseline(inp, w1q, w2q, it, w2_host)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
