"""Benchmark of the NVFP4 MoE expert path on one MI355X.

One step is one NVFP4 forward through an MoE expert layer of the moe_layer
workload (T=16384 tokens, d=4096, 384 experts, top-8, SwiGLU d_ff=1024):
quantize X -> route -> fc1 + SwiGLU -> re-quantize H -> fc2. Weights are
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


def kernel_source_digest():
    """Digest of the GEMM's code with comments and whitespace removed (so a
    comment edit keeps the counters; any code change invalidates them)."""
    import hashlib
    import re
    h = hashlib.sha256()
    for rel in TRAFFIC_SOURCES:
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


def calibration_copy(dev):
    """A plain elementwise copy of CALIB_BYTES (read once, written once): the
    counter runs read FETCH_SIZE / WRITE_SIZE of this dispatch to scale the
    GEMM's counts to bytes."""
    src = torch.ones(CALIB_BYTES // 4, dtype=torch.int32, device=dev)
    dst = torch.empty_like(src)
    torch.neg(src, out=dst)
    torch.cuda.synchronize()
    del src, dst


def flush_mall(buf):
    # A 512 MiB read evicts the 256 MB Infinity Cache and, unlike a write,
    # leaves no dirty lines whose write-back would be billed to the next kernel.
    buf.max()


def moe_layer_inputs(dev):
    c = synth.WORKLOADS["moe_layer"]
    T, d, E, k, d_ff = c["T"], c["d"], c["E"], c["k"], c["d_ff"]
    ids, weights = synth.moe_layer_routing()
    x = synth.device_normal_bf16((T, d), 1.0, 1, dev)
    return dict(T=T, d=d, E=E, k=k, d_ff=d_ff, ids=torch.from_numpy(ids).to(dev), weights=weights, x=x,
                ids_np=ids)


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


def bench_mxfp8_fwd(dev, inp, wbf16, steps, warmup, nvfp4_ms):
    """The same expert forward with MXFP8 operands (the precision the NVFP4
    forward is compared against): weights quantized once (axis 0, nearest
    even) outside the timed region; the whole forward timed as the NVFP4 step
    is, and its fc1 GEMM (E8M0-scaled FP8 MFMA, fp32 out) alone against the
    5 PF dense fp8 peak."""
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
    # fc1 alone on the forward's own quantized rows
    offs, s2a, _ = nvq.moe_route(inp["ids"], E)
    xq = nvq.mxfp8_requant_sr(inp["x"], 0, nvq.RTN, row_gather=s2a, gather_div=k)
    G = torch.empty((A, 2 * d_ff), dtype=torch.float32, device=dev)
    gws = torch.empty(1 << 20, dtype=torch.uint8, device=dev)
    for _ in range(2):
        nvq.moe_grouped_gemm_mxfp8(nvq.FWD, xq, w1m, offs, N=2 * d_ff, K=d, out=G, ws=gws)
    torch.cuda.synchronize()
    tm.start()
    for _ in range(steps):
        nvq.moe_grouped_gemm_mxfp8(nvq.FWD, xq, w1m, offs, N=2 * d_ff, K=d, out=G, ws=gws)
    fc1_ms = tm.stop_ms() / steps
    del w1m, w2m, ws, G, xq
    return {"ms_per_step": round(ms, 4), "tflops": round(flops / ms / 1e9, 2),
            "nvfp4_speedup": round(ms / nvfp4_ms, 4),
            "fc1_ms": round(fc1_ms, 4), "fc1_tflops": round(flops_fc1 / fc1_ms / 1e9, 2),
            "fc1_frac_fp8_peak": round(flops_fc1 / fc1_ms / 1e9 / MFMA_F8_PEAK_TFLOPS, 4)}


def bench_router(dev, T, E, k, steps):
    """The sigmoid top-k router at the moe_layer shape (fp32 logits N(0,1), bias N(0,1))."""
    g = torch.Generator(device=dev).manual_seed(7)
    logits = torch.randn((T, E), generator=g, device=dev)
    bias = torch.randn((E,), generator=g, device=dev)
    for _ in range(3):
        nvq.moe_router_sigmoid_topk(logits, bias, k)
    torch.cuda.synchronize()
    tm = Timer()
    tm.start()
    for _ in range(steps):
        nvq.moe_router_sigmoid_topk(logits, bias, k)
    ms = tm.stop_ms() / steps
    nbytes = T * E * 4 + E * 4 + T * k * 8
    return {"us": round(ms * 1000, 2), "gbps": round(nbytes / ms / 1e6, 1)}


def cpu_baseline(inp, w1q, w2q, it, budget_rows=2048):
    """The CPU oracle (plain C, one thread) on a bounded sample: fc1 + SwiGLU +
    fc2 for `budget_rows` expert-sorted rows of the moe_layer workload."""
    import oracle
    offs = it["offsets"].cpu().numpy()
    s2a = it["sorted2assign"].cpu().numpy()
    xq = tuple(t.cpu().numpy() for t in (it["xq_codes"], it["xq_scales"])) + (it["xq_tscale"].cpu().numpy()[0],)
    hq = tuple(t.cpu().numpy() for t in (it["hq_codes"], it["hq_scales"])) + (it["hq_tscale"].cpu().numpy()[0],)
    n = np.diff(offs)
    # the most loaded expert: rows [offs[e], offs[e] + budget_rows)
    e = int(np.argmax(n))
    rows = np.arange(offs[e], offs[e] + min(budget_rows, n[e]), dtype=np.int32)
    w1 = tuple(t[e:e + 1].cpu().numpy() for t in w1q)
    w2 = tuple(t[e:e + 1].cpu().numpy() for t in w2q)
    local_offs = np.array([0, len(rows)], np.int32)
    local_s2a = s2a[rows]
    hq_rows = (hq[0][rows], hq[1][rows], hq[2])
    d, d_ff, k = inp["d"], inp["d_ff"], inp["k"]
    t0 = time.perf_counter()
    G = oracle.moe_fc1(xq, local_offs, local_s2a, k, w1)
    oracle.swiglu(G)
    oracle.moe_fc2(hq_rows, local_offs, w2)
    dt = time.perf_counter() - t0
    flops = 2.0 * len(rows) * (2 * d_ff) * d + 2.0 * len(rows) * d * d_ff
    return dict(value=flops / dt / 1e12, unit="TFLOP/s", cores=1, kind="oracle",
                sample=f"{len(rows)} expert-sorted rows of expert {e} (fc1+SwiGLU+fc2, int64-exact), {dt:.1f} s")


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
    for _ in range(args.warmup):
        nvq.moe_expert_fwd_nvfp4(inp["x"], inp["ids"], w1q, w2q, y=y, ws=ws)
    torch.cuda.synchronize()
    log(f"[bench] timing {args.steps} forward steps")
    tm = Timer()
    tm.start()
    for _ in range(args.steps):
        nvq.moe_expert_fwd_nvfp4(inp["x"], inp["ids"], w1q, w2q, y=y, ws=ws)
    ms = tm.stop_ms() / args.steps
    flops_fc1 = 2.0 * A * (2 * d_ff) * d
    flops_fc2 = 2.0 * A * d * d_ff
    tflops = (flops_fc1 + flops_fc2) / ms / 1e9
    log(f"[bench] forward {ms:.3f} ms/step, {tflops:.1f} TFLOP/s")

    calibration_copy(dev)
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
    rt = bench_router(dev, T, E, k, args.steps)
    log(f"[bench] router {rt}")
    log("[bench] mxfp8_fwd")
    mf = bench_mxfp8_fwd(dev, inp, wbf16, args.steps, args.warmup, ms)
    log(f"[bench] mxfp8_fwd {mf}")
    del wbf16

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
                               "logits N(0,1)+bias N(0,1), X N(0,1), W N(0,0.02)",
                   "tokens": T, "d_model": d, "experts": E, "top_k": k, "d_ff": d_ff,
                   "assignments": A, "mfma_rows": wave_rows,
                   "contraction": "NVFP4 operands dequantized exactly to fp16 in LDS, fp16 MFMA, fp32 accumulate"},
        "roofline": {"bound": "mfma", "kernel": "k_grouped_gemm_nvfp4<fc1> (+SwiGLU epilogue)",
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
            "mxfp8_fwd": mf,
            "router": rt,
            "expert_load_max": int(n_e.max()), "expert_load_mean": float(n_e.mean()),
            "empty_experts": int((n_e == 0).sum()),
        },
    }
    if not args.no_cpu_baseline:
        log("[bench] cpu baseline (oracle)")
        result["cpu_baseline"] = cpu_baseline(inp, w1q, w2q, it)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
