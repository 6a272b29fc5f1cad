"""GPU parity of the NVFP4 MoE expert forward against the CPU oracle.

Staged as the fused chain requires: quantized inputs and routing bit-exact;
fc1+SwiGLU on identical NVFP4 operands within 1 bf16 ulp of the exact result;
re-quantization of an identical H bit-exact; fc2 on identical operands within
1 bf16 ulp; the fused call checked the same way on its own intermediates
(the oracle's quantization of the GPU's H equals the fused Hq; y within 1
bf16 ulp of the exact fc2 of that Hq), at small shapes and at the full
moe_layer size, and byte-identical across runs and grid sizes."""
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


def _weights_oracle(c):
    return oracle.nvfp4_quantize_batched(c["w1"]), oracle.nvfp4_quantize_batched(c["w2"])


def _dev_q(q):
    return tuple(to_dev(np.atleast_1d(a)) for a in q)


def _run_staged(c, label, grid=0):
    T, d, E, k, d_ff = c["T"], c["d"], c["E"], c["k"], c["d_ff"]
    print(f"[{label}] T={T} d={d} E={E} k={k} d_ff={d_ff}", flush=True)
    # quantized operands: the GPU's must equal the oracle's bit for bit
    w1q, w2q = _weights_oracle(c)
    g1 = nvq.nvfp4_quantize(to_dev_u16(c["w1"]), batched=True)
    g2 = nvq.nvfp4_quantize(to_dev_u16(c["w2"]), batched=True)
    for g, o in ((g1, w1q), (g2, w2q)):
        assert np.array_equal(host(g[0]), o[0]) and np.array_equal(host(g[1]), o[1])
        assert np.array_equal(host(g[2]), o[2])
    xq = oracle.nvfp4_quantize(c["x"])
    # routing
    ids = to_dev(c["topk_ids"].astype(np.int32))
    offs, s2a, tiles = nvq.moe_route(ids, E)
    o_offs, o_s2a = oracle.route(c["topk_ids"], E)
    n_valid = int(o_offs[-1])
    assert np.array_equal(host(offs), o_offs)
    assert np.array_equal(host(s2a)[:n_valid], o_s2a[:n_valid])
    n_e = np.diff(o_offs)
    assert np.array_equal(host(tiles), np.concatenate([[0], np.cumsum((n_e + 255) // 256)]))
    # fc1 + SwiGLU on identical operands
    h, gu, hmax = nvq.moe_fc1_swiglu_nvfp4(_dev_q(xq), offs, s2a, k, _dev_q(w1q), save_gu=True, workgroups=grid)
    G = oracle.moe_fc1(xq, o_offs, o_s2a, k, w1q)
    H = oracle.swiglu(G)
    hh = host(h)[:n_valid]
    nf, mx = check_bf16_close(hh, H, f"{label} H")
    print(f"[{label}] H: {nf} elements on the rms floor, max err {mx:.3f} ulp", flush=True)
    check_bf16_close(host(gu)[:n_valid, :d_ff], G[:, :d_ff], f"{label} g")
    check_bf16_close(host(gu)[:n_valid, d_ff:], G[:, d_ff:], f"{label} u")
    amax_ref = np.abs(oracle.bf16_to_f32(hh)).max()
    assert host(hmax)[0] == amax_ref
    # re-quantization of an identical H (the oracle's bf16 H)
    Hb = oracle.f64_to_bf16_fast(H)
    hq_o = oracle.nvfp4_quantize(Hb)
    hq_g = nvq.nvfp4_quantize(to_dev_u16(Hb))
    assert np.array_equal(host(hq_g[0]), hq_o[0]) and np.array_equal(host(hq_g[1]), hq_o[1])
    assert host(hq_g[2])[0] == hq_o[2]
    # fc2 on identical operands, scattered to assignment order
    y = nvq.moe_fc2_nvfp4(_dev_q(hq_o), offs, s2a, _dev_q(w2q), workgroups=grid)
    Ys = oracle.moe_fc2(hq_o, o_offs, w2q)
    yy = host(y)[o_s2a[:n_valid]]
    nf, mx = check_bf16_close(yy, Ys, f"{label} y")
    print(f"[{label}] y: {nf} elements on the rms floor, max err {mx:.3f} ulp", flush=True)
    return dict(w1q=w1q, w2q=w2q, xq=xq, H=H, G=G, o_offs=o_offs, o_s2a=o_s2a)


def _run_fused(c, ref, label, grid=0, other_grid=3):
    """The fused call against the oracle, staged as C13 of the contract:
    (i) Xq and routing exact; (ii) H within 1 bf16 ulp of silu(g)*u of the
    exact G; (iii) the oracle's quantization of the GPU's own H equals the
    fused Hq byte for byte (one tensor scale over all of H, whose maximum the
    fc1 epilogue folds from partial maxima); (iv) y within 1 bf16 ulp of the
    exact fc2 of that Hq. Then determinism: identical bytes on a second run and
    with the GEMMs on another grid size (`grid` and `other_grid`: grid caps, 0 the default)."""
    T, d, E, k, d_ff = c["T"], c["d"], c["E"], c["k"], c["d_ff"]
    x = to_dev_u16(c["x"])
    ids = to_dev(c["topk_ids"].astype(np.int32))
    w1d, w2d = _dev_q(ref["w1q"]), _dev_q(ref["w2q"])
    y, it = nvq.moe_expert_fwd_nvfp4(x, ids, w1d, w2d, export=True, save_gu=True, workgroups=grid)
    torch.cuda.synchronize()
    n_valid = int(ref["o_offs"][-1])
    # (i)
    assert np.array_equal(host(it["xq_codes"]), ref["xq"][0])
    assert np.array_equal(host(it["xq_scales"]), ref["xq"][1])
    assert host(it["xq_tscale"])[0] == ref["xq"][2]
    assert np.array_equal(host(it["offsets"]), ref["o_offs"])
    assert np.array_equal(host(it["sorted2assign"])[:n_valid], ref["o_s2a"][:n_valid])
    # (ii)
    hh = host(it["h"])[:n_valid]
    check_bf16_close(hh, ref["H"], f"{label} fused H")
    # (iii)
    hq_o = oracle.nvfp4_quantize(hh)
    assert np.array_equal(host(it["hq_codes"])[:n_valid], hq_o[0]), f"{label}: fused Hq codes differ from the oracle's"
    assert np.array_equal(host(it["hq_scales"])[:n_valid], hq_o[1]), f"{label}: fused Hq scales differ"
    assert host(it["hq_tscale"])[0] == hq_o[2], f"{label}: fused H tensor scale differs"
    # (iv)
    Ys = oracle.moe_fc2(hq_o, ref["o_offs"], ref["w2q"])
    nf, mx = check_bf16_close(host(y).reshape(T * k, d)[ref["o_s2a"][:n_valid]], Ys, f"{label} fused y")
    print(f"[{label}] fused: Hq exact, y within 1 ulp of the exact fc2 of the GPU Hq ({nf} on the rms floor, "
          f"max {mx:.3f} ulp)", flush=True)
    # determinism
    y3 = nvq.moe_expert_fwd_nvfp4(x, ids, w1d, w2d, workgroups=grid)
    assert torch.equal(y, y3)
    y4, it4 = nvq.moe_expert_fwd_nvfp4(x, ids, w1d, w2d, export=True, save_gu=True, workgroups=other_grid)
    for key in ("h", "gu", "hq_codes", "hq_scales", "hq_tscale"):
        assert torch.equal(it[key][:n_valid], it4[key][:n_valid]), f"{label}: {key} depends on the grid size"
    assert torch.equal(y, y4), f"{label}: y depends on the grid size"


def test_tiny_moe():
    c = synth.tiny_moe()
    ref = _run_staged(c, "tiny_moe")
    _run_fused(c, ref, "tiny_moe")


@pytest.mark.parametrize("case", [
    dict(T=300, d=256, E=5, k=2, d_ff=256, skew=True),      # ragged tails, skewed load
    dict(T=77, d=128, E=4, k=4, d_ff=128, skew=False),      # k == E
    dict(T=513, d=384, E=16, k=3, d_ff=128, skew=True),     # many m-tiles, empty experts likely
    dict(T=96, d=512, E=3, k=2, d_ff=512, skew=True),       # K steps in groups of four (both GEMMs)
    dict(T=64, d=1024, E=2, k=1, d_ff=384, skew=False),     # groups of four in fc1, single steps in fc2
])
def test_moe_shapes(case):
    c = synth.moe_shapes(case["T"], case["d"], case["E"], case["k"], case["d_ff"], seed=5, skew=case["skew"])
    ref = _run_staged(c, str(case))
    _run_fused(c, ref, str(case))


@pytest.mark.parametrize("case", [
    dict(T=300, d=256, E=5, k=2, d_ff=256, skew=True),      # ragged tails; single steps
    dict(T=96, d=512, E=3, k=2, d_ff=512, skew=True),       # groups of four, one group per tile (K = 512)
    dict(T=200, d=1024, E=6, k=3, d_ff=512, skew=True),     # several groups in fc1, one in fc2
])
def test_moe_shapes_few_workgroups(case):
    """Three workgroups: each walks many output tiles, so the operand stream
    runs from tile to tile across ragged, partly empty and full tiles."""
    c = synth.moe_shapes(case["T"], case["d"], case["E"], case["k"], case["d_ff"], seed=7, skew=case["skew"])
    ref = _run_staged(c, "3 workgroups " + str(case), grid=3)
    _run_fused(c, ref, "3 workgroups " + str(case), grid=3, other_grid=0)


def test_moe_degenerate_routing():
    """One expert takes every token; the other experts stay empty."""
    c = synth.moe_shapes(200, 128, 6, 1, 128, seed=6)
    c["topk_ids"] = np.full((200, 1), 4, np.int32)
    ref = _run_staged(c, "all-to-one")
    _run_fused(c, ref, "all-to-one")


def test_route_moe_layer_full_size():
    """Routing of the full moe_layer workload (16384 tokens, top-8 of 384, skewed)."""
    ids, _ = synth.moe_layer_routing()
    offs, s2a, tiles = nvq.moe_route(to_dev(ids), 384)
    o_offs, o_s2a = oracle.route(ids, 384)
    assert np.array_equal(host(offs), o_offs) and np.array_equal(host(s2a), o_s2a)
    n = np.diff(o_offs)
    print(f"moe_layer load: max {n.max()}, mean {n.mean():.1f}, empty experts {(n == 0).sum()}", flush=True)


def _sub_problem(offs, s2a, experts, rows_per_expert, rng):
    """Routing restricted to whole segments of `experts`, and sampled rows
    (segment starts and ragged ends included) in both numberings."""
    seg = [np.arange(offs[e], offs[e + 1]) for e in experts]
    sub_offs = np.concatenate([[0], np.cumsum([len(r) for r in seg])]).astype(np.int32)
    sub_s2a = np.concatenate([s2a[r] for r in seg]).astype(np.int32)
    rows_full, rows_sub = [], []
    for i, r in enumerate(seg):
        pick = np.unique(np.concatenate([r[:4], r[-4:], rng.choice(r, size=min(len(r), rows_per_expert), replace=False)]))
        rows_full.append(pick)
        rows_sub.append(pick - offs[experts[i]] + sub_offs[i])
    return sub_offs, sub_s2a, np.concatenate(rows_full), np.concatenate(rows_sub).astype(np.int32)


def test_moe_layer_gemms_full_size_sampled():
    """fc1+SwiGLU and fc2 at the full moe_layer size (T=16384, d=4096, E=384,
    top-8, d_ff=1024), launched as the benchmark times them, on sampled rows of
    three experts (the largest, the smallest non-empty one and one in between).
    The oracle quantizes the bf16 inputs itself; fc2 takes its own synthetic
    input so that no oracle operand comes from the GPU."""
    dev = torch.device("cuda:0")
    T, d, E, k, d_ff = 16384, 4096, 384, 8, 1024
    ids, _ = synth.moe_layer_routing()
    x = synth.device_normal_bf16((T, d), 1.0, 1, dev)
    w1 = synth.device_normal_bf16((E, 2 * d_ff, d), 0.02, 2, dev)
    w2 = synth.device_normal_bf16((E, d, d_ff), 0.02, 3, dev)
    xq = nvq.nvfp4_quantize(x)
    w1q = nvq.nvfp4_quantize(w1, batched=True)
    w2q = nvq.nvfp4_quantize(w2, batched=True)
    offs, s2a, _ = nvq.moe_route(to_dev(ids), E)
    h = nvq.moe_fc1_swiglu_nvfp4(xq, offs, s2a, k, w1q)[0]
    # fc2 on its own input: H-shaped N(0, 1) rows in expert-sorted order
    hin = synth.device_normal_bf16((T * k, d_ff), 1.0, 4, dev)
    hq = nvq.nvfp4_quantize(hin)
    y = nvq.moe_fc2_nvfp4(hq, offs, s2a, w2q)
    torch.cuda.synchronize()
    print("full-size fc1 and fc2 done on the GPU", flush=True)

    o_offs, o_s2a = oracle.route(ids, E)
    n_e = np.diff(o_offs)
    nz = np.flatnonzero(n_e)
    order = nz[np.argsort(n_e[nz], kind="stable")]
    experts = [int(order[-1]), int(order[0]), int(order[len(order) // 2])]
    print(f"experts {experts} with {n_e[experts].tolist()} rows", flush=True)
    rng = np.random.default_rng(11)
    sub_offs, sub_s2a, rows_full, rows_sub = _sub_problem(o_offs, o_s2a, experts, 8, rng)

    def q_sub(wb):  # oracle quantization of the sampled experts' bf16 weights
        return oracle.nvfp4_quantize_batched(wb[experts].view(torch.int16).cpu().numpy().view(np.uint16))

    xq_o = oracle.nvfp4_quantize(x.view(torch.int16).cpu().numpy().view(np.uint16))
    assert np.array_equal(host(xq[0]), xq_o[0]) and np.array_equal(host(xq[1]), xq_o[1])
    assert host(xq[2])[0] == xq_o[2]
    w1q_o, w2q_o = q_sub(w1), q_sub(w2)
    for g, o in ((w1q, w1q_o), (w2q, w2q_o)):
        assert np.array_equal(host(g[0][experts]), o[0]) and np.array_equal(host(g[1][experts]), o[1])
        assert np.array_equal(host(g[2])[experts], o[2])
    H = oracle.swiglu(oracle.moe_fc1(xq_o, sub_offs, sub_s2a, k, w1q_o, rows=rows_sub))
    nf, mx = check_bf16_close(host(h)[rows_full], H, "full-size H")
    print(f"H: {len(rows_full)} rows, {nf} elements on the rms floor, max err {mx:.3f} ulp", flush=True)

    hq_o = oracle.nvfp4_quantize(hin.view(torch.int16).cpu().numpy().view(np.uint16))
    assert np.array_equal(host(hq[0]), hq_o[0]) and np.array_equal(host(hq[1]), hq_o[1])
    seg = np.concatenate([np.arange(o_offs[e], o_offs[e + 1]) for e in experts])
    Y = oracle.moe_fc2((hq_o[0][seg], hq_o[1][seg], hq_o[2]), sub_offs, w2q_o, rows=rows_sub)
    nf, mx = check_bf16_close(host(y)[o_s2a[rows_full]], Y, "full-size y")
    print(f"y: {len(rows_full)} rows, {nf} elements on the rms floor, max err {mx:.3f} ulp", flush=True)


def _experts_to_sample(n_e):
    """The largest, the smallest non-empty and a median expert, and the
    non-empty expert of largest index (>= 256 here, so the batched weights'
    upper range is covered)."""
    nz = np.flatnonzero(n_e)
    order = nz[np.argsort(n_e[nz], kind="stable")]
    ex = [int(order[-1]), int(order[0]), int(order[len(order) // 2]), int(nz[-1])]
    assert ex[-1] >= 256
    return list(dict.fromkeys(ex))


def test_moe_layer_fused_forward_full_size():
    """moe_expert_fwd_nvfp4, the call bench.py times, at the full moe_layer size
    (T=16384, d=4096, E=384, top-8, d_ff=1024), against the oracle: Xq over the
    whole tensor and the routing exact; the H tensor scale (folded from the
    2048 fc1 partial maxima) equal to the oracle's scale of the whole GPU H;
    sampled rows of four experts: H within 1 bf16 ulp of the exact
    fc1+SwiGLU, Hq bytes equal to the oracle's encoding of the GPU's H rows
    under that scale, y within 1 bf16 ulp of the exact fc2 of the GPU's Hq."""
    dev = torch.device("cuda:0")
    T, d, E, k, d_ff = 16384, 4096, 384, 8, 1024
    A = T * k
    ids, _ = synth.moe_layer_routing()
    x = synth.device_normal_bf16((T, d), 1.0, 1, dev)
    w1 = synth.device_normal_bf16((E, 2 * d_ff, d), 0.02, 2, dev)
    w2 = synth.device_normal_bf16((E, d, d_ff), 0.02, 3, dev)
    w1q = nvq.nvfp4_quantize(w1, batched=True)
    w2q = nvq.nvfp4_quantize(w2, batched=True)
    y, it = nvq.moe_expert_fwd_nvfp4(x, to_dev(ids), w1q, w2q, export=True)
    torch.cuda.synchronize()
    print("full-size fused forward done on the GPU", flush=True)

    o_offs, o_s2a = oracle.route(ids, E)
    assert np.array_equal(host(it["offsets"]), o_offs) and np.array_equal(host(it["sorted2assign"]), o_s2a)
    bits = lambda t: t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
    xq_o = oracle.nvfp4_quantize(bits(x))
    assert np.array_equal(host(it["xq_codes"]), xq_o[0]) and np.array_equal(host(it["xq_scales"]), xq_o[1])
    assert host(it["xq_tscale"])[0] == xq_o[2]
    print("Xq and routing exact", flush=True)

    hf = oracle.bf16_to_f32(host(it["h"]))
    amax = oracle.amax_f32(hf)
    n_e = np.diff(o_offs)
    experts = _experts_to_sample(n_e)
    rng = np.random.default_rng(21)
    sub_offs, sub_s2a, rows_full, rows_sub = _sub_problem(o_offs, o_s2a, experts, 6, rng)
    print(f"experts {experts} with {n_e[experts].tolist()} rows, {len(rows_full)} rows sampled", flush=True)
    hq_rows = oracle.nvfp4_quantize_slice(hf[rows_full[0]], amax, int(rows_full[0]) * d_ff)
    assert host(it["hq_tscale"])[0] == hq_rows[2], "H tensor scale differs from the oracle's over the whole GPU H"
    gc, gs = host(it["hq_codes"]), host(it["hq_scales"])
    hq_c, hq_s = [], []
    for r in rows_full:
        oc, os_, _ = oracle.nvfp4_quantize_slice(hf[r], amax, int(r) * d_ff)
        assert np.array_equal(gc[r], oc) and np.array_equal(gs[r], os_), f"Hq row {r}"
        hq_c.append(oc)
        hq_s.append(os_)
    del hf
    w1q_o = oracle.nvfp4_quantize_batched(bits(w1[experts]))
    w2q_o = oracle.nvfp4_quantize_batched(bits(w2[experts]))
    for g, o in ((w1q, w1q_o), (w2q, w2q_o)):
        assert np.array_equal(host(g[0][experts]), o[0]) and np.array_equal(host(g[1][experts]), o[1])
        assert np.array_equal(host(g[2])[experts], o[2])
    H = oracle.swiglu(oracle.moe_fc1(xq_o, sub_offs, sub_s2a, k, w1q_o, rows=rows_sub))
    nf, mx = check_bf16_close(host(it["h"])[rows_full], H, "full-size fused H")
    print(f"H: {nf} on the rms floor, max {mx:.3f} ulp", flush=True)
    # fc2 of the GPU's Hq rows: place them at their sub-problem rows
    hq_sub_c = np.zeros((int(sub_offs[-1]), d_ff // 2), np.uint8)
    hq_sub_s = np.zeros((int(sub_offs[-1]), d_ff // 16), np.uint8)
    hq_sub_c[rows_sub] = np.stack(hq_c)
    hq_sub_s[rows_sub] = np.stack(hq_s)
    Y = oracle.moe_fc2((hq_sub_c, hq_sub_s, host(it["hq_tscale"])[0]), sub_offs, w2q_o, rows=rows_sub)
    nf, mx = check_bf16_close(host(y).reshape(A, d)[o_s2a[rows_full]], Y, "full-size fused y")
    print(f"y: {nf} on the rms floor, max {mx:.3f} ulp", flush=True)
