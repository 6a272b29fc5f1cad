"""precision_moe_numerics_amd -- the NVFP4 MoE expert path on AMD MI355X (gfx950).

A thin ctypes binding over ``libnvq.so`` (C ABI declared in ``include/nvq.h``).
The binding only marshals arguments: it passes torch tensors' device pointers
and torch's current HIP stream, and allocates outputs and workspaces with
torch. Every step of the path runs in the library's HIP kernels. There is no
CPU fallback: if the library is missing, every call raises.

Build the library with ``python -m precision_moe_numerics_amd.build``.
"""
import ctypes as C
import os

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libnvq.so")

RTN, SR = 0, 1
OUT_BF16, OUT_F32 = 0, 1
DGRAD, WGRAD, FWD = 0, 1, 2
(CVT_DQ_F16, CVT_FP4_F32, CVT_SCAN_E2M1, CVT_SCAN_E4M3_HW, CVT_SCAN_E4M3_SW, CVT_SCAN_BF16_HW,
 CVT_SCAN_BF16_SW, CVT_SR, CVT_DQ_MX_BF16, CVT_SR_E2M1_SWEEP, CVT_SR_E4M3_SWEEP, CVT_E4M3_PAIR_F32) = range(12)

_lib = None
_vp = C.c_void_p
_i64 = C.c_int64
_sz = C.c_size_t


class NvqError(RuntimeError):
    pass


def lib():
    """Load libnvq.so (once). Raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise NvqError(f"{LIB_PATH} is missing: build it with `python -m precision_moe_numerics_amd.build`")
        L = C.CDLL(LIB_PATH)
        _declare(L)
        _lib = L
    return _lib


def _declare(L):
    L.nvq_status_string.argtypes = [C.c_int]; L.nvq_status_string.restype = C.c_char_p
    L.nvq_abi_version.restype = C.c_int
    L.nvfp4_quantize_workspace_size.argtypes = [_i64, _i64, _i64]; L.nvfp4_quantize_workspace_size.restype = _sz
    L.nvfp4_quantize.argtypes = [_vp, _i64, _i64, _i64, _vp, _vp, _vp, C.c_int, C.c_uint64, C.c_uint32,
                                 _vp, _sz, _vp]
    L.nvfp4_dequantize.argtypes = [_vp, _vp, _vp, _i64, _i64, _i64, _vp, C.c_int, _vp]
    L.moe_route_workspace_size.argtypes = [_i64, _i64]; L.moe_route_workspace_size.restype = _sz
    L.moe_route.argtypes = [_vp, _i64, _i64, _vp, _vp, _vp, _vp, _sz, _vp]
    L.moe_fc1_workspace_size.argtypes = [_i64, _i64]; L.moe_fc1_workspace_size.restype = _sz
    L.moe_fc1_swiglu_nvfp4.argtypes = [_vp, _vp, _vp, _i64, _i64, _vp, _vp, C.c_int, _i64, _i64,
                                       _vp, _vp, _vp, _vp, _vp, _vp, C.c_int, _vp, _sz, _vp]
    L.moe_fc2_workspace_size.argtypes = [_i64, _i64]; L.moe_fc2_workspace_size.restype = _sz
    L.moe_fc2_nvfp4.argtypes = [_vp, _vp, _vp, _i64, _i64, _vp, _vp, _i64, _i64, _vp, _vp, _vp, _vp,
                                C.c_int, _vp, _sz, _vp]
    L.moe_expert_fwd_nvfp4_workspace_size.argtypes = [_i64, _i64, C.c_int, _i64, _i64]
    L.moe_expert_fwd_nvfp4_workspace_size.restype = _sz
    L.moe_expert_fwd_nvfp4.argtypes = [_vp, _i64, _i64, _vp, C.c_int, _i64, _i64, _vp, _vp, _vp, _vp, _vp,
                                       _vp, _vp, _vp, _vp, _sz, _vp]
    for name, args in _OPTIONAL.items():
        if hasattr(L, name):
            fn = getattr(L, name)
            fn.argtypes = args[0]
            fn.restype = args[1]


_OPTIONAL = {
    "mxfp8_axis1_ld": ([_i64, _i64], _i64),
    "mxfp8_requant_workspace_size": ([_i64, _i64], _sz),
    "mxfp8_requant_sr": ([_vp, _i64, _i64, C.c_int, _vp, C.c_int32, _vp, _i64, _i64, C.c_int, C.c_int,
                          C.c_uint64, C.c_uint32, _vp, _vp, _vp, _sz, _vp], C.c_int),
    "rht32_blockquant_workspace_size": ([_i64, _i64], _sz),
    "rht32_blockquant": ([_vp, _i64, _i64, C.c_uint64, _vp, _vp, _vp, _vp, _sz, _vp], C.c_int),
    "rht32_dequant_combine": ([_vp, _vp, _vp, _i64, C.c_int, _i64, C.c_uint64, _vp, _vp, _vp], C.c_int),
    "moe_grouped_gemm_mxfp8_workspace_size": ([C.c_int, _i64, _i64], _sz),
    "moe_grouped_gemm_mxfp8": ([C.c_int, _vp, _vp, _vp, _vp, _vp, _i64, _i64, _i64, _i64, _i64, _i64, _vp,
                                _vp, _sz, _vp], C.c_int),
    "swiglu_bwd": ([_vp, _vp, _i64, _i64, _vp, _vp], C.c_int),
    "swiglu_fwd": ([_vp, _i64, _i64, _vp, _vp], C.c_int),
    "moe_router_sigmoid_topk": ([_vp, _i64, _i64, _vp, C.c_int, _vp, _vp, _vp], C.c_int),
    "moe_expert_fwd_mxfp8_workspace_size": ([_i64, _i64, C.c_int, _i64, _i64], _sz),
    "moe_expert_fwd_mxfp8": ([_vp, _i64, _i64, _vp, C.c_int, _i64, _i64, _vp, _vp, _vp, _vp, _vp, _vp, _sz, _vp],
                             C.c_int),
    "nvq_convert_probe": ([C.c_int, _vp, _i64, _vp, _vp], C.c_int),
    "moe_fc1_swiglu_mxfp8": ([_vp, _vp, _i64, _i64, _vp, _vp, C.c_int, _i64, _i64, _vp, _vp, _vp, _vp, C.c_int,
                              _vp, _sz, _vp], C.c_int),
    "moe_fc2_mxfp8": ([_vp, _vp, _i64, _i64, _vp, _vp, _i64, _i64, _vp, _vp, _vp, C.c_int, _vp, _sz, _vp], C.c_int),
    "nvfp4_axis1_ld": ([_i64, _i64], _i64),
    "nvfp4_quantize_axis1_workspace_size": ([_i64, _i64, _i64], _sz),
    "nvfp4_quantize_axis1": ([_vp, _i64, _i64, _vp, C.c_int32, _vp, _i64, _i64, C.c_int, C.c_uint64, C.c_int, C.c_int,
                              C.c_uint64, C.c_uint32, _vp, _vp, _vp, _vp, _sz, _vp], C.c_int),
    "moe_grouped_gemm_nvfp4_bwd_workspace_size": ([C.c_int, _i64, _i64], _sz),
    "moe_grouped_gemm_nvfp4_bwd": ([C.c_int, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i64, _i64, _i64, _i64, _i64, _i64,
                                    _vp, _vp, _sz, _vp], C.c_int),
    "moe_router_softmax_topk_workspace_size": ([_i64, _i64, C.c_int], _sz),
    "moe_router_softmax_topk": ([_vp, _i64, _i64, _vp, C.c_int, _vp, _vp, _vp, _vp, _vp, _vp, _sz, _vp], C.c_int),
    "nvfp4_quantize_noalloc": ([_vp, _i64, _i64, _i64, _vp, _vp, _vp, C.c_int, C.c_uint64, C.c_uint32, _vp],
                               C.c_int),
}


# ------------------------------------------------------------------ helpers
def _ptr(t):
    return None if t is None else C.c_void_p(t.data_ptr())


def _stream():
    return C.c_void_p(torch.cuda.current_stream().cuda_stream)


def _check(rc, what):
    if rc != 0:
        msg = lib().nvq_status_string(rc).decode()
        raise NvqError(f"{what} failed: status {rc} ({msg})")


def _need(t, dtype, name):
    if not isinstance(t, torch.Tensor) or t.dtype != dtype or not t.is_cuda or not t.is_contiguous():
        raise NvqError(f"{name} must be a contiguous {dtype} CUDA tensor")


def _ws(nbytes, device, ws=None):
    if ws is not None and ws.numel() >= nbytes:
        return ws
    return torch.empty(max(int(nbytes), 256), dtype=torch.uint8, device=device)


def _as_u16(x):
    return x.view(torch.int16) if x.dtype == torch.bfloat16 else x


# ------------------------------------------------------------------ NVFP4
def nvfp4_quantize(x, round_mode=RTN, seed=0, stream_id=1, batched=False, ws=None):
    """bf16 x [R, C] (or [B, R, C] with batched=True: one tensor scale per b).
    Returns (codes u8 [..., C/2], scales u8 [..., C/16], tscale f32 [B] or [1])."""
    _need(x, torch.bfloat16, "x")
    if batched:
        B, R, Cdim = x.shape
    else:
        B, R, Cdim = 1, x.numel() // x.shape[-1], x.shape[-1]
    lead = x.shape[:-1]
    codes = torch.empty(lead + (Cdim // 2,), dtype=torch.uint8, device=x.device)
    scales = torch.empty(lead + (Cdim // 16,), dtype=torch.uint8, device=x.device)
    tscale = torch.empty(B, dtype=torch.float32, device=x.device)
    L = lib()
    w = _ws(L.nvfp4_quantize_workspace_size(B, R, Cdim), x.device, ws)
    _check(L.nvfp4_quantize(_ptr(x), B, R, Cdim, _ptr(codes), _ptr(scales), _ptr(tscale), round_mode, seed,
                            stream_id, _ptr(w), w.numel(), _stream()), "nvfp4_quantize")
    return codes, scales, tscale


def nvfp4_dequantize(codes, scales, tscale, out_dtype=torch.float32, batched=False):
    _need(codes, torch.uint8, "codes")
    _need(scales, torch.uint8, "scales")
    _need(tscale, torch.float32, "tscale")
    Cdim = codes.shape[-1] * 2
    if batched:
        B, R = codes.shape[0], codes.shape[1]
    else:
        B, R = 1, codes.numel() // codes.shape[-1]
    out = torch.empty(codes.shape[:-1] + (Cdim,), dtype=out_dtype, device=codes.device)
    mode = OUT_BF16 if out_dtype == torch.bfloat16 else OUT_F32
    _check(lib().nvfp4_dequantize(_ptr(codes), _ptr(scales), _ptr(tscale), B, R, Cdim, _ptr(out), mode,
                                  _stream()), "nvfp4_dequantize")
    return out


# ------------------------------------------------------------------ MoE forward
def moe_router_sigmoid_topk(logits, bias, k):
    """fp32 logits [T, E], fp32 bias [E] -> (int32 topk_ids [T, k], fp32 weights [T, k]); see include/nvq.h."""
    _need(logits, torch.float32, "logits")
    _need(bias, torch.float32, "bias")
    T, E = logits.shape
    ids = torch.empty((T, k), dtype=torch.int32, device=logits.device)
    w = torch.empty((T, k), dtype=torch.float32, device=logits.device)
    _check(lib().moe_router_sigmoid_topk(_ptr(logits), T, E, _ptr(bias), k, _ptr(ids), _ptr(w), _stream()),
           "moe_router_sigmoid_topk")
    return ids, w


def moe_router_softmax_topk(logits, bias, k, route=False, ws=None, ids=None, w=None):
    """fp32 logits [T, E], fp32 bias [E] or None -> (int32 topk_ids [T, k], fp32 weights [T, k]);
    with route=True also (offsets [E+1], sorted2assign [T*k], tile_offsets [E+1]) from the same call.
    ids / w: optional output tensors. See include/nvq.h."""
    _need(logits, torch.float32, "logits")
    if bias is not None:
        _need(bias, torch.float32, "bias")
    T, E = logits.shape
    dev = logits.device
    if ids is None:
        ids = torch.empty((T, k), dtype=torch.int32, device=dev)
    if w is None:
        w = torch.empty((T, k), dtype=torch.float32, device=dev)
    _need(ids, torch.int32, "ids")
    _need(w, torch.float32, "w")
    L = lib()
    if not route:
        _check(L.moe_router_softmax_topk(_ptr(logits), T, E, _ptr(bias), k, _ptr(ids), _ptr(w), None, None, None,
                                         None, 0, _stream()), "moe_router_softmax_topk")
        return ids, w
    A = T * k
    offsets = torch.empty(E + 1, dtype=torch.int32, device=dev)
    s2a = torch.full((max(A, 1),), -1, dtype=torch.int32, device=dev)[:A]
    tiles = torch.empty(E + 1, dtype=torch.int32, device=dev)
    wsb = _ws(L.moe_router_softmax_topk_workspace_size(T, E, k), dev, ws)
    _check(L.moe_router_softmax_topk(_ptr(logits), T, E, _ptr(bias), k, _ptr(ids), _ptr(w), _ptr(offsets), _ptr(s2a),
                                     _ptr(tiles), _ptr(wsb), wsb.numel(), _stream()), "moe_router_softmax_topk")
    return ids, w, (offsets, s2a, tiles)


def moe_route(topk_ids, E, ws=None):
    """int32 topk_ids [T, k] -> (offsets [E+1], sorted2assign [T*k], tile_offsets [E+1])."""
    _need(topk_ids, torch.int32, "topk_ids")
    A = topk_ids.numel()
    dev = topk_ids.device
    offsets = torch.empty(E + 1, dtype=torch.int32, device=dev)
    s2a = torch.full((max(A, 1),), -1, dtype=torch.int32, device=dev)[:A]
    tiles = torch.empty(E + 1, dtype=torch.int32, device=dev)
    L = lib()
    w = _ws(L.moe_route_workspace_size(A, E), dev, ws)
    _check(L.moe_route(_ptr(topk_ids), A, E, _ptr(offsets), _ptr(s2a), _ptr(tiles), _ptr(w), w.numel(),
                       _stream()), "moe_route")
    return offsets, s2a, tiles


def moe_fc1_swiglu_nvfp4(xq, offsets, sorted2assign, k, w1q, save_gu=False, ws=None, h=None, workgroups=0):
    """xq = (codes [T, d/2], scales [T, d/16], tscale [1]); w1q = (codes [E, 2 d_ff, d/2], scales, tscale [E]).
    Returns (h bf16 [A, d_ff], gu bf16 [A, 2 d_ff] or None, h_amax f32 [1]). workgroups: grid cap (0: default)."""
    xc, xs, xt = xq
    wc, wsc, wt = w1q
    T, d = xc.shape[0], xc.shape[1] * 2
    E, d_ff = wc.shape[0], wc.shape[1] // 2
    A = sorted2assign.numel()
    dev = xc.device
    if h is None:
        h = torch.empty((A, d_ff), dtype=torch.bfloat16, device=dev)
    gu = torch.empty((A, 2 * d_ff), dtype=torch.bfloat16, device=dev) if save_gu else None
    amax = torch.empty(1, dtype=torch.float32, device=dev)
    L = lib()
    w = _ws(L.moe_fc1_workspace_size(A, E), dev, ws)
    _check(L.moe_fc1_swiglu_nvfp4(_ptr(xc), _ptr(xs), _ptr(xt), T, d, _ptr(offsets), _ptr(sorted2assign), k, E,
                                  d_ff, _ptr(wc), _ptr(wsc), _ptr(wt), _ptr(h), _ptr(gu), _ptr(amax), int(workgroups),
                                  _ptr(w), w.numel(), _stream()), "moe_fc1_swiglu_nvfp4")
    return h, gu, amax


def moe_fc2_nvfp4(hq, offsets, sorted2assign, w2q, y=None, ws=None, workgroups=0):
    """hq = (codes [A, d_ff/2], scales [A, d_ff/16], tscale [1]); returns y bf16 [A, d] in assignment order.
    workgroups: grid cap (0: default)."""
    hc, hs, ht = hq
    wc, wsc, wt = w2q
    A, d_ff = hc.shape[0], hc.shape[1] * 2
    E, d = wc.shape[0], wc.shape[1]
    dev = hc.device
    if y is None:
        y = torch.zeros((A, d), dtype=torch.bfloat16, device=dev)
    L = lib()
    w = _ws(L.moe_fc2_workspace_size(A, E), dev, ws)
    _check(L.moe_fc2_nvfp4(_ptr(hc), _ptr(hs), _ptr(ht), A, d_ff, _ptr(offsets), _ptr(sorted2assign), E, d,
                           _ptr(wc), _ptr(wsc), _ptr(wt), _ptr(y), int(workgroups), _ptr(w), w.numel(),
                           _stream()), "moe_fc2_nvfp4")
    return y


class MoeBuffers(C.Structure):
    _fields_ = [("xq_codes", _vp), ("xq_scales", _vp), ("xq_tscale", _vp), ("offsets", _vp),
                ("sorted2assign", _vp), ("h", _vp), ("hq_codes", _vp), ("hq_scales", _vp), ("hq_tscale", _vp),
                ("gu", _vp), ("gemm_workgroups", C.c_int)]


def moe_expert_fwd_nvfp4(x, topk_ids, w1q, w2q, export=False, save_gu=False, y=None, ws=None, workgroups=0):
    """Fused NVFP4 expert forward. x bf16 [T, d]; topk_ids int32 [T, k].
    Returns y bf16 [T, k, d] (unweighted expert outputs), plus a dict of the
    intermediates when export=True. workgroups: grid cap of both GEMMs (0: default)."""
    _need(x, torch.bfloat16, "x")
    _need(topk_ids, torch.int32, "topk_ids")
    T, d = x.shape
    k = topk_ids.shape[1]
    wc1, ws1, wt1 = w1q
    wc2, ws2, wt2 = w2q
    E, d_ff = wc1.shape[0], wc1.shape[1] // 2
    A = T * k
    dev = x.device
    if y is None:
        y = torch.empty((T, k, d), dtype=torch.bfloat16, device=dev)
    inter = None
    bufs = None
    if export or save_gu or workgroups:
        inter = {}
        if export:
            inter.update(
                xq_codes=torch.empty((T, d // 2), dtype=torch.uint8, device=dev),
                xq_scales=torch.empty((T, d // 16), dtype=torch.uint8, device=dev),
                xq_tscale=torch.empty(1, dtype=torch.float32, device=dev),
                offsets=torch.empty(E + 1, dtype=torch.int32, device=dev),
                sorted2assign=torch.full((A,), -1, dtype=torch.int32, device=dev),
                h=torch.zeros((A, d_ff), dtype=torch.bfloat16, device=dev),
                hq_codes=torch.empty((A, d_ff // 2), dtype=torch.uint8, device=dev),
                hq_scales=torch.empty((A, d_ff // 16), dtype=torch.uint8, device=dev),
                hq_tscale=torch.empty(1, dtype=torch.float32, device=dev))
        if save_gu:
            inter["gu"] = torch.empty((A, 2 * d_ff), dtype=torch.bfloat16, device=dev)
        bufs = MoeBuffers(**{f: (inter[f].data_ptr() if f in inter else None) for f, _ in MoeBuffers._fields_[:-1]},
                          gemm_workgroups=int(workgroups))
    L = lib()
    w = _ws(L.moe_expert_fwd_nvfp4_workspace_size(T, d, k, E, d_ff), dev, ws)
    _check(L.moe_expert_fwd_nvfp4(_ptr(x), T, d, _ptr(topk_ids), k, E, d_ff, _ptr(wc1), _ptr(ws1), _ptr(wt1),
                                  _ptr(wc2), _ptr(ws2), _ptr(wt2), _ptr(y),
                                  C.byref(bufs) if bufs is not None else None, _ptr(w), w.numel(), _stream()),
           "moe_expert_fwd_nvfp4")
    return (y, inter) if export or save_gu else y


def moe_expert_fwd_workspace_bytes(T, d, k, E, d_ff):
    return int(lib().moe_expert_fwd_nvfp4_workspace_size(T, d, k, E, d_ff))


# ------------------------------------------------------------------ MXFP8 backward
def mxfp8_axis1_ld(R, nseg=1):
    return int(lib().mxfp8_axis1_ld(R, nseg))


def mxfp8_requant_sr(x, axis, round_mode=SR, seed=0, stream_id=None, row_gather=None, gather_div=1,
                     seg_offsets=None, R=None, ld=None, ws=None, scale_rule=0):
    """MXFP8 (E4M3 + E8M0 per 32) of bf16 x [*, C]; scale_rule 0 (OCP) or 1 (no saturation).
    axis 0 -> (elems [R, C], scales [R, C/32]); axis 1 -> (elems [C, ld], scales [C, ld/32]).
    R defaults to x's rows, or to len(row_gather) when gathering (row r reads x[row_gather[r] // gather_div])."""
    _need(x, torch.bfloat16, "x")
    Cdim = x.shape[-1]
    if R is None:
        R = x.shape[0] if row_gather is None else row_gather.numel()
    nseg = 1 if seg_offsets is None else seg_offsets.numel() - 1
    if stream_id is None:
        stream_id = 2 + axis
    dev = x.device
    if axis == 0:
        elems = torch.empty((R, Cdim), dtype=torch.uint8, device=dev)
        scales = torch.empty((R, Cdim // 32), dtype=torch.uint8, device=dev)
        ld_ = 0
    else:
        ld_ = mxfp8_axis1_ld(R, nseg) if ld is None else ld
        elems = torch.empty((Cdim, ld_), dtype=torch.uint8, device=dev)
        scales = torch.empty((Cdim, ld_ // 32), dtype=torch.uint8, device=dev)
    L = lib()
    w = _ws(L.mxfp8_requant_workspace_size(R, nseg), dev, ws)
    _check(L.mxfp8_requant_sr(_ptr(x), R, Cdim, axis, _ptr(row_gather), gather_div, _ptr(seg_offsets), nseg, ld_,
                              round_mode, int(scale_rule), seed, stream_id, _ptr(elems), _ptr(scales), _ptr(w), w.numel(),
                              _stream()), "mxfp8_requant_sr")
    return elems, scales


def moe_grouped_gemm_mxfp8(mode, a, b, seg_offsets, M=0, N=None, K=0, out=None, ws=None):
    """a = (elems, scales), b = (elems, scales) as from mxfp8_requant_sr; see include/nvq.h.
    DGRAD, FWD -> out f32 [R, N] (R = a rows); WGRAD -> out f32 [E, M, N].
    FWD: b is the expert-major stack [E*N, K] of axis-0 quantized weights."""
    ae, as_ = a
    be, bs = b
    E = seg_offsets.numel() - 1
    if N is None:
        N = be.shape[0] // E if mode == FWD else be.shape[0]
    if mode in (DGRAD, FWD):
        shape = (ae.shape[0], N)
    else:
        M = ae.shape[0] if not M else M
        shape = (E, M, N)
    if out is None:
        out = torch.empty(shape, dtype=torch.float32, device=ae.device)
    L = lib()
    w = _ws(L.moe_grouped_gemm_mxfp8_workspace_size(mode, E, ae.shape[0]), ae.device, ws)
    _check(L.moe_grouped_gemm_mxfp8(mode, _ptr(ae), _ptr(as_), _ptr(be), _ptr(bs), _ptr(seg_offsets),
                                    ae.shape[1], be.shape[1], E, M, N, K, _ptr(out), _ptr(w), w.numel(), _stream()),
           "moe_grouped_gemm_mxfp8")
    return out


def swiglu_fwd(G, out=None):
    """G f32 [n, 2 d_ff] (gate half first) -> H bf16 [n, d_ff]."""
    _need(G, torch.float32, "G")
    n, two = G.shape
    if out is None:
        out = torch.empty((n, two // 2), dtype=torch.bfloat16, device=G.device)
    _check(lib().swiglu_fwd(_ptr(G), n, two // 2, _ptr(out), _stream()), "swiglu_fwd")
    return out


def moe_fc1_swiglu_mxfp8(xq, offsets, sorted2assign, k, w1q, d_ff, save_gu=False, h=None, ws=None, workgroups=0):
    """xq = (elems [T, d], scales [T, d/32]) of the token rows; w1q = (elems [E*2*d_ff, d], scales).
    Returns (h bf16 [A, d_ff], gu bf16 [A, 2 d_ff] or None)."""
    xe, xs = xq
    we, wsc = w1q
    T, d = xe.shape
    E = we.shape[0] // (2 * d_ff)
    A = sorted2assign.numel()
    dev = xe.device
    if h is None:
        h = torch.empty((A, d_ff), dtype=torch.bfloat16, device=dev)
    gu = torch.empty((A, 2 * d_ff), dtype=torch.bfloat16, device=dev) if save_gu else None
    L = lib()
    w = _ws(L.moe_fc1_workspace_size(A, E), dev, ws)
    _check(L.moe_fc1_swiglu_mxfp8(_ptr(xe), _ptr(xs), T, d, _ptr(offsets), _ptr(sorted2assign), k, E, d_ff, _ptr(we),
                                  _ptr(wsc), _ptr(h), _ptr(gu), int(workgroups), _ptr(w), w.numel(), _stream()),
           "moe_fc1_swiglu_mxfp8")
    return h, gu


def moe_fc2_mxfp8(hq, offsets, sorted2assign, w2q, d, y=None, ws=None, workgroups=0):
    """hq = (elems [A, d_ff], scales [A, d_ff/32]); w2q = (elems [E*d, d_ff], scales) -> y bf16 [A, d] in
    assignment order (rows of dropped assignments untouched)."""
    he, hs = hq
    we, wsc = w2q
    A, d_ff = he.shape
    E = we.shape[0] // d
    dev = he.device
    if y is None:
        y = torch.zeros((A, d), dtype=torch.bfloat16, device=dev)
    L = lib()
    w = _ws(L.moe_fc2_workspace_size(A, E), dev, ws)
    _check(L.moe_fc2_mxfp8(_ptr(he), _ptr(hs), A, d_ff, _ptr(offsets), _ptr(sorted2assign), E, d, _ptr(we), _ptr(wsc),
                           _ptr(y), int(workgroups), _ptr(w), w.numel(), _stream()), "moe_fc2_mxfp8")
    return y


def moe_expert_fwd_mxfp8(x, topk_ids, w1q, w2q, y=None, ws=None):
    """MXFP8 expert forward. x bf16 [T, d]; topk_ids int32 [T, k]; w1q = (elems [E*2*d_ff, d],
    scales [E*2*d_ff, d/32]), w2q = (elems [E*d, d_ff], scales [E*d, d_ff/32]) from
    mxfp8_requant_sr(axis 0) of the stacked weights -> y bf16 [T, k, d]."""
    _need(x, torch.bfloat16, "x")
    T, d = x.shape
    k = topk_ids.shape[1]
    w1e, w1s = w1q
    w2e, w2s = w2q
    d_ff = w2e.shape[1]
    E = w1e.shape[0] // (2 * d_ff)
    if y is None:
        y = torch.empty((T, k, d), dtype=torch.bfloat16, device=x.device)
    L = lib()
    w = _ws(L.moe_expert_fwd_mxfp8_workspace_size(T, d, k, E, d_ff), x.device, ws)
    _check(L.moe_expert_fwd_mxfp8(_ptr(x), T, d, _ptr(topk_ids), k, E, d_ff, _ptr(w1e), _ptr(w1s), _ptr(w2e),
                                  _ptr(w2s), _ptr(y), _ptr(w), w.numel(), _stream()), "moe_expert_fwd_mxfp8")
    return y


def swiglu_bwd(dH, gu, out=None):
    """dH f32 [n, d_ff], gu bf16 [n, 2 d_ff] -> dA bf16 [n, 2 d_ff]."""
    _need(dH, torch.float32, "dH")
    _need(gu, torch.bfloat16, "gu")
    n, d_ff = dH.shape
    if out is None:
        out = torch.empty((n, 2 * d_ff), dtype=torch.bfloat16, device=dH.device)
    _check(lib().swiglu_bwd(_ptr(dH), _ptr(gu), n, d_ff, _ptr(out), _stream()), "swiglu_bwd")
    return out


# ------------------------------------------------------------------ RHT32 combine path
def rht32_blockquant(y, sign_seed=0, ws=None):
    """bf16 y [R, C] -> (codes [R, C/2], scales [R, C/16], tscale [1]) of z = RHT32(y)."""
    _need(y, torch.bfloat16, "y")
    R, Cdim = y.shape
    dev = y.device
    codes = torch.empty((R, Cdim // 2), dtype=torch.uint8, device=dev)
    scales = torch.empty((R, Cdim // 16), dtype=torch.uint8, device=dev)
    tscale = torch.empty(1, dtype=torch.float32, device=dev)
    L = lib()
    w = _ws(L.rht32_blockquant_workspace_size(R, Cdim), dev, ws)
    _check(L.rht32_blockquant(_ptr(y), R, Cdim, sign_seed, _ptr(codes), _ptr(scales), _ptr(tscale), _ptr(w),
                              w.numel(), _stream()), "rht32_blockquant")
    return codes, scales, tscale


def rht32_dequant_combine(q, T, k, weights, sign_seed=0, out=None):
    """q = (codes [T*k, C/2], scales, tscale); weights f32 [T, k] -> bf16 [T, C]."""
    codes, scales, tscale = q
    _need(weights, torch.float32, "weights")
    Cdim = codes.shape[-1] * 2
    if out is None:
        out = torch.empty((T, Cdim), dtype=torch.bfloat16, device=codes.device)
    _check(lib().rht32_dequant_combine(_ptr(codes), _ptr(scales), _ptr(tscale), T, k, Cdim, sign_seed,
                                       _ptr(weights), _ptr(out), _stream()), "rht32_dequant_combine")
    return out


# ------------------------------------------------------------------ converter checks
def convert_probe(which, words=None, device="cuda"):
    """Runs the conversion steps the kernels use (include/nvq.h, nvq_convert_probe).
    CVT_DQ_F16: words int32 [n, 2] -> fp16 bits int16 [n, 40];
    CVT_FP4_F32: words [n] -> float32 [n, 8];
    CVT_SR: words int32 [n, 2] (fp32 bits, draw) -> int32 [n] (E2M1 code | E4M3 byte << 8 |
            software-rule E2M1 code << 16 | software-rule E4M3 byte << 20 | bit 31 if the E2M1
            converter's eight positions disagree);
    CVT_SCAN_*: -> int32 [65536, 18] (the sweep over all fp32 bit patterns);
    CVT_DQ_MX_BF16: -> bf16 bits int16 [256, 256] (row: E8M0 scale byte, column: E4M3 byte);
    CVT_SR_E2M1_SWEEP / CVT_SR_E4M3_SWEEP: -> int64 [4] (the device comparison of the converter and
            software forms of one stochastic rounding);
    CVT_E4M3_PAIR_F32: -> float32 [65536, 2] (every byte pair as the combine decodes its scales)."""
    if which == CVT_DQ_F16:
        _need(words, torch.int32, "words")
        n = words.shape[0]
        out = torch.empty((n, 40), dtype=torch.int16, device=words.device)
        arg = _ptr(words)
    elif which == CVT_FP4_F32:
        _need(words, torch.int32, "words")
        n = words.shape[0]
        out = torch.empty((n, 8), dtype=torch.float32, device=words.device)
        arg = _ptr(words)
    elif which == CVT_SR:
        _need(words, torch.int32, "words")
        n = words.shape[0]
        out = torch.empty((n,), dtype=torch.int32, device=words.device)
        arg = _ptr(words)
    elif which == CVT_DQ_MX_BF16:
        n = 256
        out = torch.empty((256, 256), dtype=torch.int16, device=device)
        arg = None
    elif which in (CVT_SR_E2M1_SWEEP, CVT_SR_E4M3_SWEEP):
        n = 4
        out = torch.empty((4,), dtype=torch.int64, device=device)
        arg = None
    elif which == CVT_E4M3_PAIR_F32:
        n = 65536
        out = torch.empty((n, 2), dtype=torch.float32, device=device)
        arg = None
    else:
        n = 65536
        out = torch.empty((n, 18), dtype=torch.int32, device=device)
        arg = None
    _check(lib().nvq_convert_probe(which, arg, n, _ptr(out), _stream()), "nvq_convert_probe")
    return out


# ------------------------------------------------------------------ NVFP4 backward
def nvfp4_axis1_ld(R, nseg=1):
    return int(lib().nvfp4_axis1_ld(R, nseg))


def nvfp4_quantize_axis1(x, round_mode=RTN, seed=0, stream_id=1, row_gather=None, gather_div=1, seg_offsets=None,
                         nseg=1, ld=None, rht=False, sign_seed=0, per_segment=False, R=None, ws=None):
    """NVFP4 of bf16 x [*, C] along its rows, transposed and segment padded (include/nvq.h):
    -> (codes [C, ld/2], scales [C, ld/16], tscale [1], or [nseg] with per_segment)."""
    _need(x, torch.bfloat16, "x")
    Cdim = x.shape[-1]
    if R is None:
        R = x.shape[0] if row_gather is None else row_gather.numel()
    if seg_offsets is not None:
        nseg = seg_offsets.numel() - 1
    if ld is None:
        ld = R if per_segment else nvfp4_axis1_ld(R, nseg)
    dev = x.device
    codes = torch.empty((Cdim, ld // 2), dtype=torch.uint8, device=dev)
    scales = torch.empty((Cdim, ld // 16), dtype=torch.uint8, device=dev)
    tscale = torch.empty(nseg if per_segment else 1, dtype=torch.float32, device=dev)
    L = lib()
    w = _ws(L.nvfp4_quantize_axis1_workspace_size(R, Cdim, nseg), dev, ws)
    _check(L.nvfp4_quantize_axis1(_ptr(x), R, Cdim, _ptr(row_gather), gather_div, _ptr(seg_offsets), nseg, ld,
                                  int(rht), sign_seed, int(per_segment), round_mode, seed, stream_id, _ptr(codes),
                                  _ptr(scales), _ptr(tscale), _ptr(w), w.numel(), _stream()), "nvfp4_quantize_axis1")
    return codes, scales, tscale


def moe_grouped_gemm_nvfp4_bwd(mode, a, b, seg_offsets, M=0, N=None, K=0, a_gather=None, out=None, ws=None):
    """a = (codes, scales, tscale), b = (codes, scales, tscale); see include/nvq.h.
    DGRAD: out f32 [M, N] (M = A's sorted rows, K the contraction length; B [N, >= E*K]);
    WGRAD: out f32 [E, M, N] (K = the token rows the segments cover)."""
    ac, as_, at = a
    bc, bs, bt = b
    E = seg_offsets.numel() - 1
    if N is None:
        N = bc.shape[0]
    if mode == DGRAD:
        M = M or ac.shape[0]
        shape = (M, N)
    else:
        M = M or ac.shape[0]
        shape = (E, M, N)
    if out is None:
        out = torch.empty(shape, dtype=torch.float32, device=ac.device)
    L = lib()
    w = _ws(L.moe_grouped_gemm_nvfp4_bwd_workspace_size(mode, E, M), ac.device, ws)
    _check(L.moe_grouped_gemm_nvfp4_bwd(mode, _ptr(ac), _ptr(as_), _ptr(at), _ptr(a_gather), _ptr(bc), _ptr(bs),
                                        _ptr(bt), _ptr(seg_offsets), ac.shape[1] * 2, bc.shape[1] * 2, E, M, N, K,
                                        _ptr(out), _ptr(w), w.numel(), _stream()), "moe_grouped_gemm_nvfp4_bwd")
    return out
