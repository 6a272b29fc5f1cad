"""Plain CPU oracle for the NVFP4 MoE expert path (numpy in, numpy out).

TEST INFRASTRUCTURE: only ``tests/``, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` may import this package. The product path
(``precision_moe_numerics_amd``) never imports it and shares no code with it.

Each wrapper marshals numpy arrays into the C oracle (``oracle.c``), where
every function states the passage it follows and the reading it takes.
"""
import ctypes as C
import os

import numpy as np

from . import build as _build

_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_build.LIB):
            _build.build()
        _lib = C.CDLL(_build.LIB)
        _declare(_lib)
    return _lib


_u8p = C.POINTER(C.c_uint8)
_u16p = C.POINTER(C.c_uint16)
_i32p = C.POINTER(C.c_int32)
_f32p = C.POINTER(C.c_float)
_f64p = C.POINTER(C.c_double)
_i64 = C.c_int64


def _declare(L):
    L.o_bf16_to_f32.argtypes = [C.c_uint16]; L.o_bf16_to_f32.restype = C.c_float
    L.o_f64_to_bf16_rne.argtypes = [C.c_double]; L.o_f64_to_bf16_rne.restype = C.c_uint16
    for n in ("o_e2m1_decode", "o_e4m3_decode", "o_e8m0_decode"):
        getattr(L, n).argtypes = [C.c_uint8]; getattr(L, n).restype = C.c_float
    for n in ("o_e2m1_rne", "o_e4m3_rne_sat"):
        getattr(L, n).argtypes = [C.c_float]; getattr(L, n).restype = C.c_uint8
    for n in ("o_e2m1_sr", "o_e4m3_sr"):
        getattr(L, n).argtypes = [C.c_float, C.c_uint32]; getattr(L, n).restype = C.c_uint8
    L.o_philox4x32_10.argtypes = [C.POINTER(C.c_uint32), C.POINTER(C.c_uint32), C.POINTER(C.c_uint32)]
    L.o_philox4x32_10.restype = None
    L.o_draw_u16.argtypes = [C.c_uint64, C.c_uint32, C.c_uint64]; L.o_draw_u16.restype = C.c_uint32
    L.oracle_nvfp4_quantize_bf16.argtypes = [_u16p, _i64, C.c_int, C.c_uint64, C.c_uint32, _u8p, _u8p, _f32p]
    L.oracle_nvfp4_quantize_f32.argtypes = [_f32p, _i64, C.c_int, C.c_uint64, C.c_uint32, _u8p, _u8p, _f32p]
    L.oracle_nvfp4_dequantize.argtypes = [_u8p, _u8p, C.c_float, _i64, _f32p]
    L.oracle_nvfp4_quantize_f32_slice.argtypes = [_f32p, _i64, C.c_float, _i64, C.c_int, C.c_uint64, C.c_uint32,
                                                  _u8p, _u8p, _f32p]
    L.oracle_nvfp4_quantize_f32_slice.restype = C.c_int
    L.oracle_amax_f32.argtypes = [_f32p, _i64]; L.oracle_amax_f32.restype = C.c_float
    L.oracle_mxfp8_quantize.argtypes = [_u16p, _i64, _i64, C.c_int, _i32p, C.c_int32, _i32p, _i64, C.c_int,
                                        C.c_uint64, C.c_uint32, _i64, _u8p, _u8p, _i64, C.c_int]
    L.oracle_route.argtypes = [_i32p, _i64, _i64, _i32p, _i32p]
    L.oracle_router_sigmoid_topk.argtypes = [_f32p, _f32p, _i64, _i64, C.c_int, _i32p, _f64p]
    L.oracle_router_softmax_topk.argtypes = [_f32p, _f32p, _i64, _i64, C.c_int, _i32p, _f64p]
    L.oracle_moe_fc1.argtypes = [_u8p, _u8p, C.c_float, _i64, _i32p, _i32p, C.c_int32, _i64, _i64,
                                 _u8p, _u8p, _f32p, _i32p, _i64, _f64p]
    L.oracle_swiglu.argtypes = [_f64p, _i64, _i64, _f64p]
    L.oracle_moe_fc2.argtypes = [_u8p, _u8p, C.c_float, _i64, _i32p, _i64, _i64, _u8p, _u8p, _f32p,
                                 _i32p, _i64, _f64p]
    L.oracle_nvfp4_gemm_dgrad.argtypes = [_u8p, _u8p, C.c_float, _i32p, _i32p, _i64, _i64, _i64, _u8p, _u8p, _f32p,
                                          _i32p, _i64, _f64p]
    L.oracle_nvfp4_gemm_wgrad.argtypes = [_u8p, _u8p, C.c_float, _u8p, _u8p, C.c_float, _i32p, _i64, _i64, _i64,
                                          _i64, _i32p, _i64, _f64p]
    L.oracle_mxfp8_gemm_dgrad.argtypes = [_u8p, _u8p, _u8p, _u8p, _i32p, _i64, _i64, _i64, _i32p, _i64, _f64p]
    L.oracle_mxfp8_gemm_wgrad.argtypes = [_u8p, _u8p, _u8p, _u8p, _i32p, _i64, _i64, _i64, _i64, _i32p,
                                          _i64, _f64p]
    L.oracle_swiglu_bwd.argtypes = [_f32p, _u16p, _i64, _i64, _f64p]
    L.o_rht32_signs.argtypes = [C.c_uint64]; L.o_rht32_signs.restype = C.c_uint32
    L.oracle_rht32_forward.argtypes = [_u16p, _i64, C.c_uint64, _f32p]
    L.oracle_rht32_combine.argtypes = [_u8p, _u8p, C.c_float, _i64, C.c_int32, _i64, C.c_uint64, _f32p, _f64p]
    for n in ("oracle_nvfp4_quantize_bf16", "oracle_nvfp4_quantize_f32", "oracle_nvfp4_dequantize",
              "oracle_mxfp8_quantize", "oracle_route", "oracle_router_sigmoid_topk", "oracle_router_softmax_topk", "oracle_moe_fc1", "oracle_swiglu", "oracle_moe_fc2",
              "oracle_mxfp8_gemm_dgrad", "oracle_mxfp8_gemm_wgrad", "oracle_nvfp4_gemm_dgrad",
              "oracle_nvfp4_gemm_wgrad", "oracle_swiglu_bwd",
              "oracle_rht32_forward", "oracle_rht32_combine"):
        getattr(L, n).restype = C.c_int


def _p(a, t):
    if a is None:
        return None
    assert a.flags["C_CONTIGUOUS"], "oracle inputs must be C-contiguous"
    return a.ctypes.data_as(t)


def _chk(rc, name):
    if rc != 0:
        raise ValueError(f"oracle {name} failed with status {rc}")


def _c(a, dtype):
    return None if a is None else np.ascontiguousarray(a, dtype=dtype)


# ---------------------------------------------------------------- scalars
def bf16_to_f32(bits):
    """bf16 bit patterns (uint16 array) -> float32 array (exact)."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return b.view(np.float32)


def f64_to_bf16(v):
    L = lib()
    v = np.asarray(v, dtype=np.float64)
    return np.array([L.o_f64_to_bf16_rne(float(x)) for x in v.ravel()], dtype=np.uint16).reshape(v.shape)


def e2m1_decode(c):
    return lib().o_e2m1_decode(int(c))


def e4m3_decode(b):
    return lib().o_e4m3_decode(int(b))


def e8m0_decode(b):
    return lib().o_e8m0_decode(int(b))


def e2m1_rne(y):
    return lib().o_e2m1_rne(float(y))


def e2m1_sr(y, u):
    return lib().o_e2m1_sr(float(y), int(u))


def e4m3_rne_sat(v):
    return lib().o_e4m3_rne_sat(float(v))


def e4m3_sr(v, u):
    return lib().o_e4m3_sr(float(v), int(u))


def philox4x32_10(ctr, key):
    a = (C.c_uint32 * 4)(*[int(x) & 0xFFFFFFFF for x in ctr])
    k = (C.c_uint32 * 2)(*[int(x) & 0xFFFFFFFF for x in key])
    o = (C.c_uint32 * 4)()
    lib().o_philox4x32_10(a, k, o)
    return [o[i] for i in range(4)]


def draw_u16(seed, stream, idx):
    return lib().o_draw_u16(int(seed), int(stream), int(idx))


def rht32_signs(seed):
    return lib().o_rht32_signs(int(seed))


# ---------------------------------------------------------------- NVFP4
def nvfp4_quantize(x, mode=0, seed=0, stream=1):
    """x: uint16 (bf16 bits) or float32 array of any shape with size % 16 == 0.
    Returns (codes uint8 [..., C/2], scales uint8 [..., C/16], D float)."""
    x = np.asarray(x)
    shape = x.shape
    n = x.size
    codes = np.empty(shape[:-1] + (shape[-1] // 2,), np.uint8)
    scales = np.empty(shape[:-1] + (shape[-1] // 16,), np.uint8)
    D = C.c_float(0.0)
    L = lib()
    if x.dtype == np.uint16:
        xc = _c(x, np.uint16)
        rc = L.oracle_nvfp4_quantize_bf16(_p(xc, _u16p), n, mode, seed, stream, _p(codes, _u8p),
                                          _p(scales, _u8p), C.byref(D))
    else:
        xc = _c(x, np.float32)
        rc = L.oracle_nvfp4_quantize_f32(_p(xc, _f32p), n, mode, seed, stream, _p(codes, _u8p),
                                         _p(scales, _u8p), C.byref(D))
    _chk(rc, "nvfp4_quantize")
    return codes, scales, np.float32(D.value)


def amax_f32(x):
    x = _c(x, np.float32)
    return np.float32(lib().oracle_amax_f32(_p(x, _f32p), x.size))


def nvfp4_quantize_slice(x, amax, idx0, mode=0, seed=0, stream=1):
    """Encode fp32 rows x (a slice starting at element idx0 of a larger tensor
    whose maximum |x| is amax)."""
    x = _c(x, np.float32)
    codes = np.empty(x.shape[:-1] + (x.shape[-1] // 2,), np.uint8)
    scales = np.empty(x.shape[:-1] + (x.shape[-1] // 16,), np.uint8)
    D = C.c_float(0.0)
    _chk(lib().oracle_nvfp4_quantize_f32_slice(_p(x, _f32p), x.size, float(amax), int(idx0), mode, seed, stream,
                                               _p(codes, _u8p), _p(scales, _u8p), C.byref(D)), "nvfp4_quantize_slice")
    return codes, scales, np.float32(D.value)


def nvfp4_quantize_batched(x, mode=0, seed=0, stream=1):
    """One tensor scale per leading index: x [B, R, C] -> codes, scales, D [B]."""
    outs = [nvfp4_quantize(x[b], mode, seed, stream) for b in range(x.shape[0])]
    return (np.stack([o[0] for o in outs]), np.stack([o[1] for o in outs]),
            np.array([o[2] for o in outs], dtype=np.float32))


def nvfp4_dequantize(codes, scales, D):
    codes = _c(codes, np.uint8)
    scales = _c(scales, np.uint8)
    n = codes.size * 2
    out = np.empty(codes.shape[:-1] + (codes.shape[-1] * 2,), np.float32)
    _chk(lib().oracle_nvfp4_dequantize(_p(codes, _u8p), _p(scales, _u8p), float(D), n, _p(out, _f32p)),
         "nvfp4_dequantize")
    return out


# ---------------------------------------------------------------- MXFP8
def mxfp8_ld(R, nseg):
    """Row stride of the transposed (axis-1) layout: enough for every segment's
    zero-padded tail, rounded to 32."""
    return ((R + 31 * nseg) + 31) // 32 * 32


def mxfp8_quantize(x, axis, mode=0, seed=0, stream=2, row_gather=None, gather_div=1,
                   seg_offsets=None, R=None, ld=None, row0=0, rule=0):
    """row0: the logical index of the first row (the SR draw of element (r, c) is
    keyed by (row0 + r) * C + c), to encode rows of a larger tensor on their own.
    rule: 0 = floor(log2 amax) - 8 with saturating elements, 1 = ceil(log2(amax/448))."""
    x = _c(x, np.uint16)
    C_ = x.shape[-1]
    if R is None:
        R = x.shape[0] if row_gather is None else len(row_gather)
    rg = _c(row_gather, np.int32)
    so = _c(seg_offsets, np.int32)
    nseg = 1 if so is None else len(so) - 1
    if axis == 0:
        elems = np.empty((R, C_), np.uint8)
        scales = np.empty((R, C_ // 32), np.uint8)
        ld_ = 0
    else:
        ld_ = mxfp8_ld(R, nseg) if ld is None else ld
        elems = np.empty((C_, ld_), np.uint8)
        scales = np.empty((C_, ld_ // 32), np.uint8)
    rc = lib().oracle_mxfp8_quantize(_p(x, _u16p), R, C_, axis, _p(rg, _i32p), gather_div, _p(so, _i32p),
                                     nseg, mode, seed, stream, ld_, _p(elems, _u8p), _p(scales, _u8p), int(row0),
                                     int(rule))
    _chk(rc, "mxfp8_quantize")
    return elems, scales


# ---------------------------------------------------------------- routing / GEMMs
def router_sigmoid_topk(logits, bias, k):
    """logits f32 [T, E], bias f32 [E] -> (ids int32 [T, k] in choice order, weights f64 [T, k])."""
    logits = _c(logits, np.float32)
    bias = _c(bias, np.float32)
    T, E = logits.shape
    ids = np.empty((T, k), np.int32)
    w = np.empty((T, k), np.float64)
    _chk(lib().oracle_router_sigmoid_topk(_p(logits, _f32p), _p(bias, _f32p), T, E, k, _p(ids, _i32p),
                                          _p(w, _f64p)), "router_sigmoid_topk")
    return ids, w


def router_softmax_topk(logits, bias, k):
    """logits f32 [T, E], bias f32 [E] or None -> (ids int32 [T, k] in choice order,
    weights f64 [T, k]: the softmax of the chosen raw logits)."""
    logits = _c(logits, np.float32)
    bias = _c(bias, np.float32)
    T, E = logits.shape
    ids = np.empty((T, k), np.int32)
    w = np.empty((T, k), np.float64)
    _chk(lib().oracle_router_softmax_topk(_p(logits, _f32p), _p(bias, _f32p), T, E, k, _p(ids, _i32p),
                                          _p(w, _f64p)), "router_softmax_topk")
    return ids, w


def route(topk_ids, E):
    ids = _c(np.asarray(topk_ids).ravel(), np.int32)
    offsets = np.empty(E + 1, np.int32)
    s2a = np.full(ids.size, -1, np.int32)
    _chk(lib().oracle_route(_p(ids, _i32p), ids.size, E, _p(offsets, _i32p), _p(s2a, _i32p)), "route")
    return offsets, s2a


def moe_fc1(xq, offsets, s2a, topk, w1q, rows=None):
    """xq = (codes [T,d/2], scales [T,d/16], Dx); w1q = (codes [E,2dff,d/2], scales, Dw1 [E])."""
    xc, xs, Dx = xq
    wc, ws, Dw = w1q
    xc, xs, wc, ws = (_c(a, np.uint8) for a in (xc, xs, wc, ws))
    Dw = _c(Dw, np.float32)
    offsets = _c(offsets, np.int32)
    s2a = _c(s2a, np.int32)
    E = wc.shape[0]
    d_ff = wc.shape[1] // 2
    d = xc.shape[1] * 2
    rws = _c(rows, np.int32)
    nrows = int(offsets[E]) if rws is None else len(rws)
    G = np.empty((nrows, 2 * d_ff), np.float64)
    rc = lib().oracle_moe_fc1(_p(xc, _u8p), _p(xs, _u8p), float(Dx), d, _p(offsets, _i32p), _p(s2a, _i32p),
                              topk, E, d_ff, _p(wc, _u8p), _p(ws, _u8p), _p(Dw, _f32p), _p(rws, _i32p), nrows,
                              _p(G, _f64p))
    _chk(rc, "moe_fc1")
    return G


def swiglu(G):
    G = _c(G, np.float64)
    n, two_dff = G.shape
    H = np.empty((n, two_dff // 2), np.float64)
    _chk(lib().oracle_swiglu(_p(G, _f64p), n, two_dff // 2, _p(H, _f64p)), "swiglu")
    return H


def moe_fc2(hq, offsets, w2q, rows=None):
    hc, hs, DH = hq
    wc, ws, Dw = w2q
    hc, hs, wc, ws = (_c(a, np.uint8) for a in (hc, hs, wc, ws))
    Dw = _c(Dw, np.float32)
    offsets = _c(offsets, np.int32)
    E, d = wc.shape[0], wc.shape[1]
    d_ff = hc.shape[1] * 2
    rws = _c(rows, np.int32)
    nrows = int(offsets[E]) if rws is None else len(rws)
    Y = np.empty((nrows, d), np.float64)
    rc = lib().oracle_moe_fc2(_p(hc, _u8p), _p(hs, _u8p), float(DH), d_ff, _p(offsets, _i32p), E, d,
                              _p(wc, _u8p), _p(ws, _u8p), _p(Dw, _f32p), _p(rws, _i32p), nrows, _p(Y, _f64p))
    _chk(rc, "moe_fc2")
    return Y


def mxfp8_gemm_dgrad(a, b, offsets, rows=None):
    """a = (elems [R,K], scales [R,K/32]); b = (elems [E,N,K], scales [E,N,K/32])."""
    ae, as_ = (_c(t, np.uint8) for t in a)
    be, bs = (_c(t, np.uint8) for t in b)
    offsets = _c(offsets, np.int32)
    E, N, K = be.shape
    rws = _c(rows, np.int32)
    nrows = int(offsets[E]) if rws is None else len(rws)
    out = np.empty((nrows, N), np.float64)
    rc = lib().oracle_mxfp8_gemm_dgrad(_p(ae, _u8p), _p(as_, _u8p), _p(be, _u8p), _p(bs, _u8p),
                                       _p(offsets, _i32p), E, N, K, _p(rws, _i32p), nrows, _p(out, _f64p))
    _chk(rc, "mxfp8_gemm_dgrad")
    return out


def mxfp8_gemm_wgrad(a, b, pad_offsets, experts=None):
    """a = (elems [M,ld], scales [M,ld/32]); b = (elems [N,ld], scales [N,ld/32])."""
    ae, as_ = (_c(t, np.uint8) for t in a)
    be, bs = (_c(t, np.uint8) for t in b)
    po = _c(pad_offsets, np.int32)
    E = len(po) - 1
    M, ld = ae.shape
    N = be.shape[0]
    ex = _c(experts, np.int32)
    nexp = E if ex is None else len(ex)
    out = np.empty((nexp, M, N), np.float64)
    rc = lib().oracle_mxfp8_gemm_wgrad(_p(ae, _u8p), _p(as_, _u8p), _p(be, _u8p), _p(bs, _u8p), _p(po, _i32p),
                                       E, M, N, ld, _p(ex, _i32p), nexp, _p(out, _f64p))
    _chk(rc, "mxfp8_gemm_wgrad")
    return out


# ---------------------------------------------------------------- NVFP4 backward
# The backward in the forward's 4-bit format (page "Thinking Machines Details
# End-to-End 4-Bit Training for Inkling 2 Small", section "Developer quick
# start": exploring FP4 backward passes). Readings: gradients (dY, dA) use
# stochastic rounding, weights and activations nearest even; dgrad operands are
# NVFP4 along the contraction axis (the weights transposed, one tensor scale
# per expert matrix); wgrad operands are transposed into per-expert token
# segments, each 32-token chunk goes through the 32-point random Hadamard
# transform of the combine (signs first, Sylvester H32, 1/sqrt 32), and the
# result is NVFP4 along the tokens with one tensor scale per operand. The
# transform is orthogonal and applied to both operands, so it cancels in the
# product.
def _scalar(v):
    return float(np.asarray(v, dtype=np.float64).ravel()[0])


def nvfp4_gemm_dgrad(a, b, offsets, a_gather=None, rows=None):
    """a = (codes [*, K/2], scales [*, K/16], Da); b = (codes [E, N, K/2], scales, Db [E]).
    out[i][n] for listed sorted rows (all rows by default); A row of sorted row r = a_gather[r] or r."""
    ac, as_ = _c(a[0], np.uint8), _c(a[1], np.uint8)
    bc, bs = _c(b[0], np.uint8), _c(b[1], np.uint8)
    Db = _c(np.atleast_1d(b[2]), np.float32)
    offsets = _c(offsets, np.int32)
    E, N, K2 = bc.shape
    rws = _c(rows, np.int32)
    ag = _c(a_gather, np.int32)
    nrows = int(offsets[E]) if rws is None else len(rws)
    out = np.empty((nrows, N), np.float64)
    rc = lib().oracle_nvfp4_gemm_dgrad(_p(ac, _u8p), _p(as_, _u8p), _scalar(a[2]), _p(ag, _i32p), _p(offsets, _i32p),
                                       E, N, 2 * K2, _p(bc, _u8p), _p(bs, _u8p), _p(Db, _f32p), _p(rws, _i32p),
                                       nrows, _p(out, _f64p))
    _chk(rc, "nvfp4_gemm_dgrad")
    return out


def nvfp4_gemm_wgrad(a, b, pad_offsets, experts=None):
    """a = (codes [M, ld/2], scales [M, ld/16], Da); b = (codes [N, ld/2], scales, Db): out [nexp, M, N]."""
    ac, as_ = _c(a[0], np.uint8), _c(a[1], np.uint8)
    bc, bs = _c(b[0], np.uint8), _c(b[1], np.uint8)
    po = _c(pad_offsets, np.int32)
    E = len(po) - 1
    M, ld2 = ac.shape
    N = bc.shape[0]
    ex = _c(experts, np.int32)
    nexp = E if ex is None else len(ex)
    out = np.empty((nexp, M, N), np.float64)
    rc = lib().oracle_nvfp4_gemm_wgrad(_p(ac, _u8p), _p(as_, _u8p), _scalar(a[2]), _p(bc, _u8p), _p(bs, _u8p),
                                       _scalar(b[2]), _p(po, _i32p), E, M, N, 2 * ld2, _p(ex, _i32p), nexp,
                                       _p(out, _f64p))
    _chk(rc, "nvfp4_gemm_wgrad")
    return out


def nvfp4_axis1_ld(R, nseg=1):
    """Row length of the transposed segment-padded NVFP4 layout: room for every
    segment padded to 32 rows, rounded to 128, plus 128 columns of slack."""
    return 128 * ((R + 31 * nseg + 127) // 128) + 128


def nvfp4_quantize_axis1(x, mode=0, seed=0, stream=1, row_gather=None, gather_div=1, seg_offsets=None, ld=None,
                         rht_seed=None, per_segment=False):
    """NVFP4 along the rows of x (bf16 bits [R_src, C]), transposed:
      logical row r reads x[row_gather[r] // gather_div] (x[r] without a gather);
      segment s = rows [seg[s], seg[s+1]) occupies columns [pad_s, pad_s + 32 ceil(n_s / 32)) of the
      output [C, ld], zero padded (pad_0 = 0); columns past the last segment are zero;
      with rht_seed, every 32-column chunk of the segments goes through rht32_forward (the
      zero columns past the last segment stay zero);
      then NVFP4 of the [C, ld] tensor: one tensor scale over all of it, or one per segment
      (per_segment, for the weights: no transform). The stochastic draw of element (c, j) is
      keyed by c * ld + j. Returns (codes [C, ld/2], scales [C, ld/16], D [1] or [nseg])."""
    x = _c(x, np.uint16)
    Cc = x.shape[1]
    R = x.shape[0] if row_gather is None else len(row_gather)
    seg = np.array([0, R], np.int32) if seg_offsets is None else np.asarray(seg_offsets, np.int32)
    nseg = len(seg) - 1
    po = pad_offsets(seg)
    ld = nvfp4_axis1_ld(R, nseg) if ld is None else ld
    assert ld % 32 == 0 and ld >= po[-1]
    src = np.arange(R) if row_gather is None else np.asarray(row_gather, np.int64) // gather_div
    xt = np.zeros((Cc, ld), np.uint16)
    for s in range(nseg):
        r0, r1 = int(seg[s]), int(seg[s + 1])
        xt[:, po[s]:po[s] + (r1 - r0)] = x[src[r0:r1]].T
    z = bf16_to_f32(xt)
    if rht_seed is not None:
        # the chunks of the segments; the zero columns past the last segment stay zero
        assert not per_segment
        used = int(po[-1])
        z[:, :used] = rht32_forward(np.ascontiguousarray(xt[:, :used]).ravel(), rht_seed).reshape(Cc, used)
    if not per_segment:
        codes, scales, D = nvfp4_quantize(z, mode, seed, stream)
        return codes, scales, np.array([D], np.float32)
    assert mode == 0
    codes = np.zeros((Cc, ld // 2), np.uint8)
    scales = np.zeros((Cc, ld // 16), np.uint8)
    Ds = np.empty(nseg, np.float32)
    for s in range(nseg):
        a, b_ = int(po[s]), int(po[s + 1])
        c_, s_, Ds[s] = nvfp4_quantize(np.ascontiguousarray(z[:, a:b_]), 0)
        codes[:, a // 2:b_ // 2], scales[:, a // 16:b_ // 16] = c_, s_
    return codes, scales, Ds


def pad_offsets(offsets):
    """32-aligned segment starts of the transposed MXFP8 layout."""
    offsets = np.asarray(offsets, dtype=np.int64)
    n = np.diff(offsets)
    return np.concatenate([[0], np.cumsum((n + 31) // 32 * 32)]).astype(np.int32)


def swiglu_bwd(dH, gu):
    dH = _c(dH, np.float32)
    gu = _c(gu, np.uint16)
    n, d_ff = dH.shape
    dA = np.empty((n, 2 * d_ff), np.float64)
    _chk(lib().oracle_swiglu_bwd(_p(dH, _f32p), _p(gu, _u16p), n, d_ff, _p(dA, _f64p)), "swiglu_bwd")
    return dA


# ---------------------------------------------------------------- RHT
def rht32_forward(x, sign_seed=0):
    x = _c(x, np.uint16)
    z = np.empty(x.shape, np.float32)
    _chk(lib().oracle_rht32_forward(_p(x, _u16p), x.size, sign_seed, _p(z, _f32p)), "rht32_forward")
    return z


def rht32_combine(codes, scales, D, T, topk, sign_seed, w):
    codes = _c(codes, np.uint8)
    scales = _c(scales, np.uint8)
    w = _c(w, np.float32)
    Cdim = codes.shape[-1] * 2
    out = np.empty((T, Cdim), np.float64)
    _chk(lib().oracle_rht32_combine(_p(codes, _u8p), _p(scales, _u8p), float(D), T, topk, Cdim, sign_seed,
                                    _p(w, _f32p), _p(out, _f64p)), "rht32_combine")
    return out


# ---------------------------------------------------------------- chains
def moe_forward(x_bf16, topk_ids, w1q, w2q, rows=None):
    """Whole expert forward: quantize X, route, fc1 exact, SwiGLU, bf16 H,
    quantize H (one scale over all of H), fc2 exact. Returns a dict of every
    intermediate (rows=None only: H's tensor scale needs all of H)."""
    T, k = topk_ids.shape
    E = w1q[0].shape[0]
    xq = nvfp4_quantize(x_bf16)
    offsets, s2a = route(topk_ids, E)
    G = moe_fc1(xq, offsets, s2a, k, w1q)
    H = swiglu(G)
    Hb = f64_to_bf16_fast(H)
    hq = nvfp4_quantize(Hb)
    Ys = moe_fc2(hq, offsets, w2q)
    d = Ys.shape[1]
    y = np.zeros((T * k, d), np.float64)
    y[s2a[: offsets[E]]] = Ys
    return dict(xq=xq, offsets=offsets, s2a=s2a, G=G, H=H, H_bf16=Hb, hq=hq, Y_sorted=Ys, y=y.reshape(T, k, d))


def f64_to_bf16_fast(v):
    """Vectorised nearest-even fp64 -> bf16 for finite values (same rule as
    o_f64_to_bf16_rne; checked against it in the tests)."""
    v = np.asarray(v, dtype=np.float64)
    a = np.abs(v)
    _, ex = np.frexp(a)
    e = ex.astype(np.int64) - 1
    q = np.where(e < -126, np.ldexp(1.0, -133), np.ldexp(np.ones_like(a), np.maximum(e, -126) - 7))
    r = np.rint(a / q) * q
    r = np.where(a == 0, 0.0, r)
    bits = (r.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    return bits | np.where(np.signbit(v), np.uint16(0x8000), np.uint16(0))
