"""numpy front end of the CPU oracle (liboracle.so, built from rq_oracle.c).

TEST INFRASTRUCTURE ONLY: imported by the tests, by the package smoke check and
by the benchmark's CPU-baseline leg, never by the product path.

Arrays are numpy; bf16 and f16 values travel as their uint16 bit patterns.
Each function states the passage of the ResidualQuant page ("ResidualQuant:
KV Cache Quantization for Looped Transformers with 2-Bit Residuals") that its
C counterpart follows.
"""
from __future__ import annotations

import ctypes as C
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None

_u8p = np.ctypeslib.ndpointer(dtype=np.uint8, flags="C_CONTIGUOUS")
_u16p = np.ctypeslib.ndpointer(dtype=np.uint16, flags="C_CONTIGUOUS")
_f32p = np.ctypeslib.ndpointer(dtype=np.float32, flags="C_CONTIGUOUS")
_f64p = np.ctypeslib.ndpointer(dtype=np.float64, flags="C_CONTIGUOUS")
_i32p = np.ctypeslib.ndpointer(dtype=np.int32, flags="C_CONTIGUOUS")


def lib():
    """Load liboracle.so, building it with gcc first if it is missing."""
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            from oracle import build as _b
            _b.build()
        L = C.CDLL(_LIB_PATH)
        L.rqo_bf16_to_f32.restype = C.c_float
        L.rqo_bf16_to_f32.argtypes = [C.c_uint16]
        L.rqo_f16_to_f32.restype = C.c_float
        L.rqo_f16_to_f32.argtypes = [C.c_uint16]
        L.rqo_f32_to_f16.restype = C.c_uint16
        L.rqo_f32_to_f16.argtypes = [C.c_float]
        L.rqo_f32_to_f16_sat.restype = C.c_uint16
        L.rqo_f32_to_f16_sat.argtypes = [C.c_float]
        L.rqo_tree_sum.restype = C.c_float
        L.rqo_tree_sum.argtypes = [_f32p, C.c_int]
        L.rqo_dot_sum.restype = C.c_float
        L.rqo_dot_sum.argtypes = [_f32p, C.c_int]
        L.rqo_alpha_f32.restype = C.c_float
        L.rqo_alpha_f32.argtypes = [_u16p, _u16p, C.c_int]
        L.rqo_alpha_bits.restype = C.c_uint16
        L.rqo_alpha_bits.argtypes = [_u16p, _u16p, C.c_int]
        L.rqo_fwht_f32.restype = None
        L.rqo_fwht_f32.argtypes = [_f32p, C.c_int]
        L.rqo_quantize_group.restype = None
        L.rqo_quantize_group.argtypes = [_f32p, C.c_int, C.c_int, _u8p,
                                         C.POINTER(C.c_uint16), C.POINTER(C.c_uint16)]
        L.rqo_pack.restype = None
        L.rqo_pack.argtypes = [_u8p, C.c_int, C.c_int, _u8p]
        L.rqo_unpack.restype = None
        L.rqo_unpack.argtypes = [_u8p, C.c_int, C.c_int, _u8p]
        L.rqo_encode_vector.restype = None
        L.rqo_encode_vector.argtypes = [_u16p, _u16p, C.c_int, C.c_int, C.c_int, C.c_int,
                                        _u8p, _u16p, C.POINTER(C.c_uint16)]
        L.rqo_encode.restype = None
        L.rqo_encode.argtypes = [C.c_int] * 7 + [_i32p, _u16p, _u16p, C.c_int, C.c_int,
                                                 C.c_void_p, C.c_void_p, C.c_void_p]
        L.rqo_reconstruct_vector.restype = None
        L.rqo_reconstruct_vector.argtypes = [_u8p, _u16p, C.c_uint16, _u16p, C.c_int,
                                             C.c_int, C.c_int, C.c_int, _f64p]
        L.rqo_reconstruct.restype = None
        L.rqo_reconstruct.argtypes = [C.c_int] * 7 + [_u16p, _u8p, _u16p, _u16p,
                                                      C.c_int, C.c_int, _f64p]
        L.rqo_attention.restype = None
        L.rqo_attention.argtypes = [_f64p, _f64p, _f64p, C.c_int, C.c_int, C.c_double, _f64p]
        L.rqo_decode_row.restype = None
        L.rqo_decode_row.argtypes = ([C.c_int] * 8
                                     + [_u16p, _u8p, _u16p, _u16p, _u16p, _u8p, _u16p, _u16p,
                                        _u16p, C.c_int, C.c_int, C.c_int, C.c_int, C.c_double,
                                        _f64p])
        L.rqo_alpha_f32_y.restype = C.c_float
        L.rqo_alpha_f32_y.argtypes = [_u16p, _f32p, C.c_int]
        L.rqo_encode_vector_y.restype = None
        L.rqo_encode_vector_y.argtypes = [_u16p, _f32p, C.c_int, C.c_int, C.c_int, C.c_int,
                                          _u8p, _u16p, C.POINTER(C.c_uint16)]
        L.rqo_anchor_vector.restype = None
        L.rqo_anchor_vector.argtypes = [_u16p, C.c_int, C.c_int, C.c_int, C.c_int, _u8p, _u16p,
                                        _f32p]
        L.rqo_encode_anchored.restype = None
        L.rqo_encode_anchored.argtypes = [C.c_int] * 9 + [_i32p, _u16p, C.c_int, C.c_int,
                                                          C.c_void_p, C.c_void_p, C.c_void_p]
        L.rqo_dequant_f64.restype = None
        L.rqo_dequant_f64.argtypes = [_u8p, _u16p, C.c_int, C.c_int, C.c_int, C.c_int, _f64p]
        L.rqo_reconstruct_anchored.restype = None
        L.rqo_reconstruct_anchored.argtypes = ([C.c_int] * 9 + [_u8p, _u16p, C.c_void_p, C.c_void_p,
                                                                C.c_void_p, C.c_int, C.c_int,
                                                                C.c_int, _f64p])
        L.rqo_decode_row_ex.restype = None
        L.rqo_decode_row_ex.argtypes = ([C.c_int] * 8
                                        + [C.c_void_p] * 8
                                        + [C.c_int, C.c_int] + [C.c_void_p] * 6 + [C.c_int]
                                        + [_u16p, C.c_int, C.c_int, C.c_int, C.c_int, C.c_double,
                                           _f64p])
        _lib = L
    return _lib


# ---------------------------------------------------------------------------
# number formats
# ---------------------------------------------------------------------------

def f32_to_f16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> binary16 bits, round half to even (overflow -> inf)."""
    x = np.ascontiguousarray(x, dtype=np.float32).ravel()
    f = lib().rqo_f32_to_f16
    return np.fromiter((f(float(v)) for v in x), dtype=np.uint16, count=x.size)


def f16_bits_to_f32(h: np.ndarray) -> np.ndarray:
    h = np.ascontiguousarray(h, dtype=np.uint16).ravel()
    f = lib().rqo_f16_to_f32
    return np.fromiter((f(int(v)) for v in h), dtype=np.float32, count=h.size)


def bf16_bits_to_f32(h: np.ndarray) -> np.ndarray:
    h = np.ascontiguousarray(h, dtype=np.uint16).ravel()
    f = lib().rqo_bf16_to_f32
    return np.fromiter((f(int(v)) for v in h), dtype=np.float32, count=h.size)


# ---------------------------------------------------------------------------
# encoder pieces (FP32 contract)
# ---------------------------------------------------------------------------

def tree_sum(a: np.ndarray) -> float:
    a = np.array(a, dtype=np.float32)
    return float(lib().rqo_tree_sum(a, a.size))


def dot_sum(a: np.ndarray) -> float:
    a = np.array(a, dtype=np.float32)
    return float(lib().rqo_dot_sum(a, a.size))


def alpha_f32(x_bits: np.ndarray, y_bits: np.ndarray) -> float:
    x = np.ascontiguousarray(x_bits, dtype=np.uint16)
    y = np.ascontiguousarray(y_bits, dtype=np.uint16)
    return float(lib().rqo_alpha_f32(x, y, x.size))


def alpha_bits(x_bits: np.ndarray, y_bits: np.ndarray) -> int:
    x = np.ascontiguousarray(x_bits, dtype=np.uint16)
    y = np.ascontiguousarray(y_bits, dtype=np.uint16)
    return int(lib().rqo_alpha_bits(x, y, x.size))


def fwht_f32(u: np.ndarray) -> np.ndarray:
    u = np.array(u, dtype=np.float32)
    lib().rqo_fwht_f32(u, u.size)
    return u


def quantize_group(u: np.ndarray, bits: int):
    """Returns (codes uint8[g], scale_bits, zero_bits)."""
    u = np.ascontiguousarray(u, dtype=np.float32)
    codes = np.zeros(u.size, dtype=np.uint8)
    s, z = C.c_uint16(), C.c_uint16()
    lib().rqo_quantize_group(u, u.size, bits, codes, C.byref(s), C.byref(z))
    return codes, int(s.value), int(z.value)


def pack(codes: np.ndarray, bits: int) -> np.ndarray:
    codes = np.ascontiguousarray(codes, dtype=np.uint8)
    out = np.zeros(codes.size * bits // 8, dtype=np.uint8)
    lib().rqo_pack(codes, codes.size, bits, out)
    return out


def unpack(packed: np.ndarray, d: int, bits: int) -> np.ndarray:
    packed = np.ascontiguousarray(packed, dtype=np.uint8)
    out = np.zeros(d, dtype=np.uint8)
    lib().rqo_unpack(packed, d, bits, out)
    return out


def encode_vector(x_bits, y_bits, g: int, bits: int, rotate: bool):
    """One vector: returns (packed uint8[d*bits/8], meta uint16[2*d/g], alpha_bits)."""
    x = np.ascontiguousarray(x_bits, dtype=np.uint16)
    y = np.ascontiguousarray(y_bits, dtype=np.uint16)
    d = x.size
    packed = np.zeros(d * bits // 8, dtype=np.uint8)
    meta = np.zeros(2 * (d // g), dtype=np.uint16)
    a = C.c_uint16()
    lib().rqo_encode_vector(x, y, d, g, bits, int(rotate), packed, meta, C.byref(a))
    return packed, meta, int(a.value)


def anchor_vector(y_bits, g: int, bits: int, rotate: bool):
    """Quantized anchor of one vector: returns (packed uint8[d*bits/8],
    meta uint16[2*d/g], y_hat float32[d] -- the dequantized anchor)."""
    y = np.ascontiguousarray(y_bits, dtype=np.uint16)
    d = y.size
    packed = np.zeros(d * bits // 8, dtype=np.uint8)
    meta = np.zeros(2 * (d // g), dtype=np.uint16)
    yhat = np.zeros(d, dtype=np.float32)
    lib().rqo_anchor_vector(y, d, g, bits, int(rotate), packed, meta, yhat)
    return packed, meta, yhat


def encode_vector_y(x_bits, y_f32, g: int, bits: int, rotate: bool):
    """encode_vector against an FP32 reference (e.g. a dequantized anchor)."""
    x = np.ascontiguousarray(x_bits, dtype=np.uint16)
    y = np.ascontiguousarray(y_f32, dtype=np.float32)
    d = x.size
    packed = np.zeros(d * bits // 8, dtype=np.uint8)
    meta = np.zeros(2 * (d // g), dtype=np.uint16)
    a = C.c_uint16()
    lib().rqo_encode_vector_y(x, y, d, g, bits, int(rotate), packed, meta, C.byref(a))
    return packed, meta, int(a.value)


def dequant_f64(packed, meta, d: int, g: int, bits: int, rotate: bool) -> np.ndarray:
    """z + s*q per group, un-rotated, in FP64."""
    out = np.zeros(d, dtype=np.float64)
    lib().rqo_dequant_f64(np.ascontiguousarray(packed, dtype=np.uint8),
                          np.ascontiguousarray(meta, dtype=np.uint16), d, g, bits, int(rotate), out)
    return out


def anchored(layout: dict) -> bool:
    return int(layout.get("ref_bits", 0)) > 0


def ref_group(layout: dict) -> int:
    return int(layout.get("ref_group") or layout["g"])


def group_len(layout: dict) -> int:
    """Loops per anchor group (Table 8 caption: each group of loops ends in one
    INT4 anchor); the whole schedule is one group unless group_loops is set."""
    return int(layout.get("group_loops") or layout["n_loops"])


class Planes:
    """One cache side (K or V), as numpy arrays in the contract layout: the
    BF16 reference and each residual loop's codes / meta / alpha planes; with
    a quantized anchor (ref_bits > 0) no reference plane, and codes / meta
    lists one longer, the anchor's planes last."""

    def __init__(self, n_loops, batch, heads, d, g, cap, bits, ref_bits=0, ref_group=None,
                 group_loops=0):
        ga = ref_group or g
        G = group_loops or n_loops
        shape = (batch, heads, cap)
        if not ref_bits:
            self.ref = np.zeros(shape + (d,), dtype=np.uint16)
            self.codes = [np.zeros(shape + (d * bits[l] // 8,), dtype=np.uint8) for l in range(n_loops - 1)]
            self.meta = [np.zeros(shape + (d // g, 2), dtype=np.uint16) for l in range(n_loops - 1)]
            self.alpha = [np.zeros(shape, dtype=np.uint16) for l in range(n_loops - 1)]
            return
        self.ref = None
        self.codes, self.meta, self.alpha = [], [], []
        for l in range(n_loops):
            if (l + 1) % G == 0:                 # the group's anchor
                self.codes.append(np.zeros(shape + (d * ref_bits // 8,), dtype=np.uint8))
                self.meta.append(np.zeros(shape + (d // ga, 2), dtype=np.uint16))
                self.alpha.append(None)
            else:
                self.codes.append(np.zeros(shape + (d * bits[l] // 8,), dtype=np.uint8))
                self.meta.append(np.zeros(shape + (d // g, 2), dtype=np.uint16))
                self.alpha.append(np.zeros(shape, dtype=np.uint16))


def _ptrs(arrs):
    return (C.c_void_p * max(1, len(arrs)))(*[a.ctypes.data for a in arrs])


def encode(layout: dict, planes: Planes, x_bits: np.ndarray, t0: int, n: int) -> None:
    """Encode tokens [t0, t0+n) into `planes` (in place).
    layout: dict(n_loops, batch, heads, d, g, cap, rotate, bits[, ref_bits,
    ref_group]).  BF16 reference: x_bits is bf16 bits [L-1, B, H, n, d] and
    planes.ref already holds the reference.  Quantized anchor: x_bits is
    [L, B, H, n, d], the anchor's input last."""
    L, B, H = layout["n_loops"], layout["batch"], layout["heads"]
    d, g, cap = layout["d"], layout["g"], layout["cap"]
    bits = np.ascontiguousarray(layout["bits"][:L - 1], dtype=np.int32)
    x = np.ascontiguousarray(x_bits, dtype=np.uint16)
    if anchored(layout):
        assert x.shape == (L, B, H, n, d)
        G = group_len(layout)
        for g0 in range(0, L, G):             # every group on its own
            cp, mp = _ptrs(planes.codes[g0:g0 + G]), _ptrs(planes.meta[g0:g0 + G])
            ap = _ptrs(planes.alpha[g0:g0 + G - 1])
            gbits = np.ascontiguousarray(layout["bits"][g0:g0 + G - 1], dtype=np.int32)
            lib().rqo_encode_anchored(G, B, H, d, g, ref_group(layout), int(layout["ref_bits"]), cap,
                                      int(layout["rotate"]), gbits, np.ascontiguousarray(x[g0:g0 + G]),
                                      t0, n, C.cast(cp, C.c_void_p), C.cast(mp, C.c_void_p),
                                      C.cast(ap, C.c_void_p))
        return
    cp, mp, ap = _ptrs(planes.codes), _ptrs(planes.meta), _ptrs(planes.alpha)
    assert x.shape == (L - 1, B, H, n, d)
    lib().rqo_encode(L, B, H, d, g, cap, int(layout["rotate"]), bits,
                     np.ascontiguousarray(planes.ref), x, t0, n,
                     C.cast(cp, C.c_void_p), C.cast(mp, C.c_void_p), C.cast(ap, C.c_void_p))


# ---------------------------------------------------------------------------
# reconstruction and attention (FP64)
# ---------------------------------------------------------------------------

def reconstruct(layout: dict, planes: Planes, loop: int, t0: int, n: int) -> np.ndarray:
    """x_hat of loop `loop` for tokens [t0, t0+n): float64 [B, H, n, d].
    BF16 reference: loop < L-1.  Quantized anchor: any loop; loop L-1 is the
    dequantized anchor."""
    L, B, H, d = layout["n_loops"], layout["batch"], layout["heads"], layout["d"]
    out = np.zeros((B, H, n, d), dtype=np.float64)
    if anchored(layout):
        G = group_len(layout)
        an = (loop // G) * G + G - 1         # the loop's anchor
        anchor = loop == an
        li = an - 1 if anchor else loop      # stand-in residual planes (unread for the anchor)
        lib().rqo_reconstruct_anchored(B, H, d, layout["g"], ref_group(layout),
                                       int(layout["ref_bits"]), layout["cap"],
                                       int(layout["rotate"]), int(layout["bits"][li]),
                                       planes.codes[an], planes.meta[an],
                                       planes.codes[li].ctypes.data, planes.meta[li].ctypes.data,
                                       planes.alpha[li].ctypes.data, -1 if anchor else loop,
                                       t0, n, out)
        return out
    lib().rqo_reconstruct(B, H, d, layout["g"], layout["cap"], int(layout["rotate"]),
                          int(layout["bits"][loop]), planes.ref, planes.codes[loop],
                          planes.meta[loop], planes.alpha[loop], t0, n, out)
    return out


def attention(q: np.ndarray, k: np.ndarray, v: np.ndarray, scale: float) -> np.ndarray:
    q = np.ascontiguousarray(q, dtype=np.float64)
    k = np.ascontiguousarray(k, dtype=np.float64)
    v = np.ascontiguousarray(v, dtype=np.float64)
    n, d = k.shape
    out = np.zeros(d, dtype=np.float64)
    lib().rqo_attention(q, k, v, n, d, float(scale), out)
    return out


def decode_row(layout: dict, kp: Planes, vp: Planes, q_bits: np.ndarray, loop: int,
               b: int, h: int, n_ctx: int, scale: float, tail_k=None, tail_v=None) -> np.ndarray:
    """Attention output (float64 [d]) of loop `loop`'s query for (b, h) over
    the n_ctx cached tokens and then the tail rows (bf16 bits [T, d] of this
    (loop, b, h)), if given."""
    L, B, H, d = layout["n_loops"], layout["batch"], layout["heads"], layout["d"]
    # One anchor group at a time: the C side sees the group's loops as a
    # schedule of G loops whose last is the reference.
    G = group_len(layout) if anchored(layout) else L
    g0 = (loop // G) * G
    an = g0 + G - 1
    # The reference loop attends over the reference alone; its residual plane
    # arguments are ignored by the C side, so the group's first planes stand in.
    li = g0 if loop == an else loop
    bits = int(layout["bits"][li])
    q_grp = np.ascontiguousarray(np.asarray(q_bits, dtype=np.uint16)[g0:g0 + G])
    out = np.zeros(d, dtype=np.float64)
    ptr = lambda a: None if a is None else np.ascontiguousarray(a).ctypes.data
    keep = []

    def tail(t):
        if t is None:
            return None
        t = np.ascontiguousarray(t, dtype=np.uint16)
        keep.append(t)
        return t.ctypes.data
    tk, tv = tail(tail_k), tail(tail_v)
    n_tail = 0 if tail_k is None else int(np.asarray(tail_k).shape[0])
    if anchored(layout):
        abits, ga = int(layout["ref_bits"]), ref_group(layout)
        anc = (kp.codes[an], kp.meta[an], vp.codes[an], vp.meta[an])
        kref = vref = None
    else:
        abits, ga = 0, layout["g"]
        anc = (None, None, None, None)
        kref, vref = kp.ref, vp.ref
    lib().rqo_decode_row_ex(G, B, H, d, layout["g"], layout["cap"], int(layout["rotate"]), bits,
                            ptr(kref), ptr(kp.codes[li]), ptr(kp.meta[li]), ptr(kp.alpha[li]),
                            ptr(vref), ptr(vp.codes[li]), ptr(vp.meta[li]), ptr(vp.alpha[li]),
                            ga, abits, *[ptr(x) for x in anc], tk, tv, n_tail,
                            q_grp, loop - g0, b, h, n_ctx, float(scale), out)
    return out


def decode(layout: dict, kp: Planes, vp: Planes, q_bits: np.ndarray, loop_mask: int,
           n_ctx: int, scale: float, tail_k=None, tail_v=None) -> np.ndarray:
    """All rows: float64 [L, B, H, d]; rows of loops not in the mask are NaN.
    tail_k / tail_v: optional bf16 bits [L, B, H, T, d]."""
    L, B, H, d = layout["n_loops"], layout["batch"], layout["heads"], layout["d"]
    out = np.full((L, B, H, d), np.nan, dtype=np.float64)
    for l in range(L):
        if not (loop_mask >> l) & 1:
            continue
        for b in range(B):
            for h in range(H):
                tk = None if tail_k is None else tail_k[l, b, h]
                tv = None if tail_v is None else tail_v[l, b, h]
                out[l, b, h] = decode_row(layout, kp, vp, q_bits, l, b, h, n_ctx, scale, tk, tv)
    return out
