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
                                                 C.c_void_p, C.c_void_p, C.c_void_p, C.c_int]
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
                                                          C.c_void_p, C.c_void_p, C.c_void_p, C.c_int]
        L.rqo_alpha_mode_f32_y.restype = C.c_float
        L.rqo_alpha_mode_f32_y.argtypes = [_u16p, _f32p, C.c_int, C.c_int]
        L.rqo_dequant_f64.restype = None
        L.rqo_dequant_f64.argtypes = [_u8p, _u16p, C.c_int, C.c_int, C.c_int, C.c_int, _f64p]
        L.rqo_reconstruct_anchored.restype = None
        L.rqo_reconstruct_anchored.argtypes = ([C.c_int] * 9 + [_u8p, _u16p, C.c_void_p, C.c_void_p,
                                                                C.c_void_p, C.c_int, C.c_int,
                                                                C.c_int, _f64p])
        L.rqo_encode_chain.restype = None
        L.rqo_encode_chain.argtypes = ([C.c_int] * 10 + [_i32p, C.c_int, _i32p, C.c_void_p, _u16p,
                                                         C.c_int, C.c_int, C.c_void_p, C.c_void_p,
                                                         C.c_void_p])
        L.rqo_chain_rows.restype = None
        L.rqo_chain_rows.argtypes = ([C.c_int] * 6 + [_i32p, _i32p, C.c_int, C.c_void_p, C.c_void_p,
                                                      C.c_void_p, C.c_void_p, C.c_void_p, C.c_void_p,
                                                      C.c_int, C.c_int, C.c_int, _f64p])
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


def alpha_mode(layout: dict) -> int:
    """0: least squares, 1: alpha = 1, 2: norm ratio (Table 9's columns)."""
    return int(layout.get("alpha_mode", 0))


def alpha_mode_f32(x_bits, y_f32, mode: int) -> float:
    x = np.ascontiguousarray(x_bits, dtype=np.uint16)
    y = np.ascontiguousarray(y_f32, dtype=np.float32)
    return float(lib().rqo_alpha_mode_f32_y(x, y, x.size, int(mode)))


def group_len(layout: dict) -> int:
    """Loops per anchor group (Table 8 caption: each group of loops ends in one
    INT4 anchor); the whole schedule is one group unless group_loops is set."""
    return int(layout.get("group_loops") or layout["n_loops"])


def ref_first(layout: dict) -> bool:
    """First-loop reference policy (the pages' Table 1 / Table 9): each group's
    first loop is its reference instead of its last."""
    return bool(layout.get("ref_first", 0))


def anchor_loop(layout: dict, l: int) -> int:
    """The reference loop of loop l's group."""
    G = group_len(layout) if anchored(layout) else layout["n_loops"]
    g0 = (l // G) * G
    return g0 if ref_first(layout) else g0 + G - 1


def ref_chain(layout: dict) -> bool:
    """Chained references (Table 9 "Previous-loop" / "Next-loop"): each loop's
    reference is its neighbour towards the group's root loop."""
    return bool(layout.get("ref_chain", 0))


def chain_order(layout: dict, l: int):
    """(g0, root, order) of loop l's group: the group's first loop, its root
    (reference) loop, and its residual loops from the root outwards."""
    G = group_len(layout) if anchored(layout) else layout["n_loops"]
    g0 = (l // G) * G
    root = anchor_loop(layout, g0)
    if ref_first(layout):
        order = list(range(g0 + 1, g0 + G))
    else:
        order = list(range(g0 + G - 2, g0 - 1, -1))
    return g0, root, order


def _pp(arrs):
    """Array of pointers; None entries become NULL."""
    return (C.c_void_p * max(1, len(arrs)))(*[0 if a is None else a.ctypes.data for a in arrs])


def _chain_rows(layout: dict, planes: "Planes", loop: int, bh: int, t0: int, n: int) -> np.ndarray:
    g0, root, order = chain_order(layout, loop)
    G = len(order) + 1
    d = layout["d"]
    bits = np.ascontiguousarray([layout["bits"][g0 + i] if g0 + i != root else 0 for i in range(G)],
                                dtype=np.int32)
    ordi = np.ascontiguousarray([l - g0 for l in order], dtype=np.int32)
    upto = -1 if loop == root else order.index(loop)
    out = np.zeros((n, d), dtype=np.float64)
    ab = int(layout.get("ref_bits", 0))
    grp = lambda lst: [lst[g0 + i] for i in range(G)]
    lib().rqo_chain_rows(d, layout["g"], ref_group(layout), ab, layout["cap"], int(layout["rotate"]),
                         bits, ordi, upto,
                         None if ab else planes.ref.ctypes.data,
                         planes.codes[root].ctypes.data if ab else None,
                         planes.meta[root].ctypes.data if ab else None,
                         C.cast(_pp(grp(planes.codes)), C.c_void_p), C.cast(_pp(grp(planes.meta)), C.c_void_p),
                         C.cast(_pp(grp(planes.alpha)), C.c_void_p), bh, t0, n, out)
    return out


def group_order(layout: dict, l: int):
    """The loops of loop l's group as the C side takes them: the group's
    residual loops in loop order, then its reference."""
    G = group_len(layout) if anchored(layout) else layout["n_loops"]
    g0 = (l // G) * G
    an = anchor_loop(layout, g0)
    return [l for l in range(g0, g0 + G) if l != an] + [an]


class Planes:
    """One cache side (K or V), as numpy arrays in the contract layout, lists
    indexed by loop.  BF16 reference: `ref` holds it and its loop's entries are
    None.  Quantized anchors: no `ref`; an anchor loop's codes / meta are in
    the anchor format and its alpha is None."""

    def __init__(self, n_loops, batch, heads, d, g, cap, bits, ref_bits=0, ref_group=None,
                 group_loops=0, ref_first=0):
        ga = ref_group or g
        G = (group_loops or n_loops) if ref_bits else n_loops
        shape = (batch, heads, cap)
        self.ref = None if ref_bits else np.zeros(shape + (d,), dtype=np.uint16)
        self.codes, self.meta, self.alpha = [], [], []
        for l in range(n_loops):
            g0 = (l // G) * G
            if l == (g0 if ref_first else g0 + G - 1):          # a reference loop
                if ref_bits:
                    self.codes.append(np.zeros(shape + (d * ref_bits // 8,), dtype=np.uint8))
                    self.meta.append(np.zeros(shape + (d // ga, 2), dtype=np.uint16))
                else:
                    self.codes.append(None)
                    self.meta.append(None)
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
    ref_group, group_loops, ref_first, alpha_mode]).  BF16 reference: x_bits
    is bf16 bits [L-1, B, H, n, d], the non-reference loops in loop order, and
    planes.ref already holds the reference.  Quantized anchors: x_bits is
    [L, B, H, n, d], every loop in loop order."""
    L, B, H = layout["n_loops"], layout["batch"], layout["heads"]
    d, g, cap = layout["d"], layout["g"], layout["cap"]
    x = np.ascontiguousarray(x_bits, dtype=np.uint16)
    if ref_chain(layout):
        G = group_len(layout) if anchored(layout) else L
        if anchored(layout):
            assert x.shape == (L, B, H, n, d)
        else:
            assert x.shape == (L - 1, B, H, n, d)
            root = anchor_loop(layout, 0)
            full = np.zeros((L, B, H, n, d), dtype=np.uint16)
            full[[l for l in range(L) if l != root]] = x
            x = full
        for g0 in range(0, L, G):
            _, root, order = chain_order(layout, g0)
            bits = np.ascontiguousarray([layout["bits"][g0 + i] if g0 + i != root else 0 for i in range(G)],
                                        dtype=np.int32)
            ordi = np.ascontiguousarray([l - g0 for l in order], dtype=np.int32)
            grp = lambda lst: [lst[g0 + i] for i in range(G)]
            lib().rqo_encode_chain(G, B, H, d, g, ref_group(layout), int(layout.get("ref_bits", 0)), cap,
                                   int(layout["rotate"]), alpha_mode(layout), bits, root - g0, ordi,
                                   None if anchored(layout) else planes.ref.ctypes.data,
                                   np.ascontiguousarray(x[g0:g0 + G]), t0, n,
                                   C.cast(_pp(grp(planes.codes)), C.c_void_p),
                                   C.cast(_pp(grp(planes.meta)), C.c_void_p),
                                   C.cast(_pp(grp(planes.alpha)), C.c_void_p))
        return
    if anchored(layout):
        assert x.shape == (L, B, H, n, d)
        G = group_len(layout)
        for g0 in range(0, L, G):             # every group on its own
            order = group_order(layout, g0)
            res = order[:-1]
            cp, mp = _ptrs([planes.codes[l] for l in order]), _ptrs([planes.meta[l] for l in order])
            ap = _ptrs([planes.alpha[l] for l in res])
            gbits = np.ascontiguousarray([layout["bits"][l] for l in res], dtype=np.int32)
            lib().rqo_encode_anchored(G, B, H, d, g, ref_group(layout), int(layout["ref_bits"]), cap,
                                      int(layout["rotate"]), gbits, np.ascontiguousarray(x[order]),
                                      t0, n, C.cast(cp, C.c_void_p), C.cast(mp, C.c_void_p),
                                      C.cast(ap, C.c_void_p), alpha_mode(layout))
        return
    assert x.shape == (L - 1, B, H, n, d)
    res = group_order(layout, 0)[:-1]
    bits = np.ascontiguousarray([layout["bits"][l] for l in res], dtype=np.int32)
    cp = _ptrs([planes.codes[l] for l in res])
    mp = _ptrs([planes.meta[l] for l in res])
    ap = _ptrs([planes.alpha[l] for l in res])
    lib().rqo_encode(L, B, H, d, g, cap, int(layout["rotate"]), bits,
                     np.ascontiguousarray(planes.ref), x, t0, n,
                     C.cast(cp, C.c_void_p), C.cast(mp, C.c_void_p), C.cast(ap, C.c_void_p),
                     alpha_mode(layout))


# ---------------------------------------------------------------------------
# reconstruction and attention (FP64)
# ---------------------------------------------------------------------------

def reconstruct(layout: dict, planes: Planes, loop: int, t0: int, n: int) -> np.ndarray:
    """x_hat of loop `loop` for tokens [t0, t0+n): float64 [B, H, n, d].
    BF16 reference: a residual loop.  Quantized anchors: any loop; an anchor
    loop gives the dequantized anchor."""
    B, H, d = layout["batch"], layout["heads"], layout["d"]
    out = np.zeros((B, H, n, d), dtype=np.float64)
    an = anchor_loop(layout, loop)
    if ref_chain(layout):
        assert anchored(layout) or loop != an, "the BF16 reference is not reconstructed"
        for b in range(B):
            for h in range(H):
                out[b, h] = _chain_rows(layout, planes, loop, b * H + h, t0, n)
        return out
    if anchored(layout):
        anchor = loop == an
        li = group_order(layout, an)[0] if anchor else loop     # stand-in, unread for the anchor
        lib().rqo_reconstruct_anchored(B, H, d, layout["g"], ref_group(layout),
                                       int(layout["ref_bits"]), layout["cap"],
                                       int(layout["rotate"]), int(layout["bits"][li]),
                                       planes.codes[an], planes.meta[an],
                                       planes.codes[li].ctypes.data, planes.meta[li].ctypes.data,
                                       planes.alpha[li].ctypes.data, -1 if anchor else loop,
                                       t0, n, out)
        return out
    assert loop != an, "the BF16 reference is not reconstructed"
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
    B, H, d = layout["batch"], layout["heads"], layout["d"]
    if ref_chain(layout):
        k = _chain_rows(layout, kp, loop, b * H + h, 0, n_ctx)
        v = _chain_rows(layout, vp, loop, b * H + h, 0, n_ctx)
        if tail_k is not None:
            k = np.concatenate([k, bf16_bits_to_f32(np.asarray(tail_k).ravel()).reshape(-1, d).astype(np.float64)])
            v = np.concatenate([v, bf16_bits_to_f32(np.asarray(tail_v).ravel()).reshape(-1, d).astype(np.float64)])
        qv = bf16_bits_to_f32(np.asarray(q_bits, dtype=np.uint16)[loop, b, h]).astype(np.float64)
        return attention(qv, k, v, scale)
    an = anchor_loop(layout, loop)
    is_ref = loop == an
    # The C side sees a schedule of G loops whose last is the reference: the
    # row's loop is either that reference or a residual (view index 0, with
    # its own planes); every view loop carries this loop's query.
    G = len(group_order(layout, an))
    li = group_order(layout, an)[0] if is_ref else loop
    c_loop = G - 1 if is_ref else 0
    bits = int(layout["bits"][li])
    q = np.asarray(q_bits, dtype=np.uint16)
    q_view = np.ascontiguousarray(np.repeat(q[loop][None], G, axis=0))
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
                            q_view, c_loop, b, h, n_ctx, float(scale), out)
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
