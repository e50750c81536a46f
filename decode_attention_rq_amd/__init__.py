"""Python binding of librq.so: ResidualQuant KV cache on MI355X (gfx950).

Argument marshalling only: every step of encode, reconstruction and decode
runs in the library's HIP kernels (see include/rq.h).  torch supplies device
memory and the stream.  Importing this module fails if librq.so has not been
built (python decode_attention_rq_amd/build.py, or __graft_entry__.build()).

Before each call the binding checks every tensor against the layout it is
passed with: dtype, exact shape, contiguity, and (when a GPU is present)
that it lives on the GPU; a mismatch raises ValueError and nothing is
called.  The library itself checks pointers, alignment and ranges.
"""
from __future__ import annotations

import ctypes as C
import os
from dataclasses import dataclass, field
from typing import List, Optional, Sequence

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "librq.so")
RQ_MAX_LOOPS = 32

if not os.path.exists(LIB_PATH):
    raise ImportError(f"{LIB_PATH} is missing: build it with `python decode_attention_rq_amd/build.py`")

_lib = C.CDLL(LIB_PATH)


class rq_layout(C.Structure):
    _fields_ = [("n_loops", C.c_int32), ("batch", C.c_int32), ("n_heads", C.c_int32),
                ("head_dim", C.c_int32), ("group", C.c_int32), ("capacity", C.c_int32),
                ("rotate", C.c_int32), ("bits", C.c_int32 * RQ_MAX_LOOPS),
                ("ref_bits", C.c_int32), ("ref_group", C.c_int32), ("group_loops", C.c_int32),
                ("ref_first", C.c_int32), ("alpha_mode", C.c_int32), ("ref_chain", C.c_int32)]


class rq_cache(C.Structure):
    _fields_ = [("ref", C.c_void_p), ("codes", C.c_void_p * RQ_MAX_LOOPS),
                ("meta", C.c_void_p * RQ_MAX_LOOPS), ("alpha", C.c_void_p * RQ_MAX_LOOPS)]


class rq_tail(C.Structure):
    _fields_ = [("k", C.c_void_p * RQ_MAX_LOOPS), ("v", C.c_void_p * RQ_MAX_LOOPS),
                ("capacity", C.c_int32), ("n", C.c_int32)]


_P = C.POINTER
_lib.rq_status_string.restype = C.c_char_p
_lib.rq_status_string.argtypes = [C.c_int]
_lib.rq_encode.restype = C.c_int
_lib.rq_encode.argtypes = [_P(rq_layout), _P(rq_cache), _P(rq_cache), C.c_void_p, C.c_void_p,
                           C.c_int32, C.c_int32, C.c_void_p]
_lib.rq_decode_workspace_bytes.restype = C.c_size_t
_lib.rq_decode_workspace_bytes.argtypes = [_P(rq_layout), C.c_int32, C.c_int32]
_lib.rq_decode_splits.restype = C.c_int32
_lib.rq_decode_splits.argtypes = [_P(rq_layout), C.c_int32]
_lib.rq_decode_attn.restype = C.c_int
_lib.rq_decode_attn.argtypes = [_P(rq_layout), _P(rq_cache), _P(rq_cache), C.c_void_p, C.c_uint32,
                                C.c_int32, C.c_float, C.c_int32, C.c_void_p, C.c_void_p,
                                C.c_size_t, C.c_void_p]
_lib.rq_decode_attn_tail.restype = C.c_int
_lib.rq_decode_attn_tail.argtypes = [_P(rq_layout), _P(rq_cache), _P(rq_cache), _P(rq_tail), C.c_void_p,
                                     C.c_uint32, C.c_int32, C.c_float, C.c_int32, C.c_void_p,
                                     C.c_void_p, C.c_size_t, C.c_void_p]
_lib.rq_decode_attn_tail_noalloc.restype = C.c_int
_lib.rq_decode_attn_tail_noalloc.argtypes = [_P(rq_layout), _P(rq_cache), _P(rq_cache), _P(rq_tail), C.c_void_p,
                                             C.c_uint32, C.c_int32, C.c_float, C.c_int32, C.c_void_p,
                                             C.c_void_p]
_lib.rq_bf16_decode_attn.restype = C.c_int
_lib.rq_bf16_decode_attn.argtypes = [_P(rq_layout), _P(C.c_void_p), _P(C.c_void_p), C.c_void_p,
                                     C.c_uint32, C.c_int32, C.c_float, C.c_int32, C.c_void_p,
                                     C.c_void_p, C.c_size_t, C.c_void_p]
_lib.rq_probe_read_stream.restype = C.c_int
_lib.rq_probe_read_stream.argtypes = [C.c_void_p, C.c_size_t, C.c_int32, C.c_int32, C.c_int32, C.c_void_p,
                                      C.c_void_p]
_lib.rq_reconstruct.restype = C.c_int
_lib.rq_reconstruct.argtypes = [_P(rq_layout), _P(rq_cache), C.c_int32, C.c_int32, C.c_int32,
                                C.c_void_p, C.c_void_p]

STATUS = {0: "RQ_OK", -1: "RQ_ERR_INVALID_ARG", -2: "RQ_ERR_UNSUPPORTED", -3: "RQ_ERR_WORKSPACE",
          -4: "RQ_ERR_DEVICE"}


class RQError(RuntimeError):
    def __init__(self, status: int):
        self.status = status
        super().__init__(rq_status_string(status))


def rq_status_string(status: int) -> str:
    return _lib.rq_status_string(int(status)).decode()


def _check(status: int) -> None:
    if status != 0:
        raise RQError(status)


_GPU = None        # whether a GPU is present (looked up once)


def _gpu_present() -> bool:
    global _GPU
    if _GPU is None:
        _GPU = torch.cuda.is_available()
    return _GPU


def _tensor(t, name: str, dtype, shape=None, allow_none: bool = False) -> None:
    """ValueError unless t is a contiguous tensor of `dtype` and exactly
    `shape` (None: any shape), on the GPU when one is present."""
    if t is None:
        if allow_none:
            return
        raise ValueError(f"{name}: a tensor is required")
    if not isinstance(t, torch.Tensor):
        raise ValueError(f"{name}: expected a torch.Tensor, got {type(t).__name__}")
    if t.dtype != dtype:
        raise ValueError(f"{name}: dtype {t.dtype}, expected {dtype}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name}: shape {tuple(t.shape)}, expected {tuple(shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name}: must be contiguous")
    if not t.is_cuda and _gpu_present():
        raise ValueError(f"{name}: must be a GPU tensor (device {t.device})")


def _plane_key(t: torch.Tensor) -> tuple:
    """What a checked plane's validity depends on: the tensor, its data
    pointer and its version counter (which in-place changes of its shape or
    strides, and in-place writes through torch, advance)."""
    return (id(t), t.data_ptr(), t._version)


def _check_cache(layout: "Layout", c: "Cache", name: str) -> "rq_cache":
    """Every plane of c present has the dtype and shape `layout` gives it.
    Checked once per (layout, planes) pair: the result is kept on the cache
    object, keyed by the layout's fields and every plane's identity, data
    pointer and version counter (a plane replaced, or resized or restrided in
    place, is checked again).  Returns the cache's C struct."""
    fp = c._fingerprint()
    key = (layout._key(), fp)
    if getattr(c, "_checked", None) != key:
        _check_cache_planes(layout, c, name)
        c._checked = key
    return c.c(fp)


def _check_cache_planes(layout: "Layout", c: "Cache", name: str) -> None:
    B, H, d, cap = layout.batch, layout.n_heads, layout.head_dim, layout.capacity
    if len(c.codes) != layout.n_loops or len(c.meta) != layout.n_loops or len(c.alpha) != layout.n_loops:
        raise ValueError(f"{name}: planes for {len(c.codes)} loops, layout has {layout.n_loops}")
    if not layout.ref_bits:
        _tensor(c.ref, f"{name}.ref", torch.bfloat16, (B, H, cap, d), allow_none=True)
    for l in range(layout.n_loops):
        if layout.is_anchor(l):
            if layout.ref_bits:
                ga = layout.anchor_group
                _tensor(c.codes[l], f"{name}.codes[{l}]", torch.uint8, (B, H, cap, d * layout.ref_bits // 8), True)
                _tensor(c.meta[l], f"{name}.meta[{l}]", torch.float16, (B, H, cap, d // ga, 2), True)
            continue
        bits = int(layout.bits[l]) if l < len(layout.bits) else 0
        if bits not in (2, 4):
            continue            # the library reports the unsupported width
        _tensor(c.codes[l], f"{name}.codes[{l}]", torch.uint8, (B, H, cap, d * bits // 8), True)
        _tensor(c.meta[l], f"{name}.meta[{l}]", torch.float16, (B, H, cap, d // layout.group, 2), True)
        _tensor(c.alpha[l], f"{name}.alpha[{l}]", torch.float16, (B, H, cap), True)


def _check_rows(layout: "Layout", t, name: str, dtype) -> None:
    """One row per (loop, batch, head): [L, B, H, d]."""
    _tensor(t, name, dtype, (layout.n_loops, layout.batch, layout.n_heads, layout.head_dim))


def _check_workspace(ws) -> None:
    _tensor(ws, "workspace", ws.dtype if isinstance(ws, torch.Tensor) else torch.uint8)


@dataclass
class Layout:
    """Shape of one layer's cache (mirrors rq_layout)."""
    n_loops: int
    batch: int
    n_heads: int
    head_dim: int
    group: int
    capacity: int
    rotate: int = 1
    bits: Sequence[int] = field(default_factory=list)   # per residual loop
    ref_bits: int = 0        # 0: BF16 reference; 2 or 4: quantized anchor
    ref_group: int = 0       # the anchor's group size (0: group)
    group_loops: int = 0     # loops per anchor group (0: all loops, one group)
    ref_first: int = 0       # 1: each group's first loop is its reference
    alpha_mode: int = 0      # 0 least squares, 1 alpha = 1, 2 norm ratio
    ref_chain: int = 0       # 1: each loop refers to its neighbour towards the reference

    @property
    def anchor_group(self) -> int:
        return self.ref_group or self.group

    def is_anchor(self, l: int) -> bool:
        """Loop l is its group's reference (its first or last loop)."""
        G = self.group_loops or self.n_loops
        return l % G == (0 if self.ref_first else G - 1)

    def _key(self) -> tuple:
        return (self.n_loops, self.batch, self.n_heads, self.head_dim, self.group, self.capacity, self.rotate,
                tuple(self.bits), self.ref_bits, self.ref_group, self.group_loops, self.ref_first,
                self.alpha_mode, self.ref_chain)

    def c(self) -> rq_layout:
        """The C struct (built once per set of field values)."""
        key = self._key()
        memo = self.__dict__.get("_c_memo")
        if memo is not None and memo[0] == key:
            return memo[1]
        s = rq_layout(self.n_loops, self.batch, self.n_heads, self.head_dim, self.group,
                      self.capacity, self.rotate)
        for i, b in enumerate(list(self.bits)[:RQ_MAX_LOOPS]):
            s.bits[i] = int(b)
        s.ref_bits = int(self.ref_bits)
        s.ref_group = int(self.ref_group)
        s.group_loops = int(self.group_loops)
        s.ref_first = int(self.ref_first)
        s.alpha_mode = int(self.alpha_mode)
        s.ref_chain = int(self.ref_chain)
        self.__dict__["_c_memo"] = (key, s)
        return s


class Cache:
    """One side (K or V) of a layer's cache: torch tensors in the plane layout
    of include/rq.h (the library reads and writes them in place).  codes /
    meta / alpha are indexed by loop.  With a BF16 reference, `ref` holds it and
    the reference loop's entries are None.  With quantized anchors there is no
    `ref` (None); every anchor loop has anchor-format codes / meta and alpha
    None."""

    def __init__(self, layout: Layout, device="cuda", ref: Optional[torch.Tensor] = None,
                 zero: bool = True):
        """zero=False leaves the planes uninitialised (for callers that write
        every slot they later read)."""
        L, B, H, d, g, cap = (layout.n_loops, layout.batch, layout.n_heads, layout.head_dim,
                              layout.group, layout.capacity)
        new = torch.zeros if zero else torch.empty
        self.layout = layout
        self.codes: List[torch.Tensor] = []
        self.meta: List[torch.Tensor] = []
        self.alpha: List[Optional[torch.Tensor]] = []
        if layout.ref_bits:
            self.ref = None
            ga = layout.anchor_group
            for l in range(L):
                if layout.is_anchor(l):
                    self.codes.append(new(B, H, cap, d * layout.ref_bits // 8, dtype=torch.uint8, device=device))
                    self.meta.append(new(B, H, cap, d // ga, 2, dtype=torch.float16, device=device))
                    self.alpha.append(None)
                else:
                    self.codes.append(new(B, H, cap, d * layout.bits[l] // 8, dtype=torch.uint8, device=device))
                    self.meta.append(new(B, H, cap, d // g, 2, dtype=torch.float16, device=device))
                    self.alpha.append(new(B, H, cap, dtype=torch.float16, device=device))
        else:
            self.ref = ref if ref is not None else new(B, H, cap, d, dtype=torch.bfloat16, device=device)
            for l in range(L):
                if layout.is_anchor(l):
                    self.codes.append(None)
                    self.meta.append(None)
                    self.alpha.append(None)
                else:
                    self.codes.append(new(B, H, cap, d * layout.bits[l] // 8, dtype=torch.uint8, device=device))
                    self.meta.append(new(B, H, cap, d // g, 2, dtype=torch.float16, device=device))
                    self.alpha.append(new(B, H, cap, dtype=torch.float16, device=device))

    def _fingerprint(self) -> tuple:
        """_plane_key of every plane (absent planes: None): a plane replaced,
        or resized or restrided in place, changes it."""
        return tuple(None if t is None else _plane_key(t)
                     for t in [self.ref, *self.codes, *self.meta, *self.alpha])

    def c(self, fp: Optional[tuple] = None) -> rq_cache:
        """The C struct (rebuilt when a plane is replaced); fp: this cache's
        _fingerprint() if the caller has it."""
        fp = fp if fp is not None else self._fingerprint()
        memo = self.__dict__.get("_c_memo")
        if memo is not None and memo[0] == fp:
            return memo[1]
        s = rq_cache()
        s.ref = _ptr(self.ref)
        for l in range(len(self.codes)):
            s.codes[l] = _ptr(self.codes[l])
            s.meta[l] = _ptr(self.meta[l])
        for l in range(len(self.alpha)):
            s.alpha[l] = _ptr(self.alpha[l])
        self.__dict__["_c_memo"] = (fp, s)
        return s

    def batch_view(self, b0: int, b1: int, layout: Layout) -> "Cache":
        """The same planes restricted to batch entries [b0, b1) (batch is the
        outermost plane axis, so the view is contiguous), for `layout` with
        batch = b1 - b0."""
        v = Cache.__new__(Cache)
        v.layout = layout
        v.ref = None if self.ref is None else self.ref[b0:b1]
        v.codes = [None if t is None else t[b0:b1] for t in self.codes]
        v.meta = [None if t is None else t[b0:b1] for t in self.meta]
        v.alpha = [None if t is None else t[b0:b1] for t in self.alpha]
        return v

    def nbytes(self) -> int:
        t = ([] if self.ref is None else [self.ref]) + self.codes + self.meta + self.alpha
        return sum(x.numel() * x.element_size() for x in t if x is not None)


def _stream(stream) -> int:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def _ptr(t: Optional[torch.Tensor]) -> int:
    return 0 if t is None else t.data_ptr()


def rq_encode(layout: Layout, k: Cache, v: Cache, k_in: torch.Tensor, v_in: torch.Tensor,
              t0: int, n: int, stream=None) -> None:
    """k_in / v_in: bf16 [L-1, B, H, n, d] contiguous, the loops other than
    the BF16 reference in loop order; with quantized anchors [L, B, H, n, d]
    (every loop, anchors included, in loop order)."""
    kc = _check_cache(layout, k, "k")
    vc = _check_cache(layout, v, "v")
    loops = layout.n_loops if layout.ref_bits else layout.n_loops - 1
    shape = (loops, layout.batch, layout.n_heads, int(n), layout.head_dim) if n > 0 else None
    _tensor(k_in, "k_in", torch.bfloat16, shape)
    _tensor(v_in, "v_in", torch.bfloat16, shape)
    lay = layout.c()
    _check(_lib.rq_encode(C.byref(lay), C.byref(kc), C.byref(vc), _ptr(k_in), _ptr(v_in),
                          int(t0), int(n), _stream(stream)))


def rq_decode_workspace_bytes(layout: Layout, n_ctx: int, n_splits: int = 0) -> int:
    lay = layout.c()
    return int(_lib.rq_decode_workspace_bytes(C.byref(lay), int(n_ctx), int(n_splits)))


def rq_decode_splits(layout: Layout, n_ctx: int) -> int:
    lay = layout.c()
    s = int(_lib.rq_decode_splits(C.byref(lay), int(n_ctx)))
    if s < 0:
        raise RQError(s)
    return s


def rq_decode_attn(layout: Layout, k: Cache, v: Cache, q: torch.Tensor, loop_mask: int, n_ctx: int,
                   sm_scale: float, out: torch.Tensor, workspace: torch.Tensor, n_splits: int = 0,
                   stream=None) -> None:
    """q: bf16 [L, B, H, d]; out: f32 [L, B, H, d]; workspace: device bytes."""
    kc = _check_cache(layout, k, "k")
    vc = _check_cache(layout, v, "v")
    _check_rows(layout, q, "q", torch.bfloat16)
    _check_rows(layout, out, "out", torch.float32)
    _check_workspace(workspace)
    lay = layout.c()
    _check(_lib.rq_decode_attn(C.byref(lay), C.byref(kc), C.byref(vc), _ptr(q), int(loop_mask),
                               int(n_ctx), float(sm_scale), int(n_splits), _ptr(out), _ptr(workspace),
                               workspace.numel() * workspace.element_size(), _stream(stream)))


class Tail:
    """Recent BF16 tokens per loop: k[l], v[l] bf16 [B, H, capacity, d]
    (None for loops never attended); n tokens [0, n) are attended."""

    def __init__(self, k: Sequence[Optional[torch.Tensor]], v: Sequence[Optional[torch.Tensor]], n: int):
        """Every plane present must have the same capacity (the library reads
        all of them with one row stride)."""
        self.k, self.v, self.n = list(k), list(v), int(n)
        caps = {int(t.shape[2]) for t in self.k + self.v if t is not None and t.dim() == 4}
        if len(caps) > 1:
            raise ValueError(f"tail planes of different capacities {sorted(caps)}")
        self.capacity = caps.pop() if caps else 0
        if self.n < 0 or self.n > self.capacity:
            raise ValueError(f"tail: n = {self.n} outside [0, capacity {self.capacity}]")

    def _fingerprint(self) -> tuple:
        return (self.n, self.capacity) + tuple(None if t is None else _plane_key(t)
                                               for t in [*self.k, *self.v])

    def check(self, layout: "Layout") -> "rq_tail":
        """Check the planes against `layout` (once per layout and set of
        planes, as for a cache); returns the C struct."""
        fp = self._fingerprint()
        key = (layout._key(), fp)
        if self.__dict__.get("_checked") != key:
            self._check_planes(layout)
            self.__dict__["_checked"] = key
        return self.c(fp)

    def _check_planes(self, layout: "Layout") -> None:
        for side, planes in (("k", self.k), ("v", self.v)):
            for l, t in enumerate(planes):
                _tensor(t, f"tail.{side}[{l}]", torch.bfloat16,
                        (layout.batch, layout.n_heads, self.capacity, layout.head_dim), allow_none=True)

    def c(self, fp: Optional[tuple] = None) -> rq_tail:
        fp = fp if fp is not None else self._fingerprint()
        memo = self.__dict__.get("_c_memo")
        if memo is not None and memo[0] == fp:
            return memo[1]
        s = rq_tail()
        for l, t in enumerate(self.k):
            s.k[l] = _ptr(t)
        for l, t in enumerate(self.v):
            s.v[l] = _ptr(t)
        s.capacity = self.capacity
        s.n = self.n
        self.__dict__["_c_memo"] = (fp, s)
        return s


def rq_decode_attn_tail(layout: Layout, k: Cache, v: Cache, tail: Optional[Tail], q: torch.Tensor,
                        loop_mask: int, n_ctx: int, sm_scale: float, out: torch.Tensor,
                        workspace: torch.Tensor, n_splits: int = 0, stream=None) -> None:
    """rq_decode_attn over n_ctx cached tokens followed by tail.n BF16 tokens."""
    kc = _check_cache(layout, k, "k")
    vc = _check_cache(layout, v, "v")
    _check_rows(layout, q, "q", torch.bfloat16)
    _check_rows(layout, out, "out", torch.float32)
    _check_workspace(workspace)
    tc = tail.check(layout) if tail is not None else None
    lay = layout.c()
    _check(_lib.rq_decode_attn_tail(C.byref(lay), C.byref(kc), C.byref(vc),
                                    C.byref(tc) if tc is not None else None, _ptr(q),
                                    int(loop_mask), int(n_ctx), float(sm_scale), int(n_splits),
                                    _ptr(out), _ptr(workspace),
                                    workspace.numel() * workspace.element_size(), _stream(stream)))


NOALLOC_SCRATCH_BYTES = 32 << 20      # RQ_NOALLOC_SCRATCH_BYTES


def rq_decode_attn_tail_noalloc(layout: Layout, k: Cache, v: Cache, tail: Optional[Tail], q: torch.Tensor,
                                loop_mask: int, n_ctx: int, sm_scale: float, out: torch.Tensor,
                                n_splits: int = 0, stream=None) -> None:
    """rq_decode_attn_tail with the split records in the library's per-GPU
    scratch instead of a caller workspace: nothing is allocated.  Calls that
    may overlap on one GPU race on that scratch."""
    kc = _check_cache(layout, k, "k")
    vc = _check_cache(layout, v, "v")
    _check_rows(layout, q, "q", torch.bfloat16)
    _check_rows(layout, out, "out", torch.float32)
    tc = tail.check(layout) if tail is not None else None
    lay = layout.c()
    _check(_lib.rq_decode_attn_tail_noalloc(C.byref(lay), C.byref(kc), C.byref(vc),
                                            C.byref(tc) if tc is not None else None, _ptr(q),
                                            int(loop_mask), int(n_ctx), float(sm_scale), int(n_splits),
                                            _ptr(out), _stream(stream)))


def rq_bf16_decode_attn(layout: Layout, k_loops: Sequence[torch.Tensor], v_loops: Sequence[torch.Tensor],
                        q: torch.Tensor, loop_mask: int, n_ctx: int, sm_scale: float, out: torch.Tensor,
                        workspace: torch.Tensor, n_splits: int = 0, stream=None) -> None:
    """BF16-KV baseline: k_loops / v_loops are n_loops bf16 [B, H, cap, d] tensors."""
    shape = (layout.batch, layout.n_heads, layout.capacity, layout.head_dim)
    if len(k_loops) != layout.n_loops or len(v_loops) != layout.n_loops:
        raise ValueError(f"k_loops / v_loops: {layout.n_loops} entries expected")
    for l in range(layout.n_loops):
        _tensor(k_loops[l], f"k_loops[{l}]", torch.bfloat16, shape, allow_none=True)
        _tensor(v_loops[l], f"v_loops[{l}]", torch.bfloat16, shape, allow_none=True)
    _check_rows(layout, q, "q", torch.bfloat16)
    _check_rows(layout, out, "out", torch.float32)
    _check_workspace(workspace)
    lay = layout.c()
    kp = (C.c_void_p * layout.n_loops)(*[_ptr(t) for t in k_loops])
    vp = (C.c_void_p * layout.n_loops)(*[_ptr(t) for t in v_loops])
    _check(_lib.rq_bf16_decode_attn(C.byref(lay), kp, vp, _ptr(q), int(loop_mask), int(n_ctx),
                                    float(sm_scale), int(n_splits), _ptr(out), _ptr(workspace),
                                    workspace.numel() * workspace.element_size(), _stream(stream)))


def rq_reconstruct(layout: Layout, c: Cache, loop: int, t0: int, n: int, out: torch.Tensor,
                   stream=None) -> None:
    """out: f32 [B, H, n, d]."""
    cc = _check_cache(layout, c, "c")
    _tensor(out, "out", torch.float32, (layout.batch, layout.n_heads, int(n), layout.head_dim))
    lay = layout.c()
    _check(_lib.rq_reconstruct(C.byref(lay), C.byref(cc), int(loop), int(t0), int(n), _ptr(out),
                               _stream(stream)))


def workspace_for(layout: Layout, n_ctx: int, n_splits: int = 0, device="cuda") -> torch.Tensor:
    """A decode workspace of the size the library asks for."""
    nbytes = rq_decode_workspace_bytes(layout, n_ctx, n_splits)
    if nbytes == 0:
        raise RQError(-1)
    return torch.empty(nbytes, dtype=torch.uint8, device=device)


def rq_probe_read_stream(buf: torch.Tensor, nontemporal: bool, sink: torch.Tensor, pattern: int = 0,
                         stream=None) -> None:
    """Read buf once with 128-bit loads (include/rq_probe.h): pattern 0 grid
    stride, 1 one contiguous chunk per workgroup, 2 a chunk of each of 20
    planes per workgroup; sink is a device int32 tensor whose length (a
    multiple of 256) sets the number of workgroups."""
    _tensor(buf, "buf", buf.dtype if isinstance(buf, torch.Tensor) else torch.uint8)
    _tensor(sink, "sink", torch.int32)
    if sink.numel() % 256 != 0:
        raise ValueError("sink: length must be a multiple of 256")
    _check(_lib.rq_probe_read_stream(_ptr(buf), buf.numel() * buf.element_size(), int(bool(nontemporal)),
                                     int(pattern), sink.numel() // 256, _ptr(sink), _stream(stream)))
