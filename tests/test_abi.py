"""C ABI checks that need no GPU: librq.so loads, exports every entry point
include/rq.h declares, and rejects invalid arguments on the host before any
HIP call (fake, never-dereferenced device addresses are used; every case here
fails validation, so nothing is ever enqueued)."""
import ctypes as C
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADERS = [os.path.join(ROOT, "include", h) for h in sorted(os.listdir(os.path.join(ROOT, "include")))
           if h.endswith(".h")]


@pytest.fixture(scope="module")
def rq():
    import decode_attention_rq_amd as m
    return m


def declared_functions():
    text = "".join(open(h).read() for h in HEADERS)
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(rq_[a-z0-9_]+)\s*\(", text)))


def test_header_declares_the_boundary():
    names = declared_functions()
    assert names == sorted(["rq_encode", "rq_decode_workspace_bytes", "rq_decode_splits",
                            "rq_decode_attn", "rq_decode_attn_tail", "rq_decode_attn_tail_noalloc", "rq_reconstruct",
                            "rq_status_string", "rq_bf16_decode_attn", "rq_probe_read_stream"])


def test_library_exports_every_declared_symbol(rq):
    lib = C.CDLL(rq.LIB_PATH)
    for name in declared_functions():
        assert hasattr(lib, name), name


def test_status_strings(rq):
    for code, name in rq.STATUS.items():
        assert rq.rq_status_string(code).startswith(name)
    assert rq.rq_status_string(12345) == "unknown rq_status"


FAKE = 0x10000  # aligned, never dereferenced


def _layout(rq, **kw):
    lay = rq.Layout(n_loops=4, batch=2, n_heads=2, head_dim=128, group=32, capacity=64, rotate=1,
                    bits=[2, 2, 2])
    for k, v in kw.items():
        setattr(lay, k, v)
    return lay


def _cache(rq, n_loops=4, bad=None):
    c = rq.rq_cache()
    c.ref = FAKE
    for l in range(n_loops - 1):
        c.codes[l] = FAKE + 0x1000 * (l + 1)
        c.meta[l] = FAKE + 0x100000 * (l + 1)
        c.alpha[l] = FAKE + 0x10000000 * (l + 1)
    if bad:
        field, l, val = bad
        if field == "ref":
            c.ref = val
        else:
            getattr(c, field)[l] = val
    return c


def _encode(rq, lay, k=None, v=None, kin=FAKE, vin=FAKE, t0=0, n=8):
    L = lay.c()
    k = k or _cache(rq, lay.n_loops)
    v = v or _cache(rq, lay.n_loops)
    return rq._lib.rq_encode(C.byref(L), C.byref(k), C.byref(v), kin, vin, t0, n, None)


def _decode(rq, lay, mask=0b1111, n_ctx=32, scale=0.1, splits=2, out=FAKE, ws=FAKE,
            ws_bytes=1 << 30, q=FAKE, k=None, v=None):
    L = lay.c()
    k = k or _cache(rq, lay.n_loops)
    v = v or _cache(rq, lay.n_loops)
    return rq._lib.rq_decode_attn(C.byref(L), C.byref(k), C.byref(v), q, mask, n_ctx, scale, splits,
                                  out, ws, ws_bytes, None)


INVALID, UNSUPPORTED, WORKSPACE = -1, -2, -3


@pytest.mark.parametrize("kw,code", [
    (dict(n_loops=1), UNSUPPORTED), (dict(n_loops=33), UNSUPPORTED),
    (dict(batch=0), INVALID), (dict(n_heads=0), INVALID), (dict(capacity=0), INVALID),
    (dict(head_dim=96), UNSUPPORTED), (dict(head_dim=32), UNSUPPORTED),
    (dict(group=8), UNSUPPORTED), (dict(group=64), UNSUPPORTED),
    (dict(rotate=2), INVALID), (dict(bits=[2, 3, 2]), UNSUPPORTED), (dict(bits=[2, 2, 8]), UNSUPPORTED),
    (dict(batch=70000), UNSUPPORTED), (dict(batch=1024, n_heads=64, capacity=1 << 20), UNSUPPORTED),
])
def test_layout_validation(rq, kw, code):
    lay = _layout(rq, **kw)
    assert _encode(rq, lay) == code
    assert _decode(rq, lay) == code
    L = lay.c()
    c = _cache(rq, max(2, min(lay.n_loops, 32)))
    assert rq._lib.rq_reconstruct(C.byref(L), C.byref(c), 0, 0, 4, FAKE, None) == code
    assert rq._lib.rq_decode_workspace_bytes(C.byref(L), 16, 2) == 0
    assert rq._lib.rq_decode_splits(C.byref(L), 16) == INVALID


def test_null_layout_and_caches(rq):
    k = _cache(rq)
    assert rq._lib.rq_encode(None, C.byref(k), C.byref(k), FAKE, FAKE, 0, 1, None) == INVALID
    lay = _layout(rq).c()
    assert rq._lib.rq_encode(C.byref(lay), None, C.byref(k), FAKE, FAKE, 0, 1, None) == INVALID
    assert rq._lib.rq_decode_attn(C.byref(lay), C.byref(k), None, FAKE, 1, 4, 0.1, 1, FAKE, FAKE,
                                  1 << 30, None) == INVALID


@pytest.mark.parametrize("bad", [("ref", 0, 0), ("ref", 0, FAKE + 8), ("codes", 1, 0),
                                 ("meta", 2, FAKE + 4), ("alpha", 0, 0)])
def test_encode_plane_pointers(rq, bad):
    lay = _layout(rq)
    assert _encode(rq, lay, k=_cache(rq, bad=bad)) == INVALID
    assert _encode(rq, lay, v=_cache(rq, bad=bad)) == INVALID


@pytest.mark.parametrize("t0,n", [(-1, 4), (0, -1), (60, 5), (64, 1), (1 << 30, 1 << 30)])
def test_encode_token_range(rq, t0, n):
    assert _encode(rq, _layout(rq), t0=t0, n=n) == INVALID


def test_encode_inputs(rq):
    lay = _layout(rq)
    assert _encode(rq, lay, kin=0) == INVALID
    assert _encode(rq, lay, vin=FAKE + 2) == INVALID


def test_encode_empty_range_is_a_noop(rq):
    # n = 0 validates and returns before touching the device
    assert _encode(rq, _layout(rq), t0=64, n=0) == 0


@pytest.mark.parametrize("kw,code", [
    (dict(mask=0), INVALID), (dict(mask=0b10000), INVALID), (dict(mask=1 << 31), INVALID),
    (dict(n_ctx=0), INVALID), (dict(n_ctx=65), INVALID),
    (dict(scale=float("inf")), INVALID), (dict(scale=float("nan")), INVALID),
    (dict(splits=-1), INVALID), (dict(splits=33), INVALID),
    (dict(out=0), INVALID), (dict(out=FAKE + 4), INVALID), (dict(q=0), INVALID), (dict(ws=0), INVALID),
    (dict(ws_bytes=0), WORKSPACE), (dict(ws_bytes=100), WORKSPACE),
])
def test_decode_validation(rq, kw, code):
    assert _decode(rq, _layout(rq), **kw) == code


def test_decode_only_checks_planes_of_masked_loops(rq):
    lay = _layout(rq)
    k = _cache(rq, bad=("codes", 1, 0))
    assert _decode(rq, lay, mask=0b0010, k=k) == INVALID
    # loop 1 not in the mask: its null plane is not looked at; a too-small
    # workspace then shows the pointer checks passed
    assert _decode(rq, lay, mask=0b1101, k=k, ws_bytes=1) == WORKSPACE


def test_decode_rows_must_fit_32bit_offsets(rq):
    """A (batch, head)'s rows of a plane are addressed with 32-bit byte offsets:
    capacity * 2 * head_dim may reach 2^32 bytes, not more (cache and tail)."""
    edge = 1 << 23                                   # * 2 * 256 = 2^32
    # at the limit the checks pass (a too-small workspace is reported next)
    assert _decode(rq, _layout(rq, head_dim=256, capacity=edge), ws_bytes=1) == WORKSPACE
    assert _decode(rq, _layout(rq, head_dim=256, capacity=edge + 1)) == UNSUPPORTED
    assert _decode(rq, _layout(rq, head_dim=128, capacity=2 * edge + 1)) == UNSUPPORTED
    lay = _layout(rq, head_dim=256)
    assert _decode_tail(rq, lay, _tail(rq, cap=edge), ws_bytes=1) == WORKSPACE
    assert _decode_tail(rq, lay, _tail(rq, cap=edge + 1)) == UNSUPPORTED
    planes = (C.c_void_p * 4)(FAKE, FAKE, FAKE, FAKE)
    big = _layout(rq, head_dim=256, capacity=edge + 1).c()
    assert rq._lib.rq_bf16_decode_attn(C.byref(big), planes, planes, FAKE, 1, 32, 0.1, 2, FAKE, FAKE,
                                       1 << 30, None) == UNSUPPORTED


def test_workspace_size_formula(rq):
    lay = _layout(rq).c()
    # 2 splits * 4 slots * (2*2) (b,h) * (2*128+2) floats
    assert rq._lib.rq_decode_workspace_bytes(C.byref(lay), 32, 2) == 2 * 4 * 4 * 258 * 4
    # more splits than tokens are clamped to one token per split
    assert rq._lib.rq_decode_workspace_bytes(C.byref(lay), 3, 8) == 3 * 4 * 4 * 258 * 4
    # one split still has room for its records (written when a BF16 tail follows)
    assert rq._lib.rq_decode_workspace_bytes(C.byref(lay), 32, 1) == 1 * 4 * 4 * 258 * 4
    # no cached tokens (a tail alone): one split's worth
    assert rq._lib.rq_decode_workspace_bytes(C.byref(lay), 0, 1) == 1 * 4 * 4 * 258 * 4


@pytest.mark.parametrize("loop,t0,n", [(-1, 0, 4), (3, 0, 4), (0, -1, 4), (0, 0, 0), (0, 62, 4)])
def test_reconstruct_validation(rq, loop, t0, n):
    L = _layout(rq).c()
    c = _cache(rq)
    assert rq._lib.rq_reconstruct(C.byref(L), C.byref(c), loop, t0, n, FAKE, None) == INVALID
    assert rq._lib.rq_reconstruct(C.byref(L), C.byref(c), 0, 0, 4, FAKE + 8, None) == INVALID


def test_bf16_baseline_validation(rq):
    lay = _layout(rq).c()
    planes = (C.c_void_p * 4)(FAKE, FAKE, FAKE, FAKE)
    bad = (C.c_void_p * 4)(FAKE, 0, FAKE, FAKE)
    f = rq._lib.rq_bf16_decode_attn
    assert f(C.byref(lay), planes, planes, FAKE, 0, 32, 0.1, 2, FAKE, FAKE, 1 << 30, None) == INVALID
    assert f(C.byref(lay), planes, bad, FAKE, 0b0010, 32, 0.1, 2, FAKE, FAKE, 1 << 30, None) == INVALID
    assert f(C.byref(lay), None, planes, FAKE, 1, 32, 0.1, 2, FAKE, FAKE, 1 << 30, None) == INVALID
    assert f(C.byref(lay), planes, planes, FAKE, 1, 65, 0.1, 2, FAKE, FAKE, 1 << 30, None) == INVALID
    # loop 1's null plane is not looked at when loop 1 is not in the mask
    assert f(C.byref(lay), planes, bad, FAKE, 0b1101, 32, 0.1, 2, FAKE, FAKE, 1, None) == WORKSPACE


# ---------------------------------------------------------------------------
# quantized anchor and BF16 tail
# ---------------------------------------------------------------------------

def _anchor_cache(rq, n_loops=4, bad=None):
    c = _cache(rq, n_loops, bad=bad)
    if not bad or bad[0] != "ref":
        c.ref = 0                       # unused with a quantized anchor
    if not (bad and bad[1] == n_loops - 1):
        c.codes[n_loops - 1] = FAKE + 0x7000
        c.meta[n_loops - 1] = FAKE + 0x700000
    return c


@pytest.mark.parametrize("kw,code", [
    (dict(ref_bits=3), UNSUPPORTED), (dict(ref_bits=8), UNSUPPORTED), (dict(ref_bits=-1), UNSUPPORTED),
    (dict(ref_bits=4, ref_group=8), UNSUPPORTED), (dict(ref_bits=4, ref_group=64), UNSUPPORTED),
])
def test_anchor_layout_validation(rq, kw, code):
    lay = _layout(rq, **kw)
    assert _encode(rq, lay, k=_anchor_cache(rq), v=_anchor_cache(rq)) == code
    assert _decode(rq, lay, k=_anchor_cache(rq), v=_anchor_cache(rq)) == code


@pytest.mark.parametrize("bad", [("codes", 3, 0), ("meta", 3, FAKE + 4), ("codes", 0, 0)])
def test_anchor_planes_are_checked(rq, bad):
    lay = _layout(rq, ref_bits=4, ref_group=32)
    assert _encode(rq, lay, k=_anchor_cache(rq, bad=bad)) == INVALID
    assert _decode(rq, lay, v=_anchor_cache(rq, bad=bad), k=_anchor_cache(rq)) == INVALID


def test_anchor_needs_no_ref_plane(rq):
    lay = _layout(rq, ref_bits=4, ref_group=32)
    k, v = _anchor_cache(rq), _anchor_cache(rq)
    assert k.ref is None or k.ref == 0
    # everything else valid: the too-small workspace is the first complaint
    assert _decode(rq, lay, k=k, v=v, ws_bytes=1) == WORKSPACE
    # the anchor loop itself reconstructs with an anchor, never with BF16
    L = lay.c()
    assert rq._lib.rq_reconstruct(C.byref(L), C.byref(k), 3, 0, 4, FAKE + 8, None) == INVALID
    assert rq._lib.rq_reconstruct(C.byref(L), C.byref(k), 4, 0, 4, FAKE, None) == INVALID


def _tail(rq, n=4, cap=8, bad_loop=None):
    t = rq.rq_tail()
    for l in range(4):
        t.k[l] = 0 if l == bad_loop else FAKE + 0x200 * (l + 1)
        t.v[l] = FAKE + 0x400 * (l + 1)
    t.capacity, t.n = cap, n
    return t


def _decode_tail(rq, lay, tail, mask=0b1111, n_ctx=32, splits=2, ws_bytes=1 << 30):
    L = lay.c()
    k, v = _cache(rq, lay.n_loops), _cache(rq, lay.n_loops)
    return rq._lib.rq_decode_attn_tail(C.byref(L), C.byref(k), C.byref(v),
                                       C.byref(tail) if tail is not None else None, FAKE, mask,
                                       n_ctx, 0.1, splits, FAKE, FAKE, ws_bytes, None)


def test_tail_validation(rq):
    lay = _layout(rq)
    assert _decode_tail(rq, lay, _tail(rq, n=-1)) == INVALID
    assert _decode_tail(rq, lay, _tail(rq, n=9, cap=8)) == INVALID
    assert _decode_tail(rq, lay, _tail(rq, bad_loop=2)) == INVALID
    # a masked-out loop's tail rows are not looked at
    assert _decode_tail(rq, lay, _tail(rq, bad_loop=2), mask=0b1011, ws_bytes=1) == WORKSPACE
    # nothing to attend
    assert _decode_tail(rq, lay, _tail(rq, n=0), n_ctx=0) == INVALID
    assert _decode_tail(rq, lay, None, n_ctx=0) == INVALID
    # the tail alone is valid (no split count is needed); the workspace still is
    assert _decode_tail(rq, lay, _tail(rq), n_ctx=0, splits=0, ws_bytes=1) == WORKSPACE
    # plain rq_decode_attn still needs a cached token
    assert _decode(rq, lay, n_ctx=0) == INVALID


@pytest.mark.parametrize("kw,code", [
    (dict(group_loops=3), UNSUPPORTED), (dict(group_loops=1), UNSUPPORTED), (dict(group_loops=5), UNSUPPORTED),
    (dict(group_loops=2), UNSUPPORTED),                       # several groups need quantized anchors
])
def test_anchor_group_validation(rq, kw, code):
    lay = _layout(rq, **kw)
    assert _encode(rq, lay) == code
    assert _decode(rq, lay) == code


def test_anchor_groups_check_every_anchor(rq):
    lay = _layout(rq, ref_bits=4, ref_group=32, group_loops=2)
    k = _anchor_cache(rq)
    k.codes[1], k.meta[1] = FAKE + 0x9000, FAKE + 0x900000      # anchor of group 0
    v = _anchor_cache(rq)
    v.codes[1], v.meta[1] = FAKE + 0x9000, FAKE + 0x900000
    assert _decode(rq, lay, k=k, v=v, ws_bytes=1) == WORKSPACE
    k.meta[1] = 0
    assert _decode(rq, lay, k=k, v=v, mask=0b0001) == INVALID     # loop 0 needs its group's anchor
    assert _decode(rq, lay, k=k, v=v, mask=0b1100, ws_bytes=1) == WORKSPACE   # group 1 does not
    assert _encode(rq, lay, k=k, v=v) == INVALID


@pytest.mark.parametrize("kw,code", [
    (dict(alpha_mode=3), UNSUPPORTED), (dict(alpha_mode=-1), UNSUPPORTED), (dict(ref_first=2), INVALID),
])
def test_policy_validation(rq, kw, code):
    lay = _layout(rq, **kw)
    assert _encode(rq, lay) == code
    assert _decode(rq, lay) == code


def test_first_loop_policy_planes(rq):
    """With the first loop as reference, loop 0 has no residual planes and the
    last loop does."""
    lay = _layout(rq, ref_first=1, bits=[0, 2, 2, 2])
    k, v = _cache(rq), _cache(rq)
    k.codes[0] = k.meta[0] = k.alpha[0] = 0
    v.codes[0] = v.meta[0] = v.alpha[0] = 0
    k.codes[3], k.meta[3], k.alpha[3] = FAKE + 0x3000, FAKE + 0x300000, FAKE + 0x30000000
    v.codes[3], v.meta[3], v.alpha[3] = FAKE + 0x3000, FAKE + 0x300000, FAKE + 0x30000000
    assert _decode(rq, lay, k=k, v=v, ws_bytes=1) == WORKSPACE
    k.alpha[3] = 0
    assert _decode(rq, lay, k=k, v=v) == INVALID
    assert _decode(rq, lay, k=k, v=v, mask=0b0111, ws_bytes=1) == WORKSPACE


@pytest.mark.parametrize("kw,code", [
    (dict(ref_chain=2), INVALID),
    (dict(ref_chain=1, n_loops=5, bits=[2, 2, 2, 2]), UNSUPPORTED),       # 4 residual loops in a chain
    (dict(ref_chain=1, ref_bits=2, ref_group=32), UNSUPPORTED),           # INT2 anchors not chained
])
def test_chain_validation(rq, kw, code):
    lay = _layout(rq, **kw)
    k = _anchor_cache(rq, lay.n_loops) if lay.ref_bits else _cache(rq, lay.n_loops)
    v = _anchor_cache(rq, lay.n_loops) if lay.ref_bits else _cache(rq, lay.n_loops)
    assert _encode(rq, lay, k=k, v=v) == code
    assert _decode(rq, lay, k=k, v=v, mask=1) == code


def test_chain_decode_checks_every_link(rq):
    """Next-loop chain: decoding loop 0 reads loops 1 and 2 too."""
    lay = _layout(rq, ref_chain=1)
    k = _cache(rq, bad=("alpha", 1, 0))
    assert _decode(rq, lay, k=k, mask=0b0001) == INVALID
    assert _decode(rq, lay, k=k, mask=0b0100, ws_bytes=1) == WORKSPACE   # loop 2 needs only itself


def test_read_stream_probe_rejects_bad_arguments(rq):
    f = rq._lib.rq_probe_read_stream
    INVALID = -1
    assert f(None, 1024, 0, 0, 4, FAKE, None) == INVALID            # null buffer
    assert f(FAKE + 8, 1024, 0, 0, 4, FAKE, None) == INVALID        # misaligned buffer
    assert f(FAKE, 1000, 0, 0, 4, FAKE, None) == INVALID            # not a multiple of 16 bytes
    assert f(FAKE, 0, 0, 0, 4, FAKE, None) == INVALID               # empty
    assert f(FAKE, 1024, 2, 0, 4, FAKE, None) == INVALID            # bad policy flag
    assert f(FAKE, 1024, 0, 3, 4, FAKE, None) == INVALID            # bad pattern
    assert f(FAKE, 1024, 0, -1, 4, FAKE, None) == INVALID           # bad pattern
    assert f(FAKE, 1024, 0, 0, 0, FAKE, None) == INVALID            # no workgroups
    assert f(FAKE, 1024, 0, 1, 65536, FAKE, None) == INVALID        # too many
    assert f(FAKE, 1024, 0, 1, 4, None, None) == INVALID            # null sink


def _noalloc(rq, lay, mask=0b1111, n_ctx=32, splits=2, tail=None):
    L = lay.c()
    k, v = _cache(rq, lay.n_loops), _cache(rq, lay.n_loops)
    return rq._lib.rq_decode_attn_tail_noalloc(C.byref(L), C.byref(k), C.byref(v), tail, FAKE, mask, n_ctx, 0.1,
                                               splits, FAKE, None)


def test_noalloc_rejects_calls_beyond_its_scratch(rq):
    # 1024 (batch, head) pairs at head_dim 128: 4 splits need 16.9 MB of
    # records (within the 32 MiB scratch), 8 splits 33.8 MB (beyond it)
    lay = _layout(rq, batch=64, n_heads=16, capacity=4096)
    assert rq.rq_decode_workspace_bytes(lay, 4096, 8) > rq.NOALLOC_SCRATCH_BYTES
    assert rq.rq_decode_workspace_bytes(lay, 4096, 4) <= rq.NOALLOC_SCRATCH_BYTES
    assert _noalloc(rq, lay, n_ctx=4096, splits=8) == -3
    assert _noalloc(rq, lay, n_ctx=4096, splits=4, mask=0) == -1           # still validated
    assert _noalloc(rq, lay, n_ctx=0, splits=1) == -1                      # nothing to attend


def test_noalloc_device_error_path(rq, monkeypatch):
    monkeypatch.setenv("RQ_FAULT_INJECT", "launch")
    assert _noalloc(rq, _layout(rq), n_ctx=32, splits=2) == -4
