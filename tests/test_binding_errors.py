"""Error paths of the Python binding, on the CPU: every non-zero status of
the C ABI surfaces as RQError carrying that status and its text.  Invalid
arguments are rejected by the library's host-side validation before any HIP
call; the device-error path is forced with the library's RQ_FAULT_INJECT
hook (validation passes, the launch is refused), so no GPU is needed.  The
binding's own checks (dtype, shape, contiguity, device, tail capacities)
raise ValueError before the library is called."""
import pytest
import torch

import decode_attention_rq_amd as rq


def _lay(**kw):
    base = dict(n_loops=4, batch=1, n_heads=2, head_dim=128, group=32, capacity=64, rotate=1, bits=[2, 2, 2])
    base.update(kw)
    return rq.Layout(**base)


def _inputs(lay, n):
    x = torch.zeros(lay.n_loops - 1, lay.batch, lay.n_heads, n, lay.head_dim, dtype=torch.bfloat16)
    return rq.Cache(lay, "cpu"), rq.Cache(lay, "cpu"), x


def test_unsupported_layout():
    lay = _lay(bits=[3, 2, 2])
    k, v, x = _inputs(lay, 4)
    with pytest.raises(rq.RQError) as e:
        rq.rq_encode(lay, k, v, x, x, 0, 4, stream=0)
    assert e.value.status == -2
    assert str(e.value).startswith("RQ_ERR_UNSUPPORTED")


def test_invalid_range():
    lay = _lay()
    k, v, x = _inputs(lay, 4)
    with pytest.raises(rq.RQError) as e:
        rq.rq_encode(lay, k, v, x, x, 62, 4, stream=0)          # t0 + n > capacity
    assert e.value.status == -1
    assert str(e.value).startswith("RQ_ERR_INVALID_ARG")


def test_workspace_too_small():
    lay = _lay()
    k, v, _ = _inputs(lay, 4)
    q = torch.zeros(4, 1, 2, 128, dtype=torch.bfloat16)
    out = torch.empty(4, 1, 2, 128)
    ws = torch.empty(16, dtype=torch.uint8)
    with pytest.raises(rq.RQError) as e:
        rq.rq_decode_attn(lay, k, v, q, 0b1111, 32, 0.1, out, ws, n_splits=1, stream=0)
    assert e.value.status == -3


def test_device_error(monkeypatch):
    lay = _lay()
    k, v, x = _inputs(lay, 4)
    q = torch.zeros(4, 1, 2, 128, dtype=torch.bfloat16)
    out = torch.empty(4, 1, 2, 128)
    ws = rq.workspace_for(lay, 32, 1, device="cpu")
    rec = torch.empty(1, 2, 4, 128)
    monkeypatch.setenv("RQ_FAULT_INJECT", "launch")
    calls = [
        lambda: rq.rq_encode(lay, k, v, x, x, 0, 4, stream=0),
        lambda: rq.rq_decode_attn(lay, k, v, q, 0b1111, 32, 0.1, out, ws, n_splits=1, stream=0),
        lambda: rq.rq_reconstruct(lay, k, 0, 0, 4, rec, stream=0),
    ]
    for call in calls:
        with pytest.raises(rq.RQError) as e:
            call()
        assert e.value.status == -4
        assert str(e.value).startswith("RQ_ERR_DEVICE")
    # invalid arguments are still reported as such, before the launch
    with pytest.raises(rq.RQError) as e:
        rq.rq_encode(lay, k, v, x, x, 62, 4, stream=0)
    assert e.value.status == -1


def _decode_args(lay):
    k, v, _ = _inputs(lay, 4)
    q = torch.zeros(4, 1, 2, 128, dtype=torch.bfloat16)
    out = torch.empty(4, 1, 2, 128)
    ws = torch.empty(1 << 16, dtype=torch.uint8)
    return k, v, q, out, ws


@pytest.mark.parametrize("bad", ["q_dtype", "q_shape", "q_strided", "out_dtype", "out_shape", "cache_shape",
                                 "cache_dtype"])
def test_binding_rejects_mismatched_tensors(bad):
    lay = _lay()
    k, v, q, out, ws = _decode_args(lay)
    if bad == "q_dtype":
        q = q.float()
    elif bad == "q_shape":
        q = torch.zeros(4, 1, 2, 64, dtype=torch.bfloat16)
    elif bad == "q_strided":
        q = torch.zeros(4, 1, 2, 256, dtype=torch.bfloat16)[..., ::2]
    elif bad == "out_dtype":
        out = out.double()
    elif bad == "out_shape":
        out = torch.empty(3, 1, 2, 128)
    elif bad == "cache_shape":
        k = rq.Cache(_lay(batch=2), "cpu")                  # planes of another layout
    elif bad == "cache_dtype":
        k.meta[0] = k.meta[0].float()
    with pytest.raises(ValueError):
        rq.rq_decode_attn(lay, k, v, q, 0b1111, 32, 0.1, out, ws, n_splits=1, stream=0)


def test_binding_rechecks_planes_changed_in_place(monkeypatch):
    """The argument checks are kept per cache and tail object; a plane resized
    or restrided in place (same tensor, same data pointer) is checked again."""
    lay = _lay()
    k, v, q, out, ws = _decode_args(lay)
    monkeypatch.setenv("RQ_FAULT_INJECT", "launch")        # valid calls stop after validation
    with pytest.raises(rq.RQError):
        rq.rq_decode_attn(lay, k, v, q, 0b1111, 32, 0.1, out, ws, n_splits=1, stream=0)
    k.meta[1].resize_(k.meta[1].shape[0], k.meta[1].shape[1], 8, *k.meta[1].shape[3:])
    with pytest.raises(ValueError):
        rq.rq_decode_attn(lay, k, v, q, 0b1111, 32, 0.1, out, ws, n_splits=1, stream=0)
    kt = [torch.zeros(1, 2, 8, 128, dtype=torch.bfloat16) for _ in range(4)]
    tail = rq.Tail(kt, [t.clone() for t in kt], 4)
    k2, v2, _, _, _ = _decode_args(lay)
    with pytest.raises(rq.RQError):
        rq.rq_decode_attn_tail(lay, k2, v2, tail, q, 0b1111, 32, 0.1, out, ws, n_splits=1, stream=0)
    kt[2].as_strided_((1, 2, 8, 128), (2 * 8 * 128, 8 * 128, 64, 1))   # rows overlap: not contiguous
    with pytest.raises(ValueError):
        rq.rq_decode_attn_tail(lay, k2, v2, tail, q, 0b1111, 32, 0.1, out, ws, n_splits=1, stream=0)


def test_binding_rejects_encode_inputs_of_another_shape():
    lay = _lay()
    k, v, x = _inputs(lay, 4)
    with pytest.raises(ValueError):
        rq.rq_encode(lay, k, v, x, x, 0, 5, stream=0)            # x holds 4 tokens
    with pytest.raises(ValueError):
        rq.rq_encode(lay, k, v, x[:2], x[:2], 0, 4, stream=0)   # two loops, layout has three residual


def test_binding_rejects_reconstruct_output_of_another_shape():
    lay = _lay()
    k, _, _ = _inputs(lay, 4)
    with pytest.raises(ValueError):
        rq.rq_reconstruct(lay, k, 0, 0, 4, torch.empty(1, 2, 5, 128), stream=0)


def test_tail_planes_must_share_one_capacity():
    kt = [torch.zeros(1, 2, 8, 128, dtype=torch.bfloat16) for _ in range(4)]
    vt = [torch.zeros(1, 2, 8, 128, dtype=torch.bfloat16) for _ in range(3)] + \
         [torch.zeros(1, 2, 9, 128, dtype=torch.bfloat16)]
    with pytest.raises(ValueError):
        rq.Tail(kt, vt, 4)
    with pytest.raises(ValueError):
        rq.Tail(kt, kt, 9)                                      # n beyond the capacity
    t = rq.Tail(kt, [None, None, None, kt[3]], 8)
    assert t.capacity == 8


def test_binding_rejects_host_tensors_when_a_gpu_is_present(monkeypatch):
    lay = _lay()
    k, v, q, out, ws = _decode_args(lay)
    monkeypatch.setattr(rq, "_GPU", True)
    with pytest.raises(ValueError, match="GPU tensor"):
        rq.rq_decode_attn(lay, k, v, q, 0b1111, 32, 0.1, out, ws, n_splits=1, stream=0)
