"""Error paths of the Python binding, on the CPU: every non-zero status of
the C ABI surfaces as RQError carrying that status and its text.  Invalid
arguments are rejected by the library's host-side validation before any HIP
call; the device-error path is forced with the library's RQ_FAULT_INJECT
hook (validation passes, the launch is refused), so no GPU is needed."""
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
