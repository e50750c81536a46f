import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an AMD GPU (MI355X / gfx950) and the HIP library")
    config.addinivalue_line("markers", "slow: long-running CPU test")


@pytest.fixture(scope="session")
def oracle():
    from oracle import build, rq_oracle
    build.build()
    rq_oracle._lib = None
    return rq_oracle


@pytest.fixture(params=["auto", "4", "8"])
def waves(request, monkeypatch):
    """Decode workgroup shape: the library's choice, or 4 / 8 waves per split
    forced through RQ_DECODE_WAVES (which the library reads on every call)."""
    if request.param == "auto":
        monkeypatch.delenv("RQ_DECODE_WAVES", raising=False)
    else:
        monkeypatch.setenv("RQ_DECODE_WAVES", request.param)
    return request.param
