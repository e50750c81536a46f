"""Host proof of the FP32 identities the encoder uses instead of IEEE divides.

The encoder's group scale (range / (2^b - 1)) and code factor (1 / s for a
stored binary16 scale) must equal the IEEE quotients bit for bit, since the
encoded planes are compared byte for byte with the oracle.  The kernel forms
them with a multiply and fma corrections; `native/float_identities.c` checks
both identities over every input they can see (all floats in [0, 2^120], all
positive binary16 scales), using the host's IEEE binary32 arithmetic and fma.
"""
import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
def test_division_identities_exhaustive(tmp_path):
    exe = tmp_path / "float_identities"
    subprocess.run(["gcc", "-O2", "-ffp-contract=off", "-fno-fast-math", "-pthread",
                    os.path.join(HERE, "native", "float_identities.c"), "-o", str(exe), "-lm"], check=True)
    res = subprocess.run([str(exe)], capture_output=True, text=True, timeout=600)
    print(res.stdout)
    assert res.returncode == 0, res.stdout + res.stderr
    assert res.stdout.count(": 0 mismatches") == 3, res.stdout
