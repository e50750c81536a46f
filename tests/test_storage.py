"""The storage accounting reproduces every effective bit width the pages print.

Fixture: tests/golden/effective_bitwidth.json (values copied from the
ResidualQuant page's Tables 5, 8, 10 and its Abstract, each row citing where).
"""
import json
import os
from decimal import ROUND_HALF_UP, Decimal

from oracle import storage

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "effective_bitwidth.json")


def _round(x, decimals):
    q = Decimal(1).scaleb(-decimals)
    return float(Decimal(repr(round(x, 9))).quantize(q, rounding=ROUND_HALF_UP))


def _schedule(row):
    if row["schedule"] == "uniform":
        return storage.uniform(row["bits"], row["g"], residual=row["residual"])
    return storage.anchored(row["groups"], row["n_residual"], row["g"])


def test_printed_effective_bitwidths():
    data = json.load(open(GOLDEN))
    for row in data["rows"]:
        got = storage.effective_bits(_schedule(row), row["d"])
        assert _round(got, row["decimals"]) == row["printed"], (row["cite"], got)


def test_printed_storage_reduction():
    data = json.load(open(GOLDEN))
    for row in data["reduction"]:
        red = 100 * storage.storage_reduction(storage.anchored(row["groups"], row["n_residual"], row["g"]), row["d"])
        assert _round(red, row["decimals"]) == row["printed_percent"]


def test_this_layout():
    """BF16 reference + three INT2 loops with FP16 scale and zero: 812 bytes per
    (batch, head, token) for K and V, 6.34 bits per value (60.35% below BF16)."""
    assert storage.layout_bytes_per_token(4, [2, 2, 2], 32, 128) == 812
    assert storage.layout_bytes_per_token(4, [4, 2, 2], 32, 128) == 876
    assert abs(storage.layout_bits_per_value(4, [2, 2, 2], 32, 128) - 6.34375) < 1e-12
    # bytes agree with bits: 2 sides * 4 loops * 128 values * bits / 8
    assert 2 * 4 * 128 * storage.layout_bits_per_value(4, [2, 2, 2], 32, 128) / 8 == 812


def test_anchored_layout():
    """The pages' final configuration [2,2,2,4] (Fig. 6 caption: INT2 residuals
    at g=16, the INT4 anchor at g=32) in this layout, worked by hand per K or V
    side of one (batch, head, token):
      anchor: 128 * 4 / 8 = 64 B codes + 4 groups * 4 B (FP16 scale, zero) = 80 B
      INT2 loop at g=16: 32 B codes + 8 groups * 4 B + 2 B alpha = 66 B
    so the whole cache holds 2 * (80 + 3 * 66) = 556 B, and decoding one loop on
    its own reads 2 * (80 + 66) = 292 B, against 2 * 256 = 512 B for that loop's
    BF16 K and V."""
    assert storage.layout_bytes_per_token(4, [2, 2, 2], 16, 128, ref_bits=4, ref_group=32) == 556
    assert storage.loop_read_bytes_per_token(2, 16, 128, ref_bits=4, ref_group=32) == 292
    assert storage.loop_read_bytes_per_token(2, 32, 128, ref_bits=4, ref_group=32) == 2 * (80 + 50)
    # with the BF16 reference, one loop alone reads more than its BF16 K and V
    assert storage.loop_read_bytes_per_token(2, 32, 128) == 2 * (256 + 50) > 512


def test_bench_byte_accounting_matches():
    """bench.py keeps its own byte accounting (it may not import the oracle
    outside its CPU-baseline leg); it must agree with this module."""
    import importlib.util
    spec = importlib.util.spec_from_file_location(
        "bench_mod", os.path.join(os.path.dirname(os.path.dirname(__file__)), "bench.py"))
    bench = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(bench)
    for args in [(4, [2, 2, 2], 32, 128), (4, [4, 2, 2], 32, 128), (2, [2], 32, 64), (6, [2, 4, 2, 2, 4], 16, 256)]:
        assert bench.layout_bytes_per_token(*args) == storage.layout_bytes_per_token(*args)
        for rb, rg in [(4, 32), (2, 16), (4, 16)]:
            assert (bench.layout_bytes_per_token(*args, ref_bits=rb, ref_group=rg)
                    == storage.layout_bytes_per_token(*args, ref_bits=rb, ref_group=rg))
    for b, g, d in [(2, 16, 128), (4, 32, 128), (2, 32, 64)]:
        assert bench.loop_read_bytes_per_token(b, g, d) == storage.loop_read_bytes_per_token(b, g, d)
        assert (bench.loop_read_bytes_per_token(b, g, d, 4, 32)
                == storage.loop_read_bytes_per_token(b, g, d, 4, 32))
