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
