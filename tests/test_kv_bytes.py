"""Oracle byte formula against the worked numbers the pages print."""

import json
import os
from fractions import Fraction

import pytest

from oracle import kv_bytes, kv_bytes_per_token

GOLDEN = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "kv_bytes.json")))
UNIT = {"B": 1, "KiB": 1024, "GiB": 1024 ** 3, "GB": 10 ** 9}


def _formula(e):
    return kv_bytes(e["layers"], e["kv_heads"], e["head_dim"], e["bytes_per_element"], e["tokens"], e["batch"])


@pytest.mark.parametrize("e", GOLDEN["entries"], ids=[e["id"] for e in GOLDEN["entries"]])
def test_worked_values(e):
    got = _formula(e)
    printed = Fraction(str(e["printed"])) * UNIT[e["unit"]]
    if e["kind"] == "exact":
        assert got == printed
    elif e["kind"] == "rounded":
        q = Fraction(10) ** e["digits"]
        assert round(got / UNIT[e["unit"]] * q) == round(Fraction(str(e["printed"])) * q)
    elif e["kind"] == "approx":
        assert abs(got / printed - 1) <= e["rel_tol"]
    elif e["kind"] == "erratum":
        assert got == e["formula_bytes"]
        # the printed figure is not the formula rounded to the digits shown,
        # whether read in decimal or in binary units
        q = Fraction(10) ** e["digits"]
        for unit in ("GB", "GiB"):
            assert round(got / UNIT[unit] * q) != round(Fraction(str(e["printed"])) * q)
    else:
        raise AssertionError(e["kind"])


@pytest.mark.parametrize("r", GOLDEN["ratios"], ids=[r["id"] for r in GOLDEN["ratios"]])
def test_ratios(r):
    num = kv_bytes_per_token(80, r["num"]["kv_heads"], 128, r["num"]["bytes_per_element"])
    den = kv_bytes_per_token(80, r["den"]["kv_heads"], 128, r["den"]["bytes_per_element"])
    assert num / den == Fraction(r["printed"])


def test_workload_sizes_match_formula():
    """The 70B-shaped step moves 64 x 4096 tokens x 320 KiB/token of K/V."""
    assert kv_bytes(80, 8, 128, 2, 4096, 64) == 64 * 4096 * 327680 == 85_899_345_920
