"""The measurement's arithmetic against the pages' worked examples.

tests/golden/worked_examples.json holds the numbers the pages print (each
entry cites its page and section). The workload table must reproduce the
FLOP count (2MNK) and the minimum byte count, and bench.py's TFLOP/s formula
the printed rate.
"""
import json
import os

import pytest

import bench
from synthetic import workloads as W

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "worked_examples.json")
EXAMPLES = json.load(open(GOLDEN))["examples"]


@pytest.mark.parametrize("ex", EXAMPLES, ids=lambda e: f"{e['M']}x{e['N']}x{e['K']}")
def test_flop_count_matches_page(ex):
    case = W.Case("golden", "N", "N", ex["M"], ex["N"], ex["K"], 1.0, ex["beta"], seed=1)
    assert round(case.flops / 1e9, ex["flops_G_decimals"]) == ex["flops_G"], ex["cite"]


@pytest.mark.parametrize("ex", [e for e in EXAMPLES if "bytes_min" in e], ids=lambda e: f"{e['M']}^3")
def test_minimum_bytes_match_page(ex):
    case = W.Case("golden", "N", "N", ex["M"], ex["N"], ex["K"], 1.0, ex["beta"], seed=1)
    assert case.algorithmic_bytes == ex["bytes_min"], ex["cite"]


@pytest.mark.parametrize("ex", [e for e in EXAMPLES if "tflops" in e], ids=lambda e: f"{e['M']}^3")
def test_tflops_formula_matches_page(ex):
    case = W.Case("golden", "N", "N", ex["M"], ex["N"], ex["K"], 1.0, ex["beta"], seed=1)
    assert round(bench.tflops(case.flops, ex["seconds"]), ex["tflops_decimals"]) == ex["tflops"], ex["cite"]
