"""P7/P8: sizes and times the lecture prints, against the oracle's shard
ranges and the work formulas the benchmark credits.

Fixtures: tests/golden/pages_pins.json (each entry carries its citation)."""
import json
import os

import pytest

from megatron_tensor_layer_amd import workloads

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "pages_pins.json")))


@pytest.mark.parametrize("e", GOLD["shard_bytes"], ids=lambda e: e["printed"])
def test_shard_bytes(orc, e):
    t = e["t"]
    sizes = set()
    for r in range(t):
        lo, hi = orc.shard_range(e["rows"], t, r)
        sizes.add((hi - lo) * e["cols"] * e["esize"])
        assert lo == r * (e["rows"] // t)
    assert sizes == {e["expect"]}
    assert workloads.shard_bytes(e["rows"], e["cols"], t, e["esize"]) == e["expect"]
    # the rank blocks tile the dimension exactly
    assert orc.shard_range(e["rows"], t, t - 1)[1] == e["rows"]


@pytest.mark.parametrize("e", GOLD["allreduce_message"], ids=lambda e: e["printed"])
def test_allreduce_message(e):
    b = workloads.allreduce_message_bytes(e["B"], e["D"], e["esize"])
    if "expect" in e:
        assert b == e["expect"]
    else:
        assert abs(b / 1e6 - e["expect_MB"]) <= e["tol_MB"]


@pytest.mark.parametrize("e", GOLD["ring_bytes"], ids=lambda e: e["printed"])
def test_ring_bytes(e):
    assert abs(workloads.ring_allreduce_bytes_sent(e["n"], e["V"]) / 1e3 - e["expect_KB"]) <= e["tol_KB"]


@pytest.mark.parametrize("e", GOLD["case3_compute_time"], ids=lambda e: str(e["expect_us"]))
def test_case3_compute_time(e):
    # one projection of the rank's MLP share: 2*B*D*(F/n) flops
    F_local = e["F"] // e["n"]
    mlp = workloads.MlpShape(I=e["B"], D=e["D"], F_local=F_local)
    one_matrix = mlp.flops() / 3
    assert one_matrix == 2 * e["B"] * e["D"] * e["F"] / e["n"]
    us = one_matrix / (e["peak_tflops"] * 1e12) * 1e6
    assert abs(us - e["expect_us"]) <= e["tol_us"]


def test_mlp_bytes_llama_tp8():
    # compulsory bytes of the Llama-3.1-70B rank share at TP=8, decode I=1:
    # three 8192 x 3584 bf16 matrices (each the 58.7 MB shard of exercise 1)
    m = workloads.MlpShape(I=1, D=8192, F_local=3584)
    assert m.weight_bytes() == 3 * 58720256
    assert m.bytes() == 3 * 58720256 + 8192 * 2 + 8192 * 4
