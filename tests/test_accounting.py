"""Benchmark accounting pinned to the worked size examples the pages print."""
import math
import os

import pytest

from transformer_attention_fa_amd import inputs, roofline

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
UNITS = {"MiB": 2 ** 20, "GiB": 2 ** 30, "GB": 1e9, "ratio": 1, "requests": 1}


def _examples():
    rows = []
    for line in open(os.path.join(GOLDEN, "size_examples.txt")):
        line = line.strip()
        if not line or line.startswith("#"):
            continue
        name, qty, args, value, unit, _src = [c.strip() for c in line.split("|")]
        kw = dict(a.split("=") for a in args.split())
        rows.append((name, qty, kw, value, unit))
    return rows


def _evaluate(qty, kw):
    i = {k: float(v) if "." in v else int(v) for k, v in kw.items()}
    if qty == "score_matrix_bytes":
        return roofline.score_matrix_bytes(i["B"], i["H"], i["N"], i["bytes"])
    if qty == "kv_cache_bytes":
        return roofline.kv_cache_bytes(i["L"], i["N"], i["D"], i["B"], i["bytes"])
    if qty == "kv_cache_bytes_gqa":
        return roofline.kv_cache_bytes_gqa(i["L"], i["N"], i["D"], i["B"], i["bytes"], i["H"], i["G"])
    if qty == "requests_fitting":
        return math.floor(i["budget_GB"] / i["per_request_GB"])   # whole requests that fit
    if qty == "layer_kv_bytes":
        return roofline.layer_kv_bytes(i["S"], i["D"], i["bytes"])
    if qty == "layer_kv_bytes_x":
        return roofline.layer_kv_bytes(i["S"], i["D"], i["bytes"]) * i["layers"]
    if qty == "kv_head_fraction":
        return roofline.kv_head_fraction(i["H"], i["G"])
    raise KeyError(qty)


@pytest.mark.parametrize("row", _examples(), ids=lambda r: r[0])
def test_size_formula_reproduces_printed_value(row):
    name, qty, kw, value, unit = row
    got = _evaluate(qty, kw) / UNITS[unit]
    decimals = len(value.split(".")[1]) if "." in value else 0
    if unit == "requests":
        assert got == int(value)
    else:
        assert round(got, decimals) == pytest.approx(float(value)), (name, got)


def test_flop_formula_and_causal_halving():
    assert roofline.attention_flops(8, 32, 2048, 2048, 128, True) == pytest.approx(274.877906944e9)
    assert roofline.attention_flops(1, 32, 8192, 8192, 128, True) == pytest.approx(549.755813888e9)
    assert roofline.attention_flops(4, 64, 4096, 4096, 128, False) == pytest.approx(2199.023255552e9)
    for w in inputs.PREFILL_WORKLOADS:
        assert w.flops() == roofline.attention_flops(w.B, w.H, w.N_q, w.N_k, w.d, w.causal)


def test_causal_block_rule_fixture_matches_halving():
    """The rule of the causal block table: j > i skipped, j == i triangular, j < i full;
    the work left tends to half of N x N as blocks shrink relative to N."""
    grid = [l.split() for l in open(os.path.join(GOLDEN, "causal_block_rule.txt"))
            if l.strip() and not l.startswith("#")]
    nb = len(grid)
    for i in range(nb):
        for j in range(nb):
            assert grid[i][j] == ("S" if j > i else "T" if j == i else "F")
    # exact visible-pair count for a square causal problem: N(N+1)/2
    n = 2048
    pairs = sum(i + 1 for i in range(n))
    assert pairs == n * (n + 1) // 2
    assert abs(pairs / (n * n) - 0.5) < 1e-3


def test_decode_bytes_formula():
    spec = inputs.GQA_DECODE
    lens = inputs.decode_seq_lens(spec)
    assert len(lens) == spec.B
    assert lens.min() >= spec.len_lo and lens.max() <= spec.len_hi
    b = roofline.decode_kv_bytes(spec.H_kv, spec.d, lens)
    assert b == 4096 * int(lens.sum())          # 2 * 8 heads * 128 * 2 bytes per row
    assert b == inputs.decode_kv_bytes(spec, lens)


def test_peaks():
    assert roofline.PEAK_BF16_TFLOPS == pytest.approx(2516.58, abs=0.01)
    assert roofline.PEAK_HBM_GBPS == 8000.0
