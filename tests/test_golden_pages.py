"""The benchmark's FLOP count against the figures printed on the pages: every
(time, TFLOP/s) pair in tests/golden/pages_benchmark_4096.txt must satisfy
TFLOP/s = 2*M*N*K / time at M = N = K = 4096, to the printed two decimals."""
import os

import pytest

import bench

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden",
                      "pages_benchmark_4096.txt")


def rows():
    out = []
    for line in open(GOLDEN, encoding="utf-8"):
        if line.strip() and not line.startswith("#"):
            page, section, kernel, ms, tf = [f.strip() for f in line.split("|")]
            out.append((kernel, float(ms), float(tf)))
    return out


def test_golden_has_both_pages():
    assert len(rows()) == 14


@pytest.mark.parametrize("kernel,ms,tf", rows())
def test_tflops_formula_matches_printed_figures(kernel, ms, tf):
    assert round(bench.tflops(4096, 4096, 4096, ms * 1e-3), 2) == pytest.approx(tf, abs=1e-9)


def test_flop_count_definition():
    assert bench.gemm_flops(4096, 4096, 4096) == 137438953472
    assert bench.gemm_flops(4000, 3000, 4104) == 98496000000
