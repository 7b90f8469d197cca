"""The measurement accounting against figures the pages print.

The tiled-GEMM tuning note (page "企业官网建设流程全解析", section 1.1) works
the 4096^3 GEMM through by hand: FLOP count, operand bytes and arithmetic
intensity in fp32 and in bf16.  ``bench.py`` must reproduce them from its own
formulas (it also counts writing C, which the page leaves out).
"""
import json
import os

import pytest

import bench

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "tuning_note_4096_accounting.json")


@pytest.fixture(scope="module")
def page():
    with open(GOLDEN) as f:
        return json.load(f)


def test_flop_count(page):
    M, N, K = page["shape"]
    assert round(bench.gemm_flops(M, N, K) / 1e9, 1) == page["gflop"]


@pytest.mark.parametrize("dtype,elem", [("fp32", 4), ("bf16", 2)])
def test_operand_bytes_and_intensity(page, dtype, elem):
    M, N, K = page["shape"]
    # the page counts A and B only: bench's bf16 byte count minus C, rescaled
    operands_bf16 = bench.gemm_bytes(M, N, K) - 2 * M * N
    operands = operands_bf16 // 2 * elem
    assert operands / 2**20 == page[dtype]["operand_mbytes"]
    ai = bench.gemm_flops(M, N, K) / operands
    assert round(ai) == page[dtype]["ai_flop_per_byte"]


def test_ridge_point_formula(page):
    # the page's H100 bf16 ridge from its own peak and bandwidth, ~300 FLOP/B
    ridge = page["h100_bf16_tflops"] * 1e12 / (page["h100_hbm_tbps"] * 1e12)
    assert abs(ridge - page["bf16_ridge_flop_per_byte_h100"]) / 300 < 0.01
    # this chip: 2.5 PFLOP/s over 8 TB/s
    assert bench.RIDGE == pytest.approx(312.5)


def test_full_bytes_include_c(page):
    M, N, K = page["shape"]
    assert bench.gemm_bytes(M, N, K) == 2 * (M * K + N * K + M * N)
    assert bench.gemm_bytes(M, N, K, out_bytes=4) == 2 * M * K + 2 * N * K + 4 * M * N
