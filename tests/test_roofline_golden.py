"""Pins of the roofline/tiling arithmetic against the numbers the pages print."""
import json
import os

import pytest

from dense_gemm_09_amd import roofline as rl

G = os.path.join(os.path.dirname(__file__), "golden")


def load(name):
    with open(os.path.join(G, name)) as f:
        return json.load(f)


def test_reads_table():
    g = load("tiling_page_roofline.json")
    for row in g["reads_table"]:
        assert rl.reads_per_output(1, row["T"]) == row["reads_per_output_over_K"]


def test_square_4096_naive_traffic():
    g = load("tiling_page_roofline.json")["square_4096"]
    tol = g["tol"]
    reads = rl.naive_element_reads(g["M"], g["N"], g["K"])
    assert reads == pytest.approx(g["naive_element_reads"], rel=tol)
    nbytes = reads * 2
    assert nbytes == pytest.approx(g["naive_bytes_fp16"], rel=tol)
    assert nbytes / g["h100_hbm_bytes_per_s"] * 1e3 == pytest.approx(g["naive_hbm_ms"], rel=tol)
    flops = rl.gemm_flops(g["M"], g["N"], g["K"])
    assert flops / g["h100_fp16_flops"] * 1e3 == pytest.approx(g["compute_ms"], rel=tol)
    # tiling by T divides the element reads by T
    assert rl.tiled_element_reads(4096, 4096, 4096, 4) * 4 == reads


def test_intensity_and_ridge():
    g = load("tiling_page_roofline.json")
    i = g["intensity"]
    T, k, eb = i["T"], 32, i["elem_bytes"]
    assert 2 * T * T * k / (T * T * k) == i["per_tile_flops_over_T2k"]
    assert (T * k + k * T) * eb / (T * k) == i["per_tile_bytes_over_Tk"]
    assert rl.tile_intensity(T, eb) == i["intensity_at_T"]
    peak, bw = g["square_4096"]["h100_fp16_flops"], g["square_4096"]["h100_hbm_bytes_per_s"]
    assert rl.ridge_point(peak, bw) == pytest.approx(i["ridge_flop_per_byte"], rel=i["tol"])
    assert rl.tile_edge_for_ridge(peak, bw, eb) == pytest.approx(i["T_for_ridge"], rel=i["tol"])
    assert rl.bandwidth_bound_flops(T, eb, bw) / 1e12 == pytest.approx(i["bound_tflops_at_T"],
                                                                       rel=i["tol"])
    s = g["smem"]
    assert rl.tile_operand_bytes(s["BM"], s["BK"], s["elem_bytes"]) == s["tile_bytes"]
    assert rl.tile_operand_bytes(s["BM_big"], 64, s["elem_bytes"]) == s["tile_bytes_big"]
    r = g["registers"]
    assert r["register_tile"][0] * r["register_tile"][1] == r["accumulators"]


def test_deepgemm_tiling_example():
    g = load("deepgemm_page_tiling.json")
    assert rl.grid_tiles(g["M"], g["N"], g["BM"], g["BN"]) == g["blocks"] == g["grid"][0] * g["grid"][1]
    assert g["blocks"] / g["SMs"] == pytest.approx(g["blocks_per_sm_approx"], abs=0.05)
    assert rl.tile_operand_bytes(g["BM"], g["BK"], g["elem_bytes"]) == g["a_tile_bytes"]
    assert rl.tile_operand_bytes(g["BN"], g["BK"], g["elem_bytes"]) == g["b_tile_bytes"]
    assert rl.accumulators_per_thread(g["BM"], g["BN"], g["threads"]) == g["accumulators_per_thread"]


def test_mi355x_ridge():
    # dense BF16 peak over 8 TB/s
    assert rl.ridge_point(rl.MI355X_PEAK_TFLOPS["bf16"] * 1e12, rl.MI355X_HBM_GBPS * 1e9) == pytest.approx(314.6, rel=1e-3)
