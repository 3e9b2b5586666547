"""Checks against the figures the BatchLAS pages print (tests/golden/pages_figures.json).

The pages print no worked factorisation, so these pin the accounting (flop and
byte models used in every throughput report) and the accuracy class of the
oracle's factor.
"""
from __future__ import annotations

import json
import os

import numpy as np

import oracle
import synthetic as syn
from dense_linear_algebra_potrf_amd import metrics

GOLDEN = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "pages_figures.json")))


def test_flop_convention_reproduces_the_printed_rate():
    g = GOLDEN["cta_float_n155"]
    rate = metrics.potrf_flops(g["n"], g["dtype"]) * g["batch"] / (g["time_us"] * 1e-6) / 1e12
    assert abs(rate - g["tflops"]) < 0.005


def test_byte_model_reproduces_the_printed_dram_roof():
    g = GOLDEN["dram_roof_float_n8"]
    byts = metrics.potrf_bytes(g["n"], g["batch"], g["dtype"])
    assert byts - metrics.footprint_bytes(g["n"], g["batch"], g["dtype"]) == 4 * g["batch"]
    implied_tb_s = byts / (g["roof_us"] * 1e-6) / 1e12
    # the printed roof corresponds to the card's published bandwidth within 10 %
    assert 0.9 * g["card_bandwidth_tb_s"] <= implied_tb_s <= 1.01 * g["card_bandwidth_tb_s"]


def test_byte_model_counts_lines_not_elements():
    # complex-float Upper n = 64: only the lines holding the upper triangle count
    per = metrics.potrf_bytes(64, 256, "c64", "U") / 256
    assert per == 40964
    assert metrics.footprint_bytes(64, 1, "c64") + 4 == 65540
    # fp64 n = 512 Lower
    assert metrics.potrf_bytes(512, 4, "f64", "L") / 4 == 2162692
    # padded layouts touch more lines than the packed one
    lda, stride = syn.layout(33, padded=True)
    assert metrics.potrf_bytes(33, 64, "f32", "L", lda, stride) > metrics.potrf_bytes(33, 64, "f32", "L")


def test_oracle_residual_is_in_the_printed_accuracy_class():
    """Relative residual ||A - L L^H||_F / ||A||_F within a decade of the printed bands."""
    bands = GOLDEN["residual_bands"]
    for dt, n, key in (("f32", 256, "single"), ("c64", 128, "single"),
                       ("f64", 256, "double"), ("c128", 128, "double")):
        a = syn.spd_matrices(n, 2, dt, seed=77)
        f, info = oracle.potrf_matrices(a, "L")
        assert (info == 0).all()
        wide = np.complex128 if syn.is_complex(dt) else np.float64
        ll = np.tril(f).astype(wide)
        r = a.astype(wide) - ll @ np.conj(np.swapaxes(ll, 1, 2))
        rel = np.linalg.norm(r, axis=(1, 2)) / np.linalg.norm(a.astype(wide), axis=(1, 2))
        lo, hi = bands[key]
        assert (rel >= lo / 10).all() and (rel <= hi * 10).all(), (dt, rel)
