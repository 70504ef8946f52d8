"""The figures the pages print, held with their citations in
tests/golden/pages_figures.json, against the CPU oracle: the coverage of the
seven-exponent table, the 3-bit code in place of the 8-bit exponent, 11 bits
per value when no value takes the zero-point path, and the resulting ~31 %
(~30 % in the lay summary)."""
import json
import os

import numpy as np
import pytest

import oracle
from lossless_bf16_exponent_amd import workloads

HERE = os.path.dirname(os.path.abspath(__file__))
FIG = {f["name"]: f for f in json.load(open(os.path.join(HERE, "golden", "pages_figures.json")))["figures"]}


def test_every_figure_has_a_citation():
    assert FIG and all(f.get("citation") for f in FIG.values())


@pytest.mark.parametrize("sigma", [0.02, 1.0])
def test_top7_coverage(sigma):
    p = oracle.exponent_probabilities(sigma)
    assert p[list(oracle.plan_from_sigma(sigma))].sum() > FIG["top7_coverage_min"]["value"]


def test_code_width_and_eleven_bits():
    """A tensor whose exponents all lie in the table: the stream carries
    16 - exponent_bits + code_bits bits per value, plus framing that vanishes
    as n grows."""
    exps = oracle.plan_from_sigma(0.02)
    n = 1 << 20
    g = np.random.default_rng(4)
    e = np.array(exps)[g.integers(0, 7, n)]
    x = ((g.integers(0, 2, n) << 15) | (e << 7) | g.integers(0, 128, n)).astype(np.uint16)
    s = oracle.encode(x, exps)
    bits = 8.0 * s.size / n
    per_value = 16 - FIG["exponent_bits"]["value"] + FIG["code_bits"]["value"]
    assert per_value == FIG["bits_per_value_without_zero_points"]["value"]
    assert per_value <= bits < per_value + 0.01
    saving = 1.0 - per_value / 16.0
    assert abs(saving - FIG["theoretical_compression"]["value"]) <= FIG["theoretical_compression"]["tolerance"]
    assert abs(saving - FIG["lay_summary_reduction"]["value"]) <= FIG["lay_summary_reduction"]["tolerance"]
    rc, y = oracle.decode(s, n)
    assert rc == 0 and np.array_equal(y, x)


def test_gaussian_tensor_near_the_figures():
    """A near-Gaussian tensor (sigma = 0.02) lands close to the printed
    figures: about 3 % of values on the zero-point path, about 11.2 bits."""
    n = 1 << 20
    x = workloads.bf16_bits_from_f32((np.random.default_rng(0).standard_normal(n) * 0.02).astype(np.float32))
    s = oracle.encode(x, oracle.plan_from_sigma(0.02))
    zero_point_share = int.from_bytes(s[32:40].tobytes(), "little") / n
    assert zero_point_share < 1.0 - FIG["top7_coverage_min"]["value"] + 0.005
    assert 11.0 < 8.0 * s.size / n < 11.3
