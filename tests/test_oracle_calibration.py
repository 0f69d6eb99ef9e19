"""Pins of the oracle's global-scale calibration: amax against numpy's max of
|x|, and the chosen scale against closed forms and minimality over powers of
two (no block scale saturates at g, one would at g / 2), and the tight binary32
variant against exact-rational minimality."""
from fractions import Fraction

import numpy as np
import pytest
import torch

from tests.test_oracle_attention import bf16_bits


def test_amax_vs_library(oracle_lib):
    rng = np.random.default_rng(61)
    x = (rng.standard_normal((37, 3, 128)) * 5).astype(np.float32)
    x[11, 2, 77] = -123.5
    assert oracle_lib.amax(x) == float(np.abs(x).max()) == 123.5
    b = torch.tensor(x).to(torch.bfloat16)
    assert oracle_lib.amax(bf16_bits(b)) == float(b.abs().max().float())
    assert oracle_lib.amax(np.zeros((2, 1, 128), np.float32)) == 0.0


def test_global_scale_closed_forms(oracle_lib):
    assert oracle_lib.global_scale_for_amax(0.0) == 1.0
    assert oracle_lib.global_scale_for_amax(2688.0) == 1.0  # 2688 / 6 = 448 exactly
    assert oracle_lib.global_scale_for_amax(2689.0) == 2.0
    assert oracle_lib.global_scale_for_amax(1344.0) == 0.5
    assert oracle_lib.global_scale_for_amax(1.0) == 2.0 ** -11  # 1/2688 lies in (2^-12, 2^-11]


@pytest.mark.parametrize("seed", range(3))
def test_global_scale_is_the_smallest_power_of_two_without_saturation(oracle_lib, seed):
    rng = np.random.default_rng(70 + seed)
    for a in np.exp(rng.uniform(np.log(1e-6), np.log(1e9), 300)):
        g = oracle_lib.global_scale_for_amax(a)
        m, e = np.frexp(g)
        assert m == 0.5  # a power of two
        assert a / (6 * g) <= 448 < a / (6 * (g / 2))


def test_tight_global_scale_closed_forms(oracle_lib):
    assert oracle_lib.global_scale_tight_for_amax(0.0) == 1.0
    assert oracle_lib.global_scale_tight_for_amax(2688.0) == 1.0
    assert oracle_lib.global_scale_tight_for_amax(1344.0) == 0.5
    assert oracle_lib.global_scale_tight_for_amax(2688.0 * 3) == 3.0
    g = oracle_lib.global_scale_tight_for_amax(1.0)
    up = np.float32(1 / 2688)  # 1/2688 rounded up to binary32
    if Fraction(float(up)) < Fraction(1, 2688):
        up = np.nextafter(up, np.float32(1))
    assert g == float(up) and Fraction(1) <= 2688 * Fraction(g)


@pytest.mark.parametrize("seed", range(2))
def test_tight_global_scale_is_the_smallest_binary32_without_saturation(oracle_lib, seed):
    rng = np.random.default_rng(90 + seed)
    for a in np.float32(np.exp(rng.uniform(np.log(1e-6), np.log(1e9), 400))):
        a = float(a)
        g = oracle_lib.global_scale_tight_for_amax(a)
        assert np.float32(g) == g and g > 0
        below = float(np.nextafter(np.float32(g), np.float32(0)))
        assert Fraction(a) <= 2688 * Fraction(g)  # no block scale saturates at g ...
        assert Fraction(a) > 2688 * Fraction(below)  # ... and one would at the next smaller binary32
