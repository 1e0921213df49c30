"""FP8 (e4m3) MLP GEMMs against the decode tolerance, on the oracle (CPU).

[FD] §4.6 "Inference Optimization" item (4) runs the MLP layers in FP8.  The
study script tests/fp8_mlp_study.py measures the pixel error that rounding
the MLP operands to e4m3 causes on the seeded workloads; here its quantizers
are pinned and a reduced case is checked to be over the bar already.
"""
import numpy as np
import pytest

import workloads as W
from fp8_mlp_study import VARIANTS, block32, e4m3, per_tensor, study


def test_e4m3_rounding_pins():
    # e4m3: 3 mantissa bits, bias 7, largest finite 448, ties to even.
    x = np.array([1.0, 1.0625, 1.1875, 1.2, 448.0, -3.3, 2.0 ** -9, 2.0 ** -10 * 1.5, 0.0])
    ref = np.array([1.0, 1.0, 1.25, 1.25, 448.0, -3.25, 2.0 ** -9, 2.0 ** -9, 0.0])
    assert np.array_equal(e4m3(x), ref)


def test_per_tensor_scale_maps_the_max_to_448():
    x = W.standard_normal(21, 1, 64 * 96).reshape(64, 96) * 0.02
    q = per_tensor(x)
    k = np.argmax(np.abs(x))
    assert abs(q.flat[k] - x.flat[k]) <= 1e-12 * abs(x.flat[k])       # 448 is exact
    assert np.abs(q - x).max() <= np.abs(x).max() / 448.0 * 16.0     # half a step at the top


def test_block_scales_are_powers_of_two_without_clipping():
    x = W.standard_normal(21, 2, 8 * 64).reshape(8, 64) * np.exp2(np.arange(8))[:, None]
    q = block32(x)
    rel = np.abs(q - x) / np.maximum(np.abs(x), 1e-30)
    big = np.abs(x) >= np.abs(x).reshape(8, 2, 32).max(-1).repeat(32, 1) / 8.0
    assert (rel[big] <= 2.0 ** -4 + 1e-12).all()                     # normal e4m3 spacing
    # scaling by powers of two commutes with the rounding of the normal range
    assert np.array_equal(block32(x * 4.0), q * 4.0)


def test_fp8_mlp_misses_the_pixel_tolerance_even_on_one_block():
    cfg = W.CONFIGS["480p"].replace(n_layers=1)
    out = study(cfg, 1, log=lambda *_: None)
    assert set(out) == set(VARIANTS)
    for name, (ma, rl) in out.items():
        assert rl > 1e-2 and ma > 3e-2, (name, ma, rl)
