"""Pins for the oracle's quantizer, packer and dequantizer.

Symmetric per-group INT2/INT4 quantization with E4M3 scales
(paper.rainbus.top, method paragraph, Q; note.zhuruihan.top, Algorithm-System
Co-design).  Pinned by hand-computed bytes (tests/golden/packing.json), by the
level-count fact the pages state (INT2 has only 4 levels: paper.rainbus.top,
weaknesses paragraph), and by invariants of a symmetric mid-rise grid.
"""
import json
import os

import numpy as np
import pytest

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _deq(oracle, codes, scales, bits, G, d):
    H = 1
    N = codes.shape[0]
    out = oracle.decompress(codes[None], scales[None], np.zeros((1, 0, N), np.uint8),
                            np.zeros((1, 0, 1, d), np.float32), bits, G)
    return out[0]


@pytest.mark.parametrize("case", json.load(open(os.path.join(GOLD, "packing.json")))["cases"],
                         ids=lambda c: c["name"])
def test_packing_golden(oracle, case):
    r = np.array([case["row"]], np.float32)
    codes, scales = oracle.quantize(r, case["bits"], case["group"])
    assert codes[0].tolist() == case["codes"]
    assert scales[0].tolist() == case["scales"]


@pytest.mark.parametrize("bits", [2, 4])
def test_level_count_and_symmetry(oracle, bits):
    G, d = 64, 128
    # a dense ramp over [-a, a] hits every level of each group
    r = np.linspace(-5.0, 5.0, d, dtype=np.float32)[None].repeat(3, 0)
    r[1] *= 0.01
    r[2] *= 37.0
    codes, scales = oracle.quantize(r, bits, G)
    xr = _deq(oracle, codes, scales, bits, G, d)
    for i in range(3):
        for g in range(d // G):
            sh = oracle.e4m3_decode(scales[i, g])
            lv = np.unique(xr[i, g * G:(g + 1) * G])
            # the ramp of one group spans only part of [-a, a] in group 0/1
            full = (2 * np.arange(2 ** bits) - (2 ** bits - 1)) * np.float32(sh)
            assert set(lv.tolist()) <= set(full.astype(np.float32).tolist())
            # level(q) = -level(2^b-1-q)
            np.testing.assert_array_equal(full, -full[::-1])
    # a symmetric ramp in one group reaches all 2^b levels
    rr = np.linspace(-1, 1, 64, dtype=np.float32)[None]
    c, s = oracle.quantize(rr, bits, 64)
    assert len(np.unique(_deq(oracle, c, s, bits, 64, 64))) == 2 ** bits


@pytest.mark.parametrize("bits", [2, 4])
def test_error_bound(oracle, bits):
    rng = np.random.default_rng(3)
    G, d = 64, 128
    r = (rng.standard_normal((500, d)) * np.exp(rng.uniform(-8, 4, (500, 1)))).astype(np.float32)
    codes, scales = oracle.quantize(r, bits, G)
    xr = _deq(oracle, codes, scales, bits, G, d)
    L = 2 ** bits - 1
    for g in range(d // G):
        sl = slice(g * G, (g + 1) * G)
        a = np.abs(r[:, sl]).max(1)
        sh = np.array([oracle.e4m3_decode(x) for x in scales[:, g]], np.float64)
        bound = np.maximum(sh, a - L * sh) * (1 + 1e-6)
        err = np.abs(r[:, sl].astype(np.float64) - xr[:, sl]).max(1)
        assert np.all(err <= bound)
        # the top level is within E4M3 rounding of a: 2^-4 relative for
        # normal scales, half the 2^-9 subnormal step (times L) below 2^-6
        s = a / L
        normal = s >= 2.0 ** -6
        np.testing.assert_allclose(L * sh[normal], a[normal], rtol=2 ** -4 + 1e-7)
        assert np.all(np.abs(L * sh[~normal] - a[~normal]) <= L * 2.0 ** -10 * (1 + 1e-6))


@pytest.mark.parametrize("bits", [2, 4])
def test_requantize_on_grid_is_identity(oracle, bits):
    rng = np.random.default_rng(4)
    L = 2 ** bits - 1
    q = rng.integers(0, L + 1, (50, 128))
    q[:, 0] = L  # every group of 64 reaches the top level, so s_hat is reproduced
    q[:, 64] = 0
    sh = np.float32(0.375)  # exact E4M3 value
    r = ((2 * q - L) * sh).astype(np.float32)
    codes, scales = oracle.quantize(r, bits, 64)
    np.testing.assert_array_equal(_deq(oracle, codes, scales, bits, 64, 128), r)


def test_zero_group_and_saturation(oracle):
    r = np.zeros((2, 128), np.float32)
    r[1, :64] = np.linspace(-4000, 4000, 64)  # s = 4000/3 saturates to 448
    codes, scales = oracle.quantize(r, 2, 64)
    assert scales[0].tolist() == [0, 0] and scales[1].tolist() == [0x7E, 0]
    xr = _deq(oracle, codes, scales, 2, 64, 128)
    assert np.all(xr[0] == 0) and np.all(xr[1, 64:] == 0)
    assert xr[1, :64].max() == 3 * 448.0 and xr[1, :64].min() == -3 * 448.0
