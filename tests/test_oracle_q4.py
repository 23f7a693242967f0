"""Pins of the oracle's weight-only INT4 format (groups of 128 columns,
fp32 scales; "LLM inference architecture rebuild", section 5.2: an INT4
weight is used as fp16(int4_value * scale) with the scale in fp32 and
round-to-nearest).  The quantizer itself is not on the pages: symmetric,
scale = amax / 7 per (row, group)."""
import numpy as np
import pytest


def test_q4_exact_grid_round_trips(orc):
    """A group whose values are q * 2^-6 for integers |q| <= 7 with one
    |q| = 7 has scale 2^-6 exactly, codes q, and dequantizes to itself."""
    rng = np.random.default_rng(1)
    q = rng.integers(-7, 8, (6, 256))
    q[:, 5] = 7
    q[:, 128 + 9] = -7
    w = (q * 2.0 ** -6).astype(np.float16)
    codes, scales = orc.q4_quant(w)
    assert np.all(scales == np.float32(2.0 ** -6))
    got = np.array([[orc.lib().orc_q4_code(codes.ctypes.data_as(orc.C.POINTER(orc.C.c_uint8)), r * 256 + c)
                     for c in range(256)] for r in range(6)])
    assert np.array_equal(got, q)
    assert np.array_equal(orc.q4_dequant(codes, scales), w)


def test_q4_nibble_order(orc):
    """Column 2j is the low nibble of byte j, two's complement."""
    w = np.zeros((1, 128), np.float16)
    w[0, 0], w[0, 1], w[0, 2], w[0, 127] = 7, -7, 1, -3     # amax 7: scale 1
    codes, scales = orc.q4_quant(w)
    assert scales[0, 0] == 1.0
    assert codes[0, 0] == (7 | ((-7 & 15) << 4))
    assert codes[0, 1] == 1
    assert codes[0, 63] == ((-3 & 15) << 4)


@pytest.mark.parametrize("std,seed", [(0.02, 2), (1.0, 3), (300.0, 4)])
def test_q4_invariants(orc, std, seed):
    rng = np.random.default_rng(seed)
    w = (rng.standard_normal((8, 512)) * std).astype(np.float16)
    w[3, 128:256] = 0                                       # an all-zero group
    codes, scales = orc.q4_quant(w)
    deq = orc.q4_dequant(codes, scales)
    wf = w.astype(np.float32).reshape(8, 4, 128)
    amax = np.abs(wf).max(axis=2)
    # scale = amax / 7 in binary32, 1 for a zero group
    ref = np.where(amax > 0, (amax / np.float32(7)).astype(np.float32), np.float32(1))
    assert np.array_equal(scales, ref)
    # the largest magnitude of a group maps to +-7, and nothing reaches -8
    cd = np.array([[orc.lib().orc_q4_code(codes.ctypes.data_as(orc.C.POINTER(orc.C.c_uint8)), r * 512 + c)
                    for c in range(512)] for r in range(8)]).reshape(8, 4, 128)
    nz = amax > 0
    assert np.all(np.abs(cd).max(axis=2)[nz] == 7) and cd.min() >= -7
    assert np.all(cd[3, 1] == 0) and np.all(deq[3, 128:256] == 0)
    # dequantized value: fp16(float(code) * scale), binary32 product then round to nearest
    prod = (cd.astype(np.float32) * scales[:, :, None]).astype(np.float32)
    assert np.array_equal(deq.view(np.uint16), prod.astype(np.float16).reshape(8, 512).view(np.uint16))
    # round trip within half a step, plus the fp16 rounding of the result
    err = np.abs(deq.astype(np.float64).reshape(8, 4, 128) - wf.astype(np.float64))
    bound = scales[:, :, None].astype(np.float64) / 2 * (1 + 1e-6) + np.abs(wf) * 2.0 ** -11 + 2.0 ** -24
    assert np.all(err <= bound)
    # symmetric: negating the weights negates the codes, keeps the scales
    c2, s2 = orc.q4_quant(-w)
    cd2 = np.array([[orc.lib().orc_q4_code(c2.ctypes.data_as(orc.C.POINTER(orc.C.c_uint8)), r * 512 + c)
                     for c in range(512)] for r in range(8)]).reshape(8, 4, 128)
    assert np.array_equal(s2, scales) and np.array_equal(cd2, -cd)
