"""Pins of the oracle's delta quantization ("Grok-3 v3.2.4 hot update deep
dive", §3.2: adjacent-token differences of the K/V values, quantized to
INT8).  The reading (anchor row, binary32 differences of the exact values,
one adaptive-range quantizer per segment, restore by adding the differences
in row order) is the oracle's; these tests check it against values fixed by
hand and by the arithmetic, not against a second copy of its formula."""
import numpy as np
import pytest

import oracle


def h(a):
    return np.asarray(a, dtype=np.float16).view(np.uint16)


def test_delta_hand_example():
    # rows [1, -2], [1.5, -2], [0.5, 0]: differences [0.5, 0] and [-1, 2];
    # min -1, max 2: scale 3/255, zero point 85; 0.5 / (3/255) = 42.5 rounds
    # half to even to 42 -> code 127; 0 -> 85; -1 -> 0; 2 -> 255
    x = h([[1.0, -2.0], [1.5, -2.0], [0.5, 0.0]])
    anchor, codes, scale, zp = oracle.delta_seal(x)
    assert anchor.tolist() == h([1.0, -2.0]).tolist()
    assert codes.tolist() == [[127, 85], [0, 255]]
    assert zp == 85.0
    assert abs(float(scale) - 3.0 / 255.0) < 1e-9
    y = oracle.delta_restore(anchor, codes, scale, zp)
    # row 1 keeps 42 steps of 3/255 instead of 42.5: 1 + 42*3/255; row 2
    # adds -85 steps (exactly -1) to it, so the error carries on
    want = [[1.0, -2.0], [1.0 + 42 * 3 / 255, -2.0], [42 * 3 / 255, 0.0]]
    assert np.allclose(y, want, rtol=0, atol=1e-6)


def test_delta_grid_differences_restore_exactly():
    # differences k * 2^-4 with k in [-100, 155], both ends present: scale is
    # exactly 2^-4, the zero point 100 and code k + 100; every product and
    # sum is exact, so the rows come back bit for bit
    rng = np.random.default_rng(7)
    n, hd = 8, 16
    k = rng.integers(-100, 156, size=(n - 1, hd))
    k[0, 0], k[3, 5] = -100, 155
    x = np.zeros((n, hd), np.float64)
    x[0] = rng.integers(-200, 200, size=hd) / 16.0
    for p in range(1, n):
        x[p] = x[p - 1] + k[p - 1] / 16.0
    assert np.all(np.abs(x) < 128)            # exact in binary16
    anchor, codes, scale, zp = oracle.delta_seal(h(x))
    assert scale == np.float32(1 / 16) and zp == 100.0
    assert np.array_equal(codes.astype(np.int64), k + 100)   # x[p] - x[p-1], not the reverse
    y = oracle.delta_restore(anchor, codes, scale, zp)
    assert np.array_equal(y, x.astype(np.float32))


def test_delta_constant_step_is_exact():
    # the same step in every element: one difference value, the
    # constant-segment rule (scale |step|, zero point -1) keeps it exactly
    n, hd = 128, 64
    step = 0.25
    base = np.arange(hd) / 8.0 - 4.0             # multiples of 1/8: exact in binary16 here
    x = np.array([base + p * step for p in range(n)])
    anchor, codes, scale, zp = oracle.delta_seal(h(x))
    assert scale == np.float32(step) and zp == -1.0 and not codes.any()
    y = oracle.delta_restore(anchor, codes, scale, zp)
    assert np.array_equal(y, h(x).view(np.float16).astype(np.float32))


def test_delta_error_adds_up_along_the_segment():
    # each dequantized difference is within half a step of the exact one, so
    # row p is within p half-steps (plus binary32 rounding of the sums)
    rng = np.random.default_rng(11)
    for hd in (64, 128):
        x = np.cumsum(rng.normal(0, 0.05, size=(128, hd)), axis=0) + rng.normal(0, 1, size=hd)
        xb = h(x)
        xf = xb.view(np.float16).astype(np.float64)
        anchor, codes, scale, zp = oracle.delta_seal(xb)
        y = oracle.delta_restore(anchor, codes, scale, zp).astype(np.float64)
        assert np.array_equal(y[0], xf[0])
        p = np.arange(128)[:, None]
        bound = p * float(scale) / 2 * (1 + 1e-5) + p * 2.0 ** -23 * (np.abs(xf).max() + 1)
        assert np.all(np.abs(y - xf) <= bound)
        assert np.abs(y - xf).max() > float(scale) / 2   # and it does grow past one half-step


def test_delta_abrupt_token_coarsens_the_segment():
    # the page's failure mode: one abrupt token widens the range of the
    # differences, so every other row is quantized more coarsely
    rng = np.random.default_rng(5)
    x = np.cumsum(rng.normal(0, 0.01, size=(128, 64)), axis=0)
    smooth = oracle.delta_seal(h(x))
    xj = x.copy()
    xj[64:] += 8.0                               # the jump between rows 63 and 64
    jump = oracle.delta_seal(h(xj))
    assert jump[2] > 50 * smooth[2]
    err = lambda s, ref: np.abs(oracle.delta_restore(*s)[:64] - h(ref[:64]).view(np.float16).astype(np.float32)).max()
    assert err(jump, xj) > 10 * err(smooth, x)


def test_delta_one_row():
    x = h([[0.5, -3.0, 7.0]])
    anchor, codes, scale, zp = oracle.delta_seal(x)
    assert anchor.tolist() == x[0].tolist() and codes.shape == (0, 3)
    assert np.array_equal(oracle.delta_restore(anchor, codes, scale, zp), np.array([[0.5, -3.0, 7.0]], np.float32))
