"""Pins of the oracle's number formats and of the segment quantizer.

binary16 conversions are checked exhaustively against numpy's IEEE
conversions; E5M2 exhaustively against torch.float8_e5m2; the quantizer
against the worked example of "Grok-3 v3.2.4 hot update" §3.2 (golden file)
and against the invariants its definition implies.
"""
import json
import os

import numpy as np
import pytest
import torch

GOLD = os.path.join(os.path.dirname(__file__), "golden")
ALL16 = np.arange(65536, dtype=np.uint16)


def test_h2d_exhaustive(orc):
    got = orc.h2d(ALL16)
    ref = ALL16.view(np.float16).astype(np.float64)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])
    # signed zeros keep their sign
    assert np.signbit(got[0x8000]) and not np.signbit(got[0])


def test_d2h_matches_numpy_rne(orc):
    rng = np.random.default_rng(7)
    # every binary16 value, every midpoint between neighbours (ties), and
    # points a hair either side of each midpoint
    v = ALL16.view(np.float16).astype(np.float64)
    fin = v[np.isfinite(v)]
    fin = np.unique(fin)
    mids = (fin[:-1] + fin[1:]) / 2
    eps = np.abs(mids) * 1e-12 + 1e-300
    x = np.concatenate([fin, mids, mids + eps, mids - eps,
                        rng.standard_normal(200000) * np.exp(rng.uniform(-20, 12, 200000)),
                        [65504.0, 65519.999, 65520.0, 1e6, -1e6, 2.0 ** -24, 2.0 ** -25, 2.0 ** -26, 3 * 2.0 ** -26,
                         0.0, -0.0]])
    got = orc.d2h(x)
    ref = x.astype(np.float16).view(np.uint16)
    bad = np.nonzero(got != ref)[0]
    assert bad.size == 0, (x[bad[:5]], got[bad[:5]], ref[bad[:5]])
    assert orc.d2h(np.array([np.nan]))[0] & 0x7c00 == 0x7c00


def test_e5m2_exhaustive_vs_torch(orc):
    got = orc.e5m2_from_h(ALL16)
    ref = torch.from_numpy(ALL16.view(np.float16).copy()).to(torch.float8_e5m2).view(torch.uint8).numpy()
    isnan16 = np.isnan(ALL16.view(np.float16))
    # NaN: both produce a NaN code (payloads differ and do not matter)
    nan_code = lambda c: ((c & 0x7c) == 0x7c) & ((c & 3) != 0)
    assert np.all(nan_code(got[isnan16])) and np.all(nan_code(ref[isnan16]))
    assert np.array_equal(got[~isnan16], ref[~isnan16])


def test_e5m2_decode_exact_and_range(orc):
    gold = json.load(open(os.path.join(GOLD, "e5m2_range.json")))
    codes = np.arange(256, dtype=np.uint8)
    h = orc.h_from_e5m2(codes)
    vals = h.view(np.float16).astype(np.float64)
    ref = torch.from_numpy(codes.copy()).view(torch.float8_e5m2).to(torch.float64).numpy()
    fin = np.isfinite(ref)
    assert np.array_equal(vals[fin], ref[fin])
    assert np.nanmax(np.where(np.isfinite(vals), vals, np.nan)) == gold["max_finite"]
    # decoding is exact, so encode(decode(c)) == c for every non-NaN code
    nonnan = ~np.isnan(vals)
    assert np.array_equal(orc.e5m2_from_h(h)[nonnan], codes[nonnan])
    # decode is the binary16 pattern with the E5M2 byte in the high half
    assert np.array_equal(h[nonnan], codes[nonnan].astype(np.uint16) << 8)


def _seg_with(mn, mx, n=128 * 64, seed=0):
    rng = np.random.default_rng(seed)
    x = rng.uniform(mn, mx, n).astype(np.float16)
    x[3] = np.float16(mn)
    x[n - 5] = np.float16(mx)
    return x


def test_segquant_worked_example(orc):
    g = json.load(open(os.path.join(GOLD, "segment_quant_example.json")))
    x = _seg_with(g["min"], g["max"], n=g["segment_tokens"] * 64)
    codes, scale, zp = orc.seg_quant(x.view(np.uint16))
    assert abs(float(scale) - g["scale_approx"]) <= g["scale_abs_tol"]
    assert float(zp) == g["zero_point_approx"]
    t = g["exact_tie"]
    x = _seg_with(t["min"], t["max"], seed=1)
    assert float(x.min()) == t["min"] and float(x.max()) == t["max"]
    codes, scale, zp = orc.seg_quant(x.view(np.uint16))
    assert float(scale) == t["scale"]          # (max-min)/255 is exactly 2^-6 here
    assert float(zp) == t["zero_point"]        # -min/scale = 76.5 exactly: half-to-even


@pytest.mark.parametrize("lo,hi,seed", [(-1.2, 2.8, 0), (-3.0, -0.5, 1), (0.25, 9.0, 2), (-60000, 60000, 3),
                                        (-1e-3, 2e-3, 4), (-0.7, 0.7, 5)])
def test_segquant_invariants(orc, lo, hi, seed):
    x = _seg_with(lo, hi, seed=seed)
    codes, scale, zp = orc.seg_quant(x.view(np.uint16))
    xf = x.astype(np.float32)
    mn, mx = xf.min(), xf.max()
    assert scale == np.float32(np.float32(mx - mn) / np.float32(255))
    assert zp == np.float32(np.rint(np.float32(-mn) / scale))
    # the minimum maps to code 0; the maximum to 255, or 254 when both ends sit on ties
    assert codes[np.argmin(xf)] == 0
    assert codes[np.argmax(xf)] in (254, 255)
    # monotone
    o = np.argsort(xf, kind="stable")
    assert np.all(np.diff(codes[o].astype(int)) >= 0)
    # round trip within half a step (plus binary32 rounding)
    deq = orc.seg_dequant(codes, scale, zp)
    err = np.abs(deq.astype(np.float64) - xf.astype(np.float64))
    assert err.max() <= 0.5 * float(scale) * (1 + 1e-4) + 1e-6 * float(np.abs(xf).max())
    # dequantization is (code - zp) * scale in binary32
    assert np.array_equal(deq, (codes.astype(np.float32) - zp) * scale)


@pytest.mark.parametrize("c", [0.3, -0.3, 0.5, -1e-3, 60000.0, 2.0 ** -24, 0.0])
def test_segquant_degenerate(orc, c):
    """A segment of one repeated value (max == min, where the page's formula
    gives scale 0) dequantizes to that value exactly: scale |min|, zero point
    -sign(min), every code 0; an all-zero segment takes scale 1."""
    x = np.full(128 * 4, c, np.float16)
    codes, scale, zp = orc.seg_quant(x.view(np.uint16))
    v = np.float32(x[0])
    assert scale == (abs(v) if v != 0 else np.float32(1.0))
    assert zp == np.float32(-np.sign(v))
    assert np.all(codes == 0)
    assert np.all(orc.seg_dequant(codes[:4], scale, zp) == v)
