"""Pins of the oracle's building blocks: closed forms, invariants, special
cases and library routines (torch / numpy in float64)."""
import math

import numpy as np
import pytest
import torch
import torch.nn.functional as Fn


def test_rmsnorm_closed_forms(orc):
    D, eps = 64, 1e-6
    ones = np.ones(D, np.float16)
    for c in (0.0, 0.3, -2.5, 1e-4):
        y = orc.rmsnorm(np.full(D, c), ones, eps)
        assert np.allclose(y, c / math.sqrt(c * c + eps), rtol=1e-15, atol=0)
    a, j = 3.0, 5
    x = np.zeros(D)
    x[j] = a
    g = np.random.default_rng(0).uniform(0.5, 1.5, D).astype(np.float16)
    y = orc.rmsnorm(x, g, eps)
    assert y[j] == pytest.approx(float(g[j]) * a / math.sqrt(a * a / D + eps), rel=1e-15)
    assert np.count_nonzero(y) == 1


def test_rmsnorm_vs_torch(orc):
    rng = np.random.default_rng(1)
    x = rng.standard_normal(2048)
    g = rng.uniform(-2, 2, 2048).astype(np.float16)
    ref = Fn.rms_norm(torch.from_numpy(x), (2048,), torch.from_numpy(g.astype(np.float64)), eps=1e-6).numpy()
    assert np.allclose(orc.rmsnorm(x, g, 1e-6), ref, rtol=1e-13, atol=1e-15)


def test_rope_identity_norm_and_relative(orc):
    rng = np.random.default_rng(2)
    hd = 128
    q = rng.standard_normal(hd)
    k = rng.standard_normal(hd)
    assert np.array_equal(orc.rope(q, 0), q)
    for pos in (1, 7, 513, 32895):
        r = orc.rope(q, pos)
        # each (j, j+hd/2) pair keeps its length
        assert np.allclose(r[:64] ** 2 + r[64:] ** 2, q[:64] ** 2 + q[64:] ** 2, rtol=1e-12)
    # <R(m) q, R(n) k> = <R(m-n) q, k>
    for m, n in ((5, 2), (700, 699), (40, 3)):
        lhs = orc.rope(q, m) @ orc.rope(k, n)
        rhs = orc.rope(q, m - n) @ k
        assert lhs == pytest.approx(rhs, rel=1e-10, abs=1e-10)
    # pair 0 has theta_0 = 1: position 1 rotates (1, 0) by exactly one radian
    e = np.zeros(hd)
    e[0] = 1.0
    r = orc.rope(e, 1)
    assert r[0] == pytest.approx(math.cos(1.0), abs=1e-15) and r[64] == pytest.approx(math.sin(1.0), abs=1e-15)
    # the last pair has theta = base^(-(hd-2)/hd)
    e = np.zeros(hd)
    e[63] = 1.0
    r = orc.rope(e, 10)
    th = 10000.0 ** (-126 / 128)
    assert r[63] == pytest.approx(math.cos(10 * th), abs=1e-15) and r[127] == pytest.approx(math.sin(10 * th),
                                                                                             abs=1e-15)


def test_attention_vs_torch_sdpa(orc):
    rng = np.random.default_rng(3)
    for L, hd in ((1, 64), (7, 64), (64, 128), (300, 128)):
        q = rng.standard_normal(hd)
        K = rng.standard_normal((L, hd))
        V = rng.standard_normal((L, hd))
        ref = Fn.scaled_dot_product_attention(torch.from_numpy(q)[None, None, None],
                                              torch.from_numpy(K)[None, None],
                                              torch.from_numpy(V)[None, None]).numpy().reshape(hd)
        assert np.allclose(orc.attention(q, K, V), ref, rtol=1e-12, atol=1e-13)


def test_attention_special_cases(orc):
    rng = np.random.default_rng(4)
    hd = 64
    q = rng.standard_normal(hd) * 10
    v0 = rng.standard_normal((1, hd))
    assert np.array_equal(orc.attention(q, rng.standard_normal((1, hd)), v0), v0[0])
    K = np.tile(rng.standard_normal(hd), (9, 1))
    V = rng.standard_normal((9, hd))
    assert np.allclose(orc.attention(q, K, V), V.mean(0), rtol=1e-13, atol=1e-14)
    # a key far above the rest takes all the weight (max-subtraction keeps it finite)
    K = rng.standard_normal((5, hd)) * 0.01
    K[2] = q * 50
    out = orc.attention(q, K, V[:5])
    assert np.all(np.isfinite(out)) and np.allclose(out, V[2], atol=1e-12)


def test_silu(orc):
    assert orc.silu(0.0) == 0.0
    z = np.linspace(-30, 30, 601)
    ref = Fn.silu(torch.from_numpy(z)).numpy()
    got = np.array([orc.silu(v) for v in z])
    assert np.allclose(got, ref, rtol=1e-14, atol=1e-300)


def test_argmax_ties_lowest(orc):
    v = np.array([0.0, 3.0, -1.0, 3.0, 3.0])
    assert orc.argmax(v) == 1
    rng = np.random.default_rng(5)
    for _ in range(20):
        v = rng.integers(0, 5, 1000).astype(np.float64)
        assert orc.argmax(v) == int(np.argmax(v))   # numpy returns the first maximum


def test_gemv_vs_numpy(orc):
    rng = np.random.default_rng(6)
    W = (rng.standard_normal((300, 517)) * 0.02).astype(np.float16)
    x = rng.standard_normal(517)
    ref = W.astype(np.float64) @ x
    assert np.allclose(orc.gemv(W, x), ref, rtol=1e-12, atol=1e-14)
