"""Pins of the oracle's YaRN pieces (CPU only), V2 analysis page, section 3.2.

* The values the page prints (tests/golden/yarn.txt): s = 40, alpha = 1,
  beta = 32, the 160K upper limit, and the temperature factors about 1.26
  (V2's coefficient 0.0707) and 1.37 (the original 0.1) at s = 40.
* The frequency ramp at its ends and in the middle, computed here from the
  number of turns a pair makes across the original 4K window: fast pairs
  keep their frequency exactly, slow pairs are slowed by exactly s, a pair
  half way along the ramp gets the mean; factor 1 is plain RoPE.
* A fully interpolated pair at position s*p turns by the angle the plain
  frequency gives at p.
* The library's host helpers (mla_yarn_frequencies, mla_yarn_mscale) equal
  the oracle's.
"""
import math
import os

import numpy as np
import pytest

from oracle import mla_oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "yarn.txt")


def golden():
    out = {}
    for line in open(GOLDEN):
        if line.strip() and not line.startswith("#"):
            k, v, tol, _ = [x.strip() for x in line.split("|")]
            out[k] = (float(v), float(tol))
    return out


def test_printed_values():
    g = golden()
    s, alpha, beta = g["factor"][0], g["alpha"][0], g["beta"][0]
    assert (s, alpha, beta) == (40.0, 1.0, 32.0)
    assert 4 * s == g["target_window_k"][0]
    for key, coef in (("mscale_v2", 0.0707), ("mscale_original", 0.1)):
        v, tol = g[key]
        assert abs(O.yarn_mscale(s, coef) - v) <= tol, (key, O.yarn_mscale(s, coef))
    assert O.yarn_mscale(1.0) == 1.0 and O.yarn_mscale(0.5) == 1.0


def plain(d=64, base=10000.0):
    return np.array([math.pow(base, -2.0 * i / d) for i in range(d // 2)])


def test_ramp_ends_and_middle():
    d, base, s, a, b, L0 = 64, 10000.0, 40.0, 1.0, 32.0, 4096
    th = plain(d, base)
    turns = L0 * th / (2 * math.pi)
    y = O.yarn_theta(d, base, s, a, b, L0)
    fast, slow = turns >= b, turns <= a
    assert fast.any() and slow.any() and (~fast & ~slow).any()
    assert np.array_equal(y[fast], th[fast])
    assert np.array_equal(y[slow], th[slow] / s)
    mid = ~fast & ~slow
    g = (turns[mid] - a) / (b - a)
    assert np.allclose(y[mid], (1 - g) * th[mid] / s + g * th[mid], rtol=1e-15, atol=0)
    assert np.all(np.diff(y) < 0)                  # frequencies stay ordered
    # a ramp from 0 to 2 turns: the pair making 1.5 turns sits half way (ramp 0.5 .. 2.5)
    L1 = 2 * math.pi * 1.5 / th[10]
    y1 = O.yarn_theta(d, base, s, 0.5, 2.5, L1)
    assert math.isclose(y1[10], 0.5 * (th[10] / s + th[10]), rel_tol=1e-12)
    assert np.allclose(O.yarn_theta(d, base, 1.0, a, b, L0), th, rtol=1e-15, atol=0)


def test_interpolated_pair_angle():
    d, s = 64, 40.0
    y = O.yarn_theta(d, 10000.0, s, 1.0, 32.0, 4096)
    th = plain(d)
    i = d // 2 - 1                                   # the slowest pair is fully interpolated
    for p in (1, 100, 3000):
        assert math.isclose(y[i] * (s * p), th[i] * p, rel_tol=1e-15)
    # the same statement through the rotation itself
    x = np.random.default_rng(3).standard_normal((1, d))
    r1 = O.rope_rotate(x, np.array([int(s) * 77]), theta=y)
    r0 = O.rope_rotate(x, np.array([77]))
    assert np.allclose(r1[0, 2 * i:2 * i + 2], r0[0, 2 * i:2 * i + 2], rtol=0, atol=1e-12)


def test_plain_theta_reproduces_default_rope():
    x = np.random.default_rng(4).standard_normal((3, 5, 64))
    pos = np.array([0, 4095, 131071])
    assert np.array_equal(O.rope_rotate(x, pos), O.rope_rotate(x, pos, theta=plain()))


def test_library_host_helpers_equal_oracle():
    lib = os.path.join(os.path.dirname(os.path.dirname(__file__)), "mla_latent_kv_35_amd",
                       "libmla.so")
    if not os.path.exists(lib):
        pytest.skip("libmla.so not built")
    from mla_latent_kv_35_amd import binding as B
    for args in ((64, 10000.0, 40.0, 1.0, 32.0, 4096), (32, 500.0, 8.0, 0.5, 16.0, 1000),
                 (64, 10000.0, 1.0, 1.0, 32.0, 4096)):
        assert np.allclose(B.yarn_frequencies(*args), O.yarn_theta(*args), rtol=1e-15, atol=0)
    assert B.yarn_mscale(40.0, 0.0707) == O.yarn_mscale(40.0, 0.0707)
    assert B.yarn_mscale(0.5, 0.0707) == 1.0
    with pytest.raises(B.MlaError):
        B.yarn_frequencies(64, 10000.0, 0.5, 1.0, 32.0, 4096)      # factor < 1
    with pytest.raises(B.MlaError):
        B.yarn_frequencies(64, 10000.0, 40.0, 32.0, 1.0, 4096)     # beta <= alpha


def test_ramp_bounds_and_constructed_edges():
    """Every interpolated frequency lies between the fully slowed theta / s and
    the plain theta, and is continuous at both edges of the ramp: windows
    built so that one pair makes exactly alpha (exactly beta) turns give that
    pair theta / s (theta), and a window a hair longer or shorter moves it
    only a hair. A swapped alpha / beta or an inverted ramp fails these."""
    d, base, s = 64, 10000.0, 40.0
    th = plain(d, base)
    for (a, b, L0) in ((1.0, 32.0, 4096), (0.5, 4.0, 1000), (2.0, 64.0, 32768)):
        y = O.yarn_theta(d, base, s, a, b, L0)
        assert np.all(y <= th * (1 + 1e-15)) and np.all(y >= th / s * (1 - 1e-15))
    i = 20
    for turns, want in ((1.0, th[i] / s), (32.0, th[i])):
        L_edge = 2 * math.pi * turns / th[i]
        y = O.yarn_theta(d, base, s, 1.0, 32.0, L_edge)
        assert math.isclose(y[i], want, rel_tol=1e-12)
        for eps in (1e-9, -1e-9):
            y2 = O.yarn_theta(d, base, s, 1.0, 32.0, L_edge * (1 + eps))
            assert abs(y2[i] - want) <= 1e-6 * want
