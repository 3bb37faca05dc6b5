"""Pins of the oracle's bit-level exponentials ("FLAMIA: FLAsh MIcroscaling Attention
for Fast and Causally Safe Training on Blackwell", section 3.7 and appendix C).

The piecewise-linear exponential is pinned against IEEE-754 bit patterns built with
numpy (an integer read as a float32), the offsets against numerical extrema and
integrals (scipy), the code agreement against the figure the pages report, and the
attention's use of it against a brute-force weighted average on one query row.
"""
import numpy as np
import pytest
import scipy.integrate
import scipy.optimize

import synth


def bits_value(t):
    """float32 whose bits are floor(2^23 (t + 127)), clamped at 0: built from the IEEE layout"""
    u = np.floor((np.asarray(t, np.float64) + 127.0) * 2.0 ** 23)
    u = np.clip(u, 0, 2 ** 31 - 1).astype(np.uint32)
    return u.view(np.float32).astype(np.float64)


def test_exp2_bits_integers_and_fractions(orc):
    for n in range(-126, 128, 7):
        assert orc.exp2_bits(float(n)) == 2.0 ** n
        assert orc.exp2_bits(n + 0.5) == 1.5 * 2.0 ** n
        assert orc.exp2_bits(n + 0.25) == 1.25 * 2.0 ** n
    # continuous at the octave boundaries, increasing inside them
    t = np.linspace(-5.0, 3.0, 4001)
    v = orc.exp2_bits(t)
    assert np.all(np.diff(v) > 0)


def test_exp2_bits_is_the_float_bit_pattern(orc):
    """On a grid where 2^23 (t + 127) is an integer the value equals the float32 whose
    bits are that integer -- normal numbers, the subnormal piece below t = -126 and the
    clamp to +0 below t = -127."""
    rng = np.random.default_rng(3)
    k = rng.integers(-130 * 2 ** 23, 128 * 2 ** 23, 4000)
    k = np.concatenate([k, np.arange(-127 * 2 ** 23 - 5, -127 * 2 ** 23 + 5), [-126 * 2 ** 23 - 1, -126 * 2 ** 23]])
    t = k.astype(np.float64) / 2.0 ** 23
    assert np.array_equal(orc.exp2_bits(t), bits_value(t))
    assert orc.exp2_bits(-127.5) == 0.0 and orc.exp2_bits(-np.inf) == 0.0 and orc.exp2_bits(np.nan) == 0.0


def test_mitchell_offset_centres_the_error(orc):
    """delta is half the largest log2 error of the line, log2(1 + f) - f (found by a
    numerical maximization); with it the line's log2 ratio to 2^x spans [-delta, delta]."""
    res = scipy.optimize.minimize_scalar(lambda f: -(np.log2(1 + f) - f), bounds=(0, 1), method="bounded",
                                         options={"xatol": 1e-12})
    d = orc.exp_offset("mitchell")
    assert abs(d - (-res.fun) / 2) < 1e-9
    assert abs(d - 0.0430357) < 1e-6  # Mitchell's centred correction of log2(1 + f) ~ f
    x = np.concatenate([np.linspace(-3.0, 0.0, 30001), d - np.arange(1, 3)])  # with the kinks
    lr = np.log2(orc.exp2_bits(x - d)) - x
    assert abs(lr.max() - d) < 1e-6 and abs(lr.min() + d) < 1e-6
    assert np.abs(orc.exp2_bits(x - d) / 2.0 ** x - 1).max() < 0.031  # within about 3 %


def test_schraudolph_offset_averages_one(orc):
    """The ratio of the offset line to 2^x averages one over an octave (numerical
    integral); without the offset it averages 1.0407 and never falls below one."""
    d = orc.exp_offset("schraudolph")
    mean, _ = scipy.integrate.quad(lambda x: orc.exp2_bits(x - d)[()] / 2.0 ** x, -1.0, 0.0, points=[d - 1.0],
                                   epsabs=1e-13, limit=200)  # one kink, at x - d = -1
    assert abs(mean - 1.0) < 1e-9
    raw, _ = scipy.integrate.quad(lambda x: orc.exp2_bits(x)[()] / 2.0 ** x, -1.0, 0.0, epsabs=1e-13)
    assert abs(raw - 1.0407) < 1e-4
    assert orc.exp_offset("exact") == 0.0


def test_mitchell_codes_agree_with_exact_rounding(orc):
    """E2M1 codes of 6 P~ with the Mitchell-P exponential match those of the exact
    exponential on about 98 % of Gaussian scores (the pages report 98.7 % on their
    inputs); the uncentred line (offset 0) matches fewer."""
    rng = np.random.default_rng(5)
    q = rng.standard_normal((16, 128))
    k = rng.standard_normal((2048, 128))
    s = q @ k.T / np.sqrt(128)
    x = (s - s.max(1, keepdims=True)).ravel() / np.log(2.0)  # log2 units, <= 0
    x = x[x > -12.0]
    grid = orc.e2m1_values(np.arange(8)).astype(np.float64)
    mids = (grid[1:] + grid[:-1]) / 2

    def codes(p):
        return np.searchsorted(mids, 6.0 * p, side="left")

    exact = codes(2.0 ** x)
    agree = np.mean(codes(orc.exp2_bits(x - orc.exp_offset("mitchell"))) == exact)
    raw = np.mean(codes(orc.exp2_bits(x)) == exact)
    assert agree > 0.975 and agree > raw + 0.005


@pytest.mark.parametrize("mode", ["mitchell", "schraudolph"])
def test_attention_uses_the_line_on_scaled_scores(orc, mode):
    """One query row whose largest score sits in the first key tile (so the running
    maximum never moves): O and lse equal the brute-force average with weights
    w_j = line(sm_scale (s_j - max) / ln 2 - delta)."""
    N, d = 300, 64
    Q = synth.gaussian(1, 9, (N, d)).astype(np.float32)
    K = synth.gaussian(1, 10, (N, d)).astype(np.float32)
    V = synth.gaussian(1, 11, (N, d)).astype(np.float32)
    K[3] = (45.0 * Q[0] / np.dot(Q[0], Q[0])).astype(np.float32)  # score 45: row 0's maximum, in tile 0
    O, lse, _ = orc.attention(Q[None, None], K[None, None], V[None, None], orc.P_NONE, rows=np.array([0]),
                              exp_mode=mode)
    sm = 1.0 / np.sqrt(d)
    s = (Q[0].astype(np.float64) @ K.astype(np.float64).T).astype(np.float32).astype(np.float64)
    assert np.argmax(s) == 3
    w = bits_value(sm * (s - s.max()) / np.log(2.0) - orc.exp_offset(mode)).astype(np.float32).astype(np.float64)
    ref = (w @ V.astype(np.float64)) / w.sum()
    assert np.allclose(O[0], ref, rtol=0, atol=2e-6)
    assert abs(lse[0] - (np.log(w.sum()) + sm * s.max())) < 2e-5
    # the exact mode differs by the approximation (a few per cent of the weights)
    O_e, _, _ = orc.attention(Q[None, None], K[None, None], V[None, None], orc.P_NONE, rows=np.array([0]))
    assert np.abs(O_e[0] - O[0]).max() > 1e-4


def test_invalid_mode_rejected(orc):
    import ctypes
    Q = np.zeros((1, 1, 4, 8), np.float32)
    p = orc.AttnParams(orc.P_NONE, orc.Fmt(0, 0, 32, 0, 0.0), 0, 0.35, 128, 7)
    O = np.zeros((4, 8), np.float32)
    rc = orc.lib().orc_attention_ex(orc._ptr(Q, ctypes.c_float), orc._ptr(Q, ctypes.c_float),
                                    orc._ptr(Q, ctypes.c_float), None, None, None, 1, 1, 1, 4, 8, None, 0,
                                    ctypes.byref(p), None, 4, orc._ptr(O, ctypes.c_float), None, None)
    assert rc == -4
