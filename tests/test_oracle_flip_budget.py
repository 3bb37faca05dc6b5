"""Pins of the oracle's flip budget on constructed rows whose fragile decisions, and
their effect on O, are known in closed form.

One query row q = e_0 makes every score exactly the first channel of its key, so the
rows below place P~ = exp(s / sqrt(128)) where they are wanted.  The P format is
MXFP4 with the OCP rule ("MXAttention", section 2 and Table 1: e = floor(log2 M) - 2,
normalized block maximum in [4, 8), (7, 8) saturating to 6) in DIRECT mode, where
the row sum l is the sum of the unquantized P~ ("MXAttention", section 5.2).
"""
import numpy as np
import pytest

D = 128
SM = 1.0 / np.sqrt(D)


def _row(orc, scores, V, pmode=None, pfmt="mxfp4", k_extra=None):
    """Oracle output of one query row e_0 over keys with the given exact scores.
    k_extra: optional [nk, D] added to K's other channels (q ignores them unless a
    score must carry rounding error, see test_near_tie_with_inexact_scores)."""
    nk = len(scores)
    Q = np.zeros((1, 1, nk, D), np.float32)
    Q[0, 0, :, 0] = 1.0
    K = np.zeros((1, 1, nk, D), np.float32)
    K[0, 0, :, 0] = np.asarray(scores, np.float32)
    if k_extra is not None:
        K[0, 0] += k_extra
        Q[0, 0, :, 1:] = 1.0
    O, lse, fb = orc.attention(Q, K, np.asarray(V, np.float32)[None, None], orc.P_DIRECT if pmode is None else pmode,
                               pfmt, rows=np.array([0]))
    return O[0], fb[0]


def _score_for(p):
    """a float score whose P~ = exp(s SM) is p up to the rounding of s"""
    return float(np.float32(np.log(p) / SM))


def _p(s):
    return float(np.float32(np.exp(SM * float(np.float32(s)))))


def _values(nk, seed):
    rng = np.random.default_rng(seed)
    return rng.standard_normal((nk, D)).astype(np.float32)


def test_element_on_an_e2m1_midpoint(orc):
    """Key 1 at P~ = 0.1875: with the block scale 2^-2 (block maximum 1) its value
    0.75 is the midpoint of the E2M1 codes 0.5 and 1, so either code may be taken;
    the dequantized P moves by 0.5 * 2^-2 and O by 0.125 max|v_1| / l."""
    s = [0.0, _score_for(0.1875)]
    V = _values(2, 1)
    _, fb = _row(orc, s, V)
    l = np.float32(1.0) + np.float32(_p(s[1]))
    assert fb == pytest.approx(0.125 * np.abs(V[1]).max() / l, rel=1e-6)


def test_block_maximum_on_an_e8m0_boundary(orc):
    """Key 32 opens the second block alone with P~ = 0.5 = 2^-1, the boundary of the
    OCP rule: scale 2^-3 encodes it as 4 * 2^-3 = 0.5, scale 2^-4 saturates it to
    6 * 2^-4 = 0.375.  Keys 1..31 are far below (code 0), so the budget is that one
    change, 0.125 max|v_32| / l."""
    s = [0.0] + [-1.0e4] * 31 + [_score_for(0.5)]
    V = _values(33, 2)
    _, fb = _row(orc, s, V)
    l = np.float32(1.0) + np.float32(_p(s[32]))
    assert fb == pytest.approx(0.125 * np.abs(V[32]).max() / l, rel=1e-6)


def test_no_fragile_decision(orc):
    """P~ = 1 at the maximum, 0.5 on four keys (value 2 under the scale 2^-2, a grid
    point) and 0 far below: no decision lies near a threshold.  The block maximum 1
    sits exactly on an OCP boundary but is exact on both sides (the implementation
    forms it as 2^(lambda (max - m)) = 2^0), also for a tie at the maximum, since
    these scores are exact sums in FP32: the budget is 0."""
    V = _values(40, 3)
    for s in ([0.0] + [_score_for(0.5)] * 4 + [-1.0e4] * 35,
              [0.0, 0.0] + [_score_for(0.5)] * 3 + [-1.0e4] * 35):
        _, fb = _row(orc, s, V)
        assert fb == 0.0


@pytest.mark.parametrize("dist, fragile", [(2.0 ** -22, True), (2.0 ** -17, False)])
def test_window_size(orc, dist, fragile):
    """For exactly computed scores near the row maximum the window of an element is
    about 2^-20 relative (the exponential's ulps and the quantizer's products): a
    value 2^-22 from the midpoint 0.75 is fragile, one 2^-17 away is not."""
    s = [0.0, _score_for(0.1875 * (1.0 + dist))]
    _, fb = _row(orc, s, _values(2, 4))
    assert (fb > 0.0) == fragile


def test_near_tie_with_inexact_scores(orc):
    """Keys 0 and 1 score 0 and -0.01.  When every score is an exact FP32 sum the
    maximum is key 0 on both sides and P~ = 1 there is exact (budget 0).  When key
    0's score is a sum of terms 2^20, -2^20, 2^-10, -2^-10 (exact value 0, but an FP32
    sum of them may round by up to 2^-23 * 2^21 per rounding), an implementation's
    maximum may be key 1 instead, and the block maximum near 1 may fall below the
    OCP boundary: scale 2^-3 saturates both keys to 6 * 2^-3 = 0.75, a change of
    0.25 each.  The budget is 0.25 (max|v_0| + max|v_1|) / l."""
    s = [0.0, -0.01]
    V = _values(2, 5)
    _, fb0 = _row(orc, s, V)
    assert fb0 == 0.0
    extra = np.zeros((2, D), np.float32)
    extra[0, 1:5] = [2.0 ** 20, -(2.0 ** 20), 2.0 ** -10, -(2.0 ** -10)]
    _, fb1 = _row(orc, s, V, k_extra=extra)
    l = np.float32(1.0) + np.float32(_p(s[1]))
    assert fb1 == pytest.approx(0.25 * (np.abs(V[0]).max() + np.abs(V[1]).max()) / l, rel=1e-6)


def test_two_level_prescale_is_per_tile(orc):
    """Two-level P (blog "Microscaling FP4 Attention", "Two-level scaling"; SageAttention3
    notes, Q2 Eq. 5) divides each tile's P~ by its own maximum over 448 * 6 before the
    E4M3 block scales.  A tile whose scores all sit c below the row maximum is then
    quantized exactly as if it held the maximum, whatever c: its contribution to O
    scales by exp(c / sqrt(d)) and nothing else.  Tile 0 (keys 0..127) holds the row
    maximum and writes channel 0 of O, tile 1 (keys 128..255) writes channel 1; the
    ratio O_1 / O_0 must follow exp(c / sqrt(d)) exactly, which a pre-scale taken
    from the running maximum (2688 P~ for tile 1) would break by several per cent
    through its E4M3 block scales."""
    rng = np.random.default_rng(6)
    u0 = -0.25 * rng.integers(0, 40, 128).astype(np.float32)
    u0[0] = 0.0
    u1 = -0.25 * rng.integers(0, 40, 128).astype(np.float32)
    u1[0] = 0.0
    V = np.zeros((256, D), np.float32)
    V[:128, 0] = 1.0
    V[128:, 1] = 1.0
    ratios = {}
    for c in (-3.0, -5.5, -9.75):
        O, fb = _row(orc, np.concatenate([u0, c + u1]), V, pmode=orc.P_TWO_LEVEL, pfmt="nvfp4")
        assert fb == 0.0
        ratios[c] = O[1] / O[0]
    for c in (-5.5, -9.75):
        assert ratios[c] / ratios[-3.0] == pytest.approx(np.exp(SM * (c + 3.0)), rel=2e-6)
