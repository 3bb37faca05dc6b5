"""Pins of the CPU oracle's formats and quantizers against facts the pages fix.

Each test names the passage (page title and section/table) and compares the
oracle with a value printed there, a closed form, or an independent library
routine (numpy's round-half-even, torch's float8_e4m3fn cast).
"""
import math

import numpy as np
import pytest
import torch

from conftest import golden

F = golden("formats.txt")
R = golden("scale_rules.txt")
U = golden("uos.txt")
SP = golden("softmax_operand.txt")


# ---------------------------------------------------------------- E2M1 ----
def test_e2m1_grid(orc):
    """E2M1 magnitudes (blog 'NVFP4, not MXFP4'; MXAttention section 2) and
    the count of 15 distinct values (SageAttention3 analysis, Q1 C1)."""
    mags = [float(x) for x in F["e2m1_magnitudes"].split()]
    assert [orc.e2m1_value(c) for c in range(8)] == mags
    assert [orc.e2m1_value(8 | c) for c in range(8)] == [-m for m in mags]
    distinct = {orc.e2m1_value(c) for c in range(16)}  # -0 == +0
    assert len(distinct) == int(F["e2m1_distinct_values"])


def _rne_e2m1_by_rint(a):
    """Round |x| to the E2M1 grid with numpy's round-half-even per binade, then
    saturate at 6 (the OCP round-to-nearest-even convention written with a
    library rounding routine)."""
    if a < 2.0:
        v = np.rint(2.0 * a) / 2.0
    elif a < 4.0:
        v = np.rint(a)
    else:
        v = 2.0 * np.rint(a / 2.0)
    return min(v, 6.0)


def test_e2m1_rounding_matches_library_rne(orc):
    rng = np.random.default_rng(0)
    xs = list(rng.uniform(-9, 9, 20000).astype(np.float32))
    ties = [0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 7.0]
    for t in ties:
        for v in (t, -t, np.nextafter(np.float32(t), np.float32(0)), np.nextafter(np.float32(t), np.float32(9))):
            xs.append(np.float32(v))
    for x in xs:
        code = orc.e2m1_encode(float(x))
        want = _rne_e2m1_by_rint(abs(float(x)))
        assert abs(orc.e2m1_value(code)) == want, (x, code)
        assert (code >> 3) == (1 if np.signbit(x) else 0)


def test_e2m1_saturation_and_signed_zero(orc):
    """Nearest rounding with saturation to the finite range (MXAttention
    section 3): values past 6 give 6; sign kept."""
    for x in (6.0, 6.5, 7.0, 7.25, 8.0, 1e30, float("inf")):
        assert orc.e2m1_encode(x) == 7
        assert orc.e2m1_encode(-x) == 15
    assert orc.e2m1_encode(-0.1) == 8 and orc.e2m1_value(8) == 0.0


# ---------------------------------------------------------------- E4M3 ----
def test_e4m3_enumeration(orc):
    """Blog 'The probability squeeze': 127 distinct non-negative finite
    magnitudes, max 448, 35 of them in [0, 0.167]; 35 x 8 = 280."""
    vals = sorted({orc.e4m3_value(b) for b in range(256) if not math.isnan(orc.e4m3_value(b)) and orc.e4m3_value(b) >= 0})
    assert len(vals) == int(F["e4m3_distinct_nonneg"])
    assert max(vals) == float(F["e4m3_max"])
    window = [v for v in vals if v <= 0.167]
    assert len(window) == int(F["e4m3_in_0_0167"])
    assert len(window) * 8 == int(F["direct_p_value_bound"])
    assert math.isnan(orc.e4m3_value(0x7F)) and math.isnan(orc.e4m3_value(0xFF))


def test_e4m3_encode_matches_torch_cast(orc):
    """Round-to-nearest-even onto E4M3, checked against torch's float8_e4m3fn
    cast for every value below the overflow boundary 464."""
    rng = np.random.default_rng(1)
    mags = np.exp(rng.uniform(np.log(2.0 ** -12), np.log(463.9), 30000)).astype(np.float32)
    xs = np.concatenate([mags, -mags[:5000]])
    # all E4M3 midpoints and their float neighbours
    vals = np.array([orc.e4m3_value(b) for b in range(0x7F)], dtype=np.float64)
    mids = ((vals[:-1] + vals[1:]) / 2).astype(np.float32)
    xs = np.concatenate([xs, mids, np.nextafter(mids, np.float32(0)), np.nextafter(mids, np.float32(500)),
                         np.float32([0.0, -0.0, 448.0, 2.0 ** -9, 2.0 ** -10, 3 * 2.0 ** -11])])
    ref = torch.from_numpy(xs).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    got = np.array([orc.e4m3_encode(float(x)) for x in xs], dtype=np.uint8)
    np.testing.assert_array_equal(got, ref)


def test_e4m3_saturates_past_448(orc):
    for x in (448.0, 460.0, 464.0, 1000.0, 1e30):
        assert orc.e4m3_encode(x) == 0x7E
        assert orc.e4m3_encode(-x) == 0xFE


# ---------------------------------------------------------------- E8M0 ----
def _ranges():
    def parse(s):
        lo_closed, hi_closed = s[0] == "[", s[-1] == "]"
        lo, hi = (float(t) for t in s[1:-1].split(","))
        return lo, hi, lo_closed, hi_closed
    return {"ocp": parse(R["ocp_range"]), "tfs": parse(R["tfs_range"]), "uos": parse(R["uos_range"])}


RULES = {"ocp": (0, 0.0), "tfs": (1, 6.0), "uos": (1, 7.25)}


@pytest.mark.parametrize("name", ["ocp", "tfs", "uos"])
def test_e8m0_normalized_max_table1(orc, name):
    """MXAttention Table 1: normalized block maximum ranges of OCP, TFS, UOS."""
    lo, hi, lo_c, hi_c = _ranges()[name]
    rule, q = RULES[name]
    rng = np.random.default_rng(2)
    Ms = list(np.exp2(rng.uniform(-60, 60, 20000)).astype(np.float32))
    # boundaries of all three rules and their float neighbours
    for base in (1.0, 6.0, 7.25, 4.0):
        for k in range(-8, 9):
            b = np.float32(base * 2.0 ** k)
            Ms += [b, np.nextafter(b, np.float32(0)), np.nextafter(b, np.float32(1e30))]
    for M in Ms:
        e = orc.e8m0_exponent(float(M), rule, q)
        x = float(M) / 2.0 ** e
        assert (x >= lo if lo_c else x > lo) and (x <= hi if hi_c else x < hi), (name, M, e, x)


def test_e8m0_ocp_overflow_probability(orc):
    """MXAttention section 3: Pr(x_max >= 7) = log2(8/7) under log-uniform M."""
    rng = np.random.default_rng(3)
    Ms = np.exp2(rng.uniform(-20, 20, 200000)).astype(np.float32)
    hits = 0
    for M in Ms:
        e = orc.e8m0_exponent(float(M), 0, 0.0)
        hits += float(M) / 2.0 ** e >= 7.0
    p = hits / len(Ms)
    assert abs(p - float(R["p_overflow"])) < 0.004
    assert abs(math.log2(8 / 7) - float(R["p_overflow"])) < 1e-5


def test_e8m0_zero_block(orc):
    """MXAttention section 2: an all-zero block gets sigma = 1 and zero codes."""
    for f in ("mxfp4", "mxfp4_uos", "mxfp4_tfs"):
        codes, sb, s = orc.quant_block(np.zeros(32, np.float32), f)
        assert sb == 127 + int(R["zero_block_exponent"]) and s == 1.0 and not codes.any()


def test_mxfp4_block_quantization_error_bound(orc):
    """Dequantized MXFP4 values: every element is the grid point nearest to
    x/sigma (half a grid step at most) except where the OCP rule saturates."""
    rng = np.random.default_rng(4)
    for f in ("mxfp4", "mxfp4_uos", "mxfp4_tfs"):
        for _ in range(300):
            x = (rng.standard_normal(32) * np.exp(rng.uniform(-5, 5))).astype(np.float32)
            codes, sb, s = orc.quant_block(x, f)
            for xi, c in zip(x, codes):
                y = abs(float(xi)) / s
                v = abs(orc.e2m1_value(int(c)))
                gap = 1.0 if y > 2 else 0.5
                gap = 2.0 if y > 4 else gap
                assert abs(y - v) <= gap / 2 + 1e-12 or y > 6.0


# ----------------------------------------------------------------- UOS ----
def _breakpoints(orc, hi):
    val = lambda t: abs(orc.e2m1_value(orc.e2m1_encode(float(np.float32(t)))))
    xs = np.linspace(0.0, hi, 40001)
    bps, prev = [], val(xs[0])
    for a, b in zip(xs[:-1], xs[1:]):
        vb = val(b)
        if vb != prev:
            lo, h = a, b
            for _ in range(50):
                m = (lo + h) / 2
                if val(m) == prev:
                    lo = m
                else:
                    h = m
            bps.append(h)
            prev = vb
    return bps, val


def test_uos_boundary_closed_form(orc):
    """MXAttention 4.1 and appendix C.1 Table 6: Delta(q) = E(q) - 8E(q/2) with
    the oracle's E2M1 projection has its root at q* = 29/4, is positive above it
    and equals (48q^2 - 864q + 3983)/8 for q > 10."""
    bps, val = _breakpoints(orc, 30.0)

    def E(q):
        pts = [0.0] + [b for b in bps if b < q] + [q]
        tot = 0.0
        for a, b in zip(pts[:-1], pts[1:]):
            c = val((a + b) / 2)
            tot += ((b - c) ** 3 - (a - c) ** 3) / 3
        return tot

    D = lambda q: E(q) - 8 * E(q / 2)
    qs = float(U["q_star"])
    assert abs(D(qs)) < 1e-6
    for q in (0.5, 1, 3, 5, 7.0, 7.2, 7.24):
        assert D(q) < 0
    for q in (7.26, 7.5, 8, 9, 10):
        assert D(q) > 0
    a, b, c, den = (float(U[k]) for k in ("closed_form_a", "closed_form_b", "closed_form_c", "closed_form_den"))
    for q in (10.5, 11.0, 12.0, 14.0, 20.0, 25.0):
        assert abs(D(q) - (a * q * q + b * q + c) / den) < 1e-6


def test_uos_represents_row_max_exactly(orc):
    """MXAttention 4.2 / appendix J: the tile holding the row maximum contributes
    an exponential equal to 1, represented exactly under q* = 7.25."""
    x = np.zeros(32, np.float32)
    x[5] = 1.0
    x[6] = 0.3
    codes, sb, s = orc.quant_block(x, "mxfp4_uos")
    assert orc.e2m1_value(int(codes[5])) * s == 1.0


# ---------------------------------------------------- softmax operand P ----
def test_two_level_stretch_reaches_448(orc):
    """Blog 'Two-level scaling' (quant_p) and SageAttention3 Eq. 5: after the
    stretch P2 = P / (rowmax/2688) the row-max block gets scale E4M3(2688/6)=448
    and the row max is code 6, i.e. reconstructed as s_p1 * 2688."""
    stretch = float(SP["stretch"])
    assert stretch == 448.0 * 6.0
    rowmax = np.float32(0.0371)
    s1 = np.float32(rowmax / np.float32(stretch))
    p = np.array([rowmax, rowmax * 0.5, rowmax * 0.01] + [0.0] * 13, np.float32)
    codes, sb, s2 = orc.quant_block((p / s1).astype(np.float32), "nvfp4")
    assert s2 == float(SP["level2_scale_max"]) and sb == 0x7E
    assert orc.e2m1_value(int(codes[0])) == 6.0
    assert abs(orc.e2m1_value(int(codes[0])) * s2 * s1 - rowmax) <= 1e-7 * rowmax


def test_direct_nvfp4_scale_window(orc):
    """Blog 'The probability squeeze': direct P scales lie in [0, 0.167]; with
    E4M3 rounding a block holding P=1 gets 0.171875 (code 0x23), so direct
    NVFP4 P uses codes 0x00..0x23."""
    rng = np.random.default_rng(5)
    seen = set()
    for _ in range(2000):
        p = rng.uniform(0, 1, 16).astype(np.float32) ** rng.uniform(1, 30)
        codes, sb, s = orc.quant_block(p, "nvfp4")
        assert sb <= 0x23
        seen.add(sb)
    one = np.zeros(16, np.float32)
    one[0] = 1.0
    assert orc.quant_block(one, "nvfp4")[1] == 0x23
    assert orc.e4m3_value(0x22) <= float(SP["direct_scale_window"]) < orc.e4m3_value(0x23)


def test_fp8_fixed_scale_never_saturates(orc):
    """MpFA 4.1: s_P = 448 and 0 < P <= 1, so cast_e4m3(448 P) never clamps and
    is within E4M3's relative half-step of 448 P for normal values."""
    rng = np.random.default_rng(6)
    for p in rng.uniform(0, 1, 20000).astype(np.float32):
        y = np.float32(float(SP["fp8_fixed_scale"])) * p
        c = orc.e4m3_encode(float(y))
        assert c <= 0x7E
        if y >= 2.0 ** -6:
            assert abs(orc.e4m3_value(c) - float(y)) <= float(y) * 2.0 ** -4
    assert orc.e4m3_encode(448.0) == 0x7E


def test_fp8_v_round_up_exponent(orc):
    """E4M3 V with an E8M0 exponent rounded up (FLAMIA 3.2 rounds scale
    exponents upward so that no scaled value passes the largest code): the
    block maximum lands in (224, 448] and no element is clamped."""
    rng = np.random.default_rng(7)
    for _ in range(500):
        x = (rng.standard_normal(32) * np.exp(rng.uniform(-8, 8))).astype(np.float32)
        codes, sb, s = orc.quant_block(x, "fp8v")
        m = float(np.abs(x).max()) / s
        assert 224.0 < m <= 448.0
        for xi, c in zip(x, codes):
            assert abs(orc.e4m3_value(int(c))) <= 448.0
            assert abs(abs(orc.e4m3_value(int(c))) - abs(float(xi)) / s) <= max(abs(float(xi)) / s * 2 ** -4, 2 ** -10)
