"""Pins of the oracle's causally safe form of a 4-bit V ("FLAMIA: FLAsh MIcroscaling
Attention ...", section 3.2: a per-key power-of-two scale for V on the diagonal tiles,
folded into P, so that a masked future key cannot change an earlier row through a
shared V scale).  References: brute-force E2M1 rounding in numpy, a leak probe that
perturbs future keys, and the closed form that PNQ rows with V = 1 sum to one."""
import numpy as np
import pytest

import synth

E2M1 = np.array([0, 0.5, 1, 1.5, 2, 3, 4, 6])


def rne_e2m1(y):
    """nearest E2M1 magnitude index, ties to the even index, saturating at 6"""
    a = np.minimum(np.abs(y), 6.0)
    d = np.abs(a[..., None] - E2M1)
    best = d.min(-1, keepdims=True)
    cand = np.where(d == best, np.arange(8), 99)
    even = np.where(cand % 2 == 0, cand, 99).min(-1)
    idx = np.where(even < 99, even, cand.min(-1))
    return idx | np.where(np.signbit(y), 8, 0)


def test_quantize_keys_brute_force(orc):
    x = synth.bf16_to_f32(synth.f32_to_bf16((synth.gaussian(5, 1, (64, 128)) * 3).astype(np.float32)))
    x[3] = 0.0  # an all-zero key
    codes, ek = orc.quantize_keys(x, "mxfp4")  # OCP rule: e = floor(log2 amax) - 2
    amax = np.abs(x).max(1)
    e_ref = np.where(amax > 0, np.floor(np.log2(np.where(amax > 0, amax, 1))) - 2, 0).astype(np.int32)
    assert np.array_equal(ek, e_ref)
    assert np.array_equal(codes, rne_e2m1(x / np.exp2(e_ref)[:, None]).astype(np.uint8))
    codes_u, ek_u = orc.quantize_keys(x, "mxfp4_uos")  # ceiling rule: smallest e with amax <= 7.25 * 2^e
    e_u = np.where(amax > 0, np.ceil(np.log2(np.where(amax > 0, amax, 1) / 7.25)), 0).astype(np.int32)
    assert np.array_equal(ek_u, e_u)


def _case(seed, N=300, d=128):
    q = synth.gaussian(seed, 1, (1, 1, N, d)).astype(np.float32)
    k = synth.gaussian(seed, 2, (1, 1, N, d)).astype(np.float32)
    v = synth.gaussian(seed, 3, (1, 1, N, d)).astype(np.float32)
    return q, k, v


def _fwd(orc, q, k, v, pm, pf, safe, **kw):
    vc, vs = orc.quantize_cols(v[0, 0], "mxfp4")
    vd = orc.dequant_cols(vc, vs, "mxfp4")[None, None]
    if safe:
        kc, ek = orc.quantize_keys(v[0, 0], "mxfp4")
        kw.update(vkey=orc.e2m1_values(kc)[None, None], vkey_exp=ek[None, None])
    return orc.attention(q, k, vd, pm, pf, causal=True, **kw)[0]


@pytest.mark.parametrize("pm,pf", [("direct", "mxfp4"), ("pnq", "mxfp4_uos"), ("two_level", "nvfp4")])
def test_leak_probe(orc, pm, pf):
    """Multiplying the keys from 200 on by 50 changes, through the shared V scale of
    keys 192..223, the outputs of rows 192..199 of the grouped form; with the per-key
    form on the diagonal tiles every row before 200 keeps its output bit for bit."""
    pmode = {"direct": orc.P_DIRECT, "pnq": orc.P_PNQ, "two_level": orc.P_TWO_LEVEL}[pm]
    q, k, v = _case(31)
    v2 = v.copy()
    v2[..., 200:, :] *= 50.0
    before = slice(0, 200)
    grouped = [_fwd(orc, q, k, vv, pmode, pf, False) for vv in (v, v2)]
    safe = [_fwd(orc, q, k, vv, pmode, pf, True) for vv in (v, v2)]
    assert not np.array_equal(grouped[0][before], grouped[1][before])  # the leak exists
    assert np.array_equal(safe[0][before], safe[1][before])           # and is closed


def test_pnq_rows_sum_to_one_with_fold(orc):
    """With V = 1 the per-key form is code 4.0 with exponent -2 for every key, and PNQ
    divides by the sum of deq(P^') 2^-e: each output is 1 up to float rounding."""
    q, k, _ = _case(32, N=260)
    v = np.ones_like(q)
    O = _fwd(orc, q, k, v, orc.P_PNQ, "mxfp4_uos", True)
    assert np.allclose(O, 1.0, rtol=0, atol=2e-6)


def test_fold_requires_causal(orc):
    q, k, v = _case(33, N=64)
    kc, ek = orc.quantize_keys(v[0, 0], "mxfp4")
    with pytest.raises(ValueError):
        orc.attention(q, k, v, orc.P_DIRECT, "mxfp4", causal=False, vkey=orc.e2m1_values(kc)[None, None],
                      vkey_exp=ek[None, None])


def test_diagonal_tiles_are_the_query_tiles(orc):
    """The per-key form covers exactly the key tiles that start inside a row's query
    tile.  A different grouped V on keys 0..255 then reaches no row of the first query
    tile and every row after it: with 256-row query tiles rows 0..255 never read the
    grouped V below key 256; with 128-row query tiles rows 128..255 read it on key
    tile 0."""
    q, k, v = _case(34, N=600)
    vc, vs = orc.quantize_cols(v[0, 0], "mxfp4")
    vd = orc.dequant_cols(vc, vs, "mxfp4")[None, None]
    kc, ek = orc.quantize_keys(v[0, 0], "mxfp4")
    kw = dict(vkey=orc.e2m1_values(kc)[None, None], vkey_exp=ek[None, None])
    vd2 = vd.copy()
    vd2[..., :256, :] = -3.0 * vd2[..., :256, :] + 0.5
    for qt in (256, 128):
        a = orc.attention(q, k, vd, orc.P_DIRECT, "mxfp4", causal=True, q_tile=qt, **kw)[0]
        b = orc.attention(q, k, vd2, orc.P_DIRECT, "mxfp4", causal=True, q_tile=qt, **kw)[0]
        same = np.all(a == b, axis=1)
        assert same[:qt].all(), qt
        assert not same[qt:].any(), qt


def test_query_tile_must_hold_whole_key_tiles(orc):
    q, k, v = _case(35, N=64)
    kc, ek = orc.quantize_keys(v[0, 0], "mxfp4")
    with pytest.raises(ValueError):
        orc.attention(q, k, v, orc.P_DIRECT, "mxfp4", causal=True, q_tile=192, vkey=orc.e2m1_values(kc)[None, None],
                      vkey_exp=ek[None, None])
