"""Pins of the oracle's split-key decode ("MpFA ...", section 5.3: fixed partitions of
the history, local (m, l, O) states merged by log-sum-exp) against a brute-force
softmax (unquantized P: the merge is exact in real arithmetic), against the
unsplit row (one split), and on rows whose causal mask leaves a split empty."""
import numpy as np
import pytest

import synth


def _data(B, Hq, Hkv, R, N, seed):
    q = synth.gaussian(seed, 1, (B, Hq, R, 64)).astype(np.float32)
    k = synth.gaussian(seed, 2, (B, Hkv, N, 64)).astype(np.float32)
    v = synth.gaussian(seed, 3, (B, Hkv, N, 64)).astype(np.float32)
    return q, k, v


def brute(q, k, v, kv_len, sm):
    B, Hq, R, d = q.shape
    Hkv = k.shape[1]
    O = np.zeros(q.shape)
    lse = np.zeros((B, Hq, R))
    for b in range(B):
        L = kv_len[b]
        for h in range(Hq):
            hk = h * Hkv // Hq
            for r in range(R):
                pos = L - R + r
                s = sm * (k[b, hk, :pos + 1].astype(np.float64) @ q[b, h, r].astype(np.float64))
                mx = s.max()
                p = np.exp(s - mx)
                O[b, h, r] = p @ v[b, hk, :pos + 1] / p.sum()
                lse[b, h, r] = mx + np.log(p.sum())
    return O, lse


@pytest.mark.parametrize("split", [128, 256, 1024])
def test_decode_unquantized_matches_softmax(orc, split):
    q, k, v = _data(2, 4, 2, 3, 700, 51)
    kv_len = np.array([700, 333], np.int32)
    O, lse, _ = orc.decode(q, k, v, kv_len, orc.P_NONE, split=split, sm_scale=0.125)
    Ob, lseb = brute(q, k, v, kv_len, 0.125)
    assert np.allclose(O, Ob, rtol=0, atol=2e-6)
    assert np.allclose(lse, lseb, rtol=0, atol=2e-5)


@pytest.mark.parametrize("pm,pf", [("direct", "mxfp4"), ("pnq", "mxfp4_uos"), ("two_level", "nvfp4")])
def test_single_split_equals_row(orc, pm, pf):
    """with one split the merge weight is exactly 1: the row of orc_attention"""
    pmode = {"direct": orc.P_DIRECT, "pnq": orc.P_PNQ, "two_level": orc.P_TWO_LEVEL}[pm]
    N = 300
    q, k, v = _data(1, 2, 1, 1, N, 52)
    O, lse, _ = orc.decode(q, k, v, [N], pmode, pf, split=512)
    # the same rows as the last row of a causal attention over the full sequence
    Qfull = np.zeros((1, 2, N, 64), np.float32)
    Qfull[:, :, N - 1] = q[:, :, 0]
    rows = np.array([N - 1, N + N - 1], np.int64)
    Or, lr, _ = orc.attention(Qfull, k, v, pmode, pf, causal=True, rows=rows)
    assert np.array_equal(O.reshape(2, 64), Or)
    assert np.array_equal(lse.reshape(2), lr)


def test_empty_split(orc):
    """rows at positions 250..299 of a 300-key history with splits of 256: rows before
    256 see nothing of the second split, which then has weight zero"""
    q, k, v = _data(1, 1, 1, 50, 300, 53)
    O, lse, _ = orc.decode(q, k, v, [300], orc.P_NONE, split=256)
    Ob, lseb = brute(q, k, v, [300], 1 / 8)
    assert np.all(np.isfinite(O)) and np.allclose(O, Ob, rtol=0, atol=2e-6)
    assert np.allclose(lse, lseb, rtol=0, atol=2e-5)


def test_decode_rejects_bad_arguments(orc):
    q, k, v = _data(1, 1, 1, 2, 64, 54)
    with pytest.raises(ValueError):
        orc.decode(q, k, v, [64], orc.P_NONE, split=100)  # not a multiple of the tile
    with pytest.raises(ValueError):
        orc.decode(q, k, v, [1], orc.P_NONE, split=128)   # fewer keys than query rows
