"""Pins of the oracle's attention recurrence.

* Unquantized mode against brute-force softmax(Q K^T / sqrt(d)) V in float64
  (the textbook definition the online softmax reaches up to rounding order;
  MXAttention section 2, MpFA Eqs. 2-6), with causal, packed-document and GQA
  masks.
* PNQ rows sum to one (MXAttention section 4.2, Proposition 1), while direct
  quantization does not (MXAttention sections 3 and 5.5.2).
* A row that sees one key reconstructs that key's value in every P mode: the
  row maximum is represented exactly (MXAttention appendix J; two-level stretch
  2688 of the blog 'Two-level scaling'; MpFA's 448 of section 4.1).
"""
import numpy as np
import pytest

import synth

P_MODES = {"direct_mx": (1, "mxfp4"), "direct_nv": (1, "nvfp4"), "two_level": (2, "nvfp4"),
           "two_level_mx": (2, "mxfp4"), "pnq_uos": (3, "mxfp4_uos"), "fp8": (4, None)}


def _inputs(B, Hq, Hkv, N, seed=0, kind="kmean"):
    x = synth.make_inputs(kind, B, Hq, Hkv, N, 128, seed)
    return (synth.bf16_to_f32(x["q"]), synth.bf16_to_f32(x["k"]), synth.bf16_to_f32(x["v"]))


def _brute(Q, K, V, causal=False, doc_off=None):
    B, Hq, N, d = Q.shape
    Hkv = K.shape[1]
    O = np.zeros((B, Hq, N, d))
    lse = np.zeros((B, Hq, N))
    mask = np.ones((N, N), bool)
    if doc_off is not None:
        doc = np.searchsorted(doc_off, np.arange(N), side="right") - 1
        mask &= doc[:, None] == doc[None, :]
    if causal:
        mask &= np.tril(np.ones((N, N), bool))
    for b in range(B):
        for h in range(Hq):
            hk = h * Hkv // Hq
            S = Q[b, h].astype(np.float64) @ K[b, hk].astype(np.float64).T / np.sqrt(d)
            S = np.where(mask, S, -np.inf)
            m = S.max(axis=1, keepdims=True)
            P = np.exp(S - m)
            l = P.sum(axis=1, keepdims=True)
            O[b, h] = P @ V[b, hk].astype(np.float64) / l
            lse[b, h] = (np.log(l) + m)[:, 0]
    return O.reshape(-1, d), lse.reshape(-1)


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("shape", [(1, 2, 2, 300), (2, 4, 2, 200), (1, 3, 1, 129)])
def test_unquantized_matches_brute_force(orc, causal, shape):
    B, Hq, Hkv, N = shape
    Q, K, V = _inputs(B, Hq, Hkv, N)
    O, lse, fb = orc.attention(Q, K, V, orc.P_NONE, causal=causal)
    Ob, lseb = _brute(Q, K, V, causal)
    assert np.abs(O - Ob).max() <= 2e-6 * np.abs(Ob).max()
    assert np.abs(lse - lseb).max() <= 2e-6 * np.abs(lseb).max()
    assert not fb.any()


@pytest.mark.parametrize("causal", [False, True])
def test_unquantized_packed_documents(orc, causal):
    Q, K, V = _inputs(1, 2, 2, 400)
    doc_off = np.array([0, 37, 180, 181, 400], np.int32)
    O, lse, _ = orc.attention(Q, K, V, orc.P_NONE, causal=causal, doc_off=doc_off)
    Ob, lseb = _brute(Q, K, V, causal, doc_off)
    assert np.abs(O - Ob).max() <= 2e-6 * np.abs(Ob).max()
    assert np.abs(lse - lseb).max() <= 2e-6 * np.abs(lseb).max()


def test_unquantized_tile_width_invariance(orc):
    """Online softmax is traversal-invariant in exact arithmetic (MpFA 4.1)."""
    Q, K, V = _inputs(1, 1, 1, 333)
    a = orc.attention(Q, K, V, orc.P_NONE, kv_tile=128)[0]
    b = orc.attention(Q, K, V, orc.P_NONE, kv_tile=64)[0]
    assert np.abs(a - b).max() <= 2e-6 * np.abs(a).max()


@pytest.mark.parametrize("pfmt", ["mxfp4_uos", "mxfp4", "nvfp4"])
def test_pnq_rows_sum_to_one(orc, pfmt):
    """MXAttention Prop. 1: with V = 1 every PNQ output is 1 (FP32 rounding)."""
    Q, K, _ = _inputs(1, 2, 2, 500, kind="lowrank")
    V = np.ones_like(K)
    O, _, _ = orc.attention(Q, K, V, orc.P_PNQ, pfmt=pfmt)
    assert np.abs(O - 1.0).max() <= 4e-6


def test_direct_rows_do_not_sum_to_one(orc):
    """Direct placement updates l from the unquantized tile (MXAttention 3 and
    5.2), so with V = 1 outputs drift from 1."""
    Q, K, _ = _inputs(1, 2, 2, 500)
    V = np.ones_like(K)
    O, _, _ = orc.attention(Q, K, V, orc.P_DIRECT, pfmt="mxfp4")
    assert np.abs(O - 1.0).mean() > 1e-3


@pytest.mark.parametrize("mode", list(P_MODES))
def test_single_visible_key_reconstructs_value(orc, mode):
    """Causal row 0 sees only key 0, whose exponential is exactly 1 and is
    represented exactly by every P quantizer except direct NVFP4, whose scale
    E4M3(1/6) = 0.171875 turns 1 into 6 x 0.171875 = 1.03125 while l stays 1
    (blog 'The probability squeeze': direct scales live near 1/6), and the
    two-level scheme with an E8M0 level-2 scale, where the stretched maximum
    2688 takes sigma = 2^9 (OCP rule) and 2688/512 = 5.25 rounds to 6, i.e. 3072.
    In both cases l comes from the unquantized P~ = 1."""
    pm, pf = P_MODES[mode]
    Q, K, V = _inputs(1, 1, 1, 64)
    O, lse, _ = orc.attention(Q, K, V, pm, pfmt=pf, causal=True)
    factor = {"direct_nv": 6 * 0.171875, "two_level_mx": 3072.0 / 2688.0}.get(mode, 1.0)
    assert np.abs(O[0] - factor * V[0, 0, 0]).max() <= 1e-6 * np.abs(V[0, 0, 0]).max()


@pytest.mark.parametrize("mode", list(P_MODES))
def test_causal_rows_ignore_future_keys(orc, mode):
    pm, pf = P_MODES[mode]
    Q, K, V = _inputs(1, 1, 1, 300)
    O1, _, _ = orc.attention(Q, K, V, pm, pfmt=pf, causal=True)
    K2, V2 = K.copy(), V.copy()
    K2[0, 0, 200:] = K2[0, 0, 200:] * 3 + 1
    V2[0, 0, 200:] = -V2[0, 0, 200:]
    O2, _, _ = orc.attention(Q, K2, V2, pm, pfmt=pf, causal=True)
    assert np.array_equal(O1.reshape(300, -1)[:200], O2.reshape(300, -1)[:200])
    assert not np.array_equal(O1.reshape(300, -1)[200:], O2.reshape(300, -1)[200:])


@pytest.mark.parametrize("mode", list(P_MODES))
def test_gqa_equals_repeated_heads(orc, mode):
    pm, pf = P_MODES[mode]
    Q, K, V = _inputs(1, 4, 2, 150)
    Og, _, _ = orc.attention(Q, K, V, pm, pfmt=pf)
    Km, Vm = np.repeat(K, 2, axis=1), np.repeat(V, 2, axis=1)
    Om, _, _ = orc.attention(Q, Km, Vm, pm, pfmt=pf)
    assert np.array_equal(Og, Om)


@pytest.mark.parametrize("mode", list(P_MODES))
def test_packed_documents_equal_separate_calls(orc, mode):
    """Packed documents (FLAMIA 3.6) behave as independent sequences: tiles and
    P blocks start at each document's first token."""
    pm, pf = P_MODES[mode]
    Q, K, V = _inputs(1, 2, 2, 420)
    doc_off = np.array([0, 130, 131, 300, 420], np.int32)
    Op, _, _ = orc.attention(Q, K, V, pm, pfmt=pf, causal=True, doc_off=doc_off)
    Op = Op.reshape(2, 420, -1)
    for a, b in zip(doc_off[:-1], doc_off[1:]):
        Od, _, _ = orc.attention(Q[:, :, a:b], K[:, :, a:b], V[:, :, a:b], pm, pfmt=pf, causal=True)
        assert np.array_equal(Op[:, a:b].reshape(-1, 128), Od)


def test_quantized_modes_close_to_exact(orc):
    """Quantized outputs stay near the exact ones (context only: the pages'
    cosine figures come from other data and are parity unpinned)."""
    Q, K, V = _inputs(1, 2, 2, 512)
    Oe, _, _ = orc.attention(Q, K, V, orc.P_NONE)
    for mode, (pm, pf) in P_MODES.items():
        O, _, _ = orc.attention(Q, K, V, pm, pfmt=pf)
        cos = (O * Oe).sum() / np.sqrt((O * O).sum() * (Oe * Oe).sum())
        assert cos > 0.9, mode
