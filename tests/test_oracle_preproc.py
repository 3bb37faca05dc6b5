"""Pins of the oracle's outlier pre-processing against independent routines.

Passages: per-channel means and centering ([MPFA] "MpFA: Hardware-Efficient Train-Free
QK4V8 FlashAttention Kernels on Blackwell GPUs", section 4.2, Eq. 7), the compensation
vector and where it enters the scores (section 4.3, Eqs. 8-10), smooth-K ("Microscaling
FP4 Attention: Why the Softmax Operand Needs Two Scale Factors", "Smooth-K is the
smaller lever"), the normalized Hadamard rotation ("FLAMIA: FLAsh MIcroscaling Attention
...", section 3.4 and appendix A.2).  References are numpy float64 means and products,
scipy's Sylvester Hadamard matrix, exact rationals and a brute-force softmax.
"""
from fractions import Fraction

import numpy as np
import pytest
import scipy.linalg

import synth


def bf16_data(shape, seed, scale=1.0, shift=0.0):
    x = synth.gaussian(seed, 7, shape, std=scale) + np.float32(shift)
    return synth.bf16_to_f32(synth.f32_to_bf16(x.astype(np.float32)))


# ------------------------------------------------------------ channel mean ----
def test_mean_constant_and_empty(orc):
    x = np.full((13, 8), 0.375, dtype=np.float32)
    assert np.array_equal(orc.channel_mean(x), np.full((1, 8), 0.375, np.float32))
    # an empty document (offsets 5, 5) gets 0
    m = orc.channel_mean(x, doc_off=[0, 5, 5, 13])
    assert np.array_equal(m[1], np.zeros(8, np.float32))
    assert np.array_equal(m[0], m[2])


def test_mean_matches_numpy(orc):
    """Sums of bf16 values of moderate span are exact in double, so any summation
    order (numpy's pairwise sum) gives the same double; dividing by L and rounding
    to float then gives the oracle's value bit for bit."""
    x = bf16_data((301, 128), 1, scale=3.0, shift=0.7)
    ref = (x.astype(np.float64).sum(0) / 301).astype(np.float32)
    assert np.array_equal(orc.channel_mean(x)[0], ref)
    doc = np.array([0, 40, 41, 200, 301], np.int32)
    m = orc.channel_mean(x, doc_off=doc)
    for k in range(4):
        seg = x[doc[k]:doc[k + 1]].astype(np.float64)
        assert np.array_equal(m[k], (seg.sum(0) / len(seg)).astype(np.float32)), k


# -------------------------------------------------------------- pre-process ----
def test_preprocess_identity_and_centering(orc):
    x = bf16_data((50, 64), 2)
    assert np.array_equal(orc.preprocess_rows(x), x)
    mu = orc.channel_mean(x)
    # x - mu is one correctly rounded float subtraction
    assert np.array_equal(orc.preprocess_rows(x, mean=mu), x - mu[0])
    # documents: each token uses its own document's mean
    doc = np.array([0, 17, 50], np.int32)
    md = orc.channel_mean(x, doc_off=doc)
    y = orc.preprocess_rows(x, mean=md, doc_off=doc)
    assert np.array_equal(y[:17], x[:17] - md[0]) and np.array_equal(y[17:], x[17:] - md[1])


def test_hadamard_unit_vectors_give_scipy_rows(orc):
    """e_i H / sqrt(d) is row i of the Sylvester matrix (scipy.linalg.hadamard)
    times fl32(1/sqrt(d)): pins the sign pattern and the normalization."""
    d = 128
    H = scipy.linalg.hadamard(d)
    c = np.float32(1.0 / np.sqrt(np.float64(d)))
    out = orc.preprocess_rows(np.eye(d, dtype=np.float32), hadamard=True)
    assert np.array_equal(out, H.astype(np.float32) * c)


def test_hadamard_matches_exact_product(orc):
    """Random bf16 rows, centered and rotated: the double product (x - mu) H is
    exact for these spans, so it equals the oracle's sum before the scaling."""
    d = 128
    x = bf16_data((40, d), 3, scale=2.0, shift=-1.5)
    mu = orc.channel_mean(x)
    H = scipy.linalg.hadamard(d).astype(np.float64)
    y = x.astype(np.float64) - mu[0].astype(np.float64)
    ref = ((y @ H) * (1.0 / np.sqrt(np.float64(d)))).astype(np.float32)
    got = orc.preprocess_rows(x, mean=mu, hadamard=True)
    assert np.array_equal(got, ref)
    # one row against exact rationals, rounded once to double before the scaling
    i = 5
    z = [sum(Fraction(float(y[i, k])) * int(H[k, j]) for k in range(d)) for j in range(d)]
    zz = np.array([float(v) for v in z]) * (1.0 / np.sqrt(np.float64(d)))
    assert np.array_equal(got[i], zz.astype(np.float32))


def test_hadamard_is_orthogonal(orc):
    """The normalized rotation keeps norms and dot products (to float rounding)."""
    a = bf16_data((2, 128), 4)
    r = orc.preprocess_rows(a, hadamard=True).astype(np.float64)
    a64 = a.astype(np.float64)
    assert abs(np.dot(r[0], r[1]) - np.dot(a64[0], a64[1])) <= 1e-5 * np.linalg.norm(a64[0]) * np.linalg.norm(a64[1])
    assert np.allclose(np.linalg.norm(r, axis=1), np.linalg.norm(a64, axis=1), rtol=1e-6)


# ------------------------------------------------------------- compensation ----
def test_center_comp_exact(orc):
    """delta[j] = qmean . (K[j] - kmean): within half an ulp of the exact rational
    value (the double sum adds less than 2^-40 relative here)."""
    d = 64
    K = bf16_data((20, d), 5, shift=0.5)
    Q = bf16_data((30, d), 6, shift=-0.25)
    km, qm = orc.channel_mean(K), orc.channel_mean(Q)
    delta = orc.center_comp(qm, K, km)
    for j in range(20):
        exact = sum(Fraction(float(qm[0, c])) * (Fraction(float(K[j, c])) - Fraction(float(km[0, c])))
                    for c in range(d))
        ulp = np.spacing(np.float32(abs(float(exact))))
        assert abs(float(delta[j]) - float(exact)) <= 0.5 * float(ulp) * (1 + 1e-6), j


def test_center_decomposition(orc):
    """Eq. 8: Q K^T - (Q_c K_c^T + 1 delta^T) is constant along each row (it is
    q_i . kmean), so the softmax of the restored scores equals softmax(Q K^T)."""
    d = 32
    K = bf16_data((24, d), 7, shift=2.0)
    Q = bf16_data((9, d), 8, shift=-1.0)
    km, qm = orc.channel_mean(K), orc.channel_mean(Q)
    Qc = orc.preprocess_rows(Q, mean=qm).astype(np.float64)
    Kc = orc.preprocess_rows(K, mean=km).astype(np.float64)
    delta = orc.center_comp(qm, K, km).astype(np.float64)
    S = Q.astype(np.float64) @ K.astype(np.float64).T
    diff = S - (Qc @ Kc.T + delta[None, :])
    rowc = Q.astype(np.float64) @ km[0].astype(np.float64)
    assert np.allclose(diff, rowc[:, None], rtol=0, atol=1e-4)
    # a wrong sign on delta would leave a key-dependent residue of 2 delta
    assert np.abs(S - (Qc @ Kc.T - delta[None, :]) - rowc[:, None]).max() > 0.1


# ----------------------------------------------------------- score bias ----
def brute(Q, K, V, bias, sm, causal):
    S = (Q.astype(np.float64) @ K.astype(np.float64).T + bias[None, :]) * sm
    if causal:
        S = np.where(np.tril(np.ones_like(S, dtype=bool)), S, -np.inf)
    P = np.exp(S - S.max(1, keepdims=True))
    return (P / P.sum(1, keepdims=True)) @ V.astype(np.float64)


@pytest.mark.parametrize("causal", [False, True])
def test_attention_bias_brute_force(orc, causal):
    """Unquantized online softmax (tiles of 128) with a per-key bias equals the
    softmax of Q K^T + bias; under a causal mask, a huge bias on future keys changes
    nothing (the bias enters before the mask)."""
    N, d = 300, 64
    Q, K, V = (bf16_data((N, d), s) for s in (9, 10, 11))
    bias = bf16_data((N,), 12, scale=4.0)
    if causal:
        bias = bias.copy()
        bias[200:] += 1e4  # only ever seen by rows >= 200 once visible
    O, _, _ = orc.attention(Q[None, None], K[None, None], V[None, None], orc.P_NONE, causal=causal,
                            bias=bias[None, None])
    ref = brute(Q, K, V, bias.astype(np.float64), 1 / np.sqrt(d), causal)
    rows = np.arange(200) if causal else np.arange(N)
    assert np.allclose(O[rows], ref[rows], rtol=0, atol=2e-5)


def test_centering_end_to_end(orc):
    """Attention of the centered operands with the compensation bias equals the
    attention of the original operands (unquantized P, float rounding only)."""
    N, d = 260, 128
    Q = bf16_data((N, d), 13, shift=1.0)
    K = bf16_data((N, d), 14, shift=-2.0)
    V = bf16_data((N, d), 15)
    qm, km = orc.channel_mean(Q), orc.channel_mean(K)
    Qc, Kc = orc.preprocess_rows(Q, mean=qm), orc.preprocess_rows(K, mean=km)
    delta = orc.center_comp(qm, K, km)
    O1, _, _ = orc.attention(Qc[None, None], Kc[None, None], V[None, None], orc.P_NONE, bias=delta[None, None])
    O0, _, _ = orc.attention(Q[None, None], K[None, None], V[None, None], orc.P_NONE)
    assert np.allclose(O1, O0, rtol=0, atol=2e-5)
    # smooth-K alone (K centered, no compensation) also leaves the softmax unchanged
    O2, _, _ = orc.attention(Q[None, None], Kc[None, None], V[None, None], orc.P_NONE)
    assert np.allclose(O2, O0, rtol=0, atol=2e-5)
