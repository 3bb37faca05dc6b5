"""The unquantized route of mxattn_fwd (Q, K, V in bf16, pmode NONE) against a
float64 brute-force softmax(Q K^T / sqrt(d)) V of the same bf16 values ("MXAttention"
section 2; "MpFA" section 3, Eq. 2), through the C ABI.

Bound per output element, from the route's arithmetic: the scores are exact bf16
products summed in FP32 (error at most 128 * 2^-24 * sum_c |q_c k_c| each), the
exponent and the FP32 exponential add a few ulps, and P~ is rounded to bf16 (8
significant bits: relative error at most 2^-8) for the PV product while l sums the FP32 P~.  So with p_j the exact softmax
weights, |dO_c| <= sum_j p_j |v_jc| (2^-8 + 2 delta) + 2^-20 max|O|, delta bounding
the relative change of the weights from the score and exponential errors (computed
per row below).  The test asserts that bound, checks the MFMA layout, masks, GQA
head mapping and packed documents, and that bf16 output is the FP32 output rounded."""
import numpy as np
import pytest

import synth
from helpers import gpu_available

pytestmark = [pytest.mark.gpu, pytest.mark.skipif(not gpu_available(), reason="needs a GPU")]


def brute(q, k, v, causal, doc_off):
    """q [Hq,N,d], k/v [Hkv,N,d] float64 -> O [Hq,N,d], weights row sums of |v| terms, delta"""
    Hq, N, d = q.shape
    Hkv = k.shape[0]
    sm = 1.0 / np.sqrt(d)
    O = np.zeros_like(q)
    absw = np.zeros_like(q)
    delta = np.zeros((Hq, N))
    doc = np.zeros(N, np.int64) if doc_off is None else np.searchsorted(doc_off, np.arange(N), side="right") - 1
    for h in range(Hq):
        hk = h * Hkv // Hq
        S = q[h] @ k[hk].T
        A = np.abs(q[h]) @ np.abs(k[hk]).T  # sum_c |q_c k_c|
        vis = doc[:, None] == doc[None, :]
        if causal:
            vis &= np.arange(N)[None, :] <= np.arange(N)[:, None]
        S = np.where(vis, S, -np.inf)
        m = S.max(axis=1, keepdims=True)
        P = np.exp(sm * (S - m))
        P /= P.sum(axis=1, keepdims=True)
        O[h] = P @ v[hk]
        absw[h] = P @ np.abs(v[hk])
        # score error 128 * 2^-24 * A on every visible score and on the row maximum,
        # times sm / ln 2 in the exponent's argument, plus the argument's and the
        # exponential's own roundings (a few ulps of relative error)
        e_arg = 2 * sm * 128 * 2.0 ** -24 * np.where(vis, A, 0).max(axis=1)
        delta[h] = np.expm1(e_arg) + 2.0 ** -20
    return O, absw, delta


def run(B, Hq, Hkv, N, causal=False, doc_off=None, seed=0, out_fp32=True):
    import torch
    import microscaling_fp4_attention_amd as mx
    x = synth.make_inputs("kmean", B, Hq, Hkv, N, 128, seed)
    dev = "cuda:0"
    t = {n: torch.from_numpy(x[n].astype(np.int16)).view(torch.bfloat16).to(dev) for n in ("q", "k", "v")}
    cu = None if doc_off is None else torch.from_numpy(np.asarray(doc_off, np.int32)).to(dev)
    Q = mx.quantize(t["q"], mx.ROLE_QK, "bf16")
    K = mx.quantize(t["k"], mx.ROLE_QK, "bf16")
    V = mx.quantize(t["v"], mx.ROLE_V, "bf16", cu_seqlens=cu)
    ws, nd = (None, 0) if doc_off is None else (mx.fwd_plan(doc_off, N, causal), len(doc_off) - 1)
    p = mx.fwd_params("none", "bf16", causal=causal, out_fp32=out_fp32)
    lse = torch.empty((B, Hq, N), dtype=torch.float32, device=dev)
    out = mx.fwd(Q, K, V, p, lse=lse, workspace=ws, ndocs=nd)
    torch.cuda.synchronize()
    assert torch.equal(Q.codes_view(), t["q"]) and torch.equal(V.codes_view(), t["v"])  # the copies
    O = out.float().cpu().numpy()
    qf, kf, vf = (synth.bf16_to_f32(x[n]).astype(np.float64) for n in ("q", "k", "v"))
    worst = 0.0
    for b in range(B):
        Or, absw, delta = brute(qf[b], kf[b], vf[b], causal, None if doc_off is None else np.asarray(doc_off))
        bound = absw * (2.0 ** -8 + 2 * delta[..., None]) + 2.0 ** -20 * np.abs(Or).max()
        if not out_fp32:
            bound += 2.0 ** -8 * np.abs(Or)  # bf16 output rounding
        err = np.abs(O[b] - Or)
        worst = max(worst, float((err / bound).max()))
        # the log-sum-exp of the row, natural log
        S = np.einsum("hnd,hmd->hnm", qf[b], np.repeat(kf[b], Hq // Hkv, axis=0)) / np.sqrt(128)
        doc = np.zeros(N, np.int64) if doc_off is None else np.searchsorted(doc_off, np.arange(N), side="right") - 1
        vis = doc[:, None] == doc[None, :]
        if causal:
            vis = vis & (np.arange(N)[None, :] <= np.arange(N)[:, None])
        S = np.where(vis[None], S, -np.inf)
        mm = S.max(axis=2)
        lse_ref = mm + np.log(np.exp(S - mm[..., None]).sum(axis=2))
        assert np.allclose(lse.cpu().numpy()[b], lse_ref, rtol=0, atol=1e-4)
    print(f"unquantized B{B} Hq{Hq} Hkv{Hkv} N{N} causal={causal} docs={doc_off is not None}: max |dO|/bound {worst:.3e}")
    assert np.all(np.isfinite(O))
    assert worst <= 1.0
    return out


def test_unquantized_noncausal():
    run(2, 4, 2, 300)


def test_unquantized_causal_gqa():
    run(1, 8, 2, 257, causal=True, seed=1)


def test_unquantized_packed_documents():
    run(1, 2, 2, 700, causal=True, doc_off=np.array([0, 100, 101, 357, 490, 700]), seed=2)
    run(1, 2, 1, 700, causal=False, doc_off=np.array([0, 100, 101, 357, 490, 700]), seed=3)


def test_unquantized_small_shapes_and_bf16_output():
    for N in (1, 128, 129):
        run(1, 1, 1, N, seed=4)
    run(1, 2, 2, 200, causal=True, seed=5, out_fp32=False)
