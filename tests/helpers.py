"""Shared helpers of the GPU tests: run the HIP path and the CPU oracle on the
same seeded inputs and compare them.

The oracle side quantizes with its own C routines; the GPU side with
mxattn_quantize.  Quantized bytes must agree exactly; the forward output (FP32)
must satisfy |dO| <= 2e-3 * max|O_oracle| + flip budget of the row, where the
flip budget bounds the effect of the rounding decisions whose input lies within
its window of a threshold (the oracle derives each window from a bound on how
far FP32 arithmetic can move that input and reports the budget per row).
Every comparison is recorded in PARITY, which tests/conftest.py prints at the end
of the session (worst |dO|/bound and the share of rows with a nonzero budget).
"""
from __future__ import annotations

import numpy as np

import oracle
import synth

TOL = 2e-3
# Rows whose flip budget is nonzero, as a share of the rows compared, must stay below
# FRAGILE_CAP on the exact exponential over rows of at most a few thousand keys; and on
# every comparison the median row's budget must stay below the plain tolerance, so the
# bound is not mostly budget.  (The share grows with the keys per row: a row of 32K keys
# makes 32 times the decisions of one of 1K; the bit-level exponentials keep 16 fraction
# bits of their argument, so their window is 2^-15 instead of about 2^-20.)
FRAGILE_CAP = 0.10

# (case, worst |dO| / bound, rows with a nonzero flip budget, rows compared, median budget / tolerance)
PARITY: list = []


def record_parity(name, ratio, fb_over_tol, cap_share=FRAGILE_CAP):
    """Keep one comparison for the session summary and check how much of its bound is
    flip budget.  fb_over_tol: each compared row's budget over the plain tolerance
    2e-3 max|O|; cap_share: the largest share of rows with a budget (None: not
    checked, for long rows and the bit-level exponentials)."""
    r = np.asarray(fb_over_tol, np.float64).ravel()
    n_fragile, n_rows = int((r > 0).sum()), int(r.size)
    med = float(np.median(r)) if r.size else 0.0
    PARITY.append((name, float(ratio), n_fragile, n_rows, med))
    assert med <= 1.0, f"{name}: the median row's flip budget is {med:.2f} times the tolerance"
    if cap_share is not None:
        cap = max(3, int(cap_share * n_rows))
        assert n_fragile <= cap, f"{name}: {n_fragile} of {n_rows} rows have a flip budget (cap {cap})"


def score_rounds(qfmt) -> int:
    """FP32 roundings in the HIP path's score sums: two chained FP4 MFMAs (64 channels
    each) for MXFP4 Q/K, at most eight chained f16 (or, in the single-buffer kernel, bf16)
    MFMAs (16 channels each; four of 32 in the 16-column decode) for NVFP4 Q/K; the
    oracle widens the window of every decision by what they can move a score."""
    return 8 if str(qfmt).startswith("nvfp4") else 2


def gpu_available() -> bool:
    try:
        import torch
        return torch.cuda.is_available()
    except Exception:
        return False


def unpack_nibbles(b: np.ndarray) -> np.ndarray:
    """uint8 [..., n] -> uint8 [..., 2n] with the low nibble first."""
    out = np.empty(b.shape[:-1] + (2 * b.shape[-1],), dtype=np.uint8)
    out[..., 0::2] = b & 15
    out[..., 1::2] = b >> 4
    return out


def v_slots(N, doc_off, block):
    """token -> padded key slot of the V layout (document-local blocks)."""
    if doc_off is None:
        return np.arange(N)
    slots = np.empty(N, dtype=np.int64)
    voff = 0
    for k in range(len(doc_off) - 1):
        s, e = int(doc_off[k]), int(doc_off[k + 1])
        slots[s:e] = voff + np.arange(e - s)
        voff += (e - s + block - 1) // block * block
    return slots


def gpu_codes_qk(qt) -> np.ndarray:
    """GPU QK codes as one code per byte [B, H, N, d]."""
    return unpack_nibbles(qt.codes_view().cpu().numpy()) if qt.desc.fmt.elem == 0 else qt.codes_view().cpu().numpy()


def gpu_codes_v(qt, N, doc_off) -> tuple[np.ndarray, np.ndarray]:
    """GPU V codes and scales in the oracle's layout: codes [B, H, d, N] by token,
    scales [B, H, d, nblk] (document by document)."""
    c = qt.codes_view().cpu().numpy()
    if qt.desc.fmt.elem == 0:
        c = unpack_nibbles(c)
    slots = v_slots(N, doc_off, qt.desc.fmt.block)
    nblk = oracle.v_nblocks(N, doc_off, qt.desc.fmt.block)
    return c[..., slots], qt.scales_view().cpu().numpy()[..., :nblk]


def oracle_quant_qk(x: np.ndarray, fmt):
    codes, scales = oracle.quantize_rows(x, fmt)
    return codes, scales, oracle.dequant_rows(codes, scales, fmt)


def oracle_quant_v(x: np.ndarray, fmt, doc_off=None):
    """x [B, H, N, d] -> codes [B, H, d, N], scales [B, H, d, nblk], dequantized [B, H, N, d]."""
    B, H, N, d = x.shape
    nblk = oracle.v_nblocks(N, doc_off, oracle.fmt(fmt).block)
    codes = np.zeros((B, H, d, N), np.uint8)
    scales = np.zeros((B, H, d, nblk), np.uint8)
    deq = np.zeros_like(x, dtype=np.float32)
    for b in range(B):
        for h in range(H):
            c, s = oracle.quantize_cols(x[b, h], fmt, doc_off)
            codes[b, h], scales[b, h] = c, s
            deq[b, h] = oracle.dequant_cols(c, s, fmt, doc_off)
    return codes, scales, deq


PM_ORACLE = {"direct": oracle.P_DIRECT, "two_level": oracle.P_TWO_LEVEL, "pnq": oracle.P_PNQ,
             "fp8": oracle.P_FP8_FIXED}


def oracle_preproc(xf, doc_off, mean_on, hadamard):
    """Oracle pre-processing of Q or K [B, H, N, d] head by head: (means or None, y)."""
    B, H, N, d = xf.shape
    nd = 1 if doc_off is None else len(doc_off) - 1
    means = np.zeros((B, H, nd, d), np.float32) if mean_on else None
    y = np.empty_like(xf)
    for b in range(B):
        for h in range(H):
            m = oracle.channel_mean(xf[b, h], doc_off) if mean_on else None
            if mean_on:
                means[b, h] = m
            y[b, h] = oracle.preprocess_rows(xf[b, h], m, doc_off, hadamard)
    return means, y


def oracle_comp(qmeans, kf, kmeans, Hq, doc_off):
    B, Hkv, N, d = kf.shape
    delta = np.zeros((B, Hq, N), np.float32)
    for b in range(B):
        for h in range(Hq):
            hk = h * Hkv // Hq
            delta[b, h] = oracle.center_comp(qmeans[b, h], kf[b, hk], kmeans[b, hk], doc_off)
    return delta


def ulp_diff(a: np.ndarray, b: np.ndarray) -> int:
    """largest distance in float32 units in the last place (finite values)"""
    ia = a.astype(np.float32).view(np.int32).astype(np.int64)
    ib = b.astype(np.float32).view(np.int32).astype(np.int64)
    ia = np.where(ia < 0, -(ia & 0x7FFFFFFF), ia)
    ib = np.where(ib < 0, -(ib & 0x7FFFFFFF), ib)
    return int(np.abs(ia - ib).max()) if ia.size else 0


def gpu_codes_vkey(qt, N, doc_off):
    """GPU per-key V form in the oracle's layout: codes [B, H, N, d] (by token), exponents [B, H, N]."""
    c = unpack_nibbles(qt.codes_view().cpu().numpy())  # [B, H, d, np]
    slots = v_slots(N, doc_off, qt.desc.fmt.block)
    codes = np.ascontiguousarray(np.swapaxes(c[..., slots], -1, -2))
    ek = qt.scales_view().cpu().numpy()[..., slots].astype(np.int32) - 127
    return codes, ek


def oracle_vkey(vf, vfmt):
    """oracle per-key form of V [B, H, N, d]: (codes [B,H,N,d], values [B,H,N,d], exponents [B,H,N])"""
    B, H, N, d = vf.shape
    codes = np.zeros((B, H, N, d), np.uint8)
    ek = np.zeros((B, H, N), np.int32)
    for b in range(B):
        for h in range(H):
            codes[b, h], ek[b, h] = oracle.quantize_keys(vf[b, h], vfmt)
    return codes, oracle.e2m1_values(codes), ek


def run_case(qfmt, vfmt, pmode, pfmt, B, Hq, Hkv, N, causal=False, kind="kmean", seed=0, doc_off=None,
             rows=None, check_bytes=True, inputs=None, pre=None, safe=False, exp_mode="exact"):
    """Run one forward on the GPU and on the oracle; returns a dict of results.

    pre: None, or a dict of outlier pre-processing for Q and K: {"center": both means
    subtracted and the compensation passed as score bias, "smoothk": K's mean only,
    "hadamard": normalized rotation} (keys absent = off).  exp_mode: the exponential of
    P~ ("exact", "mitchell", "schraudolph") on both sides."""
    import torch
    import microscaling_fp4_attention_amd as mx

    x = inputs if inputs is not None else synth.make_inputs(kind, B, Hq, Hkv, N, 128, seed)
    qf, kf, vf = (synth.bf16_to_f32(x[n]) for n in ("q", "k", "v"))
    dev = torch.device("cuda:0")

    def to_dev(a):
        return torch.from_numpy(a.astype(np.int16)).view(torch.bfloat16).to(dev)

    qg, kg, vg = to_dev(x["q"]), to_dev(x["k"]), to_dev(x["v"])
    cu = None if doc_off is None else torch.from_numpy(np.asarray(doc_off, np.int32)).to(dev)
    pre = pre or {}
    center, smoothk, had = bool(pre.get("center")), bool(pre.get("smoothk")), bool(pre.get("hadamard"))
    qmean_g = mx.channel_mean(qg, cu) if center else None
    kmean_g = mx.channel_mean(kg, cu) if (center or smoothk) else None
    if center or smoothk or had:
        Qq = mx.quantize(qg, mx.ROLE_QK, qfmt, cu_seqlens=cu, mean=qmean_g, hadamard=had)
        Kq = mx.quantize(kg, mx.ROLE_QK, qfmt, cu_seqlens=cu, mean=kmean_g, hadamard=had)
    else:
        Qq = mx.quantize(qg, mx.ROLE_QK, qfmt)
        Kq = mx.quantize(kg, mx.ROLE_QK, qfmt)
    Vq = mx.quantize(vg, mx.ROLE_V, vfmt, cu_seqlens=cu)
    delta_g = mx.center_comp(qmean_g, kg, kmean_g, cu) if center else None
    Vk = mx.quantize(vg, mx.ROLE_VKEY, vfmt, cu_seqlens=cu) if safe else None
    params = mx.fwd_params(pmode, pfmt, causal=causal, score_bias=delta_g, vkey=Vk, exp_mode=exp_mode)
    ws, nd = None, 0
    if doc_off is not None:
        ws = mx.fwd_plan(doc_off, N, causal)
        nd = len(doc_off) - 1
    lse = torch.empty((B, Hq, N), dtype=torch.float32, device=dev)
    out = mx.fwd(Qq, Kq, Vq, params, lse=lse, workspace=ws, ndocs=nd)
    torch.cuda.synchronize()
    O_gpu = out.cpu().numpy().reshape(-1, 128)
    lse_gpu = lse.cpu().numpy().reshape(-1)

    res = {}
    # oracle pre-processing (means bit-exact, compensation within one float ulp)
    bias = None
    if center or smoothk or had:
        qmeans, qf_in = oracle_preproc(qf, doc_off, center, had)
        kmeans, kf_in = oracle_preproc(kf, doc_off, center or smoothk, had)
        if center:
            assert np.array_equal(qmean_g.cpu().numpy(), qmeans), "Q means differ"
        if center or smoothk:
            assert np.array_equal(kmean_g.cpu().numpy(), kmeans), "K means differ"
        if center:
            bias = oracle_comp(qmeans, kf, kmeans, Hq, doc_off)
            res["delta_ulp"] = ulp_diff(delta_g.cpu().numpy(), bias)
            assert res["delta_ulp"] <= 1, f"compensation differs by {res['delta_ulp']} ulp"
    else:
        qf_in, kf_in = qf, kf
    # oracle quantization (bytes must match the GPU's)
    qc, qs, qd = oracle_quant_qk(qf_in, qfmt)
    kc, ks, kd = oracle_quant_qk(kf_in, qfmt)
    vc, vs, vd = oracle_quant_v(vf, vfmt, doc_off)
    if check_bytes:
        assert np.array_equal(gpu_codes_qk(Qq), qc), "Q codes differ"
        assert np.array_equal(Qq.scales_view().cpu().numpy(), qs), "Q scales differ"
        assert np.array_equal(gpu_codes_qk(Kq), kc), "K codes differ"
        assert np.array_equal(Kq.scales_view().cpu().numpy(), ks), "K scales differ"
        gc, gs = gpu_codes_v(Vq, N, doc_off)
        assert np.array_equal(gc, vc), "V codes differ"
        assert np.array_equal(gs, vs), "V scales differ"
    vk_vals = vk_exp = None
    if safe:
        vk_codes, vk_vals, vk_exp = oracle_vkey(vf, vfmt)
        if check_bytes:
            gkc, gke = gpu_codes_vkey(Vk, N, doc_off)
            assert np.array_equal(gkc, vk_codes), "per-key V codes differ"
            assert np.array_equal(gke, vk_exp), "per-key V exponents differ"
    O_ref, lse_ref, fb = oracle.attention(qd, kd, vd, PM_ORACLE[pmode], pfmt, causal=causal, doc_off=doc_off,
                                          rows=rows, bias=bias, vkey=vk_vals, vkey_exp=vk_exp, exp_mode=exp_mode,
                                          score_rounds=score_rounds(qfmt))
    sel = np.arange(B * Hq * N) if rows is None else np.asarray(rows)
    Og = O_gpu[sel]
    err = np.abs(Og - O_ref)
    amax = np.abs(O_ref).max()
    bound = TOL * amax + fb[:, None]
    res.update(err=err, bound=bound, amax=amax, fb=fb, O_ref=O_ref, O_gpu=Og, lse_ref=lse_ref, lse_gpu=lse_gpu[sel],
               O_gpu_all=O_gpu,
               ratio=float((err / bound).max()) if err.size else 0.0, n_fragile=int((fb > 0).sum()))
    return res
