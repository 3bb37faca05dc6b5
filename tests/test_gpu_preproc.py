"""GPU outlier pre-processing against the oracle: channel means (bit-exact), the
centered / rotated Q and K quantization (bytes bit-exact), the centering compensation
(within one float ulp) and the forward with the compensation as score bias, for every
forward kernel, causal masks, grouped-query heads and packed documents."""
import numpy as np
import pytest

import oracle
import synth
from helpers import (TOL, gpu_available, gpu_codes_qk, oracle_comp, oracle_preproc, oracle_quant_qk, record_parity,
                     run_case, score_rounds, ulp_diff)

pytestmark = [pytest.mark.gpu, pytest.mark.skipif(not gpu_available(), reason="needs a GPU")]


def _dev(a):
    import torch
    return torch.from_numpy(a.astype(np.int16)).view(torch.bfloat16).to("cuda:0")


def _inputs(B, H, N, seed, shift=1.5):
    """bf16 tensor [B, H, N, 128] with a per-channel offset and a few outlier channels"""
    x = synth.gaussian(seed, 3, (B, H, N, 128)) + np.float32(shift) * synth.gaussian(seed, 4, (1, 1, 1, 128))
    x[..., 7] *= 12.0
    return synth.f32_to_bf16(x.astype(np.float32))


DOCS8 = [0, 1, 130, 131, 700, 1500, 2600, 2601, 3000]  # 8 documents, two of one token


@pytest.mark.parametrize("B,H,N,docs", [(2, 3, 1000, None), (1, 2, 777, [0, 1, 300, 301, 777]), (1, 1, 1, None),
                                        (1, 16, 3000, DOCS8), (1, 17, 3000, DOCS8), (4, 40, 300, None)])
def test_channel_mean_bitexact(B, H, N, docs):
    """including 128, 136 and 160 (batch, head, document) units: documents of one
    token, units numbered document-major over several XCD rounds"""
    import torch
    import microscaling_fp4_attention_amd as mx
    h = _inputs(B, H, N, 11)
    cu = None if docs is None else torch.tensor(docs, dtype=torch.int32, device="cuda:0")
    m = mx.channel_mean(_dev(h), cu).cpu().numpy()
    xf = synth.bf16_to_f32(h)
    for b in range(B):
        for hh in range(H):
            assert np.array_equal(m[b, hh], oracle.channel_mean(xf[b, hh], docs)), (b, hh)


def test_channel_mean_strided_input():
    """a [B, N, H, d] activation read through its [B, H, N, d] view"""
    import torch
    import microscaling_fp4_attention_amd as mx
    h = _inputs(1, 3, 500, 12)
    x = _dev(h)[0].permute(1, 0, 2).contiguous().permute(1, 0, 2)[None]  # strides (., 128, 384, 1)
    assert x.stride(2) == 3 * 128
    m = mx.channel_mean(x).cpu().numpy()
    xf = synth.bf16_to_f32(h)
    for hh in range(3):
        assert np.array_equal(m[0, hh], oracle.channel_mean(xf[0, hh]))


@pytest.mark.parametrize("fmt", ["mxfp4", "mxfp4_uos", "nvfp4"])
@pytest.mark.parametrize("mean_on,had", [(True, False), (False, True), (True, True)])
@pytest.mark.parametrize("docs", [None, [0, 129, 130, 600]])
def test_quantize_pre_bytes(fmt, mean_on, had, docs):
    import torch
    import microscaling_fp4_attention_amd as mx
    B = 1 if docs is not None else 2
    N = 600
    h = _inputs(B, 2, N, 13)
    x = _dev(h)
    cu = None if docs is None else torch.tensor(docs, dtype=torch.int32, device="cuda:0")
    mean = mx.channel_mean(x, cu) if mean_on else None
    qt = mx.quantize(x, mx.ROLE_QK, fmt, cu_seqlens=cu, mean=mean, hadamard=had)
    means, y = oracle_preproc(synth.bf16_to_f32(h), docs, mean_on, had)
    codes, scales, _ = oracle_quant_qk(y, fmt)
    assert np.array_equal(gpu_codes_qk(qt), codes)
    assert np.array_equal(qt.scales_view().cpu().numpy(), scales)


@pytest.mark.parametrize("docs", [None, [0, 5, 200, 333]])
def test_center_comp(docs):
    import torch
    import microscaling_fp4_attention_amd as mx
    B = 2 if docs is None else 1
    hq, hk = _inputs(B, 4, 333, 14, shift=2.0), _inputs(B, 2, 333, 15, shift=-1.0)
    cu = None if docs is None else torch.tensor(docs, dtype=torch.int32, device="cuda:0")
    qg, kg = _dev(hq), _dev(hk)
    qm, km = mx.channel_mean(qg, cu), mx.channel_mean(kg, cu)
    delta = mx.center_comp(qm, kg, km, cu).cpu().numpy()
    ref = oracle_comp(qm.cpu().numpy(), synth.bf16_to_f32(hk), km.cpu().numpy(), 4, docs)
    assert ulp_diff(delta, ref) <= 1
    assert np.mean(delta == ref) > 0.99


# (Q/K format, V format, P mode, P format): one route per forward kernel
BIAS_ROUTES = {
    "mxfp4_uos_pnq": ("mxfp4_uos", "mxfp4_uos", "pnq", "mxfp4_uos"),      # ping-pong, FP4 PV
    "mxfp4_two_level_e4m3": ("mxfp4", "mxfp4", "two_level", "nvfp4"),    # ping-pong, bf16 PV
    "qk4pv8": ("nvfp4", "fp8v", "fp8", None),                            # ping-pong, bf16 QK, FP8 PV
    "nvfp4_two_level": ("nvfp4", "nvfp4", "two_level", "nvfp4"),          # NVFP4-V kernel
}


def _check(res, name):
    print(f"{name}: max err/bound {res['ratio']:.3f}, delta ulp {res.get('delta_ulp')}, amax {res['amax']:.3f}")
    record_parity(name, res["ratio"], res["fb"] / (TOL * res["amax"]))
    assert np.all(np.isfinite(res["O_gpu"]))
    assert res["ratio"] <= 1.0, name


@pytest.mark.parametrize("route", list(BIAS_ROUTES))
@pytest.mark.parametrize("causal", [False, True])
def test_fwd_centered(route, causal):
    q, v, pm, pf = BIAS_ROUTES[route]
    res = run_case(q, v, pm, pf, B=1, Hq=4, Hkv=2, N=300, causal=causal, kind="kmean", seed=21,
                   pre={"center": True})
    _check(res, f"{route} centered causal={causal}")


@pytest.mark.parametrize("route", ["mxfp4_uos_pnq", "qk4pv8", "nvfp4_two_level"])
def test_fwd_centered_documents(route):
    q, v, pm, pf = BIAS_ROUTES[route]
    doc_off = np.array([0, 100, 101, 357, 490, 700], np.int32)
    res = run_case(q, v, pm, pf, B=1, Hq=2, Hkv=2, N=700, causal=True, kind="outlier", seed=22, doc_off=doc_off,
                   pre={"center": True})
    _check(res, f"{route} centered docs")


@pytest.mark.parametrize("pre", [{"smoothk": True}, {"hadamard": True}, {"center": True, "hadamard": True}])
def test_fwd_other_preprocessing(pre):
    res = run_case("mxfp4", "mxfp4", "two_level", "nvfp4", B=1, Hq=2, Hkv=1, N=400, causal=False, kind="outlier",
                   seed=23, pre=pre)
    _check(res, f"pre={pre}")


@pytest.mark.parametrize("route", [("mxfp4", "mxfp4", "two_level", "nvfp4"), ("mxfp4_uos", "mxfp4_uos", "pnq", "mxfp4_uos"),
                                   ("nvfp4", "fp8v", "fp8", None), ("nvfp4", "nvfp4", "direct", "nvfp4")])
def test_fwd_smoothk_packed_causal(route):
    """smooth-K alone (each document's K mean, no compensation: a row's visible keys all
    share it) under the causal mask with packed documents, on both forward kernels"""
    doc_off = np.array([0, 1, 300, 301, 777], np.int32)
    res = run_case(*route, B=1, Hq=4, Hkv=2, N=777, causal=True, kind="outlier", seed=24, doc_off=doc_off,
                   pre={"smoothk": True})
    _check(res, f"smooth-K docs causal {route[2]} {route[0]}")


def test_fullsize_gqa_causal_centered():
    """The GQA causal 32K workload (NVFP4 Q/K, FP8 P and V) with sequence centering
    and the compensation bias, in the launch shape bench.py times, on sampled rows
    of a few heads; means bit-exact, compensation within one ulp, bytes bit-exact."""
    import torch
    import microscaling_fp4_attention_amd as mx
    from helpers import PM_ORACLE, TOL, oracle_quant_v, gpu_codes_v

    x = synth.workload("c4_gqa_causal_32k")
    B, Hq, Hkv, N = x["B"], x["Hq"], x["Hkv"], x["N"]
    qg, kg, vg = _dev(x["q"]), _dev(x["k"]), _dev(x["v"])
    qm, km = mx.channel_mean(qg), mx.channel_mean(kg)
    Q = mx.quantize(qg, mx.ROLE_QK, "nvfp4", mean=qm)
    K = mx.quantize(kg, mx.ROLE_QK, "nvfp4", mean=km)
    V = mx.quantize(vg, mx.ROLE_V, "fp8v")
    delta = mx.center_comp(qm, kg, km)
    out = mx.fwd(Q, K, V, mx.fwd_params("fp8", None, causal=True, out_fp32=True, score_bias=delta))
    torch.cuda.synchronize()
    rng = np.random.default_rng(7)
    heads = sorted({0, Hq - 1, int(rng.integers(0, Hq))})
    rows = sorted({0, N - 1, *map(int, rng.integers(0, N, 10))})
    qcodes, kcodes = gpu_codes_qk(Q), gpu_codes_qk(K)
    dg = delta.cpu().numpy()
    worst, fbt = 0.0, []
    for h in heads:
        hk = h * Hkv // Hq
        qf = synth.bf16_to_f32(x["q"][:1, h:h + 1])
        kf = synth.bf16_to_f32(x["k"][:1, hk:hk + 1])
        vf = synth.bf16_to_f32(x["v"][:1, hk:hk + 1])
        qmean, qy = oracle_preproc(qf, None, True, False)
        kmean, ky = oracle_preproc(kf, None, True, False)
        assert np.array_equal(qm[0, h].cpu().numpy(), qmean[0, 0]) and np.array_equal(km[0, hk].cpu().numpy(), kmean[0, 0])
        qc, qs, qd = oracle_quant_qk(qy, "nvfp4")
        kc, ks, kd = oracle_quant_qk(ky, "nvfp4")
        assert np.array_equal(qcodes[0, h], qc[0, 0]) and np.array_equal(kcodes[0, hk], kc[0, 0])
        _, _, vd = oracle_quant_v(vf, "fp8v")
        bias = oracle_comp(qmean, kf, kmean, 1, None)
        assert ulp_diff(dg[0, h], bias[0, 0]) <= 1
        O_ref, _, fb = oracle.attention(qd, kd, vd, PM_ORACLE["fp8"], None, causal=True,
                                        rows=np.array(rows, np.int64), bias=bias, score_rounds=score_rounds("nvfp4"))
        O_gpu = out[0, h].cpu().numpy()[rows]
        bound = TOL * np.abs(O_ref).max() + fb[:, None]
        worst = max(worst, float((np.abs(O_gpu - O_ref) / bound).max()))
        fbt.append(fb / (TOL * np.abs(O_ref).max()))
    print(f"c4 centered: heads {heads}, {len(rows)} rows, max |dO|/bound = {worst:.2e}")
    record_parity("full size c4 centered", worst, np.concatenate(fbt), None)
    assert worst <= 1.0


@pytest.mark.parametrize("had", [False, True])
def test_fullsize_varlen_causal_centered(had):
    """The packed-document causal 64K workload (MXFP4 Q/K/V, two-level P with E4M3/16
    level 2) with per-document centering and the compensation bias, with and without the
    normalized Hadamard rotation of the centered Q and K, in the launch shape bench.py times, on sampled rows of a few heads (each document's first and last row
    among them); means bit-exact, compensation within one ulp, bytes bit-exact."""
    import torch
    import microscaling_fp4_attention_amd as mx
    from helpers import PM_ORACLE, oracle_quant_v, gpu_codes_v

    x = synth.workload("c5_varlen_causal_64k")
    B, Hq, Hkv, N, doc_off = x["B"], x["Hq"], x["Hkv"], x["N"], x["doc_off"]
    nd = len(doc_off) - 1
    cu = torch.tensor(doc_off, dtype=torch.int32, device="cuda:0")
    qg, kg, vg = _dev(x["q"]), _dev(x["k"]), _dev(x["v"])
    qm, km = mx.channel_mean(qg, cu), mx.channel_mean(kg, cu)
    Q = mx.quantize(qg, mx.ROLE_QK, "mxfp4", cu_seqlens=cu, mean=qm, hadamard=had)
    K = mx.quantize(kg, mx.ROLE_QK, "mxfp4", cu_seqlens=cu, mean=km, hadamard=had)
    V = mx.quantize(vg, mx.ROLE_V, "mxfp4", cu_seqlens=cu)
    delta = mx.center_comp(qm, kg, km, cu)
    ws = mx.fwd_plan(doc_off, N, True)
    out = mx.fwd(Q, K, V, mx.fwd_params("two_level", "nvfp4", causal=True, out_fp32=True, score_bias=delta),
                 workspace=ws, ndocs=nd)
    torch.cuda.synchronize()
    rng = np.random.default_rng(8)
    heads = sorted({0, Hq - 1, int(rng.integers(0, Hq))})
    starts, ends = doc_off[:-1], doc_off[1:] - 1
    rows = sorted({0, N - 1, *map(int, starts[:4]), *map(int, ends[:4]), *map(int, rng.integers(0, N, 8))})
    qcodes, kcodes = gpu_codes_qk(Q), gpu_codes_qk(K)
    gvc, gvs = gpu_codes_v(V, N, doc_off)
    dg = delta.cpu().numpy()
    worst, fbt = 0.0, []
    for h in heads:
        hk = h * Hkv // Hq
        qf = synth.bf16_to_f32(x["q"][:1, h:h + 1])
        kf = synth.bf16_to_f32(x["k"][:1, hk:hk + 1])
        vf = synth.bf16_to_f32(x["v"][:1, hk:hk + 1])
        qmean, qy = oracle_preproc(qf, doc_off, True, had)
        kmean, ky = oracle_preproc(kf, doc_off, True, had)
        assert np.array_equal(qm[0, h].cpu().numpy(), qmean[0, 0]) and np.array_equal(km[0, hk].cpu().numpy(), kmean[0, 0])
        qc, qs, qd = oracle_quant_qk(qy, "mxfp4")
        kc, ks, kd = oracle_quant_qk(ky, "mxfp4")
        assert np.array_equal(qcodes[0, h], qc[0, 0]) and np.array_equal(kcodes[0, hk], kc[0, 0])
        vc, vs, vd = oracle_quant_v(vf, "mxfp4", doc_off)
        assert np.array_equal(gvc[0, hk], vc[0, 0]) and np.array_equal(gvs[0, hk], vs[0, 0])
        bias = oracle_comp(qmean, kf, kmean, 1, doc_off)
        assert ulp_diff(dg[0, h], bias[0, 0]) <= 1
        O_ref, _, fb = oracle.attention(qd, kd, vd, PM_ORACLE["two_level"], "nvfp4", causal=True, doc_off=doc_off,
                                        rows=np.array(rows, np.int64), bias=bias, score_rounds=score_rounds("mxfp4"))
        O_gpu = out[0, h].cpu().numpy()[rows]
        bound = TOL * np.abs(O_ref).max() + fb[:, None]
        worst = max(worst, float((np.abs(O_gpu - O_ref) / bound).max()))
        fbt.append(fb / (TOL * np.abs(O_ref).max()))
    name = "full size c5 centered" + (" + Hadamard" if had else "")
    print(f"{name}: {nd} documents, heads {heads}, {len(rows)} rows, max |dO|/bound = {worst:.2e}")
    record_parity(name, worst, np.concatenate(fbt), None)
    assert worst <= 1.0
