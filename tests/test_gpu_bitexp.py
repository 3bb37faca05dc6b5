"""GPU forward with the bit-level exponentials ("FLAMIA: FLAsh MIcroscaling Attention
for Fast and Causally Safe Training on Blackwell", section 3.7 and appendix C)
against the oracle's piecewise-linear exponential: |dO| <= 2e-3 max|O| + the row's
flip budget, on every ping-pong kernel route, causal and packed-document masks,
grouped-query heads, the centering bias and causally safe V scales, plus the two
full-size workloads in bench.py's launch shape on sampled rows."""
import numpy as np
import pytest

import oracle
import synth
from helpers import PM_ORACLE, TOL, gpu_available, record_parity, run_case, score_rounds

pytestmark = [pytest.mark.gpu, pytest.mark.skipif(not gpu_available(), reason="needs a GPU")]

# ping-pong kernel routes: (Q/K format, V format, P mode, P format)
ROUTES = {
    "mxfp4_direct": ("mxfp4", "mxfp4", "direct", "mxfp4"),
    "mxfp4_uos_pnq": ("mxfp4_uos", "mxfp4_uos", "pnq", "mxfp4_uos"),
    "mxfp4_two_level_e8m0": ("mxfp4", "mxfp4", "two_level", "mxfp4"),
    "mxfp4_two_level_e4m3": ("mxfp4", "mxfp4", "two_level", "nvfp4"),
    "mxfp4_pnq_e4m3p": ("mxfp4", "mxfp4", "pnq", "nvfp4"),
    "qk4pv8": ("nvfp4", "fp8v", "fp8", None),
    "mxfp4_qk_pv8": ("mxfp4", "fp8v", "fp8", None),
}
# the form each route is meant for: Mitchell-P for a 4-bit P, Schraudolph's for FP8 P
MEANT = {r: ("schraudolph" if ROUTES[r][2] == "fp8" else "mitchell") for r in ROUTES}


def lse_bound(res):
    """1e-3 relative, plus (PNQ: the row sum is taken from P^) the largest relative change
    of the row sum that the row's fragile P decisions can make: the flip budget fb is
    (fb_O + fb_l max|o|) / l, so fb_l / l <= fb / max|o|"""
    omax = np.abs(res["O_ref"]).max(1)
    flips = np.where(omax > 0, res["fb"] / np.maximum(omax, 1e-30), 0.0)
    return 1e-3 * np.maximum(1.0, np.abs(res["lse_ref"])) + np.log1p(flips)


def _check(res, name):
    print(f"{name}: max err/bound {res['ratio']:.3f}, fragile rows {res['n_fragile']}, amax {res['amax']:.3f}")
    record_parity(name, res["ratio"], res["fb"] / (TOL * res["amax"]), None)
    assert np.all(np.isfinite(res["O_gpu"]))
    assert res["ratio"] <= 1.0, name
    lg, lr = res["lse_gpu"], res["lse_ref"]
    same_inf = np.isinf(lg) & (lg == lr)
    d = np.where(same_inf, 0.0, np.abs(lg - lr))
    r = d / lse_bound(res)
    i = int(np.argmax(r))
    print(f"  lse: worst row {i} |d| {d[i]:.3e} bound {lse_bound(res)[i]:.3e} fb {res['fb'][i]:.3e}")
    assert np.all(r <= 1.0), name


@pytest.mark.parametrize("route", list(ROUTES))
@pytest.mark.parametrize("exp_mode", ["mitchell", "schraudolph"])
def test_bits_noncausal(route, exp_mode):
    q, v, pm, pf = ROUTES[route]
    res = run_case(q, v, pm, pf, B=1, Hq=2, Hkv=2, N=300, kind="kmean", seed=31, exp_mode=exp_mode)
    _check(res, f"{route} {exp_mode}")


@pytest.mark.parametrize("route", list(ROUTES))
def test_bits_causal_gqa(route):
    q, v, pm, pf = ROUTES[route]
    res = run_case(q, v, pm, pf, B=2, Hq=4, Hkv=2, N=257, causal=True, kind="kmean", seed=32, exp_mode=MEANT[route])
    _check(res, f"{route} {MEANT[route]} causal gqa")


@pytest.mark.parametrize("route", ["mxfp4_uos_pnq", "mxfp4_two_level_e4m3", "qk4pv8"])
@pytest.mark.parametrize("causal", [False, True])
def test_bits_packed_documents(route, causal):
    q, v, pm, pf = ROUTES[route]
    doc_off = np.array([0, 100, 101, 357, 490, 700], np.int32)
    res = run_case(q, v, pm, pf, B=1, Hq=2, Hkv=2, N=700, causal=causal, kind="outlier", seed=33, doc_off=doc_off,
                   exp_mode=MEANT[route])
    _check(res, f"{route} {MEANT[route]} docs causal={causal}")


@pytest.mark.parametrize("route", ["mxfp4_uos_pnq", "mxfp4_two_level_e4m3", "qk4pv8"])
def test_bits_with_centering_bias(route):
    q, v, pm, pf = ROUTES[route]
    res = run_case(q, v, pm, pf, B=1, Hq=4, Hkv=2, N=300, causal=True, kind="kmean", seed=34, pre={"center": True},
                   exp_mode=MEANT[route])
    _check(res, f"{route} {MEANT[route]} centered")


@pytest.mark.parametrize("route", ["mxfp4_uos_pnq", "mxfp4_direct", "mxfp4_two_level_e4m3", "mxfp4_two_level_e8m0"])
def test_bits_causally_safe_v(route):
    """Mitchell-P with the per-key V form on the diagonal tiles (the page's 4-bit P
    route with its causally safe scales)."""
    q, v, pm, pf = ROUTES[route]
    doc_off = np.array([0, 129, 130, 500, 777], np.int32)
    res = run_case(q, v, pm, pf, B=1, Hq=2, Hkv=1, N=777, causal=True, kind="outlier", seed=35, doc_off=doc_off,
                   safe=True, exp_mode="mitchell")
    _check(res, f"{route} mitchell causally safe")


def test_bits_change_the_result():
    """The bit-level run is not the exact run: the two outputs differ by about the
    approximation, and the masked-out future keys still contribute nothing."""
    q, v, pm, pf = ROUTES["mxfp4_uos_pnq"]
    x = synth.make_inputs("kmean", 1, 2, 2, 300, 128, 36)
    r_e = run_case(q, v, pm, pf, B=1, Hq=2, Hkv=2, N=300, causal=True, inputs=x)
    r_m = run_case(q, v, pm, pf, B=1, Hq=2, Hkv=2, N=300, causal=True, inputs=x, exp_mode="mitchell")
    d = np.abs(r_e["O_gpu_all"] - r_m["O_gpu_all"]).max()
    print(f"max |O_exact - O_mitchell| = {d:.4f} (amax {r_e['amax']:.3f})")
    assert d > 1e-3 * r_e["amax"]
    assert d < 0.2 * r_e["amax"]
    # row 0 sees key 0 only: O = V[0] dequantized up to P's own rounding in both modes
    assert np.allclose(r_m["O_gpu_all"][0], r_e["O_gpu_all"][0], atol=0.05 * r_e["amax"])


def test_bits_refused_where_not_built():
    """The 4-wave kernel's routes (E4M3-scaled V, NVFP4 Q/K with a 4-bit PV) and the
    split-key decode refuse the bit-level modes with MXATTN_E_UNSUPPORTED."""
    import torch
    import microscaling_fp4_attention_amd as mx
    x = synth.make_inputs("kmean", 1, 1, 1, 128, 128, 37)
    t = {n: torch.from_numpy(x[n].astype(np.int16)).view(torch.bfloat16).to("cuda:0") for n in "qkv"}
    for qf, vf, pm, pf in [("nvfp4", "nvfp4", "two_level", "nvfp4"), ("nvfp4", "mxfp4", "pnq", "mxfp4")]:
        Q = mx.quantize(t["q"], mx.ROLE_QK, qf)
        K = mx.quantize(t["k"], mx.ROLE_QK, qf)
        V = mx.quantize(t["v"], mx.ROLE_V, vf)
        mx.fwd(Q, K, V, mx.fwd_params(pm, pf))  # the exact mode runs
        with pytest.raises(RuntimeError, match="unsupported"):
            mx.fwd(Q, K, V, mx.fwd_params(pm, pf, exp_mode="mitchell"))
    Q = mx.quantize(t["q"][:, :, -1:], mx.ROLE_QK, "mxfp4")
    K = mx.quantize(t["k"], mx.ROLE_QK, "mxfp4")
    V = mx.quantize(t["v"], mx.ROLE_V, "mxfp4")
    ws = torch.empty(mx.decode_workspace_bytes(1, 1, 1, 128), dtype=torch.uint8, device="cuda:0")
    with pytest.raises(RuntimeError, match="unsupported"):
        mx.decode(Q, K, V, mx.fwd_params("two_level", "mxfp4", causal=True, exp_mode="mitchell"), workspace=ws)
    Qf = mx.quantize(t["q"], mx.ROLE_QK, "mxfp4")
    mx.fwd(Qf, K, V, mx.fwd_params("two_level", "mxfp4", exp_mode="mitchell"))
    with pytest.raises(RuntimeError, match="invalid"):
        mx.fwd(Qf, K, V, mx.fwd_params("two_level", "mxfp4", exp_mode=9))


@pytest.mark.parametrize("name,exp_mode", [("c3_video_dit_32k", "mitchell"), ("c4_gqa_causal_32k", "schraudolph")])
def test_bits_fullsize_sampled_rows(name, exp_mode):
    """The video-DiT 32K workload with Mitchell-P and the GQA causal 32K workload with
    Schraudolph's form, all heads launched as bench.py launches them, checked on
    sampled rows of a few heads."""
    import torch
    import microscaling_fp4_attention_amd as mx
    from helpers import oracle_quant_qk, oracle_quant_v
    cases = {"c3_video_dit_32k": ("mxfp4_uos", "mxfp4_uos", "pnq", "mxfp4_uos"),
             "c4_gqa_causal_32k": ("nvfp4", "fp8v", "fp8", None)}
    qf, vf, pm, pf = cases[name]
    x = synth.workload(name)
    B, Hq, Hkv, N, causal = x["B"], x["Hq"], x["Hkv"], x["N"], x["causal"]
    t = {n: torch.from_numpy(x[n].astype(np.int16)).view(torch.bfloat16).to("cuda:0") for n in "qkv"}
    Q = mx.quantize(t["q"], mx.ROLE_QK, qf)
    K = mx.quantize(t["k"], mx.ROLE_QK, qf)
    V = mx.quantize(t["v"], mx.ROLE_V, vf)
    out = mx.fwd(Q, K, V, mx.fwd_params(pm, pf, causal=causal, out_fp32=True, exp_mode=exp_mode))
    torch.cuda.synchronize()
    rng = np.random.default_rng(2024)
    heads = sorted({0, Hq - 1, int(rng.integers(0, Hq))})
    rows = sorted({0, N - 1, *map(int, rng.integers(0, N, 10))})
    worst, fbt = 0.0, []
    for h in heads:
        hk = h * Hkv // Hq
        _, _, qd = oracle_quant_qk(synth.bf16_to_f32(x["q"][:1, h:h + 1]), qf)
        _, _, kd = oracle_quant_qk(synth.bf16_to_f32(x["k"][:1, hk:hk + 1]), qf)
        _, _, vd = oracle_quant_v(synth.bf16_to_f32(x["v"][:1, hk:hk + 1]), vf)
        O_ref, _, fb = oracle.attention(qd, kd, vd, PM_ORACLE[pm], pf, causal=causal, rows=np.array(rows, np.int64),
                                        exp_mode=exp_mode, score_rounds=score_rounds(qf))
        O_gpu = out[0, h].cpu().numpy()[rows]
        assert np.all(np.isfinite(O_gpu))
        bound = TOL * np.abs(O_ref).max() + fb[:, None]
        worst = max(worst, float((np.abs(O_gpu - O_ref) / bound).max()))
        fbt.append(fb / (TOL * np.abs(O_ref).max()))
    print(f"{name} {exp_mode}: heads {heads}, {len(rows)} rows, max |dO|/bound = {worst:.2e}")
    record_parity(f"full size {name} {exp_mode}", worst, np.concatenate(fbt), None)
    assert worst <= 1.0
