"""Parity at the full sizes of the five measured workloads, in the launch shape
bench.py times (all heads, full sequence), on sampled query rows the oracle
computes one by one: first and last rows, rows at document boundaries and seeded
random rows of a few heads.  FP32 output: |dO| <= 2e-3 max|O| + flip budget; the
quantized bytes of the sampled heads must match the oracle's exactly."""
import numpy as np
import pytest

import oracle
import synth
from helpers import (PM_ORACLE, TOL, gpu_available, gpu_codes_qk, gpu_codes_v, gpu_codes_vkey, oracle_quant_qk,
                     oracle_quant_v, oracle_vkey, record_parity, score_rounds)

pytestmark = [pytest.mark.gpu, pytest.mark.skipif(not gpu_available(), reason="needs a GPU")]

# case -> (workload, Q/K format, V format, P mode, P format), as bench.py runs them; the
# two-level cases at N = 32K take the video-DiT inputs with both readings of the
# level-2 block format (E4M3 per 16 keys, E8M0 per 32 keys); "_safe": with causally
# safe V scales (bench.py --causal-safe)
CASES = {
    "c1_single_head": ("c1_single_head", "mxfp4", "mxfp4", "two_level", "nvfp4"),
    "c2_mha_4k": ("c2_mha_4k", "mxfp4", "mxfp4", "two_level", "nvfp4"),
    "c3_video_dit_32k": ("c3_video_dit_32k", "mxfp4_uos", "mxfp4_uos", "pnq", "mxfp4_uos"),
    "c4_gqa_causal_32k": ("c4_gqa_causal_32k", "nvfp4", "fp8v", "fp8", None),
    "c5_varlen_causal_64k": ("c5_varlen_causal_64k", "mxfp4", "mxfp4", "two_level", "nvfp4"),
    "two_level_e4m3_32k": ("c3_video_dit_32k", "mxfp4", "mxfp4", "two_level", "nvfp4"),
    "two_level_e8m0_32k": ("c3_video_dit_32k", "mxfp4", "mxfp4", "two_level", "mxfp4"),
    "c5_varlen_causal_64k_safe": ("c5_varlen_causal_64k", "mxfp4", "mxfp4", "two_level", "nvfp4"),
    # the same with the bit-level Mitchell-P exponential (bench.py --causal-safe --exp mitchell)
    "c5_varlen_causal_64k_safe_mitchell": ("c5_varlen_causal_64k", "mxfp4", "mxfp4", "two_level", "nvfp4"),
}


def _sample_rows(N, doc_off, rng, n_random=10):
    rows = {0, N - 1}
    if doc_off is not None:
        for s in doc_off[1:-1][:6]:
            rows.update({int(s) - 1, int(s)})
    rows.update(int(r) for r in rng.integers(0, N, n_random))
    return sorted(r for r in rows if 0 <= r < N)


@pytest.mark.parametrize("name", list(CASES))
def test_fullsize_sampled_rows(name):
    import torch
    import microscaling_fp4_attention_amd as mx

    wl, qf, vf, pm, pf = CASES[name]
    x = synth.workload(wl)
    B, Hq, Hkv, N = x["B"], x["Hq"], x["Hkv"], x["N"]
    causal, doc_off = x["causal"], x["doc_off"]
    dev = "cuda:0"
    t = {n: torch.from_numpy(x[n].astype(np.int16)).view(torch.bfloat16).to(dev) for n in "qkv"}
    cu = None if doc_off is None else torch.from_numpy(doc_off.astype(np.int32)).to(dev)
    Q = mx.quantize(t["q"], mx.ROLE_QK, qf)
    K = mx.quantize(t["k"], mx.ROLE_QK, qf)
    V = mx.quantize(t["v"], mx.ROLE_V, vf, cu_seqlens=cu)
    exp_mode = "mitchell" if name.endswith("_mitchell") else "exact"
    safe = name.endswith("_safe") or name.endswith("_safe_mitchell")
    Vk = mx.quantize(t["v"], mx.ROLE_VKEY, vf, cu_seqlens=cu) if safe else None
    ws, nd = None, 0
    if doc_off is not None:
        ws = mx.fwd_plan(doc_off, N, causal)
        nd = len(doc_off) - 1
    out = mx.fwd(Q, K, V, mx.fwd_params(pm, pf, causal=causal, out_fp32=True, vkey=Vk, exp_mode=exp_mode),
                 workspace=ws, ndocs=nd)
    torch.cuda.synchronize()

    rng = np.random.default_rng(12345)
    heads = sorted({0, Hq - 1, int(rng.integers(0, Hq))})
    rows = _sample_rows(N, doc_off, rng)
    qcodes, kcodes = gpu_codes_qk(Q), gpu_codes_qk(K)
    vcodes, vscales = gpu_codes_v(V, N, doc_off)
    if safe:
        gkc, gke = gpu_codes_vkey(Vk, N, doc_off)
    worst, fbt = 0.0, []
    for h in heads:
        hk = h * Hkv // Hq
        qh = synth.bf16_to_f32(x["q"][:1, h:h + 1])
        kh = synth.bf16_to_f32(x["k"][:1, hk:hk + 1])
        vh = synth.bf16_to_f32(x["v"][:1, hk:hk + 1])
        qc, qs, qd = oracle_quant_qk(qh, qf)
        kc, ks, kd = oracle_quant_qk(kh, qf)
        vc, vs, vd = oracle_quant_v(vh, vf, doc_off)
        assert np.array_equal(qcodes[0, h], qc[0, 0]) and np.array_equal(Q.scales_view()[0, h].cpu().numpy(), qs[0, 0])
        assert np.array_equal(kcodes[0, hk], kc[0, 0]) and np.array_equal(K.scales_view()[0, hk].cpu().numpy(), ks[0, 0])
        assert np.array_equal(vcodes[0, hk], vc[0, 0]) and np.array_equal(vscales[0, hk], vs[0, 0])
        vk_vals = vk_exp = None
        if safe:
            vk_codes, vk_vals, vk_exp = oracle_vkey(vh, vf)
            assert np.array_equal(gkc[0, hk], vk_codes[0, 0]) and np.array_equal(gke[0, hk], vk_exp[0, 0])
        O_ref, _, fb = oracle.attention(qd, kd, vd, PM_ORACLE[pm], pf, causal=causal, doc_off=doc_off,
                                        rows=np.array(rows, np.int64), score_rounds=score_rounds(qf),
                                        vkey=vk_vals, vkey_exp=vk_exp, exp_mode=exp_mode)
        O_gpu = out[0, h].cpu().numpy()[rows]
        # the bound uses max|O| of the sampled rows of this head
        bound = TOL * np.abs(O_ref).max() + fb[:, None]
        ratio = float((np.abs(O_gpu - O_ref) / bound).max())
        worst = max(worst, ratio)
        fbt.append(fb / (TOL * np.abs(O_ref).max()))
        assert np.all(np.isfinite(O_gpu))
    print(f"{name}: heads {heads}, {len(rows)} rows each, max |dO| / bound = {worst:.2e}")
    # rows of up to 64K keys: the share of rows with a budget is not capped, the median is
    record_parity(f"full size {name}", worst, np.concatenate(fbt), None)
    assert worst <= 1.0
