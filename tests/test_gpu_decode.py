"""GPU split-key decode (mxattn_decode) against the oracle's split decode ("MpFA ...",
section 5.3): the same quantized bytes, splits of 256 keys merged by log-sum-exp,
|dO| <= 2e-3 max|O| + the merged flip budget; ragged histories, several newest rows,
packed GQA groups, and a 32:8 GQA decode over 32K keys, for the MXFP4 routes and the
QK4PV8 route (NVFP4 Q/K, FP8 P and V).  Up to 16 packed query columns
(query heads per KV head x newest rows) run on the 16-column kernel, 17 to 32 on the
32-column one; both are covered for every P mode."""
import numpy as np
import pytest

import oracle
import synth
from helpers import (PM_ORACLE, TOL, gpu_available, gpu_codes_qk, gpu_codes_v, oracle_quant_qk, oracle_quant_v,
                     FRAGILE_CAP, record_parity, score_rounds, unpack_nibbles)

pytestmark = [pytest.mark.gpu, pytest.mark.skipif(not gpu_available(), reason="needs a GPU")]

FMT = {"direct": ("mxfp4", "mxfp4"), "pnq": ("mxfp4_uos", "mxfp4_uos"), "two_level": ("mxfp4", "mxfp4"),
       "fp8": ("nvfp4", "fp8v")}  # QK4PV8: NVFP4 Q/K, P = E4M3(448 P~), FP8 V


def _bf16(shape, seed, stream, shift=0.0):
    x = synth.gaussian(seed, stream, shape) + np.float32(shift)
    return synth.f32_to_bf16(x.astype(np.float32))


def run_decode(pm, B, Hq, Hkv, R, N, kv_len, seed, qfmt=None, cap=FRAGILE_CAP):
    import torch
    import microscaling_fp4_attention_amd as mx
    qf_, vf_ = FMT[pm]
    qf_ = qfmt or qf_
    pf_ = None if pm == "fp8" else qf_
    q, k, v = _bf16((B, Hq, R, 128), seed, 1), _bf16((B, Hkv, N, 128), seed, 2, 0.3), _bf16((B, Hkv, N, 128), seed, 3)
    dev = "cuda:0"
    t = {n: torch.from_numpy(a.astype(np.int16)).view(torch.bfloat16).to(dev) for n, a in (("q", q), ("k", k), ("v", v))}
    Q = mx.quantize(t["q"], mx.ROLE_QK, qf_)
    K = mx.quantize(t["k"], mx.ROLE_QK, qf_)
    V = mx.quantize(t["v"], mx.ROLE_V, vf_)
    kl = None if kv_len is None else torch.tensor(kv_len, dtype=torch.int32, device=dev)
    lse = torch.empty((B, Hq, R), dtype=torch.float32, device=dev)
    out = mx.decode(Q, K, V, mx.fwd_params(pm, pf_, causal=True, out_fp32=True), kv_len=kl, lse=lse)
    torch.cuda.synchronize()
    qc, qs, qd = oracle_quant_qk(synth.bf16_to_f32(q), qf_)
    kc, ks, kd = oracle_quant_qk(synth.bf16_to_f32(k), qf_)
    vc, vs, vd = oracle_quant_v(synth.bf16_to_f32(v), vf_)
    assert np.array_equal(gpu_codes_qk(Q), qc) and np.array_equal(gpu_codes_qk(K), kc)
    gc, gs = gpu_codes_v(V, N, None)
    assert np.array_equal(gc, vc) and np.array_equal(gs, vs)
    kvl = np.full(B, N, np.int32) if kv_len is None else np.asarray(kv_len, np.int32)
    O_ref, lse_ref, fb = oracle.decode(qd, kd, vd, kvl, PM_ORACLE[pm], pf_, split=256, score_rounds=score_rounds(qf_))
    O_gpu = out.cpu().numpy()
    bound = TOL * np.abs(O_ref).max() + fb[..., None]
    ratio = float((np.abs(O_gpu - O_ref) / bound).max())
    lse_err = float(np.abs(lse.cpu().numpy() - lse_ref).max())
    print(f"decode {pm} {qf_} B{B} Hq{Hq} Hkv{Hkv} R{R} N{N}: max |dO|/bound {ratio:.3f}, |dlse| {lse_err:.2e}")
    record_parity(f"decode {pm} {qf_} B{B} Hq{Hq} Hkv{Hkv} R{R} N{N}", ratio, fb / (TOL * np.abs(O_ref).max()),
                  None if N > 4096 else cap)
    assert np.all(np.isfinite(O_gpu))
    assert ratio <= 1.0
    assert lse_err <= 1e-3 * max(1.0, float(np.abs(lse_ref).max()))


@pytest.mark.parametrize("pm", ["direct", "pnq", "two_level"])
def test_decode_ragged(pm):
    run_decode(pm, B=2, Hq=8, Hkv=2, R=1, N=700, kv_len=[700, 333], seed=61)


@pytest.mark.parametrize("R", [4, 8])
def test_decode_several_rows(R):
    """R newest rows per request with a causal mask among them; 4 x 8 fills all 32 columns"""
    run_decode("pnq", B=1, Hq=4, Hkv=1, R=R, N=1300, kv_len=None, seed=62)


@pytest.mark.parametrize("pm", ["direct", "pnq", "two_level"])
@pytest.mark.parametrize("Hq,Hkv,R", [(8, 1, 3), (17, 1, 1), (16, 2, 2), (4, 1, 4)])
def test_decode_column_forms(pm, Hq, Hkv, R):
    """24 and 17 packed columns (the 32-column kernel) and 16 (the 16-column kernel at
    its limit), over a ragged history"""
    run_decode(pm, B=2, Hq=Hq, Hkv=Hkv, R=R, N=1100, kv_len=[1100, 517], seed=66)


@pytest.mark.parametrize("qf", ["nvfp4", "mxfp4"])
@pytest.mark.parametrize("Hq,Hkv,R,N,kv_len", [(8, 2, 1, 700, [700, 333]), (8, 1, 3, 1100, [1100, 517]),
                                               (4, 1, 8, 1300, None), (2, 2, 2, 260, [2, 257]),
                                               (16, 1, 1, 900, [900, 450])])
def test_decode_qk4pv8(qf, Hq, Hkv, R, N, kv_len):
    """The QK4PV8 route ("MpFA", sections 4.1 and 5.3): NVFP4 (or MXFP4) Q/K, an FP8 V,
    P = E4M3(448 P~): ragged histories, several newest rows, up to 32 packed columns
    (16 at most on the 16-column kernel, which the 2-, 4- and 16-column cases take)"""
    run_decode("fp8", B=2 if kv_len is not None and len(kv_len) == 2 else 1, Hq=Hq, Hkv=Hkv, R=R, N=N, kv_len=kv_len,
               seed=71, qfmt=qf)


def test_decode_minimal_history():
    run_decode("direct", B=3, Hq=2, Hkv=2, R=2, N=260, kv_len=[2, 130, 257], seed=63)


@pytest.mark.parametrize("N,kv_len", [(40, [40, 3]), (97, [97, 64]), (129, [129, 128])])
def test_decode_short_histories(N, kv_len):
    """histories shorter than a tile or a split (the last tile partly past N: its K rows
    repeat row N - 1 and its keys are masked)"""
    run_decode("two_level", B=2, Hq=4, Hkv=2, R=1, N=N, kv_len=kv_len, seed=65)


def test_decode_gqa_32_8_long():
    run_decode("two_level", B=1, Hq=32, Hkv=8, R=1, N=32768, kv_len=None, seed=64)


def test_decode_qk4pv8_gqa_32_8_long():
    run_decode("fp8", B=1, Hq=32, Hkv=8, R=1, N=32768, kv_len=None, seed=67)


@pytest.mark.parametrize("pm,B,Hq,Hkv,R,N,kv_len", [("direct", 2, 8, 2, 1, 700, [700, 333]),
                                                      ("pnq", 1, 4, 1, 8, 1300, None),
                                                      ("two_level", 2, 4, 2, 1, 129, [129, 128]),
                                                      ("two_level", 1, 32, 8, 1, 32768, None),
                                                      ("two_level", 2, 8, 1, 3, 1100, [1100, 517]),
                                                      ("fp8", 2, 8, 2, 1, 700, [700, 333]),
                                                      ("fp8", 1, 32, 8, 1, 32768, None),
                                                      ("fp8", 2, 8, 1, 3, 1100, [1100, 517])])
def test_decode_vt_equals_v(pm, B, Hq, Hkv, R, N, kv_len):
    """The decode over role VT (V tile-major) gives exactly the decode over role V, and
    role VT holds role V's bytes moved tile by tile."""
    import torch
    import microscaling_fp4_attention_amd as mx
    qf_, vf_ = FMT[pm]
    pf_ = None if pm == "fp8" else qf_
    q, k, v = _bf16((B, Hq, R, 128), 71, 1), _bf16((B, Hkv, N, 128), 71, 2, 0.3), _bf16((B, Hkv, N, 128), 71, 3)
    dev = "cuda:0"
    t = {n: torch.from_numpy(a.astype(np.int16)).view(torch.bfloat16).to(dev) for n, a in (("q", q), ("k", k), ("v", v))}
    Q, K = mx.quantize(t["q"], mx.ROLE_QK, qf_), mx.quantize(t["k"], mx.ROLE_QK, qf_)
    kl = None if kv_len is None else torch.tensor(kv_len, dtype=torch.int32, device=dev)
    p = mx.fwd_params(pm, pf_, causal=True, out_fp32=True)
    res, vq = [], []
    for role in (mx.ROLE_V, mx.ROLE_VT):
        lse = torch.empty((B, Hq, R), dtype=torch.float32, device=dev)
        V = mx.quantize(t["v"], role, vf_)
        out = mx.decode(Q, K, V, p, kv_len=kl, lse=lse)
        res.append((out, lse))
        vq.append(V)
    torch.cuda.synchronize()
    assert torch.equal(res[0][0], res[1][0]) and torch.equal(res[0][1], res[1][1])
    cv, ct = vq[0].codes_view(), vq[1].codes_view()  # [B,H,d,np*b/8] and [B,H,np/128,d,128*b/8]
    nt = ct.shape[2]
    assert torch.equal(cv.reshape(B, Hkv, 128, nt, -1).permute(0, 1, 3, 2, 4), ct)
    sv, st = vq[0].scales_view(), vq[1].scales_view()
    assert torch.equal(sv.reshape(B, Hkv, 128, nt, 4).permute(0, 1, 3, 2, 4), st)


@pytest.mark.parametrize("pm", ["two_level", "fp8"])
def test_decode_bench_size(pm):
    """The decode in the shape bench.py times: 4 requests, GQA 32:8, one new token each
    over 131072 keys (256 chunk states per row to merge), V tile-major (role VT).  The
    four requests hold one history and one query, so request 0 is checked against the
    oracle and the others must equal it bit for bit."""
    import torch
    import microscaling_fp4_attention_amd as mx
    B, Hq, Hkv, N = 4, 32, 8, 131072
    qf_, vf_ = FMT[pm]
    pf_ = None if pm == "fp8" else qf_
    q, k, v = _bf16((1, Hq, 1, 128), 68, 1), _bf16((1, Hkv, N, 128), 68, 2, 0.3), _bf16((1, Hkv, N, 128), 68, 3)
    dev = "cuda:0"
    t = {n: torch.from_numpy(a.astype(np.int16)).view(torch.bfloat16).to(dev).repeat(B, 1, 1, 1)
         for n, a in (("q", q), ("k", k), ("v", v))}
    Q, K = mx.quantize(t["q"], mx.ROLE_QK, qf_), mx.quantize(t["k"], mx.ROLE_QK, qf_)
    V = mx.quantize(t["v"], mx.ROLE_VT, vf_)
    lse = torch.empty((B, Hq, 1), dtype=torch.float32, device=dev)
    out = mx.decode(Q, K, V, mx.fwd_params(pm, pf_, causal=True, out_fp32=True), lse=lse)
    torch.cuda.synchronize()
    assert all(torch.equal(out[b], out[0]) and torch.equal(lse[b], lse[0]) for b in range(1, B))
    qc, qs, qd = oracle_quant_qk(synth.bf16_to_f32(q), qf_)
    kc, ks, kd = oracle_quant_qk(synth.bf16_to_f32(k), qf_)
    vc, vs, vd = oracle_quant_v(synth.bf16_to_f32(v), vf_)
    assert np.array_equal(gpu_codes_qk(Q)[:1], qc) and np.array_equal(gpu_codes_qk(K)[:1], kc)
    # role VT [B, H, tile, d, 128 keys] holds role V's channel rows [B, H, d, keys] tile by tile
    ct, st = V.codes_view()[:1], V.scales_view()[:1]
    gc = ct.permute(0, 1, 3, 2, 4).reshape(1, Hkv, 128, -1).cpu().numpy()
    gs = st.permute(0, 1, 3, 2, 4).reshape(1, Hkv, 128, -1).cpu().numpy()
    if V.desc.fmt.elem == 0:
        gc = unpack_nibbles(gc)
    assert np.array_equal(gc[..., :N], vc) and np.array_equal(gs[..., :vs.shape[-1]], vs)
    O_ref, lse_ref, fb = oracle.decode(qd, kd, vd, np.array([N], np.int32), PM_ORACLE[pm], pf_, split=256,
                                       score_rounds=score_rounds(qf_))
    O_gpu = out[:1].cpu().numpy()
    bound = TOL * np.abs(O_ref).max() + fb[..., None]
    ratio = float((np.abs(O_gpu - O_ref) / bound).max())
    lse_err = float(np.abs(lse[:1].cpu().numpy() - lse_ref).max())
    name = f"decode {pm} {qf_} B{B} Hq{Hq} Hkv{Hkv} R1 N{N} VT"
    print(f"{name}: max |dO|/bound {ratio:.3f}, |dlse| {lse_err:.2e}")
    record_parity(name, ratio, fb / (TOL * np.abs(O_ref).max()), None)
    assert np.all(np.isfinite(O_gpu))
    assert ratio <= 1.0
    assert lse_err <= 1e-3 * max(1.0, float(np.abs(lse_ref).max()))


def test_decode_refused():
    import torch
    import microscaling_fp4_attention_amd as mx
    dev = "cuda:0"
    q = torch.from_numpy(_bf16((1, 8, 5, 128), 65, 1).astype(np.int16)).view(torch.bfloat16).to(dev)
    k = torch.from_numpy(_bf16((1, 1, 300, 128), 65, 2).astype(np.int16)).view(torch.bfloat16).to(dev)
    Q = mx.quantize(q, mx.ROLE_QK, "mxfp4")
    K = mx.quantize(k, mx.ROLE_QK, "mxfp4")
    V = mx.quantize(k, mx.ROLE_V, "mxfp4")
    with pytest.raises(mx.MxattnError) as e:  # 8 heads x 5 rows > 32 columns
        mx.decode(Q, K, V, mx.fwd_params("direct", "mxfp4", causal=True))
    assert e.value.status == -2
    Q1 = mx.quantize(q[:, :1], mx.ROLE_QK, "mxfp4")
    with pytest.raises(mx.MxattnError):  # decode rows are the newest tokens: causal only
        mx.decode(Q1, K, V, mx.fwd_params("direct", "mxfp4", causal=False))
    with pytest.raises(mx.MxattnError) as e:  # FP8 P takes an FP8 V
        mx.decode(Q1, K, V, mx.fwd_params("fp8", None, causal=True))
    assert e.value.status == -2
    with pytest.raises(mx.MxattnError) as e:  # FP8 P takes an FP8 V in the tile-major form too
        mx.decode(Q1, K, mx.quantize(k, mx.ROLE_VT, "mxfp4"), mx.fwd_params("fp8", None, causal=True))
    assert e.value.status == -2
    torch.cuda.synchronize()
