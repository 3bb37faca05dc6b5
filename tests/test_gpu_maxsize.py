"""Parity near the largest sequence the forward accepts: the kernels address one head's
K and V with 32-bit offsets, so N and the padded V length must stay at or below 2^24
(an FP8 V row is n_padded bytes: 127 rows reach 2.1e9 bytes, above 2^31).  Here B=1,
two query heads over one KV head, 16651776 packed tokens in 4045 documents
(block-diagonal causal), a total chosen so that the padded V length (each document's
V blocks start at its first token) is exactly 2^24, the largest accepted; every tensor
is several GB.  Inputs are seeded blocks of 8191 tokens repeated along the sequence:
8191 shares no factor with a power of two, so reading at an offset wrong by any
power-of-two stride yields different data.  The oracle computes sampled rows of the
first, a middle and the last documents, each as a sequence of its own (the packed
forward's document-local tiles and V blocks make that the same computation).
FP32 output: |dO| <= 2e-3 max|O| + flip budget."""
import numpy as np
import pytest

import oracle
import synth
from helpers import PM_ORACLE, TOL, gpu_available, oracle_quant_qk, oracle_quant_v, record_parity, score_rounds

pytestmark = [pytest.mark.gpu, pytest.mark.skipif(not gpu_available(), reason="needs a GPU")]

PERIOD = 8191
N_TOTAL = 16651776  # padded V length exactly 2^24 for the documents below
ROUTES = {  # (Q/K format, V format, P mode, P format)
    "mxfp4_uos_pnq": ("mxfp4_uos", "mxfp4_uos", "pnq", "mxfp4_uos"),
    "qk4pv8": ("nvfp4", "fp8v", "fp8", None),
}


def _documents(rng):
    lens = []
    while sum(lens) < N_TOTAL:
        lens.append(int(rng.integers(2048, 6145)))
    lens[-1] -= sum(lens) - N_TOTAL
    if lens[-1] < 1:
        lens[-2] += lens[-1] - 1
        lens[-1] = 1
    return np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)


@pytest.mark.parametrize("route", list(ROUTES))
def test_fwd_near_max_length(route):
    import torch
    import microscaling_fp4_attention_amd as mx
    qf, vf, pm, pf = ROUTES[route]
    Hq, Hkv = 2, 1
    rng = np.random.default_rng(2024)
    doc_off = _documents(rng)
    ndocs = len(doc_off) - 1
    base = {"q": synth.f32_to_bf16(synth.gaussian(9, 1, (Hq, PERIOD, 128))),
            "k": synth.f32_to_bf16(synth.gaussian(9, 2, (Hkv, PERIOD, 128))),
            "v": synth.f32_to_bf16(synth.gaussian(9, 3, (Hkv, PERIOD, 128)))}
    dev = "cuda:0"
    reps = (N_TOTAL + PERIOD - 1) // PERIOD
    t = {}
    for n, a in base.items():
        b = torch.from_numpy(a.astype(np.int16)).view(torch.bfloat16).to(dev)
        t[n] = b.repeat(1, reps, 1)[:, :N_TOTAL].unsqueeze(0).contiguous()  # [1, H, N, 128]
    cu = torch.from_numpy(doc_off.astype(np.int32)).to(dev)
    Q = mx.quantize(t["q"], mx.ROLE_QK, qf)
    K = mx.quantize(t["k"], mx.ROLE_QK, qf)
    V = mx.quantize(t["v"], mx.ROLE_V, vf, cu_seqlens=cu)
    del t
    assert V.n_padded == 1 << 24
    ws = mx.fwd_plan(doc_off, N_TOTAL, True)
    out = mx.fwd(Q, K, V, mx.fwd_params(pm, pf, causal=True, out_fp32=True), workspace=ws, ndocs=ndocs)
    torch.cuda.synchronize()

    worst, fbt = 0.0, []
    for d in (0, ndocs // 2, ndocs - 2, ndocs - 1):
        s, L = int(doc_off[d]), int(doc_off[d + 1] - doc_off[d])
        idx = (s + np.arange(L)) % PERIOD
        rows = sorted({0, L - 1} | {int(r) for r in rng.integers(0, L, 24)})
        kh = synth.bf16_to_f32(base["k"][:, idx])[None]  # [1, 1, L, 128]
        vh = synth.bf16_to_f32(base["v"][:, idx])[None]
        _, _, kd = oracle_quant_qk(kh, qf)
        _, _, vd = oracle_quant_v(vh, vf)
        for h in range(Hq):
            qh = synth.bf16_to_f32(base["q"][h:h + 1, idx])[None]
            _, _, qd = oracle_quant_qk(qh, qf)
            O_ref, _, fb = oracle.attention(qd, kd, vd, PM_ORACLE[pm], pf, causal=True, rows=np.array(rows, np.int64),
                                            score_rounds=score_rounds(qf))
            O_gpu = out[0, h, s:s + L].cpu().numpy()[rows]
            assert np.all(np.isfinite(O_gpu))
            bound = TOL * np.abs(O_ref).max() + fb[:, None]
            ratio = float((np.abs(O_gpu - O_ref) / bound).max())
            worst = max(worst, ratio)
            fbt.append(fb / (TOL * np.abs(O_ref).max()))
            assert ratio <= 1.0, (route, d, h, ratio)
    print(f"{route}: {ndocs} documents, n_padded {V.n_padded}, worst |dO| / bound = {worst:.3f}")
    record_parity(f"largest size {route}", worst, np.concatenate(fbt), None)
