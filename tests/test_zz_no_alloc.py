"""The allocation-free decode (mxattn_decode_noalloc) against mxattn_decode, through
the C ABI: the same kernels on the library's static scratch instead of a caller
workspace, so the outputs and log-sum-exps must be equal bit for bit.  Two calls in
a row, the second smaller (the scratch keeps the first call's contents), and a call
beyond the scratch's limit, which must be refused with the sizes in the error text."""
import numpy as np
import pytest

import synth
from helpers import gpu_available

pytestmark = [pytest.mark.gpu, pytest.mark.skipif(not gpu_available(), reason="needs a GPU")]


def _case(mx, torch, B, Hq, Hkv, R, N, kv_len, pm, seed):
    dev = "cuda:0"

    def bf(shape, k):
        a = synth.f32_to_bf16(synth.gaussian(seed, k, shape).astype(np.float32))
        return torch.from_numpy(a.astype(np.int16)).view(torch.bfloat16).to(dev)

    qkf, vf, pf = ("nvfp4", "fp8v", None) if pm == "fp8" else ("mxfp4", "mxfp4", "mxfp4")  # fp8: QK4PV8
    Q = mx.quantize(bf((B, Hq, R, 128), 1), mx.ROLE_QK, qkf)
    K = mx.quantize(bf((B, Hkv, N, 128), 2), mx.ROLE_QK, qkf)
    V = mx.quantize(bf((B, Hkv, N, 128), 3), mx.ROLE_VT, vf)
    kl = torch.tensor(kv_len, dtype=torch.int32, device=dev)
    p = mx.fwd_params(pm, pf, causal=True, out_fp32=True)
    return Q, K, V, kl, p


@pytest.mark.parametrize("pm", ["pnq", "two_level", "fp8"])
def test_decode_noalloc_equals_decode(pm):
    import torch
    import microscaling_fp4_attention_amd as mx
    # first a large call (GQA 32:8, 4 requests over up to 40K keys), then a smaller one
    for (B, Hq, Hkv, R, N, kv_len, seed) in [(4, 32, 8, 1, 40000, [40000, 12345, 39999, 700], 1),
                                              (2, 8, 2, 3, 3000, [3000, 1500], 2)]:
        Q, K, V, kl, p = _case(mx, torch, B, Hq, Hkv, R, N, kv_len, pm, seed)
        lse_a = torch.empty((B, Hq, R), dtype=torch.float32, device="cuda:0")
        lse_b = torch.empty_like(lse_a)
        out_a = mx.decode(Q, K, V, p, kv_len=kl, lse=lse_a)
        out_b = mx.decode_noalloc(Q, K, V, p, kv_len=kl, lse=lse_b)
        torch.cuda.synchronize()
        print(f"decode_noalloc {pm} B{B} Hq{Hq} R{R} N{N}: max |a - b| "
              f"{float((out_a - out_b).abs().max()):.3e}")
        assert torch.equal(out_a, out_b)
        assert torch.equal(lse_a, lse_b)
        assert bool(torch.isfinite(out_b).all())


def test_decode_noalloc_refuses_beyond_the_scratch():
    import torch
    import microscaling_fp4_attention_amd as mx
    B, Hq, Hkv, R = 4, 32, 8, 1
    N = 512 * 509  # 4 * 32 * 509 = 65152 split rows > 65027
    assert mx.decode_workspace_bytes(B, Hq, R, N) > mx.DECODE_SCRATCH_BYTES
    assert mx.decode_workspace_bytes(B, Hq, R, 512 * 508) <= mx.DECODE_SCRATCH_BYTES
    # descriptors only: the call is refused before any device work
    Q = mx.quantize(torch.zeros((B, Hq, R, 128), dtype=torch.bfloat16, device="cuda:0"), mx.ROLE_QK, "mxfp4")
    K = mx.quantize(torch.zeros((B, Hkv, 128, 128), dtype=torch.bfloat16, device="cuda:0"), mx.ROLE_QK, "mxfp4")
    V = mx.quantize(torch.zeros((B, Hkv, 128, 128), dtype=torch.bfloat16, device="cuda:0"), mx.ROLE_VT, "mxfp4")
    K.desc.N = V.desc.N = N
    V.desc.n_padded = N
    with pytest.raises(mx.MxattnError) as ei:
        mx.decode_noalloc(Q, K, V, mx.fwd_params("pnq", "mxfp4", causal=True))
    assert ei.value.status == mx.E_WORKSPACE
    assert "static scratch" in str(ei.value)
