"""GPU causally safe V scales ("FLAMIA ...", section 3.2) against the oracle: the
per-key form of V (bytes bit-exact, with and without documents), the forward with the
per-key fold on each row's diagonal tiles (the key tiles inside its 256-row query tile)
for every 4-bit-V route of the ping-pong kernel (parity), a channel small enough to
split the f16 shift between the bf16 operands, a leak probe (future keys leave earlier
rows bit-identical), and the refused combinations."""
import numpy as np
import pytest

import synth
from helpers import TOL, gpu_available, record_parity, run_case

pytestmark = [pytest.mark.gpu, pytest.mark.skipif(not gpu_available(), reason="needs a GPU")]

# (Q/K format, V format, P mode, P format)
SAFE_ROUTES = {
    "mxfp4_direct": ("mxfp4", "mxfp4", "direct", "mxfp4"),
    "mxfp4_uos_pnq": ("mxfp4_uos", "mxfp4_uos", "pnq", "mxfp4_uos"),
    "mxfp4_two_level_e8m0": ("mxfp4", "mxfp4", "two_level", "mxfp4"),
    "mxfp4_two_level_e4m3": ("mxfp4", "mxfp4", "two_level", "nvfp4"),
    "mxfp4_pnq_e4m3p": ("mxfp4", "mxfp4", "pnq", "nvfp4"),
}


def _check(res, name):
    print(f"{name}: max err/bound {res['ratio']:.3f}, fragile rows {res['n_fragile']}, amax {res['amax']:.3f}")
    record_parity(name, res["ratio"], res["fb"] / (TOL * res["amax"]))
    assert np.all(np.isfinite(res["O_gpu"]))
    assert res["ratio"] <= 1.0, name


@pytest.mark.parametrize("route", list(SAFE_ROUTES))
def test_fwd_causal_safe(route):
    q, v, pm, pf = SAFE_ROUTES[route]
    res = run_case(q, v, pm, pf, B=2, Hq=4, Hkv=2, N=600, causal=True, kind="outlier", seed=41, safe=True)
    _check(res, route + " causal safe")


@pytest.mark.parametrize("route", ["mxfp4_uos_pnq", "mxfp4_two_level_e4m3"])
def test_fwd_causal_safe_documents(route):
    q, v, pm, pf = SAFE_ROUTES[route]
    doc_off = np.array([0, 100, 101, 357, 490, 700], np.int32)
    res = run_case(q, v, pm, pf, B=1, Hq=2, Hkv=2, N=700, causal=True, kind="outlier", seed=42, doc_off=doc_off,
                   safe=True)
    _check(res, route + " causal safe docs")


def test_fwd_causal_safe_with_centering():
    res = run_case("mxfp4", "mxfp4", "two_level", "nvfp4", B=1, Hq=2, Hkv=1, N=520, causal=True, kind="kmean",
                   seed=43, safe=True, pre={"center": True})
    _check(res, "causal safe + centering")


@pytest.mark.parametrize("route", ["mxfp4_two_level_e4m3", "mxfp4_pnq_e4m3p"])
def test_fwd_causal_safe_tiny_channel(route):
    """One V channel 2^-118 times the others: its f16 shift exceeds 125, so the per-key
    tiles' bf16 products split the shift between the two operands (V 2^(vshift - sigma),
    P^' 2^sigma with sigma > 0).  A sigma missing on either side would scale every
    channel's diagonal-tile contribution by 2^sigma."""
    q, v, pm, pf = SAFE_ROUTES[route]
    x = synth.make_inputs("outlier", 1, 2, 2, 600, 128, 46)
    vf = synth.bf16_to_f32(x["v"])
    vf[..., 7] *= 2.0 ** -118
    assert np.abs(vf[..., 7]).max() < 2.0 ** -110  # largest E8M0 block exponent below -112
    x = dict(x, v=synth.f32_to_bf16(vf))
    res = run_case(q, v, pm, pf, 1, 2, 2, 600, causal=True, inputs=x, safe=True)
    _check(res, route + " causal safe tiny channel")


@pytest.mark.parametrize("route", ["mxfp4_direct", "mxfp4_two_level_e4m3"])
def test_leak_probe(route):
    """Scaling the values of keys >= 200 (inside the V block of keys 192..223) changes
    rows 192..199 through the grouped V scales; with the per-key form on the diagonal
    tiles every row before 200 is bit-identical."""
    q, v, pm, pf = SAFE_ROUTES[route]
    x = synth.make_inputs("outlier", 1, 2, 2, 700, 128, 44)
    x2 = dict(x)
    vf = synth.bf16_to_f32(x["v"])
    vf[:, :, 200:, :] *= 50.0
    x2["v"] = synth.f32_to_bf16(vf)
    out = {}
    for safe in (False, True):
        a = run_case(q, v, pm, pf, 1, 2, 2, 700, causal=True, inputs=x, check_bytes=False, safe=safe)["O_gpu_all"]
        b = run_case(q, v, pm, pf, 1, 2, 2, 700, causal=True, inputs=x2, check_bytes=False, safe=safe)["O_gpu_all"]
        rows = np.concatenate([h * 700 + np.arange(200) for h in range(2)])
        out[safe] = np.array_equal(a[rows], b[rows])
    assert not out[False], "expected the grouped V scales to leak"
    assert out[True], "rows before the perturbed keys changed with the per-key form"


def test_refused_combinations():
    import torch
    import microscaling_fp4_attention_amd as mx
    x = synth.make_inputs("kmean", 1, 2, 2, 256, 128, 45)
    dev = "cuda:0"
    t = {n: torch.from_numpy(x[n].astype(np.int16)).view(torch.bfloat16).to(dev) for n in "qkv"}
    V = mx.quantize(t["v"], mx.ROLE_V, "mxfp4")
    Vk = mx.quantize(t["v"], mx.ROLE_VKEY, "mxfp4")
    Q = mx.quantize(t["q"], mx.ROLE_QK, "mxfp4")
    K = mx.quantize(t["k"], mx.ROLE_QK, "mxfp4")
    with pytest.raises(mx.MxattnError):  # needs a causal mask
        mx.fwd(Q, K, V, mx.fwd_params("direct", "mxfp4", causal=False, vkey=Vk))
    Qn = mx.quantize(t["q"], mx.ROLE_QK, "nvfp4")
    Kn = mx.quantize(t["k"], mx.ROLE_QK, "nvfp4")
    with pytest.raises(mx.MxattnError) as e:  # NVFP4 Q/K with MXFP4 V runs on the 4-wave kernel
        mx.fwd(Qn, Kn, V, mx.fwd_params("direct", "mxfp4", causal=True, vkey=Vk))
    assert e.value.status == -2
    V8 = mx.quantize(t["v"], mx.ROLE_V, "fp8v")
    with pytest.raises(mx.MxattnError):  # an FP8 V takes round-up exponents, not a per-key form
        mx.fwd(Qn, Kn, V8, mx.fwd_params("fp8", None, causal=True, vkey=Vk))
    torch.cuda.synchronize()
