"""GPU forward (mxattn_fwd) against the oracle, element by element in FP32:
|dO| <= 2e-3 * max|O_oracle| + the row's flip budget.  Shapes span several key
tiles with a ragged tail; the cases cover every operand route, causal masks,
grouped-query heads and packed documents."""
import numpy as np
import pytest

import synth
from helpers import TOL, gpu_available, record_parity, run_case

pytestmark = [pytest.mark.gpu, pytest.mark.skipif(not gpu_available(), reason="needs a GPU")]

# (Q/K format, V format, P mode, P format)
ROUTES = {
    "mxfp4_direct": ("mxfp4", "mxfp4", "direct", "mxfp4"),
    "mxfp4_uos_pnq": ("mxfp4_uos", "mxfp4_uos", "pnq", "mxfp4_uos"),
    "mxfp4_two_level_e8m0": ("mxfp4", "mxfp4", "two_level", "mxfp4"),
    "mxfp4_two_level_e4m3": ("mxfp4", "mxfp4", "two_level", "nvfp4"),
    "mxfp4_direct_e4m3p": ("mxfp4", "mxfp4", "direct", "nvfp4"),
    "nvfp4_direct": ("nvfp4", "nvfp4", "direct", "nvfp4"),
    "nvfp4_two_level": ("nvfp4", "nvfp4", "two_level", "nvfp4"),
    "nvfp4_pnq": ("nvfp4", "nvfp4", "pnq", "nvfp4"),
    "nvfp4_qk_mxfp4_pv": ("nvfp4", "mxfp4", "pnq", "mxfp4"),
    "qk4pv8": ("nvfp4", "fp8v", "fp8", None),
    "mxfp4_qk_pv8": ("mxfp4", "fp8v", "fp8", None),
}


def _check(res, name):
    print(f"{name}: max err/bound {res['ratio']:.3f}, fragile rows {res['n_fragile']}, amax {res['amax']:.3f}")
    assert np.all(np.isfinite(res["O_gpu"]))
    record_parity(name, res["ratio"], res["fb"] / (TOL * res["amax"]))
    assert res["ratio"] <= 1.0, name


@pytest.mark.parametrize("route", list(ROUTES))
def test_fwd_route_noncausal(route):
    q, v, pm, pf = ROUTES[route]
    res = run_case(q, v, pm, pf, B=1, Hq=2, Hkv=2, N=300, kind="kmean")
    _check(res, route)


@pytest.mark.parametrize("route", ["mxfp4_direct", "mxfp4_uos_pnq", "mxfp4_two_level_e4m3", "nvfp4_two_level",
                                   "qk4pv8"])
def test_fwd_causal_gqa(route):
    q, v, pm, pf = ROUTES[route]
    res = run_case(q, v, pm, pf, B=2, Hq=4, Hkv=2, N=257, causal=True, kind="kmean", seed=3)
    _check(res, route + " causal gqa")
    lse_ok = np.abs(res["lse_gpu"] - res["lse_ref"]) <= 1e-3 * np.maximum(1.0, np.abs(res["lse_ref"]))
    assert lse_ok.all()


@pytest.mark.parametrize("route", ["mxfp4_uos_pnq", "mxfp4_two_level_e4m3", "mxfp4_two_level_e8m0", "qk4pv8"])
@pytest.mark.parametrize("causal", [False, True])
def test_fwd_packed_documents(route, causal):
    q, v, pm, pf = ROUTES[route]
    doc_off = np.array([0, 100, 101, 357, 490, 700], np.int32)  # includes a 1-token document
    res = run_case(q, v, pm, pf, B=1, Hq=2, Hkv=2, N=700, causal=causal, kind="outlier", seed=4, doc_off=doc_off)
    _check(res, route + f" docs causal={causal}")


def test_fwd_config1_all_rows():
    """Single head, N = 1024, K with a per-channel mean: the four direct/two-level
    modes of the smallest configuration, every row."""
    x = synth.workload("c1_single_head")
    for qf, pm in [("nvfp4", "direct"), ("nvfp4", "two_level"), ("mxfp4", "direct"), ("mxfp4", "two_level")]:
        res = run_case(qf, qf, pm, "nvfp4" if pm == "two_level" else qf, B=1, Hq=1, Hkv=1, N=1024, inputs=x)
        _check(res, f"c1 {qf} {pm}")


def test_fwd_small_and_degenerate_shapes():
    # one token, one tile exactly, and a tail of one key
    for N in (1, 128, 129):
        res = run_case("mxfp4_uos", "mxfp4_uos", "pnq", "mxfp4_uos", B=1, Hq=1, Hkv=1, N=N, kind="plain", seed=5)
        _check(res, f"N={N}")


@pytest.mark.parametrize("case", [("mxfp4_two_level_e4m3", False), ("mxfp4_two_level_e4m3", True),
                                  ("qk4pv8", False), ("mxfp4_uos_pnq", True)])
def test_fwd_boundary_lengths(case):
    """Causal lengths at the edges of the 128-key tiles and of the 256-row query tiles
    (the causally safe form folds on a query tile's two key tiles, the second of which
    may be partial or absent)"""
    route, safe = case
    q, v, pm, pf = ROUTES[route]
    for N in (1, 2, 127, 128, 129, 255, 256, 257):
        res = run_case(q, v, pm, pf, B=1, Hq=2, Hkv=1, N=N, causal=True, kind="outlier", seed=6, safe=safe)
        _check(res, f"{route}{' safe' if safe else ''} causal N={N}")


def test_fwd_deterministic():
    import torch
    import microscaling_fp4_attention_amd as mx
    x = synth.make_inputs("lowrank", 1, 2, 2, 700, 128, 6)
    dev = "cuda:0"
    t = {n: torch.from_numpy(x[n].astype(np.int16)).view(torch.bfloat16).to(dev) for n in "qkv"}
    outs = []
    for _ in range(2):
        Q = mx.quantize(t["q"], mx.ROLE_QK, "mxfp4_uos")
        K = mx.quantize(t["k"], mx.ROLE_QK, "mxfp4_uos")
        V = mx.quantize(t["v"], mx.ROLE_V, "mxfp4_uos")
        outs.append(mx.fwd(Q, K, V, mx.fwd_params("pnq", "mxfp4_uos")).cpu())
    assert torch.equal(outs[0], outs[1])


def test_fwd_pnq_rows_sum_to_one():
    """PNQ (MXAttention Proposition 1): with V = 1 (MXFP4 encodes 1 exactly) every
    output entry is 1 up to FP32 rounding, whatever the scores."""
    import torch
    import microscaling_fp4_attention_amd as mx
    x = synth.make_inputs("lowrank", 1, 2, 2, 400, 128, 8)
    dev = "cuda:0"
    q = torch.from_numpy(x["q"].astype(np.int16)).view(torch.bfloat16).to(dev)
    k = torch.from_numpy(x["k"].astype(np.int16)).view(torch.bfloat16).to(dev)
    v = torch.ones((1, 2, 400, 128), dtype=torch.bfloat16, device=dev)
    Q = mx.quantize(q, mx.ROLE_QK, "mxfp4_uos")
    K = mx.quantize(k, mx.ROLE_QK, "mxfp4_uos")
    V = mx.quantize(v, mx.ROLE_V, "mxfp4_uos")
    o = mx.fwd(Q, K, V, mx.fwd_params("pnq", "mxfp4_uos")).cpu().numpy()
    assert np.abs(o - 1.0).max() <= 1e-5


def test_fwd_bf16_output_matches_fp32():
    import torch
    import microscaling_fp4_attention_amd as mx
    x = synth.make_inputs("kmean", 1, 2, 2, 300, 128, 9)
    dev = "cuda:0"
    t = {n: torch.from_numpy(x[n].astype(np.int16)).view(torch.bfloat16).to(dev) for n in "qkv"}
    Q = mx.quantize(t["q"], mx.ROLE_QK, "mxfp4")
    K = mx.quantize(t["k"], mx.ROLE_QK, "mxfp4")
    V = mx.quantize(t["v"], mx.ROLE_V, "mxfp4")
    o32 = mx.fwd(Q, K, V, mx.fwd_params("direct", "mxfp4", out_fp32=True))
    o16 = mx.fwd(Q, K, V, mx.fwd_params("direct", "mxfp4", out_fp32=False))
    assert torch.equal(o32.to(torch.bfloat16), o16)


@pytest.mark.parametrize("route", ["mxfp4_uos_pnq", "qk4pv8", "nvfp4_two_level"])
@pytest.mark.parametrize("causal", [False, True])
def test_fwd_empty_documents(route, causal):
    """packed documents with empty ones in the middle and at the end (repeated offsets):
    the empty documents own no rows, no work items and no V blocks"""
    q, v, pm, pf = ROUTES[route]
    doc_off = np.array([0, 100, 100, 357, 357, 700, 700], np.int32)
    res = run_case(q, v, pm, pf, B=1, Hq=2, Hkv=1, N=700, causal=causal, kind="outlier", seed=9, doc_off=doc_off)
    _check(res, route + f" empty docs causal={causal}")


def _scaled_v(x, scale_of_channel):
    """inputs x with V's channel c multiplied by scale_of_channel[c] (powers of two: exact)"""
    v = synth.bf16_to_f32(x["v"]) * np.asarray(scale_of_channel, np.float32)
    y = dict(x)
    y["v"] = synth.f32_to_bf16(v)
    return y


@pytest.mark.parametrize("route", ["mxfp4_two_level_e4m3", "mxfp4_direct_e4m3p"])
@pytest.mark.parametrize("case", ["huge", "tiny", "tiny_zero_blocks", "split_channels"])
def test_fwd_f16_pv_v_range(route, case):
    """E4M3-scaled P with MXFP4 V runs its PV product in f16 with each V channel shifted
    by a power of two into f16's range.  V far above f16's largest value (x 2^40), far
    below its smallest (x 2^-60; also with two all-zero 32-key blocks, whose scale byte is
    that of 2^0), and channels 2^60 apart (half x 2^30, half x 2^-30): each channel group
    is checked against its own scale."""
    q, v, pm, pf = ROUTES[route]
    x = synth.make_inputs("kmean", 1, 2, 2, 300, 128, 7)
    ch = np.ones(128, np.float32)
    if case == "huge":
        ch[:] = 2.0 ** 40
    elif case == "split_channels":
        ch[:64], ch[64:] = 2.0 ** 30, 2.0 ** -30
    if case.startswith("tiny"):
        ch[:] = 2.0 ** -60
    xs = _scaled_v(x, ch)
    if case == "tiny_zero_blocks":
        va = xs["v"].copy()
        va[:, :, 64:128, :] = 0  # keys 64..127 of every channel: two zero blocks
        xs["v"] = va
    res = run_case(q, v, pm, pf, B=1, Hq=2, Hkv=2, N=300, inputs=xs)
    assert np.all(np.isfinite(res["O_gpu"]))
    groups = [np.arange(128)] if case != "split_channels" else [np.arange(64), np.arange(64, 128)]
    vmax = float(np.abs(synth.bf16_to_f32(xs["v"])).max())
    for g in groups:
        Og, Or = res["O_gpu"][:, g], res["O_ref"][:, g]
        # the flip budget bounds |dp^| max|v| / l over all channels; this group's share
        # scales with its own largest |v|
        vg = float(np.abs(synth.bf16_to_f32(xs["v"])[..., g]).max())
        bound = TOL * np.abs(Or).max() + res["fb"][:, None] * (vg / vmax)
        ratio = float((np.abs(Og - Or) / bound).max())
        record_parity(f"{route} V range {case} channels {g[0]}..{g[-1]}", ratio,
                      res["fb"] * (vg / vmax) / (TOL * np.abs(Or).max()))
        assert ratio <= 1.0, (case, g[0], ratio)


@pytest.mark.parametrize("bad", ["unplanned", "causal_flag", "doc_count"])
def test_fwd_mismatched_plan_gives_nan(bad):
    """A workspace whose plan does not match the call (none written, another causal
    flag, another document count over the same tokens) is detected by the kernel from
    the plan's header: every output row and LSE is NaN, and nothing is read out of
    bounds."""
    import torch
    import microscaling_fp4_attention_amd as mx
    N = 700
    doc_off = np.array([0, 100, 101, 357, 490, 700], np.int32)
    x = synth.make_inputs("plain", 1, 2, 2, N, 128, 11)
    dev = "cuda:0"
    t = {n: torch.from_numpy(x[n].astype(np.int16)).view(torch.bfloat16).to(dev) for n in ("q", "k", "v")}
    cu = torch.from_numpy(doc_off).to(dev)
    Q = mx.quantize(t["q"], mx.ROLE_QK, "mxfp4_uos")
    K = mx.quantize(t["k"], mx.ROLE_QK, "mxfp4_uos")
    V = mx.quantize(t["v"], mx.ROLE_V, "mxfp4_uos", cu_seqlens=cu)
    p = mx.fwd_params("pnq", "mxfp4_uos", causal=True, out_fp32=True)
    nd = len(doc_off) - 1
    if bad == "unplanned":
        ws = torch.zeros(mx.fwd_workspace_bytes(N, nd), dtype=torch.uint8, device=dev)
    elif bad == "causal_flag":
        ws = mx.fwd_plan(doc_off, N, False)
    else:  # a plan of 2 documents, padded to the byte size of the 5-document one
        ws2 = mx.fwd_plan(np.array([0, 350, 700], np.int32), N, True)
        ws = torch.zeros(mx.fwd_workspace_bytes(N, nd), dtype=torch.uint8, device=dev)
        ws[:ws2.numel()] = ws2
    lse = torch.empty((1, 2, N), dtype=torch.float32, device=dev)
    out = mx.fwd(Q, K, V, p, lse=lse, workspace=ws, ndocs=nd)
    torch.cuda.synchronize()
    assert bool(torch.isnan(out).all()) and bool(torch.isnan(lse).all()), bad
    # the matching plan gives finite rows
    out = mx.fwd(Q, K, V, p, lse=lse, workspace=mx.fwd_plan(doc_off, N, True), ndocs=nd)
    torch.cuda.synchronize()
    assert bool(torch.isfinite(out).all())


@pytest.mark.parametrize("route", ["mxfp4_uos_pnq", "mxfp4_two_level_e4m3", "nvfp4_direct"])
def test_fwd_work_order_independence(route):
    """The plan's work lists (document, query tile) are ordered longest first only for
    load balance: any order gives the same output bit for bit.  The lists are shuffled
    in place in the workspace (header: int32 n_items, ndocs, causal, magic, n_items256,
    cap128, n_tokens, pad; then 16-byte document entries; then cap128 entries of the
    128-row list and the 256-row list, 8 bytes each) and the forward is run again."""
    import torch
    import microscaling_fp4_attention_amd as mx
    q, v, pm, pf = ROUTES[route]
    doc_off = np.array([0, 700, 701, 1500, 1800, 3000, 3333], np.int32)
    N, nd = int(doc_off[-1]), len(doc_off) - 1
    x = synth.make_inputs("outlier", 1, 2, 2, N, 128, 12)
    dev = "cuda:0"
    t = {n: torch.from_numpy(x[n].astype(np.int16)).view(torch.bfloat16).to(dev) for n in ("q", "k", "v")}
    cu = torch.from_numpy(doc_off).to(dev)
    Q = mx.quantize(t["q"], mx.ROLE_QK, q)
    K = mx.quantize(t["k"], mx.ROLE_QK, q)
    V = mx.quantize(t["v"], mx.ROLE_V, v, cu_seqlens=cu)
    p = mx.fwd_params(pm, pf, causal=True, out_fp32=True)
    ws = mx.fwd_plan(doc_off, N, True)
    lse1 = torch.empty((1, 2, N), dtype=torch.float32, device=dev)
    out1 = mx.fwd(Q, K, V, p, lse=lse1, workspace=ws, ndocs=nd)
    torch.cuda.synchronize()
    h = ws.cpu().numpy()
    hdr = h[:32].view(np.int32)
    n128, n256, cap128 = int(hdr[0]), int(hdr[4]), int(hdr[5])
    off = 32 + 16 * nd
    l128 = h[off:off + 8 * cap128].view(np.int32).reshape(-1, 2)
    l256 = h[off + 8 * cap128:].view(np.int32)[:2 * n256].reshape(-1, 2)
    rng = np.random.default_rng(5)
    l128[:n128] = l128[:n128][rng.permutation(n128)]
    l256[:n256] = l256[:n256][rng.permutation(n256)]
    ws2 = torch.from_numpy(h).to(dev)
    lse2 = torch.empty_like(lse1)
    out2 = mx.fwd(Q, K, V, p, lse=lse2, workspace=ws2, ndocs=nd)
    torch.cuda.synchronize()
    assert not np.array_equal(ws.cpu().numpy(), h)  # the order did change
    assert torch.equal(out1, out2) and torch.equal(lse1, lse2)
    assert bool(torch.isfinite(out1).all())
