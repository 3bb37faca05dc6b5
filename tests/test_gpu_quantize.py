"""GPU quantize pass (mxattn_quantize) against the oracle: every code and scale
byte must be identical (MXAttention section 2 and Table 1 for the E8M0 rules;
blog "NVFP4, not MXFP4" for s = E4M3(amax/6); MpFA section 4.1 and FLAMIA
section 3.2 for E4M3 V with a power-of-two scale per 32 keys)."""
import numpy as np
import pytest

import synth
from helpers import gpu_available, gpu_codes_qk, gpu_codes_v, oracle_quant_qk, oracle_quant_v

pytestmark = [pytest.mark.gpu, pytest.mark.skipif(not gpu_available(), reason="needs a GPU")]


def _dev(a):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a).astype(np.int16)).view(torch.bfloat16).to("cuda:0")


def _edge_values(n_rows):
    """Rows that exercise zero blocks, -0, rounding ties at every E2M1 midpoint,
    saturation, tiny and huge magnitudes, bf16 subnormals and the largest bf16."""
    rng = np.random.default_rng(7)
    rows = []
    mids = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 7.0, 6.5, 5.5, 0.1, 0.0])
    for r in range(n_rows):
        x = np.zeros(128, np.float32)
        kind = r % 8
        if kind == 0:
            pass  # all zero
        elif kind == 1:
            x[:] = -0.0
        elif kind == 2:  # ties relative to a block max of 6 (scale 1 under OCP: M=6 -> e=0)
            x[:] = np.resize(np.concatenate([mids, -mids]), 128)
            x[::32] = 6.0
        elif kind == 3:  # ties at scale 2^-3
            x[:] = np.resize(np.concatenate([mids, -mids]), 128) * 0.125
            x[::16] = 0.75
        elif kind == 4:
            x[:] = rng.standard_normal(128) * 1e-38  # subnormal range
        elif kind == 5:
            x[:] = rng.standard_normal(128) * 1e37
            x[5] = 3.3895314e38  # largest bf16
        elif kind == 6:  # block maxima exactly at 7.25 * 2^k and just around it
            x[:] = rng.uniform(-1, 1, 128)
            x[0], x[32], x[64], x[96] = 7.25, 7.25 * 2 ** -5, np.nextafter(np.float32(7.25), 9), 3.625
            x[16], x[48], x[80], x[112] = 6.0, 6.0 * 2 ** 3, np.nextafter(np.float32(6.0), 0), 448.0
        else:
            x[:] = rng.standard_normal(128) * 3.0
        rows.append(x)
    return synth.f32_to_bf16(np.stack(rows))


QK_FMTS = ["mxfp4", "mxfp4_uos", "mxfp4_tfs", "nvfp4"]
V_FMTS = ["mxfp4", "mxfp4_uos", "nvfp4", "fp8v"]


@pytest.mark.parametrize("fmt", QK_FMTS)
@pytest.mark.parametrize("kind", ["kmean_outlier", "lowrank"])
def test_quantize_qk_bytes(fmt, kind):
    import microscaling_fp4_attention_amd as mx
    x = synth.make_inputs(kind, 2, 3, 3, 300, 128, seed=1)["k"]
    qt = mx.quantize(_dev(x), mx.ROLE_QK, fmt)
    c, s, _ = oracle_quant_qk(synth.bf16_to_f32(x), fmt)
    assert np.array_equal(gpu_codes_qk(qt), c)
    assert np.array_equal(qt.scales_view().cpu().numpy(), s)


@pytest.mark.parametrize("fmt", QK_FMTS)
def test_quantize_qk_edge_cases(fmt):
    import microscaling_fp4_attention_amd as mx
    x = _edge_values(40).reshape(1, 1, 40, 128)
    qt = mx.quantize(_dev(x), mx.ROLE_QK, fmt)
    c, s, _ = oracle_quant_qk(synth.bf16_to_f32(x), fmt)
    assert np.array_equal(gpu_codes_qk(qt), c)
    assert np.array_equal(qt.scales_view().cpu().numpy(), s)


def test_quantize_qk_strided_input():
    """A [B, N, H, d] tensor viewed as [B, H, N, d] (non-contiguous heads)."""
    import microscaling_fp4_attention_amd as mx
    x = synth.make_inputs("plain", 1, 4, 4, 200, 128, seed=3)["q"]
    g = _dev(x.transpose(0, 2, 1, 3).copy()).permute(0, 2, 1, 3)
    assert not g.is_contiguous()
    qt = mx.quantize(g, mx.ROLE_QK, "mxfp4")
    c, s, _ = oracle_quant_qk(synth.bf16_to_f32(x), "mxfp4")
    assert np.array_equal(gpu_codes_qk(qt), c)
    assert np.array_equal(qt.scales_view().cpu().numpy(), s)


@pytest.mark.parametrize("fmt", ["mxfp4", "mxfp4_uos"])
@pytest.mark.parametrize("N", [1000, 4500])
def test_quantize_vt_is_v_tile_major(fmt, N):
    """Role VT holds role V's bytes with key tile t of channel c moved to [t][c]."""
    import microscaling_fp4_attention_amd as mx
    x = _dev(synth.make_inputs("plain", 2, 3, 3, N, 128, seed=5)["v"])
    v, vt = mx.quantize(x, mx.ROLE_V, fmt), mx.quantize(x, mx.ROLE_VT, fmt)
    assert vt.n_padded == v.n_padded
    nt = v.n_padded // 128
    cv = v.codes_view().reshape(2, 3, 128, nt, 64).permute(0, 1, 3, 2, 4)
    sv = v.scales_view().reshape(2, 3, 128, nt, 4).permute(0, 1, 3, 2, 4)
    assert torch_equal(vt.codes_view(), cv) and torch_equal(vt.scales_view(), sv)


def torch_equal(a, b):
    import torch
    return bool(torch.equal(a.contiguous(), b.contiguous()))


def _e4m3_value(c):
    e, m = (c >> 3) & 15, c & 7
    return m * 2.0 ** -9 if e == 0 else (1 + m / 8) * 2.0 ** (e - 7)


def test_quantize_nvfp4_every_element_under_every_scale():
    """Every nonzero E4M3 block scale s (codes 1..126), each with blocks whose maximum is
    6 s exactly (so the scale is s), and every positive bf16 magnitude up to that
    maximum in both signs as the other 15 elements: the codes of x / s, including every
    value on or next to an E2M1 rounding midpoint, byte-exact against the oracle."""
    import microscaling_fp4_attention_amd as mx
    mags = np.arange(0, 0x7F80, dtype=np.uint32)  # every finite non-negative bf16
    vals = (mags << 16).view(np.float32)
    blocks = []
    for c in range(1, 127):
        M = np.float32(6.0 * _e4m3_value(c))
        assert synth.bf16_to_f32(synth.f32_to_bf16(np.array([M])))[0] == M
        m = vals[vals <= M]
        el = np.empty(2 * m.size, np.float32)
        el[0::2], el[1::2] = m, -m
        el = np.concatenate([el, np.zeros((-el.size) % 15, np.float32)]).reshape(-1, 15)
        blocks.append(np.concatenate([np.full((el.shape[0], 1), M, np.float32), el], axis=1))
    b = np.concatenate(blocks)
    b = np.concatenate([b, np.zeros(((-b.shape[0]) % 8, 16), np.float32)])
    x = synth.f32_to_bf16(b.reshape(1, 1, -1, 128))
    assert x.shape[2] > 30000
    qt = mx.quantize(_dev(x), mx.ROLE_QK, "nvfp4")
    c, sc, _ = oracle_quant_qk(synth.bf16_to_f32(x), "nvfp4")
    assert np.array_equal(qt.scales_view().cpu().numpy(), sc)
    assert np.array_equal(gpu_codes_qk(qt), c)


@pytest.mark.parametrize("fmt", V_FMTS)
@pytest.mark.parametrize("docs", [None, [0, 37, 100, 229, 300], [0, 300]])
def test_quantize_v_bytes(fmt, docs):
    import torch
    import microscaling_fp4_attention_amd as mx
    x = synth.make_inputs("plain", 1, 2, 2, 300, 128, seed=2)["v"]
    doc_off = None if docs is None else np.array(docs, np.int32)
    cu = None if docs is None else torch.tensor(docs, dtype=torch.int32, device="cuda:0")
    qt = mx.quantize(_dev(x), mx.ROLE_V, fmt, cu_seqlens=cu)
    c, s, _ = oracle_quant_v(synth.bf16_to_f32(x), fmt, doc_off)
    gc, gs = gpu_codes_v(qt, 300, doc_off)
    assert np.array_equal(gc, c)
    assert np.array_equal(gs, s)
    # padding slots hold code 0 and padding-only blocks the all-zero scale
    full = qt.codes_view().cpu().numpy()
    nb = qt.n_padded
    assert full.shape[-1] * (2 if qt.desc.fmt.elem == 0 else 1) == nb


@pytest.mark.parametrize("fmt", ["mxfp4_uos", "fp8v"])
@pytest.mark.parametrize("docs", [None, [0, 9000, 9001, 30517, 48852]])
def test_quantize_v_bytes_several_runs(fmt, docs):
    # B=1, H=16, 48852 tokens: 382+ tiles of 128 key slots per head, enough for the
    # quantizer to give each workgroup runs of 8 tiles with a ragged last run (its scale
    # bytes are collected per run); codes and scales byte-exact
    import torch
    import microscaling_fp4_attention_amd as mx
    N = 48852
    x = synth.f32_to_bf16(synth.gaussian(4, 7, (1, 16, N, 128)))
    doc_off = None if docs is None else np.array(docs, np.int32)
    cu = None if docs is None else torch.tensor(docs, dtype=torch.int32, device="cuda:0")
    qt = mx.quantize(_dev(x), mx.ROLE_V, fmt, cu_seqlens=cu)
    ntiles = qt.n_padded // 128
    assert ntiles % 8 != 0 and 16 * ((ntiles + 7) // 8) >= 768
    c, s, _ = oracle_quant_v(synth.bf16_to_f32(x), fmt, doc_off)
    gc, gs = gpu_codes_v(qt, N, doc_off)
    assert np.array_equal(gc, c)
    assert np.array_equal(gs, s)


@pytest.mark.parametrize("fmt", V_FMTS)
def test_quantize_v_edge_cases(fmt):
    import microscaling_fp4_attention_amd as mx
    x = _edge_values(128).reshape(1, 1, 128, 128)
    qt = mx.quantize(_dev(x), mx.ROLE_V, fmt)
    c, s, _ = oracle_quant_v(synth.bf16_to_f32(x), fmt)
    gc, gs = gpu_codes_v(qt, 128, None)
    assert np.array_equal(gc, c)
    assert np.array_equal(gs, s)
