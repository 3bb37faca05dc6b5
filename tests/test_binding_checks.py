"""The binding refuses caller tensors whose addresses must not reach the library: host
tensors (a host address in a kernel faults the device), outputs of the wrong element
type or shape (the kernels write through the descriptor's sizes), short LSE, bias or
length buffers.  No GPU is needed: every call below raises before any library call.
"""
import pytest
import torch


@pytest.fixture(scope="module")
def mx():
    import microscaling_fp4_attention_amd as mx
    try:
        mx.lib()
    except ImportError as e:  # the library is built by __graft_entry__.build()
        pytest.skip(str(e))
    return mx


def fake_qtensor(mx, role, B=1, H=2, N=8):
    d = mx.QTensorC()
    d.fmt, d.role, d.ndocs, d.B, d.H, d.N, d.d = mx.qfmt("mxfp4"), role, 1, B, H, N, 128
    d.n_padded = 128 if role != mx.ROLE_QK else N
    z = torch.zeros(16, dtype=torch.uint8)
    return mx.QTensor(z, z, d)


def test_need_helper(mx):
    t = torch.zeros((2, 3), dtype=torch.float32)
    with pytest.raises(ValueError, match="must be torch.bfloat16"):
        mx._need(t, "t", dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="shape"):
        mx._need(t, "t", shape=(3, 2))
    with pytest.raises(ValueError, match="elements"):
        mx._need(t, "t", numel=5)
    with pytest.raises(ValueError, match="contiguous"):
        mx._need(t.t(), "t", contiguous=True)
    with pytest.raises(ValueError, match="device tensor"):
        mx._need(t, "t", dtype=torch.float32, shape=(2, 3), numel=6, contiguous=True)


def test_fwd_output_checks(mx):
    q, k, v = fake_qtensor(mx, mx.ROLE_QK), fake_qtensor(mx, mx.ROLE_QK), fake_qtensor(mx, mx.ROLE_V)
    p32 = mx.fwd_params("pnq", "mxfp4", out_fp32=True)
    with pytest.raises(ValueError, match="out must be torch.float32"):  # bf16 buffer, FP32 output
        mx.fwd(q, k, v, p32, out=torch.empty((1, 2, 8, 128), dtype=torch.bfloat16))
    with pytest.raises(ValueError, match="out must have shape"):
        mx.fwd(q, k, v, p32, out=torch.empty((1, 2, 4, 128), dtype=torch.float32))
    with pytest.raises(ValueError, match="out must be a device tensor"):
        mx.fwd(q, k, v, p32, out=torch.empty((1, 2, 8, 128), dtype=torch.float32))
    with pytest.raises(ValueError, match="device tensor"):  # the default output follows Q's (host) codes
        mx.fwd(q, k, v, mx.fwd_params("pnq", "mxfp4", out_fp32=False))


def test_decode_output_checks(mx):
    q = fake_qtensor(mx, mx.ROLE_QK, H=4, N=1)
    k, v = fake_qtensor(mx, mx.ROLE_QK, N=256), fake_qtensor(mx, mx.ROLE_V, N=256)
    p = mx.fwd_params("pnq", "mxfp4", causal=True, out_fp32=False)
    with pytest.raises(ValueError, match="out must be torch.bfloat16"):
        mx.decode(q, k, v, p, out=torch.empty((1, 4, 1, 128), dtype=torch.float32))
    with pytest.raises(ValueError, match="out must have shape"):
        mx.decode(q, k, v, p, out=torch.empty((1, 4, 2, 128), dtype=torch.bfloat16))


def test_host_inputs_are_refused(mx):
    x = torch.zeros((1, 2, 8, 128), dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="x must be a device tensor"):
        mx.quantize(x, mx.ROLE_QK, "mxfp4")
    with pytest.raises(ValueError, match="x must be a device tensor"):
        mx.quantize(x, mx.ROLE_V, "mxfp4")
    with pytest.raises(ValueError, match="x must be a device tensor"):
        mx.channel_mean(x)
    with pytest.raises(ValueError, match="k must be a device tensor"):
        mx.center_comp(torch.zeros((1, 2, 1, 128)), x, torch.zeros((1, 2, 1, 128)))
    with pytest.raises(ValueError, match="bfloat16"):
        mx.quantize(x.float(), mx.ROLE_QK, "mxfp4")
    with pytest.raises(ValueError, match="score_bias"):
        mx.fwd_params("pnq", score_bias=torch.zeros((4, 2)).t())
