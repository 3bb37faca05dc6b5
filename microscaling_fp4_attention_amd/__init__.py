"""Python binding of libmxattn (include/mxattn.h): argument marshalling only.

Every step of the attention path runs in the HIP kernels of the library; this
module sizes and allocates buffers with PyTorch (device memory and streams only),
fills the C structs and calls the C entry points through ctypes.  Importing it
fails loudly when the built library is missing; there is no fallback.
"""
from __future__ import annotations

import ctypes
import math
import os
from dataclasses import dataclass

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmxattn.so")

# enums of mxattn.h
OK, E_INVALID, E_UNSUPPORTED, E_ALIGN, E_WORKSPACE, E_HIP = 0, -1, -2, -3, -4, -5
ELEM_E2M1, ELEM_E4M3, ELEM_BF16 = 0, 1, 2
SCALE_E8M0, SCALE_E4M3, SCALE_NONE = 0, 1, 2
RULE_OCP, RULE_CEIL = 0, 1
ROLE_QK, ROLE_V, ROLE_VKEY, ROLE_VT = 0, 1, 2, 3
P_NONE, P_DIRECT, P_TWO_LEVEL, P_PNQ, P_FP8_FIXED = 0, 1, 2, 3, 4
EXP_EXACT, EXP_MITCHELL, EXP_SCHRAUDOLPH = 0, 1, 2


ABI_VERSION = 8  # MXATTN_ABI_VERSION of include/mxattn.h
DECODE_SCRATCH_BYTES = 32 << 20  # MXATTN_DECODE_SCRATCH_BYTES


class QFmt(ctypes.Structure):
    _fields_ = [("elem", ctypes.c_int32), ("scale", ctypes.c_int32), ("block", ctypes.c_int32),
                ("rule", ctypes.c_int32), ("qmax", ctypes.c_float)]


class QTensorC(ctypes.Structure):
    _fields_ = [("codes", ctypes.c_void_p), ("scales", ctypes.c_void_p), ("fmt", QFmt), ("role", ctypes.c_int32),
                ("ndocs", ctypes.c_int32), ("B", ctypes.c_int64), ("H", ctypes.c_int64), ("N", ctypes.c_int64),
                ("d", ctypes.c_int64), ("n_padded", ctypes.c_int64)]


class FwdParams(ctypes.Structure):
    _fields_ = [("pmode", ctypes.c_int32), ("pfmt", QFmt), ("causal", ctypes.c_int32), ("sm_scale", ctypes.c_float),
                ("kv_tile", ctypes.c_int32), ("out_fp32", ctypes.c_int32), ("score_bias", ctypes.c_void_p),
                ("vkey", ctypes.c_void_p), ("exp_mode", ctypes.c_int32)]


class PreProc(ctypes.Structure):
    _fields_ = [("mean", ctypes.c_void_p), ("hadamard", ctypes.c_int32)]


# block formats named as on the pages
FORMATS = {
    "mxfp4": (ELEM_E2M1, SCALE_E8M0, 32, RULE_OCP, 0.0),        # OCP MX: E8M0 per 32, floor rule
    "mxfp4_uos": (ELEM_E2M1, SCALE_E8M0, 32, RULE_CEIL, 7.25),  # MXAttention unified optimal scaling
    "mxfp4_tfs": (ELEM_E2M1, SCALE_E8M0, 32, RULE_CEIL, 6.0),   # truncation-free scaling
    "nvfp4": (ELEM_E2M1, SCALE_E4M3, 16, RULE_OCP, 0.0),        # 1x16 blocks, E4M3 scale amax/6
    "fp8v": (ELEM_E4M3, SCALE_E8M0, 32, RULE_CEIL, 448.0),      # E4M3 values, E8M0 per 32, round up
    "bf16": (ELEM_BF16, SCALE_NONE, 0, RULE_OCP, 0.0),          # unquantized route
}
PMODES = {"none": P_NONE, "direct": P_DIRECT, "two_level": P_TWO_LEVEL, "pnq": P_PNQ, "fp8": P_FP8_FIXED}
EXP_MODES = {"exact": EXP_EXACT, "mitchell": EXP_MITCHELL, "schraudolph": EXP_SCHRAUDOLPH}


def qfmt(f) -> QFmt:
    if isinstance(f, QFmt):
        return f
    return QFmt(*FORMATS[f])


class MxattnError(RuntimeError):
    def __init__(self, status: int, what: str):
        msg = _lib().mxattn_status_str(status).decode()
        extra = _lib().mxattn_last_error().decode() if status in (E_HIP, E_WORKSPACE) else ""
        super().__init__(f"{what}: {msg} ({status}) {extra}".strip())
        self.status = status


_LIB = None


def _lib():
    global _LIB
    if _LIB is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is not built; run `python -m microscaling_fp4_attention_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        P = ctypes.POINTER
        i64, vp, i32 = ctypes.c_int64, ctypes.c_void_p, ctypes.c_int
        L.mxattn_abi_version.restype = i32
        if L.mxattn_abi_version() != ABI_VERSION:
            raise ImportError(f"{LIB_PATH} has ABI {L.mxattn_abi_version()}, this binding needs {ABI_VERSION}; rebuild")
        L.mxattn_status_str.restype = ctypes.c_char_p
        L.mxattn_status_str.argtypes = [i32]
        L.mxattn_last_error.restype = ctypes.c_char_p
        L.mxattn_last_hip_error.restype = ctypes.c_char_p
        L.mxattn_debug_fail_launches.restype = i32
        L.mxattn_debug_fail_launches.argtypes = [i32]
        L.mxattn_qtensor_bytes.restype = i32
        L.mxattn_qtensor_bytes.argtypes = [P(QFmt), i32, i64, i64, i64, i64, i32, P(ctypes.c_size_t),
                                           P(ctypes.c_size_t), P(i64)]
        L.mxattn_quantize.restype = i32
        L.mxattn_quantize.argtypes = [vp, P(i64), i64, i64, i64, i64, i32, P(QFmt), vp, i32, P(QTensorC), vp]
        L.mxattn_channel_mean.restype = i32
        L.mxattn_channel_mean.argtypes = [vp, P(i64), i64, i64, i64, i64, vp, i32, vp, vp]
        L.mxattn_quantize_pre.restype = i32
        L.mxattn_quantize_pre.argtypes = [vp, P(i64), i64, i64, i64, i64, i32, P(QFmt), P(PreProc), vp, i32,
                                          P(QTensorC), vp]
        L.mxattn_center_comp.restype = i32
        L.mxattn_center_comp.argtypes = [vp, vp, P(i64), vp, i64, i64, i64, i64, i64, vp, i32, vp, vp]
        L.mxattn_decode_workspace_bytes.restype = ctypes.c_size_t
        L.mxattn_decode_workspace_bytes.argtypes = [i64, i64, i64, i64]
        L.mxattn_decode.restype = i32
        L.mxattn_decode.argtypes = [P(QTensorC), P(QTensorC), P(QTensorC), P(FwdParams), vp, vp, P(i64), vp, vp,
                                    ctypes.c_size_t, vp]
        L.mxattn_decode_noalloc.restype = i32
        L.mxattn_decode_noalloc.argtypes = [P(QTensorC), P(QTensorC), P(QTensorC), P(FwdParams), vp, vp, P(i64), vp,
                                            vp]
        L.mxattn_fwd_workspace_bytes.restype = ctypes.c_size_t
        L.mxattn_fwd_workspace_bytes.argtypes = [i64, i32]
        L.mxattn_fwd_plan.restype = i32
        L.mxattn_fwd_plan.argtypes = [P(ctypes.c_int32), i32, i64, i32, vp, ctypes.c_size_t, vp]
        L.mxattn_fwd.restype = i32
        L.mxattn_fwd.argtypes = [P(QTensorC), P(QTensorC), P(QTensorC), P(FwdParams), i32, vp, P(i64), vp, vp,
                                 ctypes.c_size_t, vp]
        _LIB = L
    return _LIB


def lib():
    """The loaded ctypes library (raises ImportError when it is not built)."""
    return _lib()


def _check(rc: int, what: str):
    if rc != OK:
        raise MxattnError(rc, what)


def _stream(stream=None) -> ctypes.c_void_p:
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _i64(vals):
    return (ctypes.c_int64 * len(vals))(*[int(v) for v in vals])


@dataclass
class QTensor:
    """A quantized tensor: codes and scales (uint8 device tensors) plus its descriptor."""
    codes: torch.Tensor
    scales: torch.Tensor
    desc: QTensorC

    @property
    def n_padded(self) -> int:
        return int(self.desc.n_padded)

    def codes_view(self) -> torch.Tensor:
        """role QK: [B, H, N, d*bits/8]; role V: [B, H, d, n_padded*bits/8];
        role VT: [B, H, n_padded/128, d, 128*bits/8]."""
        d = self.desc
        if d.fmt.elem == ELEM_BF16:  # the values, [B, H, N, d]
            return self.codes.view(torch.bfloat16).view(d.B, d.H, d.N, d.d)
        bits = 4 if d.fmt.elem == ELEM_E2M1 else 8
        if d.role == ROLE_QK:
            return self.codes.view(d.B, d.H, d.N, d.d * bits // 8)
        if d.role == ROLE_VT:
            return self.codes.view(d.B, d.H, d.n_padded // 128, d.d, 128 * bits // 8)
        return self.codes.view(d.B, d.H, d.d, d.n_padded * bits // 8)

    def scales_view(self) -> torch.Tensor:
        """role QK: [B, H, N, d/block]; role V: [B, H, d, n_padded/block]; role VKEY:
        [B, H, n_padded]; role VT: [B, H, n_padded/128, d, 4]."""
        d = self.desc
        if d.role == ROLE_QK:
            return self.scales.view(d.B, d.H, d.N, d.d // d.fmt.block)
        if d.role == ROLE_VKEY:
            return self.scales.view(d.B, d.H, d.n_padded)
        if d.role == ROLE_VT:
            return self.scales.view(d.B, d.H, d.n_padded // 128, d.d, 4)
        return self.scales.view(d.B, d.H, d.d, d.n_padded // d.fmt.block)


def qtensor_bytes(fmt, role: int, B: int, H: int, N: int, d: int = 128, ndocs: int = 0):
    cb, sb, npad = ctypes.c_size_t(0), ctypes.c_size_t(0), ctypes.c_int64(0)
    f = qfmt(fmt)
    _check(_lib().mxattn_qtensor_bytes(ctypes.byref(f), role, B, H, N, d, ndocs, ctypes.byref(cb), ctypes.byref(sb),
                                       ctypes.byref(npad)), "mxattn_qtensor_bytes")
    return cb.value, sb.value, npad.value


def _cu(cu_seqlens):
    if cu_seqlens is None:
        return None, 0
    if cu_seqlens.dtype != torch.int32 or not cu_seqlens.is_cuda:
        raise ValueError("cu_seqlens must be an int32 device tensor")
    return ctypes.c_void_p(cu_seqlens.data_ptr()), cu_seqlens.numel() - 1


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _need(t: torch.Tensor, name: str, dtype=None, shape=None, numel=None, contiguous=False):
    """Check a caller tensor before its address reaches the library: the kernels take
    raw device pointers and write through the sizes the descriptors give, so a host
    tensor, a wrong element type or a short buffer must be refused here."""
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if numel is not None and t.numel() != numel:
        raise ValueError(f"{name} must have {numel} elements, got {t.numel()}")
    if contiguous and not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor, got one on {t.device}")


def channel_mean(x: torch.Tensor, cu_seqlens: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """Per-channel means of a bf16 tensor x [B, H, N, d] over each document's tokens:
    float32 [B, H, max(ndocs, 1), d] (mxattn_channel_mean)."""
    if x.dtype != torch.bfloat16 or x.dim() != 4:
        raise ValueError("x must be a 4-D bfloat16 tensor [B, H, N, d]")
    _need(x, "x")
    B, H, N, d = x.shape
    cu, ndocs = _cu(cu_seqlens)
    mean = torch.empty((B, H, max(ndocs, 1), d), dtype=torch.float32, device=x.device)
    _check(_lib().mxattn_channel_mean(_ptr(x), _i64(x.stride()), B, H, N, d, cu, ndocs, _ptr(mean),
                                      _stream(stream)), "mxattn_channel_mean")
    return mean


def center_comp(qmean: torch.Tensor, k: torch.Tensor, kmean: torch.Tensor, cu_seqlens: torch.Tensor | None = None,
                stream=None) -> torch.Tensor:
    """Centering compensation delta [B, Hq, N] (float32) for the forward's score_bias
    (mxattn_center_comp): qmean [B, Hq, nd, d], k bf16 [B, Hkv, N, d], kmean [B, Hkv, nd, d]."""
    _need(k, "k", dtype=torch.bfloat16)
    if k.dim() != 4 or qmean.dim() != 4:
        raise ValueError("k must be [B, Hkv, N, d] and qmean [B, Hq, nd, d]")
    B, Hkv, N, d = k.shape
    Hq = qmean.shape[1]
    cu, ndocs = _cu(cu_seqlens)
    nd = max(ndocs, 1)
    _need(qmean, "qmean", dtype=torch.float32, shape=(B, Hq, nd, d))
    _need(kmean, "kmean", dtype=torch.float32, shape=(B, Hkv, nd, d))
    delta = torch.empty((B, Hq, N), dtype=torch.float32, device=k.device)
    _check(_lib().mxattn_center_comp(_ptr(qmean.contiguous()), _ptr(k), _i64(k.stride()), _ptr(kmean.contiguous()),
                                     B, Hq, Hkv, N, d, cu, ndocs, _ptr(delta), _stream(stream)), "mxattn_center_comp")
    return delta


def quantize(x: torch.Tensor, role: int, fmt, cu_seqlens: torch.Tensor | None = None, stream=None,
             mean: torch.Tensor | None = None, hadamard: bool = False) -> QTensor:
    """Quantize a bf16 tensor x [B, H, N, d] (any strides with a unit channel stride).

    cu_seqlens: int32 device tensor of document offsets (role V: the document layout;
    role QK with a mean: each token's mean row), or None.
    mean / hadamard (role QK only): subtract the per-document channel means (from
    channel_mean) and/or rotate by the normalized Hadamard matrix before quantizing
    (mxattn_quantize_pre).
    """
    if x.dtype != torch.bfloat16 or x.dim() != 4:
        raise ValueError("x must be a 4-D bfloat16 tensor [B, H, N, d]")
    _need(x, "x")
    B, H, N, d = x.shape
    if mean is not None or hadamard:
        if role != ROLE_QK:
            raise ValueError("pre-processing applies to role QK only")
        if mean is not None:
            nd = 1 if cu_seqlens is None else max(cu_seqlens.numel() - 1, 1)
            _need(mean, "mean", dtype=torch.float32, shape=(B, H, nd, d))
        cb, sb, _ = qtensor_bytes(fmt, role, B, H, N, d, 0)
        codes = torch.empty(max(cb, 16), dtype=torch.uint8, device=x.device)[:cb]
        scales = torch.empty(max(sb, 16), dtype=torch.uint8, device=x.device)[:sb]
        desc = QTensorC()
        desc.codes = codes.data_ptr() if cb else None
        desc.scales = scales.data_ptr() if sb else None
        f = qfmt(fmt)
        mean_c = None if mean is None else mean.contiguous()
        pre = PreProc(None if mean_c is None else mean_c.data_ptr(), int(bool(hadamard)))
        cu, ndocs = _cu(cu_seqlens)
        _check(_lib().mxattn_quantize_pre(_ptr(x), _i64(x.stride()), B, H, N, d, role, ctypes.byref(f),
                                          ctypes.byref(pre), cu, ndocs, ctypes.byref(desc), _stream(stream)),
               "mxattn_quantize_pre")
        return QTensor(codes, scales, desc)
    if role == ROLE_QK:
        cu_seqlens = None  # documents do not change a plain Q/K quantization
    ndocs = 0 if cu_seqlens is None else cu_seqlens.numel() - 1
    cb, sb, _ = qtensor_bytes(fmt, role, B, H, N, d, ndocs)
    codes = torch.empty(max(cb, 16), dtype=torch.uint8, device=x.device)[:cb]
    scales = torch.empty(max(sb, 16), dtype=torch.uint8, device=x.device)[:sb]
    desc = QTensorC()
    desc.codes = codes.data_ptr() if cb else None
    desc.scales = scales.data_ptr() if sb else None
    f = qfmt(fmt)
    cu = None
    if cu_seqlens is not None:
        if cu_seqlens.dtype != torch.int32 or not cu_seqlens.is_cuda:
            raise ValueError("cu_seqlens must be an int32 device tensor")
        cu = ctypes.c_void_p(cu_seqlens.data_ptr())
    _check(_lib().mxattn_quantize(ctypes.c_void_p(x.data_ptr()), _i64(x.stride()), B, H, N, d, role,
                                  ctypes.byref(f), cu, ndocs, ctypes.byref(desc), _stream(stream)), "mxattn_quantize")
    return QTensor(codes, scales, desc)


def fwd_workspace_bytes(N: int, ndocs: int) -> int:
    return int(_lib().mxattn_fwd_workspace_bytes(N, ndocs))


def fwd_plan(cu_seqlens_host, N: int, causal: bool, device="cuda", stream=None) -> torch.Tensor:
    """Build the work list of a packed-document forward; returns the workspace tensor."""
    cu = [int(v) for v in cu_seqlens_host]
    ndocs = len(cu) - 1
    nbytes = fwd_workspace_bytes(N, ndocs)
    ws = torch.empty(max(nbytes, 16), dtype=torch.uint8, device=device)
    arr = (ctypes.c_int32 * len(cu))(*cu)
    _check(_lib().mxattn_fwd_plan(arr, ndocs, N, int(bool(causal)), ctypes.c_void_p(ws.data_ptr()), nbytes,
                                  _stream(stream)), "mxattn_fwd_plan")
    return ws


def fwd_params(pmode, pfmt="mxfp4", causal=False, sm_scale=None, d=128, out_fp32=True, kv_tile=128,
               score_bias: torch.Tensor | None = None, vkey: "QTensor | None" = None,
               exp_mode="exact") -> FwdParams:
    """score_bias: float32 device tensor [B, Hq, N] added to each key's scores (the
    centering compensation from center_comp), or None.  vkey: the role-VKEY quantization
    of the same V (causally safe V scales on the diagonal tiles), or None.  The params
    keep references to both.  exp_mode: "exact", "mitchell" or "schraudolph" (the
    exponential of P~; the bit-level ones are approximations for inference)."""
    pm = PMODES[pmode] if isinstance(pmode, str) else int(pmode)
    if sm_scale is None:
        sm_scale = 1.0 / math.sqrt(d)
    pf = qfmt(pfmt if pfmt is not None else "mxfp4")
    if score_bias is not None and (score_bias.dtype != torch.float32 or not score_bias.is_contiguous()):
        raise ValueError("score_bias must be a contiguous float32 tensor [B, Hq, N]")
    p = FwdParams(pm, pf, int(bool(causal)), float(sm_scale), kv_tile, int(bool(out_fp32)),
                  None if score_bias is None else score_bias.data_ptr(),
                  None if vkey is None else ctypes.addressof(vkey.desc),
                  EXP_MODES[exp_mode] if isinstance(exp_mode, str) else int(exp_mode))
    p._score_bias_ref = score_bias
    p._vkey_ref = vkey
    return p


def fwd(q: QTensor, k: QTensor, v: QTensor, params: FwdParams, out: torch.Tensor | None = None,
        lse: torch.Tensor | None = None, workspace: torch.Tensor | None = None, ndocs: int = 0,
        stream=None) -> torch.Tensor:
    """Attention forward; returns out [B, Hq, N, 128] (float32 or bfloat16 per params.out_fp32)."""
    B, Hq, N, d = q.desc.B, q.desc.H, q.desc.N, q.desc.d
    dt = torch.float32 if params.out_fp32 else torch.bfloat16
    if out is None:
        out = torch.empty((B, Hq, N, d), dtype=dt, device=q.codes.device)
    _need(out, "out", dtype=dt, shape=(B, Hq, N, d))
    if lse is not None:
        _need(lse, "lse", dtype=torch.float32, numel=B * Hq * N, contiguous=True)
    bias = getattr(params, "_score_bias_ref", None)
    if bias is not None:
        _need(bias, "score_bias", dtype=torch.float32, numel=B * Hq * N, contiguous=True)
    ws_ptr, ws_bytes = None, 0
    if workspace is not None:
        _need(workspace, "workspace", dtype=torch.uint8)
        ws_ptr, ws_bytes = ctypes.c_void_p(workspace.data_ptr()), workspace.numel()
    lse_ptr = None if lse is None else ctypes.c_void_p(lse.data_ptr())
    _check(_lib().mxattn_fwd(ctypes.byref(q.desc), ctypes.byref(k.desc), ctypes.byref(v.desc), ctypes.byref(params),
                             ndocs, ctypes.c_void_p(out.data_ptr()), _i64(out.stride()), lse_ptr, ws_ptr, ws_bytes,
                             _stream(stream)), "mxattn_fwd")
    return out


def decode_workspace_bytes(B: int, Hq: int, R: int, N: int) -> int:
    return int(_lib().mxattn_decode_workspace_bytes(B, Hq, R, N))


def decode(q: QTensor, k: QTensor, v: QTensor, params: FwdParams, kv_len: torch.Tensor | None = None,
           out: torch.Tensor | None = None, lse: torch.Tensor | None = None, workspace: torch.Tensor | None = None,
           stream=None) -> torch.Tensor:
    """Split-key decode (mxattn_decode): q [B, Hq, R, 128] quantized (the R newest tokens),
    k / v over the [B, Hkv, N] history; kv_len: int32 device tensor [B] or None.
    Returns out [B, Hq, R, 128] (float32 or bfloat16 per params.out_fp32)."""
    B, Hq, R, d = q.desc.B, q.desc.H, q.desc.N, q.desc.d
    N = k.desc.N
    dt = torch.float32 if params.out_fp32 else torch.bfloat16
    if out is None:
        out = torch.empty((B, Hq, R, d), dtype=dt, device=q.codes.device)
    _need(out, "out", dtype=dt, shape=(B, Hq, R, d))
    if lse is not None:
        _need(lse, "lse", dtype=torch.float32, numel=B * Hq * R, contiguous=True)
    nbytes = decode_workspace_bytes(B, Hq, R, N)
    if workspace is None:
        workspace = torch.empty(max(nbytes, 16), dtype=torch.uint8, device=q.codes.device)
    _need(workspace, "workspace", dtype=torch.uint8)
    if kv_len is not None:
        _need(kv_len, "kv_len", dtype=torch.int32, numel=B, contiguous=True)
    _check(_lib().mxattn_decode(ctypes.byref(q.desc), ctypes.byref(k.desc), ctypes.byref(v.desc), ctypes.byref(params),
                                _ptr(kv_len), _ptr(out), _i64(out.stride()), _ptr(lse), _ptr(workspace),
                                workspace.numel(), _stream(stream)), "mxattn_decode")
    return out


def decode_noalloc(q: QTensor, k: QTensor, v: QTensor, params: FwdParams, kv_len: torch.Tensor | None = None,
                   out: torch.Tensor | None = None, lse: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """mxattn_decode_noalloc: decode() with the split states in the library's static
    scratch (no workspace, no allocation in the library; pass `out` to allocate nothing
    here either).  Calls that overlap on one GPU race."""
    B, Hq, R, d = q.desc.B, q.desc.H, q.desc.N, q.desc.d
    dt = torch.float32 if params.out_fp32 else torch.bfloat16
    if out is None:
        out = torch.empty((B, Hq, R, d), dtype=dt, device=q.codes.device)
    _need(out, "out", dtype=dt, shape=(B, Hq, R, d))
    if lse is not None:
        _need(lse, "lse", dtype=torch.float32, numel=B * Hq * R, contiguous=True)
    if kv_len is not None:
        _need(kv_len, "kv_len", dtype=torch.int32, numel=B, contiguous=True)
    _check(_lib().mxattn_decode_noalloc(ctypes.byref(q.desc), ctypes.byref(k.desc), ctypes.byref(v.desc),
                                        ctypes.byref(params), _ptr(kv_len), _ptr(out), _i64(out.stride()), _ptr(lse),
                                        _stream(stream)), "mxattn_decode_noalloc")
    return out
