"""ctypes wrapper of the CPU oracle (oracle.c).

TEST INFRASTRUCTURE ONLY: imported by tests/, __graft_entry__.smoke() and the
CPU-baseline leg of bench.py.  The GPU library never imports or links it.
Functions take and return numpy arrays; all arithmetic happens in oracle.c.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SO = os.path.join(_HERE, "liboracle.so")

# enum values of oracle.h
ELEM_E2M1, ELEM_E4M3 = 0, 1
SCALE_E8M0, SCALE_E4M3 = 0, 1
RULE_OCP, RULE_CEIL = 0, 1
P_NONE, P_DIRECT, P_TWO_LEVEL, P_PNQ, P_FP8_FIXED = 0, 1, 2, 3, 4
EXP_EXACT, EXP_MITCHELL, EXP_SCHRAUDOLPH = 0, 1, 2
EXP_MODES = {"exact": EXP_EXACT, "mitchell": EXP_MITCHELL, "schraudolph": EXP_SCHRAUDOLPH}


class Fmt(ctypes.Structure):
    _fields_ = [("elem", ctypes.c_int), ("scale", ctypes.c_int), ("block", ctypes.c_int),
                ("rule", ctypes.c_int), ("qmax", ctypes.c_float)]


class AttnParams(ctypes.Structure):
    _fields_ = [("pmode", ctypes.c_int), ("pfmt", Fmt), ("causal", ctypes.c_int),
                ("sm_scale", ctypes.c_float), ("kv_tile", ctypes.c_int), ("exp_mode", ctypes.c_int),
                ("score_rounds", ctypes.c_int), ("q_tile", ctypes.c_int)]


# named formats (the presets of the pages)
FORMATS = {
    "mxfp4": Fmt(ELEM_E2M1, SCALE_E8M0, 32, RULE_OCP, 0.0),        # OCP MX rule
    "mxfp4_uos": Fmt(ELEM_E2M1, SCALE_E8M0, 32, RULE_CEIL, 7.25),  # MXAttention UOS
    "mxfp4_tfs": Fmt(ELEM_E2M1, SCALE_E8M0, 32, RULE_CEIL, 6.0),   # truncation-free
    "nvfp4": Fmt(ELEM_E2M1, SCALE_E4M3, 16, RULE_OCP, 0.0),        # 1x16, E4M3 scale
    "fp8v": Fmt(ELEM_E4M3, SCALE_E8M0, 32, RULE_CEIL, 448.0),      # E4M3 with E8M0/32
}


def build(force: bool = True) -> str:
    """Compile oracle.c into liboracle.so with gcc (no fast-math, no contraction)."""
    if force or not os.path.exists(_SO):
        cmd = ["gcc", "-std=c99", "-O2", "-ffp-contract=off", "-fno-fast-math", "-fPIC", "-shared",
               "-Wall", "-o", _SO, os.path.join(_HERE, "oracle.c"), "-lm"]
        subprocess.run(cmd, check=True)
    return _SO


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_SO):
            build()
        L = ctypes.CDLL(_SO)
        P = ctypes.POINTER
        f32p, u8p, i32p, i64p, f64p = (P(ctypes.c_float), P(ctypes.c_uint8), P(ctypes.c_int32),
                                       P(ctypes.c_int64), P(ctypes.c_double))
        L.orc_e2m1_value.restype = ctypes.c_double
        L.orc_e2m1_value.argtypes = [ctypes.c_int]
        L.orc_e2m1_encode.restype = ctypes.c_int
        L.orc_e2m1_encode.argtypes = [ctypes.c_float]
        L.orc_e4m3_value.restype = ctypes.c_double
        L.orc_e4m3_value.argtypes = [ctypes.c_int]
        L.orc_e4m3_encode.restype = ctypes.c_int
        L.orc_e4m3_encode.argtypes = [ctypes.c_float]
        L.orc_e8m0_exponent.restype = ctypes.c_int
        L.orc_e8m0_exponent.argtypes = [ctypes.c_float, ctypes.c_int, ctypes.c_float, ctypes.c_int]
        L.orc_quant_block.restype = ctypes.c_float
        L.orc_quant_block.argtypes = [f32p, ctypes.c_int, P(Fmt), u8p, u8p]
        L.orc_quantize_rows.argtypes = [f32p, ctypes.c_int64, ctypes.c_int, P(Fmt), u8p, u8p]
        L.orc_dequant_rows.argtypes = [u8p, u8p, ctypes.c_int64, ctypes.c_int, P(Fmt), f32p]
        L.orc_v_nblocks.restype = ctypes.c_int64
        L.orc_v_nblocks.argtypes = [ctypes.c_int, i32p, ctypes.c_int, ctypes.c_int]
        L.orc_quantize_cols.argtypes = [f32p, ctypes.c_int, ctypes.c_int, i32p, ctypes.c_int, P(Fmt), u8p, u8p]
        L.orc_dequant_cols.argtypes = [u8p, u8p, ctypes.c_int, ctypes.c_int, i32p, ctypes.c_int, P(Fmt), f32p]
        L.orc_attention_bias.restype = ctypes.c_int
        L.orc_attention_bias.argtypes = [f32p, f32p, f32p, f32p, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                         ctypes.c_int, ctypes.c_int, i32p, ctypes.c_int, P(AttnParams), i64p,
                                         ctypes.c_int64, f32p, f32p, f64p]
        L.orc_attention_ex.restype = ctypes.c_int
        L.orc_attention_ex.argtypes = [f32p, f32p, f32p, f32p, f32p, i32p, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                       ctypes.c_int, ctypes.c_int, i32p, ctypes.c_int, P(AttnParams), i64p,
                                       ctypes.c_int64, f32p, f32p, f64p]
        L.orc_decode.restype = ctypes.c_int
        L.orc_decode.argtypes = [f32p, f32p, f32p, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                 ctypes.c_int, ctypes.c_int, i32p, ctypes.c_int, P(AttnParams), f32p, f32p, f64p]
        L.orc_quantize_keys.argtypes = [f32p, ctypes.c_int, ctypes.c_int, P(Fmt), u8p, i32p]
        L.orc_channel_mean.argtypes = [f32p, ctypes.c_int, ctypes.c_int, i32p, ctypes.c_int, f32p]
        L.orc_preprocess_rows.argtypes = [f32p, ctypes.c_int, ctypes.c_int, f32p, i32p, ctypes.c_int,
                                          ctypes.c_int, f32p]
        L.orc_center_comp.argtypes = [f32p, f32p, f32p, ctypes.c_int, ctypes.c_int, i32p, ctypes.c_int, f32p]
        L.orc_attention.restype = ctypes.c_int
        L.orc_attention.argtypes = [f32p, f32p, f32p, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                    ctypes.c_int, i32p, ctypes.c_int, P(AttnParams), i64p, ctypes.c_int64,
                                    f32p, f32p, f64p]
        _lib = L
    return _lib


def _ptr(a, ctype):
    if a is None:
        return None
    return a.ctypes.data_as(ctypes.POINTER(ctype))


def fmt(name_or_fmt) -> Fmt:
    return FORMATS[name_or_fmt] if isinstance(name_or_fmt, str) else name_or_fmt


# ---- scalar formats ----
def e2m1_value(code: int) -> float:
    return lib().orc_e2m1_value(code)


def e2m1_encode(x: float) -> int:
    return lib().orc_e2m1_encode(x)


def e4m3_value(b: int) -> float:
    return lib().orc_e4m3_value(b)


def e4m3_encode(x: float) -> int:
    return lib().orc_e4m3_encode(x)


def e8m0_exponent(amax: float, rule: int, qmax: float = 0.0, elem: int = ELEM_E2M1) -> int:
    return lib().orc_e8m0_exponent(amax, rule, qmax, elem)


def quant_block(x, f):
    """Quantize one block; returns (codes uint8[n], scale byte, scale float)."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    codes = np.zeros(len(x), dtype=np.uint8)
    sb = ctypes.c_uint8(0)
    s = lib().orc_quant_block(_ptr(x, ctypes.c_float), len(x), ctypes.byref(fmt(f)),
                              _ptr(codes, ctypes.c_uint8), ctypes.byref(sb))
    return codes, sb.value, s


# ---- tensors ----
def quantize_rows(x, f):
    """x: float32 [..., d] -> (codes uint8 [..., d], scales uint8 [..., d/block])."""
    f = fmt(f)
    x = np.ascontiguousarray(x, dtype=np.float32)
    d = x.shape[-1]
    rows = x.size // d
    codes = np.zeros(x.shape, dtype=np.uint8)
    scales = np.zeros(x.shape[:-1] + (d // f.block,), dtype=np.uint8)
    lib().orc_quantize_rows(_ptr(x, ctypes.c_float), rows, d, ctypes.byref(f),
                            _ptr(codes, ctypes.c_uint8), _ptr(scales, ctypes.c_uint8))
    return codes, scales


def dequant_rows(codes, scales, f):
    f = fmt(f)
    codes = np.ascontiguousarray(codes, dtype=np.uint8)
    scales = np.ascontiguousarray(scales, dtype=np.uint8)
    d = codes.shape[-1]
    out = np.zeros(codes.shape, dtype=np.float32)
    lib().orc_dequant_rows(_ptr(codes, ctypes.c_uint8), _ptr(scales, ctypes.c_uint8), codes.size // d, d,
                           ctypes.byref(f), _ptr(out, ctypes.c_float))
    return out


def v_nblocks(N, doc_off, block):
    d = None if doc_off is None else np.ascontiguousarray(doc_off, dtype=np.int32)
    return lib().orc_v_nblocks(N, _ptr(d, ctypes.c_int32), 0 if d is None else len(d) - 1, block)


def quantize_cols(x, f, doc_off=None):
    """x: float32 [N, d] (one head) -> (codes uint8 [d, N], scales uint8 [d, nblk])."""
    f = fmt(f)
    x = np.ascontiguousarray(x, dtype=np.float32)
    N, d = x.shape
    dd = None if doc_off is None else np.ascontiguousarray(doc_off, dtype=np.int32)
    nd = 0 if dd is None else len(dd) - 1
    nblk = v_nblocks(N, dd, f.block)
    codes = np.zeros((d, N), dtype=np.uint8)
    scales = np.zeros((d, nblk), dtype=np.uint8)
    lib().orc_quantize_cols(_ptr(x, ctypes.c_float), N, d, _ptr(dd, ctypes.c_int32), nd, ctypes.byref(f),
                            _ptr(codes, ctypes.c_uint8), _ptr(scales, ctypes.c_uint8))
    return codes, scales


def dequant_cols(codes, scales, f, doc_off=None):
    """codes [d, N], scales [d, nblk] -> float32 [N, d]."""
    f = fmt(f)
    d, N = codes.shape
    dd = None if doc_off is None else np.ascontiguousarray(doc_off, dtype=np.int32)
    nd = 0 if dd is None else len(dd) - 1
    out = np.zeros((N, d), dtype=np.float32)
    lib().orc_dequant_cols(_ptr(np.ascontiguousarray(codes), ctypes.c_uint8),
                           _ptr(np.ascontiguousarray(scales), ctypes.c_uint8), N, d, _ptr(dd, ctypes.c_int32),
                           nd, ctypes.byref(f), _ptr(out, ctypes.c_float))
    return out


def attention(Q, K, V, pmode, pfmt=None, causal=False, sm_scale=None, kv_tile=128, doc_off=None,
              rows=None, bias=None, vkey=None, vkey_exp=None, exp_mode="exact", score_rounds=2, q_tile=256):
    """Q [B,Hq,N,d], K/V [B,Hkv,N,d] float32 (dequantized); bias: None or float32 [B,Hq,N]
    added to each key's scores; vkey [B,Hkv,N,d] / vkey_exp [B,Hkv,N]: the per-key form
    of V used on each row's diagonal tiles (causal only): the key tiles that start inside
    the row's query tile of q_tile rows; exp_mode: "exact", "mitchell" or "schraudolph"
    (the exponential of P~); score_rounds: FP32 roundings in the score sums of the
    implementation under test (flip-budget window only).
    Returns (O [nrows,d], lse, fb)."""
    Q = np.ascontiguousarray(Q, dtype=np.float32)
    K = np.ascontiguousarray(K, dtype=np.float32)
    V = np.ascontiguousarray(V, dtype=np.float32)
    B, Hq, N, d = Q.shape
    Hkv = K.shape[1]
    if sm_scale is None:
        sm_scale = 1.0 / np.sqrt(d)
    pf = fmt(pfmt) if pfmt is not None else Fmt(0, 0, 32, 0, 0.0)
    p = AttnParams(pmode, pf, int(bool(causal)), float(sm_scale), kv_tile, EXP_MODES[exp_mode], score_rounds,
                   q_tile)
    r = None if rows is None else np.ascontiguousarray(rows, dtype=np.int64)
    nrows = B * Hq * N if r is None else len(r)
    O = np.zeros((nrows, d), dtype=np.float32)
    lse = np.zeros(nrows, dtype=np.float32)
    fb = np.zeros(nrows, dtype=np.float64)
    dd = None if doc_off is None else np.ascontiguousarray(doc_off, dtype=np.int32)
    bb = None if bias is None else np.ascontiguousarray(bias, dtype=np.float32)
    if bb is not None and bb.shape != (B, Hq, N):
        raise ValueError("bias must be [B, Hq, N]")
    vk = None if vkey is None else np.ascontiguousarray(vkey, dtype=np.float32)
    ek = None if vkey_exp is None else np.ascontiguousarray(vkey_exp, dtype=np.int32)
    if (vk is None) != (ek is None):
        raise ValueError("vkey and vkey_exp go together")
    rc = lib().orc_attention_ex(_ptr(Q, ctypes.c_float), _ptr(K, ctypes.c_float), _ptr(V, ctypes.c_float),
                                _ptr(bb, ctypes.c_float), _ptr(vk, ctypes.c_float), _ptr(ek, ctypes.c_int32), B, Hq,
                                Hkv, N, d, _ptr(dd, ctypes.c_int32), 0 if dd is None else len(dd) - 1,
                                ctypes.byref(p), _ptr(r, ctypes.c_int64), nrows, _ptr(O, ctypes.c_float),
                                _ptr(lse, ctypes.c_float), _ptr(fb, ctypes.c_double))
    if rc != 0:
        raise ValueError(f"orc_attention failed with {rc}")
    return O, lse, fb


# ---- outlier pre-processing (one head at a time) ----
def _docs(doc_off):
    dd = None if doc_off is None else np.ascontiguousarray(doc_off, dtype=np.int32)
    return dd, (0 if dd is None else len(dd) - 1)


def channel_mean(x, doc_off=None):
    """x: float32 [N, d] -> per-document channel means float32 [max(ndocs,1), d]."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    N, d = x.shape
    dd, nd = _docs(doc_off)
    mean = np.zeros((max(nd, 1), d), dtype=np.float32)
    lib().orc_channel_mean(_ptr(x, ctypes.c_float), N, d, _ptr(dd, ctypes.c_int32), nd, _ptr(mean, ctypes.c_float))
    return mean


def preprocess_rows(x, mean=None, doc_off=None, hadamard=False):
    """x: float32 [N, d] -> fl32(((x - mean[doc]) H) / sqrt(d)) (rotation optional), [N, d]."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    N, d = x.shape
    dd, nd = _docs(doc_off)
    m = None if mean is None else np.ascontiguousarray(mean, dtype=np.float32)
    out = np.zeros((N, d), dtype=np.float32)
    lib().orc_preprocess_rows(_ptr(x, ctypes.c_float), N, d, _ptr(m, ctypes.c_float), _ptr(dd, ctypes.c_int32), nd,
                              int(bool(hadamard)), _ptr(out, ctypes.c_float))
    return out


def center_comp(qmean, K, kmean, doc_off=None):
    """qmean, kmean: float32 [max(ndocs,1), d]; K: float32 [N, d] -> delta float32 [N]."""
    K = np.ascontiguousarray(K, dtype=np.float32)
    N, d = K.shape
    dd, nd = _docs(doc_off)
    delta = np.zeros(N, dtype=np.float32)
    lib().orc_center_comp(_ptr(np.ascontiguousarray(qmean, dtype=np.float32), ctypes.c_float),
                          _ptr(K, ctypes.c_float), _ptr(np.ascontiguousarray(kmean, dtype=np.float32), ctypes.c_float),
                          N, d, _ptr(dd, ctypes.c_int32), nd, _ptr(delta, ctypes.c_float))
    return delta


# ---- causally safe per-key form of a 4-bit V ----
def quantize_keys(x, f):
    """x float32 [N, d] -> (codes uint8 [N, d], exponents int32 [N]): one E8M0 scale per
    token over its d channels (f's rule), element codes of x / 2^e."""
    f = fmt(f)
    x = np.ascontiguousarray(x, dtype=np.float32)
    N, d = x.shape
    codes = np.zeros((N, d), np.uint8)
    ek = np.zeros(N, np.int32)
    lib().orc_quantize_keys(_ptr(x, ctypes.c_float), N, d, ctypes.byref(f), _ptr(codes, ctypes.c_uint8),
                            _ptr(ek, ctypes.c_int32))
    return codes, ek


def e2m1_values(codes):
    """E2M1 codes -> their values (unit scale), float32"""
    table = np.array([e2m1_value(c) for c in range(16)], np.float32)
    return table[np.asarray(codes) & 15]


# ---- decode with split keys ----
def decode(Q, K, V, kv_len, pmode, pfmt=None, split=256, sm_scale=None, kv_tile=128, exp_mode="exact",
           score_rounds=2):
    """Q [B,Hq,R,d] (the R newest tokens), K/V [B,Hkv,N,d] dequantized float32, kv_len [B]:
    split-key decode merged by log-sum-exp.  Returns (O [B,Hq,R,d], lse [B,Hq,R], fb [B,Hq,R])."""
    Q = np.ascontiguousarray(Q, dtype=np.float32)
    K = np.ascontiguousarray(K, dtype=np.float32)
    V = np.ascontiguousarray(V, dtype=np.float32)
    B, Hq, R, d = Q.shape
    Hkv, N = K.shape[1], K.shape[2]
    if sm_scale is None:
        sm_scale = 1.0 / np.sqrt(d)
    pf = fmt(pfmt) if pfmt is not None else Fmt(0, 0, 32, 0, 0.0)
    p = AttnParams(pmode, pf, 1, float(sm_scale), kv_tile, EXP_MODES[exp_mode], score_rounds)
    kl = np.ascontiguousarray(kv_len, dtype=np.int32)
    O = np.zeros((B, Hq, R, d), np.float32)
    lse = np.zeros((B, Hq, R), np.float32)
    fb = np.zeros((B, Hq, R), np.float64)
    rc = lib().orc_decode(_ptr(Q, ctypes.c_float), _ptr(K, ctypes.c_float), _ptr(V, ctypes.c_float), B, Hq, Hkv, R,
                          N, d, _ptr(kl, ctypes.c_int32), split, ctypes.byref(p), _ptr(O, ctypes.c_float),
                          _ptr(lse, ctypes.c_float), _ptr(fb, ctypes.c_double))
    if rc != 0:
        raise ValueError(f"orc_decode failed with {rc}")
    return O, lse, fb


# ---- bit-level exponentials ----
def exp2_bits(t):
    """Mitchell's piecewise-linear 2^t read from a float's bits, with the clamp (orc_exp2_bits)."""
    f = lib().orc_exp2_bits
    f.restype, f.argtypes = ctypes.c_double, [ctypes.c_double]
    return np.array([f(float(v)) for v in np.ravel(t)], np.float64).reshape(np.shape(t))


def exp_offset(mode):
    """the offset delta of a bit-level mode ("mitchell", "schraudolph"; 0 for "exact")"""
    f = lib().orc_exp_offset
    f.restype, f.argtypes = ctypes.c_double, [ctypes.c_int]
    return f(EXP_MODES[mode])
