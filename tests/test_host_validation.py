"""Host-side argument checks of mxattn_fwd and mxattn_decode (include/mxattn.h: "host
validation runs first; on failure the call returns a negative status and enqueues
nothing").  No GPU is needed: every case below is rejected before any HIP call, so the
descriptors carry fake, suitably aligned device addresses that are never dereferenced.
"""
import ctypes

import pytest

INVALID, UNSUPPORTED, ALIGN, WORKSPACE = -1, -2, -3, -4
FAKE = 0x7F0000000000  # 16-byte aligned address, never touched by the host checks


@pytest.fixture(scope="module")
def mx():
    import microscaling_fp4_attention_amd as mx
    try:
        mx.lib()
    except ImportError as e:  # the library is built by __graft_entry__.build()
        pytest.skip(str(e))
    return mx


def qt(mx, role, fmt="mxfp4", B=1, H=4, N=1000, d=128, ndocs=1, addr=FAKE):
    t = mx.QTensorC()
    t.codes, t.scales = addr, addr + 0x100000
    t.fmt = mx.qfmt(fmt)
    t.role, t.ndocs, t.B, t.H, t.N, t.d = role, ndocs, B, H, N, d
    t.n_padded = (N + 127) // 128 * 128 if role != mx.ROLE_QK else N
    return t


def params(mx, pmode="pnq", pfmt="mxfp4", **kw):
    p = mx.FwdParams()
    p.pmode, p.pfmt, p.causal, p.sm_scale = mx.PMODES[pmode], mx.qfmt(pfmt), 0, 128 ** -0.5
    p.kv_tile, p.out_fp32, p.score_bias, p.vkey, p.exp_mode = 128, 1, None, None, mx.EXP_EXACT
    for k, v in kw.items():
        setattr(p, k, v)
    return p


def fwd(mx, q, k, v, p, ndocs=0, out=FAKE, os=(4 * 1000 * 128, 1000 * 128, 128, 1), ws=None, ws_bytes=0):
    by = ctypes.byref
    return mx.lib().mxattn_fwd(by(q) if q is not None else None, by(k), by(v), by(p), ndocs, out,
                               mx._i64(os), None, ws, ws_bytes, None)


def base(mx, **over):
    """a well-formed MXFP4 GQA problem (Hq 4, Hkv 2, N 1000); `over` replaces parts"""
    q = over.pop("q", qt(mx, mx.ROLE_QK))
    k = over.pop("k", qt(mx, mx.ROLE_QK, H=2))
    v = over.pop("v", qt(mx, mx.ROLE_V, H=2))
    p = over.pop("p", params(mx))
    return q, k, v, p, over


def test_fwd_descriptor_checks(mx):
    q, k, v, p, _ = base(mx)
    assert fwd(mx, None, k, v, p) == INVALID                               # null descriptor
    assert fwd(mx, qt(mx, mx.ROLE_V), k, v, p) == INVALID                  # Q with role V
    assert fwd(mx, q, k, qt(mx, mx.ROLE_QK, H=2), p) == INVALID            # V with role QK
    assert fwd(mx, qt(mx, mx.ROLE_QK, d=64), k, v, p) == UNSUPPORTED       # d != 128
    assert fwd(mx, qt(mx, mx.ROLE_QK, B=2), k, v, p) == INVALID            # batch mismatch
    assert fwd(mx, qt(mx, mx.ROLE_QK, N=999), k, v, p) == INVALID          # length mismatch
    assert fwd(mx, qt(mx, mx.ROLE_QK, H=3), k, v, p) == INVALID            # Hq not a multiple of Hkv
    assert fwd(mx, q, k, qt(mx, mx.ROLE_V, H=4), p) == INVALID             # K and V heads differ
    assert fwd(mx, q, qt(mx, mx.ROLE_QK, "mxfp4_uos", H=2), v, p) == UNSUPPORTED  # Q/K formats differ
    assert fwd(mx, qt(mx, mx.ROLE_QK, "fp8v"), qt(mx, mx.ROLE_QK, "fp8v", H=2), v, p) == UNSUPPORTED


def test_fwd_parameter_checks(mx):
    q, k, v, p, _ = base(mx)
    assert fwd(mx, q, k, v, params(mx, kv_tile=64)) == UNSUPPORTED
    for s in (0.0, -1.0, float("inf"), float("nan")):
        assert fwd(mx, q, k, v, params(mx, sm_scale=s)) == INVALID
    assert fwd(mx, q, k, v, p, ndocs=-1) == INVALID
    bad = params(mx)
    bad.pmode = 9
    assert fwd(mx, q, k, v, bad) == INVALID                                 # unknown P mode
    assert fwd(mx, q, k, v, params(mx, "fp8")) == UNSUPPORTED               # FP8 P needs an FP8 V
    assert fwd(mx, q, k, v, params(mx, pfmt="fp8v")) == UNSUPPORTED         # P block format must be 4-bit
    bad = params(mx)
    bad.exp_mode = 7
    assert fwd(mx, q, k, v, bad) == INVALID                                 # unknown exponential
    nv = qt(mx, mx.ROLE_V, "nvfp4", H=2)
    assert fwd(mx, q, k, nv, params(mx, exp_mode=mx.EXP_MITCHELL)) == UNSUPPORTED  # bit-level exp: E8M0 V only
    assert fwd(mx, q, k, v, p, os=(0, 0, 128, 2)) == INVALID                # inner output stride must be 1
    assert fwd(mx, q, k, v, p, os=(-1, 0, 128, 1)) == INVALID


def test_fwd_size_pointer_and_alignment_checks(mx):
    q, k, v, p, _ = base(mx)
    big = 1 << 24
    assert fwd(mx, qt(mx, mx.ROLE_QK, N=big + 1), qt(mx, mx.ROLE_QK, H=2, N=big + 1),
               qt(mx, mx.ROLE_V, H=2, N=big + 1), p) == UNSUPPORTED        # 32-bit head offsets
    assert fwd(mx, q, k, v, p, out=None) == INVALID
    assert fwd(mx, qt(mx, mx.ROLE_QK, addr=0), k, v, p) == INVALID          # null codes
    assert fwd(mx, qt(mx, mx.ROLE_QK, addr=FAKE + 8), k, v, p) == ALIGN     # codes not 16-byte aligned
    assert fwd(mx, q, k, v, p, out=FAKE + 4) == ALIGN
    assert fwd(mx, q, k, v, p, os=(4 * 1000 * 128, 1000 * 128, 130, 1)) == ALIGN  # row stride of 520 bytes
    bias = params(mx)
    bias.score_bias = FAKE + 4
    assert fwd(mx, q, k, v, bias) == ALIGN


def test_fwd_document_and_workspace_checks(mx):
    p = params(mx, causal=1)
    q = qt(mx, mx.ROLE_QK, N=1000)
    k = qt(mx, mx.ROLE_QK, H=2, N=1000)
    v3 = qt(mx, mx.ROLE_V, H=2, N=1000, ndocs=3)
    need = mx.fwd_workspace_bytes(1000, 3)
    assert fwd(mx, q, k, v3, p, ndocs=3, ws=None) == WORKSPACE              # no plan
    assert fwd(mx, q, k, v3, p, ndocs=3, ws=FAKE, ws_bytes=need - 1) == WORKSPACE
    assert fwd(mx, q, k, v3, p, ndocs=3, ws=FAKE + 8, ws_bytes=need) == ALIGN
    assert fwd(mx, q, k, qt(mx, mx.ROLE_V, H=2, N=1000, ndocs=2), p, ndocs=3, ws=FAKE, ws_bytes=need) == INVALID
    q2, k2 = qt(mx, mx.ROLE_QK, B=2), qt(mx, mx.ROLE_QK, B=2, H=2)
    assert fwd(mx, q2, k2, qt(mx, mx.ROLE_V, B=2, H=2, ndocs=3), p, ndocs=3, ws=FAKE, ws_bytes=need) == INVALID
    # the per-key V form: causal only, the same V slot layout, a 4-bit V with E8M0 scales
    vk = qt(mx, mx.ROLE_VKEY, H=2, N=1000)
    nc = params(mx, causal=0, vkey=ctypes.addressof(vk))
    assert fwd(mx, q, k, qt(mx, mx.ROLE_V, H=2), nc) == INVALID
    wrong = qt(mx, mx.ROLE_VKEY, H=2, N=1000)
    wrong.n_padded += 128
    assert fwd(mx, q, k, qt(mx, mx.ROLE_V, H=2), params(mx, causal=1, vkey=ctypes.addressof(wrong))) == INVALID
    fp8 = params(mx, "fp8", causal=1, vkey=ctypes.addressof(vk))
    assert fwd(mx, q, k, qt(mx, mx.ROLE_V, "fp8v", H=2), fp8) == UNSUPPORTED


def test_fwd_empty_problem_is_ok_without_device_work(mx):
    q, k, v, p, _ = base(mx)
    z = [qt(mx, r, H=h, N=0, addr=0) for r, h in ((mx.ROLE_QK, 4), (mx.ROLE_QK, 2), (mx.ROLE_V, 2))]
    assert fwd(mx, *z, p, out=None) == 0


def dec(mx, q, k, v, p, out=FAKE, os=(4 * 128, 128, 128, 1), ws=FAKE, ws_bytes=1 << 30):
    by = ctypes.byref
    return mx.lib().mxattn_decode(by(q), by(k), by(v), by(p), None, out, mx._i64(os), None, ws, ws_bytes, None)


def test_decode_checks(mx):
    k = qt(mx, mx.ROLE_QK, H=2, N=4096)
    v = qt(mx, mx.ROLE_V, H=2, N=4096)
    q = qt(mx, mx.ROLE_QK, H=8, N=1)                                        # one new row per request
    p = params(mx, causal=1)
    assert dec(mx, q, k, v, params(mx, causal=0)) == INVALID                # decode rows are causal
    assert dec(mx, q, k, v, params(mx, causal=1, exp_mode=mx.EXP_MITCHELL)) == UNSUPPORTED
    assert dec(mx, qt(mx, mx.ROLE_QK, H=8, N=9), k, v, p) == UNSUPPORTED    # 4 heads x 9 rows > 32 columns
    assert dec(mx, qt(mx, mx.ROLE_QK, H=8, N=4097), k, v, p) == UNSUPPORTED  # more rows than keys
    assert dec(mx, q, k, v, params(mx, "fp8", causal=1)) == UNSUPPORTED      # FP8 P needs an FP8 V
    nq, nk = qt(mx, mx.ROLE_QK, "nvfp4", H=8, N=1), qt(mx, mx.ROLE_QK, "nvfp4", H=2, N=4096)
    assert dec(mx, nq, nk, v, params(mx, "fp8", causal=1)) == UNSUPPORTED    # ... also with NVFP4 Q/K
    assert dec(mx, nq, k, qt(mx, mx.ROLE_V, "fp8v", H=2, N=4096), params(mx, "fp8", causal=1)) == UNSUPPORTED
    assert dec(mx, nq, nk, v, p) == UNSUPPORTED                              # NVFP4 Q/K decode with 4-bit P
    assert dec(mx, q, k, v, params(mx, pfmt="nvfp4", causal=1)) == UNSUPPORTED
    assert dec(mx, q, k, qt(mx, mx.ROLE_V, H=2, N=4096, ndocs=2), p) == INVALID
    need = mx.lib().mxattn_decode_workspace_bytes(1, 8, 1, 4096)
    assert dec(mx, q, k, v, p, ws=None) == WORKSPACE
    assert dec(mx, q, k, v, p, ws_bytes=need - 1) == WORKSPACE
    assert dec(mx, q, k, v, p, ws=FAKE + 4, ws_bytes=need) == ALIGN
    assert dec(mx, q, k, v, p, out=FAKE + 2) == ALIGN


def test_role_vt_checks(mx):
    # the tile-major V of the decode: role V's sizes, no documents, E8M0 per 32 (MXFP4 or FP8 V)
    assert mx.qtensor_bytes("mxfp4_uos", mx.ROLE_VT, 2, 3, 1000) == mx.qtensor_bytes("mxfp4_uos", mx.ROLE_V, 2, 3, 1000)
    with pytest.raises(mx.MxattnError) as e:
        mx.qtensor_bytes("mxfp4", mx.ROLE_VT, 1, 2, 1000, ndocs=3)
    assert e.value.status == INVALID
    with pytest.raises(mx.MxattnError) as e:  # E4M3 block scales have no tile-major form
        mx.qtensor_bytes("nvfp4", mx.ROLE_VT, 1, 2, 1000)
    assert e.value.status == UNSUPPORTED
    assert mx.qtensor_bytes("fp8v", mx.ROLE_VT, 2, 3, 1000) == mx.qtensor_bytes("fp8v", mx.ROLE_V, 2, 3, 1000)
    # the prefill takes role V only
    q, k, v, p, _ = base(mx)
    assert fwd(mx, q, k, qt(mx, mx.ROLE_VT, H=2), p) == INVALID


def test_grid_size_limits_are_unsupported(mx):
    """Launch grids of 16 threads per row (pre-quantizer, compensation) or per 4 rows (Q/K
    quantizer) use 32-bit thread ids: sizes past them are refused on the host as
    unsupported, before any device work (not reported later as a HIP error)."""
    by = ctypes.byref
    L = mx.lib()
    out = mx.QTensorC()
    out.codes, out.scales = FAKE, FAKE + 0x100000
    f = mx.qfmt("mxfp4")
    big = (1 << 20, 8, 128)  # B*H*N = 2^30 rows
    strides = mx._i64((8 * 128 * 128, 128 * 128, 128, 1))
    assert L.mxattn_quantize(FAKE, strides, *big, 128, mx.ROLE_QK, by(f), None, 0, by(out), None) == UNSUPPORTED
    pre = mx.PreProc()
    pre.mean, pre.hadamard = None, 1
    mid = (1 << 18, 8, 128)  # 2^28 rows
    assert L.mxattn_quantize_pre(FAKE, strides, *mid, 128, mx.ROLE_QK, by(f), by(pre), None, 0, by(out),
                                 None) == UNSUPPORTED
    assert L.mxattn_center_comp(FAKE, FAKE, strides, FAKE, 1 << 18, 8, 8, 128, 128, None, 0, FAKE,
                                None) == UNSUPPORTED


def test_forced_launch_failure_reports_hip_error(mx):
    """The test hook makes the next submission fail after the host checks: the call
    returns MXATTN_E_HIP and mxattn_last_error() names the call and the HIP error; the
    binding raises MxattnError with that text.  No device work is made.  The hook and
    the error text are per thread: the case runs on a thread of its own and leaves this
    one's state untouched."""
    import threading
    by = ctypes.byref
    L = mx.lib()
    q, k, v, p, _ = base(mx)
    before = L.mxattn_last_error()
    failures = []

    def case():
        try:
            assert L.mxattn_debug_fail_launches(1) == 0
            assert fwd(mx, q, k, v, p) == -5
            err = L.mxattn_last_error().decode()
            assert "mxattn_fwd launch" in err, err
            assert L.mxattn_last_hip_error().decode() == err  # the same text under both names
            assert L.mxattn_debug_fail_launches(0) == 0  # the one forced failure was used
            # the plan builder's copy takes the same path
            cu = (ctypes.c_int32 * 3)(0, 500, 1000)
            L.mxattn_debug_fail_launches(1)
            ws = mx.fwd_workspace_bytes(1000, 2)
            assert L.mxattn_fwd_plan(cu, 2, 1000, 1, FAKE, ws, None) == -5
            assert "mxattn_fwd_plan copy" in L.mxattn_last_error().decode()
            with pytest.raises(mx.MxattnError) as ei:
                L.mxattn_debug_fail_launches(1)
                mx._check(fwd(mx, q, k, v, p), "mxattn_fwd")
            assert ei.value.status == mx.E_HIP and "mxattn_fwd launch" in str(ei.value)
            L.mxattn_debug_fail_launches(0)
        except BaseException as e:  # reported on the test's own thread
            failures.append(e)

    t = threading.Thread(target=case)
    t.start()
    t.join()
    if failures:
        raise failures[0]
    assert L.mxattn_last_error() == before
    assert L.mxattn_debug_fail_launches(0) == 0


def test_unquantized_route_checks(mx):
    """Q, K and V in bf16 (scale NONE) with pmode NONE is the unquantized route; any
    mix with quantized operands or P modes is unsupported.  Acceptance is seen through
    the launch hook: the call passes its host checks and stops at the forced failure."""
    L = mx.lib()
    qb, kb = qt(mx, mx.ROLE_QK, "bf16"), qt(mx, mx.ROLE_QK, "bf16", H=2)
    vb = qt(mx, mx.ROLE_V, "bf16", H=2)
    vb.n_padded = 1000
    pn = params(mx, "none", "bf16")
    os = (4 * 1000 * 128, 1000 * 128, 128, 1)
    rcs = []

    def accepted():  # on a thread of its own: the hook and the error text are per thread
        L.mxattn_debug_fail_launches(1)
        rcs.append(fwd(mx, qb, kb, vb, pn, os=os))
        L.mxattn_debug_fail_launches(0)

    import threading
    t = threading.Thread(target=accepted)
    t.start()
    t.join()
    assert rcs == [-5]                                                             # accepted
    q, k, v, p, _ = base(mx)
    assert fwd(mx, qb, kb, vb, params(mx, "pnq", "mxfp4")) == UNSUPPORTED          # quantized P on bf16
    assert fwd(mx, q, k, v, pn) == UNSUPPORTED                                     # P NONE on quantized
    assert fwd(mx, qb, kb, v, pn) == UNSUPPORTED                                   # mixed V
    assert fwd(mx, qb, kb, vb, params(mx, "none", "bf16", exp_mode=mx.EXP_MITCHELL)) == UNSUPPORTED
    bad = params(mx, "none", "bf16")
    bad.pmode = 9
    assert fwd(mx, qb, kb, vb, bad) == INVALID
    cb, sb, npad = ctypes.c_size_t(), ctypes.c_size_t(), ctypes.c_int64()
    f = mx.qfmt("bf16")
    by = ctypes.byref
    assert L.mxattn_qtensor_bytes(by(f), mx.ROLE_VT, 1, 2, 100, 128, 0, by(cb), by(sb), by(npad)) == UNSUPPORTED
    g = mx.qfmt("bf16")
    g.scale = mx.SCALE_E8M0
    assert L.mxattn_qtensor_bytes(by(g), mx.ROLE_QK, 1, 2, 100, 128, 0, by(cb), by(sb), by(npad)) == INVALID
    assert L.mxattn_qtensor_bytes(by(f), mx.ROLE_V, 1, 2, 100, 128, 5, by(cb), by(sb), by(npad)) == 0
    assert (cb.value, sb.value, npad.value) == (2 * 100 * 128 * 2, 0, 100)
