"""The C ABI without a GPU: the built library loads, exports every function that
include/mxattn.h declares, reports the header's ABI version, and its host-side
validation answers as documented (calls that return before any HIP call)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "mxattn.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)  # drop comments
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[a-z_0-9]+\s*\*?\s*(mxattn_[a-z_0-9]+)\s*\(", text, flags=re.M)))


@pytest.fixture(scope="module")
def mx():
    import microscaling_fp4_attention_amd as m
    if not os.path.exists(m.LIB_PATH):
        pytest.skip("libmxattn.so is not built (run __graft_entry__.build())")
    return m


def test_header_declares_the_entry_points():
    names = declared_functions()
    for n in ["mxattn_quantize", "mxattn_quantize_pre", "mxattn_channel_mean", "mxattn_center_comp", "mxattn_fwd",
              "mxattn_fwd_plan", "mxattn_fwd_workspace_bytes", "mxattn_qtensor_bytes", "mxattn_abi_version",
              "mxattn_status_str", "mxattn_last_error"]:
        assert n in names, n


def test_library_exports_every_declared_symbol(mx):
    lib = ctypes.CDLL(mx.LIB_PATH)
    missing = [n for n in declared_functions() if not hasattr(lib, n)]
    assert not missing, missing


def test_abi_version_matches_header(mx):
    v = int(re.search(r"#define MXATTN_ABI_VERSION (\d+)", open(HEADER).read()).group(1))
    assert mx.lib().mxattn_abi_version() == v == mx.ABI_VERSION


def test_status_strings(mx):
    for code in (0, -1, -2, -3, -4, -5):
        assert mx.lib().mxattn_status_str(code)
    assert mx.lib().mxattn_last_error() == b""


def test_host_validation(mx):
    # sizes: MXFP4 role QK = 64 code bytes + 4 scale bytes per token; role V pads to 128 slots
    cb, sb, npad = mx.qtensor_bytes("mxfp4", mx.ROLE_QK, 2, 3, 100)
    assert (cb, sb, npad) == (2 * 3 * 100 * 64, 2 * 3 * 100 * 4, 100)
    cb, sb, npad = mx.qtensor_bytes("mxfp4", mx.ROLE_V, 1, 2, 300, ndocs=3)
    assert npad == 512 and cb == 2 * 128 * 512 // 2 and sb == 2 * 128 * 512 // 32
    with pytest.raises(mx.MxattnError) as e:
        mx.qtensor_bytes("mxfp4", mx.ROLE_QK, 1, 1, 10, d=64)
    assert e.value.status == -2  # d != 128 is unsupported
    # a zero-sized tensor is quantized without any device work
    L = mx.lib()
    desc = mx.QTensorC()
    f = mx.qfmt("mxfp4")
    rc = L.mxattn_quantize(None, mx._i64([0, 0, 128, 1]), 0, 1, 5, 128, mx.ROLE_QK, ctypes.byref(f), None, 0,
                           ctypes.byref(desc), None)
    assert rc == 0 and desc.N == 5
    # role V cannot be pre-processed; bad strides are rejected before any launch
    pre = mx.PreProc(None, 1)
    assert L.mxattn_quantize_pre(None, mx._i64([0, 0, 128, 1]), 1, 1, 5, 128, mx.ROLE_V, ctypes.byref(f),
                                 ctypes.byref(pre), None, 0, ctypes.byref(desc), None) == -1
    assert L.mxattn_channel_mean(None, mx._i64([0, 0, 128, 2]), 1, 1, 5, 128, None, 0, None, None) == -1
    assert L.mxattn_center_comp(None, None, mx._i64([0, 0, 128, 1]), None, 1, 3, 2, 5, 128, None, 0, None,
                                None) == -1  # Hq not a multiple of Hkv
    assert mx.fwd_workspace_bytes(1000, 0) == 0 and mx.fwd_workspace_bytes(1000, 4) > 0


def test_struct_layouts_match_the_header(mx, tmp_path):
    """The binding's ctypes structures have the C structures' sizes and field offsets
    (a C program built from include/mxattn.h with gcc prints them)."""
    import subprocess
    src = tmp_path / "layout.c"
    src.write_text("""#include <stddef.h>
#include <stdio.h>
#include "mxattn.h"
#define F(T, f) printf(#T " " #f " %zu\\n", offsetof(T, f))
int main(void) {
  printf("mxattn_fwd_params size %zu\\n", sizeof(mxattn_fwd_params));
  printf("mxattn_qtensor size %zu\\n", sizeof(mxattn_qtensor));
  printf("mxattn_preproc size %zu\\n", sizeof(mxattn_preproc));
  F(mxattn_fwd_params, pmode); F(mxattn_fwd_params, pfmt); F(mxattn_fwd_params, causal);
  F(mxattn_fwd_params, sm_scale); F(mxattn_fwd_params, kv_tile); F(mxattn_fwd_params, out_fp32);
  F(mxattn_fwd_params, score_bias); F(mxattn_fwd_params, vkey); F(mxattn_fwd_params, exp_mode);
  F(mxattn_qtensor, codes); F(mxattn_qtensor, scales); F(mxattn_qtensor, fmt); F(mxattn_qtensor, role);
  F(mxattn_qtensor, ndocs); F(mxattn_qtensor, B); F(mxattn_qtensor, n_padded);
  F(mxattn_preproc, mean); F(mxattn_preproc, hadamard);
  return 0;
}
""")
    exe = tmp_path / "layout"
    subprocess.run(["gcc", "-std=c99", "-I", os.path.join(ROOT, "include"), str(src), "-o", str(exe)], check=True)
    lines = subprocess.run([str(exe)], check=True, capture_output=True, text=True).stdout.split("\n")
    py = {"mxattn_fwd_params": mx.FwdParams, "mxattn_qtensor": mx.QTensorC, "mxattn_preproc": mx.PreProc}
    for line in filter(None, lines):
        t, f, v = line.split()
        if f == "size":
            assert ctypes.sizeof(py[t]) == int(v), t
        else:
            assert getattr(py[t], f).offset == int(v), (t, f)
