"""Host-side pieces of bench.py that decide what a result line reports: the counted
FLOP and the route peaks the roofline divides by, the source hash that ties a
committed profile's HBM traffic to the code it measured (comments do not count, code
does) and the traffic lookup that refuses a stale profile."""
import os
import sys

sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
import bench  # noqa: E402


def test_code_only_strips_comments_not_literals():
    text = ('int a = 1;  // note\n/* block\n   comment */ const char* s = "x // y \\" z";\n\n'
            "  char q = '/'; /* */ int b;\n")
    assert bench._code_only(text) == 'int a = 1;\n const char* s = "x // y \\" z";\n  char q = \'/\';  int b;'


def test_hash_follows_code_not_comments(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    src = tmp_path / "k.hip"
    src.write_text("__global__ void k(float* x) { x[0] = 1.0f; }\n")
    h0 = bench.kernel_source_sha256(["k.hip"])
    src.write_text("// a kernel\n__global__ void k(float* x) { x[0] = 1.0f; }  // one store\n\n")
    assert bench.kernel_source_sha256(["k.hip"]) == h0
    src.write_text("__global__ void k(float* x) { x[0] = 2.0f; }\n")
    assert bench.kernel_source_sha256(["k.hip"]) != h0


def test_stale_profile_reports_no_traffic(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    (tmp_path / "k.hip").write_text("__global__ void k() {}\n")
    prof = tmp_path / "p.txt"
    prof.write_text(f"traffic_bytes_per_launch = 123\nkernel_source_sha256 = {bench.kernel_source_sha256(['k.hip'])}\n")
    assert bench.read_traffic("p.txt", ["k.hip"]) == 123
    (tmp_path / "k.hip").write_text("__global__ void k() { }  // edited\n__device__ int z;\n")
    assert bench.read_traffic("p.txt", ["k.hip"]) is None


def test_counted_flop_follows_the_metric():
    """4 B H N^2 d for non-causal runs; causal and packed documents count the visible
    pairs, 4 H d sum L (L + 1) / 2 (the metric's dense figure halved on the diagonal)."""
    import numpy as np
    assert bench.counted_flop(1, 24, 32768, 128, False, None) == 4 * 24 * 32768 ** 2 * 128
    assert bench.counted_flop(2, 16, 4096, 128, True, None) == 4 * 2 * 16 * 128 * (4096 * 4097 / 2)
    doc = np.array([0, 3, 10, 10, 17])  # lengths 3, 7, 0, 7
    assert bench.counted_flop(1, 16, 17, 128, True, doc) == 4 * 16 * 128 * (6 + 28 + 0 + 28)
    assert bench.counted_flop(1, 16, 17, 128, False, doc) == 4 * 16 * 128 * (9 + 49 + 0 + 49)


def test_route_peaks():
    """Each product is half of the counted FLOP, so a route's peak is the harmonic
    combination of its two MFMA peaks."""
    name, peak = bench.route_peak("mxfp4_uos", "mxfp4_uos", "pnq", "mxfp4_uos")
    assert name == "QK fp4, PV fp4" and peak == bench.FP4_PEAK_TFLOPS
    name, peak = bench.route_peak("mxfp4", "mxfp4", "two_level", "nvfp4")
    assert name == "QK fp4, PV f16"
    assert abs(peak - 1.0 / (0.5 / bench.FP4_PEAK_TFLOPS + 0.5 / bench.BF16_PEAK_TFLOPS)) < 1e-9
    name, peak = bench.route_peak("nvfp4", "fp8v", "fp8", None)
    assert name == "QK f16, PV fp8"
    assert abs(peak - 1.0 / (0.5 / bench.BF16_PEAK_TFLOPS + 0.5 / bench.FP8_PEAK_TFLOPS)) < 1e-9
