"""Host-side pieces of bench.py that decide what a result line reports: the source hash
that ties a committed profile's HBM traffic to the code it measured (comments do not
count, code does) and the traffic lookup that refuses a stale profile."""
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
