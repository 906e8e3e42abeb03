"""Host-side pieces of bench.py that need no GPU."""
from __future__ import annotations

import subprocess
import sys

import bench


def test_traffic_summary_matches_current_kernel_or_is_ignored(tmp_path):
    got = bench.measured_traffic()
    # either the committed summary was taken on this exact kernel source, or it is ignored
    for key, val in got.items():
        assert key.count(":") == 1 and val > 0
    fake = tmp_path / "t.txt"
    fake.write_text("source_sha256 = " + "0" * 64 + "\ntraffic_bytes[f16:8192] = 5\n")
    assert bench.measured_traffic(str(fake)) == {}


def test_source_hash_ignores_comments_not_code(tmp_path):
    src = ("__device__ int f(int x) { return x + 1; }  // one\n"
           "// host side\nstruct Config {\n  int a;  // field\n};\nint validate(")
    a, b, c = (tmp_path / n for n in ("a.hip", "b.hip", "c.hip"))
    a.write_text(src)
    b.write_text(src.replace("// one", "// another comment").replace("  int a;", "\n    int a;\n"))
    c.write_text(src.replace("x + 1", "x + 2"))
    ha, hb, hc = (bench.kernel_source_sha(str(p)) for p in (a, b, c))
    assert ha == hb and ha != hc


def test_multi_gpu_request_is_refused():
    r = subprocess.run([sys.executable, bench.__file__, "--gpus", "2"], capture_output=True, text=True)
    assert r.returncode == 2 and "one GPU" in r.stderr


def test_trace_summary_of_a_small_trace(tmp_path):
    csv = tmp_path / "k.csv"
    csv.write_text('"Kernel_Name","Grid_Size","Workgroup_Size","Start_Timestamp","End_Timestamp"\n'
                   '"void (anonymous namespace)::gemm_kernel<0, 256, 256, 128, 128, 4>((anonymous namespace)::Args)",262144,256,1000,3000\n'
                   '"void (anonymous namespace)::gemm_kernel<0, 256, 256, 128, 128, 4>((anonymous namespace)::Args)",262144,256,5000,9000\n')
    r = subprocess.run([sys.executable, bench.__file__, "--trace-summary", str(csv)], capture_output=True, text=True)
    assert r.returncode == 0 and "3.00" in r.stdout and "gemm_kernel<0, 256, 256, 128, 128, 4>" in r.stdout


def test_telemetry_is_absent_without_a_gpu():
    # amdsmi finds no device here: the section is reported as null, the step is never run
    ran = []
    assert bench.sample_power(lambda: ran.append(1), 1.0) is None
    assert not ran


def test_roofline_names_the_kernel_that_runs():
    # the library's host-side tile choice needs no GPU
    import precision_dense_gemm_amd as pd
    assert bench.kernel_name(pd, "f16", 8192) == "gemm_mf16_kernel"
    assert bench.kernel_name(pd, "i8", 8192) == "gemm_mf16_kernel"
    assert bench.kernel_name(pd, "i4", 8192) == "gemm_kernel"    # without a workspace: nibble planes
    assert bench.kernel_name(pd, "i4", 8192, "fp6") == "gemm_f6_kernel"
    assert bench.kernel_name(pd, "f16", 512) == "gemm_kernel"   # a smaller tile, 32 x 32 MFMAs
    assert bench.kernel_name(pd, "i8", 2048) == "gemm_mf16_kernel"   # 128 x 128, 16 x 16 MFMAs
    assert bench.kernel_name(pd, "i4", 2048) == "gemm_kernel"
    assert bench.kernel_name(pd, "f16", 1024) == "gemm_kernel"   # 64 x 64
