"""Host-side parts of bench.py (no GPU): the --gpus guard, the conversion of
rocprofv3 counter files into bytes per launch, the source-hash check that
voids stale traffic figures, and the CPU oracle baseline's sample."""
import csv
import json
import os
import subprocess
import sys

import pytest

import bench
import workloads as W

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
FIELDS = ["Correlation_Id", "Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"]


def write_counters(d, counter, rows):
    os.makedirs(d, exist_ok=True)
    with open(os.path.join(d, "run_counter_collection.csv"), "w", newline="") as fh:
        w = csv.DictWriter(fh, fieldnames=FIELDS)
        w.writeheader()
        for i, (name, val) in enumerate(rows):
            w.writerow({"Correlation_Id": i, "Dispatch_Id": i, "Kernel_Name": name,
                        "Counter_Name": counter, "Counter_Value": val})


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, cwd=ROOT)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def test_write_traffic_scales_by_the_copy_kernel(tmp_path, monkeypatch):
    nc = "void fa::fwd_wide_kernel<4, false, false>(fa::FwdParams)"
    ca = "void fa::fwd_wide_kernel<4, true, true>(fa::FwdParams)"
    cp = "__amd_rocclr_copyBuffer"
    # the copy moves 2^30 bytes each way; FETCH_SIZE reads half of it (x2),
    # WRITE_SIZE all of it (x1), in KiB
    # small copies (input set-up) come with the 1 GiB one; only the largest
    # sets the scale
    write_counters(tmp_path / "f", "FETCH_SIZE",
                   [(cp, 3.0), (nc, 1000.0), (nc, 1002.0), (ca, 500.0), (cp, 524288.0)])
    write_counters(tmp_path / "w", "WRITE_SIZE",
                   [(cp, 6.0), (nc, 300.0), (ca, 301.0), (cp, 1048576.0)])
    out_file = tmp_path / "traffic.json"
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(out_file))
    t = bench.write_traffic(str(tmp_path / "f"), str(tmp_path / "w"))
    assert t["scale"] == {"FETCH_SIZE": 2.0, "WRITE_SIZE": 1.0}
    k = t["kernels"]["fwd_noncausal_d128"]
    assert k["read_bytes"] == round(1001.0 * 1024 * 2)
    assert k["write_bytes"] == 300 * 1024
    assert k["bytes_per_launch"] == k["read_bytes"] + k["write_bytes"]
    assert t["kernels"]["fwd_causal_d128"]["read_bytes"] == 500 * 1024 * 2
    assert json.loads(out_file.read_text()) == t
    assert (k["unit"] == "fa_fwd_wide.hip"
            and k["source_hash"] == bench.kernel_source_hash("fa_fwd_wide.hip"))
    # read back only while the kernel's sources are unchanged
    assert bench.measured_traffic("fwd_noncausal_d128") == k["bytes_per_launch"]
    stale = json.loads(json.dumps(t))
    stale["kernels"]["fwd_noncausal_d128"]["source_hash"] = "0" * 16
    out_file.write_text(json.dumps(stale))
    assert bench.measured_traffic("fwd_noncausal_d128") is None
    assert bench.measured_traffic("fwd_causal_d128") is not None
    # counters of another instance under the same tag are not used either
    other = json.loads(json.dumps(t))
    other["kernels"]["fwd_noncausal_d128"]["kernel"] = "void fa::fwd_kernel<128, 8, 1, false, false>"
    out_file.write_text(json.dumps(other))
    assert bench.measured_traffic("fwd_noncausal_d128") is None


def test_write_traffic_needs_the_copy_kernel(tmp_path, monkeypatch):
    write_counters(tmp_path / "f", "FETCH_SIZE", [("fwd_kernel<128, 8, 1, false, false>", 1.0)])
    write_counters(tmp_path / "w", "WRITE_SIZE", [("fwd_kernel<128, 8, 1, false, false>", 1.0)])
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(tmp_path / "t.json"))
    with pytest.raises(SystemExit):
        bench.write_traffic(str(tmp_path / "f"), str(tmp_path / "w"))


def test_committed_traffic_file_is_well_formed():
    with open(bench.TRAFFIC_FILE) as fh:
        t = json.load(fh)
    for k in t["kernels"].values():
        assert len(k["source_hash"]) == 16 and k["unit"].endswith(".hip")
        assert k["bytes_per_launch"] == k["read_bytes"] + k["write_bytes"] > 0


def test_cpu_baseline_reports_its_sample():
    r = bench.cpu_baseline(W.WORKLOADS[1], budget_s=0.05)
    assert r["kind"] == "oracle" and r["unit"] == "TFLOP/s"
    assert r["value"] > 0 and r["cores"] >= 1
    assert "single_head_n256_d64" in r["sample"]


def test_source_hash_ignores_comments_only(tmp_path):
    src = tmp_path / "csrc"
    src.mkdir()
    (src / "k.hip").write_text("// header\nint f(int x) {  // doubled\n  return 2 * x;\n}\n")
    h0 = bench.kernel_source_hash("k.hip", str(src))
    (src / "k.hip").write_text("/* new\n   header */\n\nint f(int x) {\n  return 2 * x;  // twice\n}\n")
    assert bench.kernel_source_hash("k.hip", str(src)) == h0
    (src / "k.hip").write_text("int f(int x) {\n  return 3 * x;\n}\n")
    assert bench.kernel_source_hash("k.hip", str(src)) != h0


def test_source_hash_covers_the_unit_and_its_headers_only(tmp_path):
    src = tmp_path / "csrc"
    src.mkdir()
    (src / "a.hpp").write_text("int g();\n")
    (src / "b.hpp").write_text('#include "a.hpp"\n')
    (src / "k.hip").write_text('#include "b.hpp"\nint f();\n')
    (src / "other.hip").write_text("int h();\n")
    assert bench.unit_files("k.hip", str(src)) == ["a.hpp", "b.hpp", "k.hip"]
    h0 = bench.kernel_source_hash("k.hip", str(src))
    (src / "other.hip").write_text("int h2();\n")      # another unit: no effect
    assert bench.kernel_source_hash("k.hip", str(src)) == h0
    (src / "a.hpp").write_text("int g2();\n")          # an included header: stale
    assert bench.kernel_source_hash("k.hip", str(src)) != h0


def test_source_hash_does_not_depend_on_the_checkout_path(tmp_path):
    """The same sources hash the same from another directory (the build
    options name the checkout's include path)."""
    import shutil
    import subprocess
    import sys
    dst = tmp_path / "copy"
    dst.mkdir()
    # only what the hash reads: bench.py, its input module, the package
    # sources and build script, and the public header
    for f in ("bench.py", "workloads.py"):
        shutil.copy(os.path.join(ROOT, f), dst / f)
    shutil.copytree(os.path.join(ROOT, "include"), dst / "include")
    shutil.copytree(os.path.join(ROOT, "exact_attention_84_amd"), dst / "exact_attention_84_amd",
                    ignore=shutil.ignore_patterns("_build", "*.so", "__pycache__"))
    code = "import bench; print(bench.kernel_source_hash('fa_fwd.hip'))"
    a = subprocess.run([sys.executable, "-c", code], cwd=ROOT, capture_output=True, text=True)
    b = subprocess.run([sys.executable, "-c", code], cwd=dst, capture_output=True, text=True)
    assert a.stdout.strip() and a.stdout.strip() == b.stdout.strip(), (a.stderr, b.stderr)
