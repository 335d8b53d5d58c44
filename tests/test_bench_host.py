"""Host-side logic of bench.py (no GPU): the rocprofv3 summaries that the
committed profiles come from, and the rule that a traffic figure is reported
only for the kernel source it was measured on."""
import csv
import json
import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402

POOL = "void ct::(anonymous namespace)::avgpool3d_k3s2p1_vec_kernel<false>(float const*, float*)"
CONV = "void ct::(anonymous namespace)::convT1d_f32_wave_kernel<32, 5, 3, 4, 8>(float const*)"
COPY = "__amd_rocclr_copyBuffer"


def _write_csv(path, fields, rows):
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=fields)
        w.writeheader()
        w.writerows(rows)


def test_kernel_names_map_to_ops():
    assert bench.kernel_key(POOL)[0] == "avgpool3d"
    assert bench.kernel_key("ct::avgpool3d_k3s2p1_elem_kernel(...)")[0] == "avgpool3d"
    assert bench.kernel_key(CONV)[0] == "convT1d"
    assert bench.kernel_key("ct::avgpool3d_generic_kernel<2>")[0] == "avgpool3d_generic"
    assert bench.kernel_key(COPY) is None


def test_summarize_trace_averages_durations(tmp_path, capsys):
    rows = [{"Kernel_Name": POOL, "Start_Timestamp": 0, "End_Timestamp": 1600000},
            {"Kernel_Name": POOL, "Start_Timestamp": 5000000, "End_Timestamp": 6610000},
            {"Kernel_Name": CONV, "Start_Timestamp": 0, "End_Timestamp": 700000}]
    _write_csv(tmp_path / "kt_kernel_trace.csv", ["Kernel_Name", "Start_Timestamp", "End_Timestamp"], rows)
    bench.summarize_trace(str(tmp_path))
    out = capsys.readouterr().out
    pool = [l for l in out.splitlines() if l.startswith("| avgpool3d")][0].split("|")
    assert pool[2].strip() == "2" and pool[3].strip() == "1605.0"
    assert pool[4].strip() == "1600.0" and pool[5].strip() == "1610.0"
    # algorithmic bytes per launch / average duration
    assert pool[7].strip() == f"{9663676416 / 1605.0 / 1e3:.0f}"
    conv = [l for l in out.splitlines() if l.startswith("| convT1d")][0].split("|")
    assert conv[3].strip() == "700.0"


def test_summarize_counters_scales_by_the_copy(tmp_path, capsys):
    fields = ["Kernel_Name", "Counter_Name", "Counter_Value", "Grid_Size"]
    fd, wd = tmp_path / "f", tmp_path / "w"
    fd.mkdir(), wd.mkdir()
    # the 1 GiB copy reads 2^19 KiB and writes 2^20 KiB: read scale 2, write scale 1;
    # a small upload (grid below 2^17) must not count as the calibration copy
    _write_csv(fd / "p_counter_collection.csv", fields, [
        {"Kernel_Name": COPY, "Counter_Name": "FETCH_SIZE", "Counter_Value": 524288, "Grid_Size": 131072},
        {"Kernel_Name": COPY, "Counter_Name": "FETCH_SIZE", "Counter_Value": 10, "Grid_Size": 64},
        {"Kernel_Name": POOL, "Counter_Name": "FETCH_SIZE", "Counter_Value": 4000000, "Grid_Size": 524288},
        {"Kernel_Name": POOL, "Counter_Name": "FETCH_SIZE", "Counter_Value": 4200000, "Grid_Size": 524288}])
    _write_csv(wd / "p_counter_collection.csv", fields, [
        {"Kernel_Name": COPY, "Counter_Name": "WRITE_SIZE", "Counter_Value": 1048576, "Grid_Size": 131072},
        {"Kernel_Name": POOL, "Counter_Name": "WRITE_SIZE", "Counter_Value": 1048576, "Grid_Size": 524288}])
    dst = tmp_path / "traffic.json"
    bench.summarize_counters(str(fd), str(wd), dst=str(dst))
    t = json.load(open(dst))["avgpool3d"]
    assert t["fetch_scale"] == 2.0 and t["write_scale"] == 1.0
    assert t["read_bytes"] == 4100000 * 1024 * 2
    assert t["write_bytes"] == 1 << 30
    assert t["bytes_per_launch"] == t["read_bytes"] + t["write_bytes"]
    assert t["source"] == "avgpool3d.hip"
    assert t["source_sha256_16"] == bench.source_hash("avgpool3d")


def test_summarize_counters_needs_the_copy(tmp_path):
    fields = ["Kernel_Name", "Counter_Name", "Counter_Value", "Grid_Size"]
    _write_csv(tmp_path / "c.csv", fields, [
        {"Kernel_Name": POOL, "Counter_Name": "FETCH_SIZE", "Counter_Value": 1, "Grid_Size": 1}])
    with pytest.raises(SystemExit):
        bench.summarize_counters(str(tmp_path), str(tmp_path), dst=str(tmp_path / "t.json"))


def test_traffic_reported_only_for_the_measured_source(tmp_path, monkeypatch):
    src_dir = tmp_path / "transposed_conv_pooling_amd" / "csrc"
    src_dir.mkdir(parents=True)
    (tmp_path / "profiles").mkdir()
    (src_dir / "avgpool3d.hip").write_text("kernel v1\n")
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    h = bench.source_hash("avgpool3d")
    json.dump({"avgpool3d": {"bytes_per_launch": 123, "source_sha256_16": h}},
              open(tmp_path / "profiles" / "traffic.json", "w"))
    assert bench.measured_traffic("avgpool3d") == 123
    (src_dir / "avgpool3d.hip").write_text("kernel v2\n")      # source changed since
    assert bench.measured_traffic("avgpool3d") is None


def test_more_than_one_gpu_exits_with_a_message():
    import subprocess
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode != 0
    assert "exactly one GPU" in r.stdout + r.stderr


def test_every_traced_kernel_maps_to_an_op():
    """Each kernel named in the committed kernel-trace summaries resolves to an
    op, a source file and its algorithmic bytes (a renamed or new kernel that
    the table misses would drop out of the traffic and roofline figures)."""
    import re
    names = set()
    for f in ("bench_kernel_trace.md", "extra_ops_kernel_trace.md"):
        text = open(os.path.join(bench.ROOT, "profiles", f)).read()
        names |= set(re.findall(r"\(`(ct::[^`]+)`\)", text))
    assert names, "no kernel names found in the trace summaries"
    for n in sorted(names):
        key = bench.kernel_key(n)
        assert key is not None, n
        op, src, nbytes = key
        assert op and nbytes > 0 and os.path.exists(
            os.path.join(bench.ROOT, "transposed_conv_pooling_amd", "csrc", src)), (n, key)


def test_rotation_keeps_every_call_cold():
    """Buffer sets per op: a set whose traffic exceeds 512 MB alone is enough;
    otherwise at least 4 sets, more than 512 MB in all and more than 512 MB of
    inputs alone (the fused workloads' inputs are 25 MB and 17 MB)."""
    import bench
    mb = 1 << 20
    assert bench.rotation_count(1200 * mb, 25 * mb) == 1
    assert bench.rotation_count(9600 * mb) == 1
    for set_mb, in_mb in [(137, 24), (72, 16), (152, 24), (200, 190), (1, 1)]:
        n = bench.rotation_count(set_mb * mb, in_mb * mb)
        assert n >= 4 and n * set_mb * mb > bench.COLD_BYTES and n * in_mb * mb > bench.COLD_BYTES
