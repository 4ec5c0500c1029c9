"""Host-side checks of bench.py's counter tooling: kernel names from rocprofv3, per-dispatch
counter sums, the copy calibration, the per-kernel source sets and their hashes."""
import json

import bench


def test_short_name_strips_parameters_and_namespaces():
    raw = ("void vsa::(anonymous namespace)::attend_kernel<vsa::(anonymous namespace)::Bf16Core<128>, "
           "12, 4, 1, false>(vsa::Geo, int, unsigned short const*)")
    assert bench._short_name(raw) == "vsa::attend_kernel<vsa::Bf16Core<128>, 12, 4, 1, false>"
    assert bench._short_name("__amd_rocclr_copyBuffer") == "__amd_rocclr_copyBuffer"


def test_kernel_sources_follow_local_includes():
    base, srcs = bench._kernel_sources("vsa::attend_kernel<vsa::Bf16Core<128>, 12, 4, 1, false>")
    assert base == "attend_kernel"
    assert srcs[0].endswith("csrc/attend.hip")
    assert any(p.endswith("attn_core.h") for p in srcs) and any(p.endswith("include/vsa.h") for p in srcs)
    assert bench._kernel_sources("vsa::fine_attend_kernel<128, 2>")[1][0].endswith("csrc/fine.hip")
    assert bench._kernel_sources("at::native::elementwise_kernel<128>")[1] is None


def test_source_hash_ignores_comments_and_whitespace(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    (tmp_path / "a.hip").write_text("int f(int x) {\n  return x + 1;  // one\n}\n")
    (tmp_path / "b.hip").write_text("/* doc */ int f(int x)\n{ return x + 1; }\n")
    (tmp_path / "c.hip").write_text("int f(int x) { return x + 2; }\n")
    assert bench._src_hash(["a.hip"]) == bench._src_hash(["b.hip"])
    assert bench._src_hash(["a.hip"]) != bench._src_hash(["c.hip"])


def _csv(path, counter, rows):
    head = ("Correlation_Id,Dispatch_Id,Agent_Id,Queue_Id,Process_Id,Thread_Id,Grid_Size,Kernel_Id,"
            "Kernel_Name,Workgroup_Size,LDS_Block_Size,Scratch_Size,VGPR_Count,Accum_VGPR_Count,"
            "SGPR_Count,Counter_Name,Counter_Value,Start_Timestamp,End_Timestamp\n")
    lines = [head]
    for disp, name, val in rows:
        lines.append(f'{disp},{disp},"Agent 1",1,1,1,64,1,"{name}",64,0,0,8,0,16,"{counter}",{val},0,1\n')
    path.write_text("".join(lines))


def test_write_traffic_calibrates_and_takes_medians(tmp_path, monkeypatch):
    out = tmp_path / "traffic.json"
    monkeypatch.setattr(bench, "TRAFFIC_JSON", str(out))
    k = "void vsa::(anonymous namespace)::layout_kernel<128, false>(vsa::Geo)"
    copy = "__amd_rocclr_copyBuffer"
    # the copy of 1 GiB reads as half its bytes on FETCH_SIZE, all of them on WRITE_SIZE; a
    # dispatch may report a counter in several rows (summed); the median of three dispatches
    _csv(tmp_path / "f.csv", "FETCH_SIZE", [(1, copy, 524288.0), (2, k, 100.0), (2, k, 100.0),
                                             (3, k, 300.0), (4, k, 900.0), (5, copy, 10.0)])
    _csv(tmp_path / "w.csv", "WRITE_SIZE", [(1, copy, 1048576.0), (2, k, 50.0), (3, k, 60.0),
                                             (4, k, 70.0)])
    bench.write_traffic("toy", str(tmp_path / "f.csv"), str(tmp_path / "w.csv"), "cmd")
    data = json.loads(out.read_text())["workloads"]["toy"]
    assert data["calibration"]["fetch_factor"] == 0.5 and data["calibration"]["write_factor"] == 1.0
    e = data["kernels"]["vsa::layout_kernel<128, false>"]
    # dispatch 2 sums its two rows (200); the median of 200, 300, 900 is 300
    assert e["dispatches"] == 3 and e["fetch_kib_raw"] == 300.0 and e["write_kib_raw"] == 60.0
    assert e["fetch_bytes"] == 300 * 1024 * 2 and e["write_bytes"] == 60 * 1024
    assert e["bytes_per_launch"] == e["fetch_bytes"] + e["write_bytes"]
    assert copy not in data["kernels"]  # only the library's own kernels are recorded
    # the stage lookup checks the kernel's current sources
    assert bench._traffic("layout_kernel<", "toy") == e["bytes_per_launch"]
    assert bench._traffic("attend_kernel<", "toy") is None
