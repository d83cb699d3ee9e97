"""Host-side helpers that read rocprofv3 output: the comment-free source hash
that ties a committed counter summary to the kernel it was measured on, and
bench.py's use of it."""
import os

from bit_quantized_expert_router_amd.profsum import code_sha256, strip_comments

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_strip_comments_keeps_code_and_literals():
    src = ('#include "a.h"  // header\n'
           '/* block\n   comment */ int x = 1;   \n'
           '\n'
           'const char* s = "http://x /* not */";  // tail\n'
           "char c = '/'; int y = 2 / 3; /* a */ int z;\n")
    assert strip_comments(src) == ('#include "a.h"\n'
                                   '  int x = 1;\n'
                                   'const char* s = "http://x /* not */";\n'
                                   "char c = '/'; int y = 2 / 3;   int z;\n")


def test_code_sha_ignores_comments_only(tmp_path):
    a, b, c = tmp_path / "a.hip", tmp_path / "b.hip", tmp_path / "c.hip"
    a.write_text("int f() { return 1; }  // one\n")
    b.write_text("// a different note\n\nint f() { return 1; }\n")
    c.write_text("int f() { return 2; }  // one\n")
    assert code_sha256([a]) == code_sha256([b])
    assert code_sha256([a]) != code_sha256([c])
    assert code_sha256([a, c]) != code_sha256([c, a])


def test_bench_reads_traffic_only_for_matching_sources(tmp_path, monkeypatch):
    import bench
    src = tmp_path / "k.hip"
    src.write_text("__global__ void k() {}\n")
    prof = tmp_path / "profiles"
    prof.mkdir()
    body = ("kernel: k\ntraffic_bytes_per_launch: 1234\nsources: k.hip\n"
            f"source_sha256: {code_sha256([src])}\n")
    (prof / "t.txt").write_text(body)
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    assert bench.pmc_traffic("t.txt", "k") == 1234.0
    assert bench.pmc_traffic("t.txt", "other") is None
    src.write_text("// note\n__global__ void k() {}\n")
    assert bench.pmc_traffic("t.txt", "k") == 1234.0
    src.write_text("__global__ void k() { }\n")
    assert bench.pmc_traffic("t.txt", "k") is None
    assert bench.pmc_traffic("missing.txt", "k") is None


def test_counters_summary(tmp_path):
    from bit_quantized_expert_router_amd.profsum import counters
    d = tmp_path / "run"
    d.mkdir()
    head = ("Correlation_Id,Dispatch_Id,Grid_Size,Kernel_Name,Counter_Name,Counter_Value,"
            "Start_Timestamp,End_Timestamp\n")
    rows = []
    name = '"void moeq2::(anonymous namespace)::prefill_gateup_kernel<12>(moeq2::LayerArgs)"'
    for did, t0 in ((1, 1000), (2, 5000)):
        # 2 us per dispatch; GRBM over 8 XCDs at 2.4 GHz; MFMA busy a quarter of 1024 SIMDs
        rows.append(f"{did},{did},4096,{name},GRBM_GUI_ACTIVE,{8 * 4800},{t0},{t0 + 2000}")
        rows.append(f"{did},{did},4096,{name},SQ_VALU_MFMA_BUSY_CYCLES,{4800 * 1024 / 4},{t0},{t0 + 2000}")
        rows.append(f"{did},{did},4096,{name},SQ_INSTS_MFMA,100,{t0},{t0 + 2000}")
        rows.append(f"{did},{did},4096,{name},SQ_INSTS_VALU,{100 + 4800 * 1024 / 8 / 4},{t0},{t0 + 2000}")
    rows.append(f"3,3,64,\"other_kernel\",GRBM_GUI_ACTIVE,1,0,10")
    (d / "run_counter_collection.csv").write_text(head + "\n".join(rows) + "\n")
    out = counters(str(tmp_path))
    assert len(out) == 1
    r = out[0]
    assert r["kernel"] == "prefill_gateup_kernel<12>" and r["grid"] == 4096 and r["dispatches"] == 2
    assert abs(r["avg_us"] - 2.0) < 1e-9
    assert abs(r["clock_GHz"] - 2.4) < 1e-9
    assert abs(r["mfma_busy_pct"] - 25.0) < 1e-9
    assert abs(r["valu_issue_pct"] - 12.5) < 1e-9


def test_segments_cut_dispatches_in_start_order(tmp_path):
    from bit_quantized_expert_router_amd.profsum import segments
    d = tmp_path / "run"
    d.mkdir()
    lines = ['"Kind","Kernel_Name","Start_Timestamp","End_Timestamp"']
    # dispatches of k listed out of order; durations 1, 2, 3, 10, 20 us by start time; another kernel between
    for start, dur, name in ((3000, 3000, "void moeq2::k<1>(int)"), (0, 1000, "void moeq2::k<1>(int)"),
                             (500, 99000, "void moeq2::other(int)"), (1000, 2000, "void moeq2::k<1>(int)"),
                             (9000, 10000, "void moeq2::k<1>(int)"), (30000, 20000, "void moeq2::k<1>(int)")):
        lines.append(f'"KERNEL_DISPATCH","{name}",{start},{start + dur}')
    (d / "x_kernel_trace.csv").write_text("\n".join(lines) + "\n")
    parts = segments(str(tmp_path), "k", [3, 2])
    assert [p["calls"] for p in parts] == [3, 2]
    assert parts[0]["avg_us"] == 2.0 and parts[0]["max_us"] == 3.0
    assert parts[1]["avg_us"] == 15.0 and parts[1]["min_us"] == 10.0
