"""Host-side checks of the rocprofv3 summary helpers and the bench's traffic record."""

import os

from causal_streaming_decoding_amd import profiling

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_short_name_strips_return_type_and_arguments():
    assert profiling.short_name("void wedlm::k_window_attn_bf16<4>(wedlm::AttnArgs)") == \
        "wedlm::k_window_attn_bf16<4>"
    assert profiling.short_name("wedlm::k_entropy_select(int, int)") == "wedlm::k_entropy_select"
    assert profiling.short_name("__amd_rocclr_copyBuffer") == "__amd_rocclr_copyBuffer"


def _record(tmp_path, sha, workload="w", steps=256):
    p = tmp_path / "t.txt"
    p.write_text(f"kernel: k\nsource_sha256: {sha}\nworkload: {workload}\nsteps: {steps}\n"
                 "fetch_bytes_per_launch: 100\nwrite_bytes_per_launch: 20\n"
                 "algorithmic_bytes_per_launch: 96\n")
    return str(p)


def test_traffic_record_applies_only_to_the_measured_source(tmp_path):
    good = _record(tmp_path, profiling.attn_source_hash())
    # the counted / algorithmic ratio, whatever the step count of the reader
    assert profiling.read_traffic(good, "w") == 120.0 / 96.0
    assert profiling.read_traffic(good, "other") is None
    stale = _record(tmp_path, "0" * 64)
    assert profiling.read_traffic(stale, "w") is None
    assert profiling.read_traffic(str(tmp_path / "missing.txt"), "w") is None


def test_committed_record_is_well_formed():
    path = os.path.join(ROOT, "profiles", "k_window_attn_bf16_qwen3_36L_bs16_stream256_traffic.txt")
    rec = dict(ln.rstrip("\n").split(": ", 1) for ln in open(path) if ": " in ln)
    assert len(rec["source_sha256"]) == 64
    fetch = float(rec["fetch_bytes_per_launch"])
    write = float(rec["write_bytes_per_launch"])
    alg = float(rec["algorithmic_bytes_per_launch"])
    assert 0.9 < (fetch + write) / alg < 1.2


def test_config_summary_from_files(tmp_path):
    import json
    hist = {"bins": ["[0,1)", "[1,2)"], "counts": [0, 3], "min": 1.5, "median": 1.7,
            "mask_slots": 3, "mask_slots_below_tau": 1}
    lines = []
    for w in ("w", "x"):
        lines.append({"workload": w, "step_us": {"median": 10.0, "p10": 9.0, "p90": 11.0},
                      "eager_step_us": {"median": 12.0}, "chained_step_us": {"median": 8.5},
                      "eager_separate_entropy_step_us": {"median": 13.0},
                      "overlap_step_us": {"median": 11.0},
                      "attn_segment_us": {"median": 6.0},
                      "entropy_tail_segment_us": {"median": 3.0}, "step_hbm_gbps_at_median": 80.0,
                      "attn_hbm_gbps_at_segment_median": 100.0,
                      "entropy_hbm_gbps_at_segment_median": 50.0, "entropy_histogram": hist})
    (tmp_path / "c.jsonl").write_text("\n".join(json.dumps(x) for x in lines) + "\n")
    hdr = "Kernel_Name,Grid_Size_X,Grid_Size_Y,Workgroup_Size_X,Start_Timestamp,End_Timestamp\n"
    for d, rows in (("tw", ['"void wedlm::k_a<4>(int)",1024,1,256,0,5000',
                            '"void wedlm::k_a<4>(int)",1024,1,256,0,7000', '"other_kernel",64,1,64,0,1']),
                    ("tx", ['"void wedlm::k_a<4>(int)",1024,1,256,0,9000'])):
        (tmp_path / d).mkdir()
        (tmp_path / d / "run_kernel_trace.csv").write_text(hdr + "\n".join(rows) + "\n")
    out = tmp_path / "o.md"
    profiling.summarize_configs(str(tmp_path / "c.jsonl"),
                                [("w", str(tmp_path / "tw")), ("x", str(tmp_path / "tx"))],
                                str(out), "b", "t")
    text = out.read_text()
    assert ("| `w` | 10.0 | 9.0 | 11.0 | 12.0 | 8.5 | 13.0 | 11.0 | 6.0 | 3.0 | 80 | 100 | "
            "1.50 / 1.70 | 1 of 3 |") in text
    # each workload's kernels in their own table: the same launch shape twice
    assert "| `wedlm::k_a<4>` | 4 x 1 | 256 | 2 | 6.00 |" in text
    assert "| `wedlm::k_a<4>` | 4 x 1 | 256 | 1 | 9.00 |" in text
    assert "other_kernel" not in text
    assert "* `w`: [1,2) 3" in text


def _write_csv(path, header, rows):
    path.parent.mkdir(parents=True, exist_ok=True)
    path.write_text(",".join(header) + "\n" + "\n".join(",".join(str(x) for x in r) for r in rows) + "\n")


def test_entropy_summary_from_files(tmp_path):
    # one bf16 workload: 2 rows x 20000 logits -> 2 chunks of 16384, grid 2 x 256 x 2 threads
    rows, V = 2, 20000
    grid_x, grid_y = 2 * 256, rows
    k = '"void wedlm::k_entropy_partial<unsigned short, true>(unsigned short const*, int)"'
    _write_csv(tmp_path / "tr" / "run_kernel_trace.csv",
               ["Kernel_Name", "Start_Timestamp", "End_Timestamp", "Grid_Size_X", "Grid_Size_Y",
                "Grid_Size_Z"],
               [[k, 1000, 5000, grid_x, grid_y, 1], [k, 9000, 11000, grid_x, grid_y, 1],
                ['"void wedlm::k_other(int)"', 0, 99999, grid_x, grid_y, 1]])
    cal = ['"__amd_rocclr_copyBuffer"', 1 << 20]
    for name, counter, kib, cal_kib in (("fe", "FETCH_SIZE", 40.0, 1 << 19), ("wr", "WRITE_SIZE", 0.5, 1 << 20)):
        _write_csv(tmp_path / name / "run_counter_collection.csv",
                   ["Dispatch_Id", "Kernel_Name", "Grid_Size", "Counter_Name", "Counter_Value"],
                   [[1, k, grid_x * grid_y, counter, kib], [2, k, grid_x * grid_y, counter, kib],
                    [3, cal[0], cal[1], counter, cal_kib]])
    out = tmp_path / "e.md"
    items = [("w", rows, V, 2, str(tmp_path / "tr"), str(tmp_path / "fe"), str(tmp_path / "wr"))]
    profiling.summarize_entropy(items, str(out), ["cmd"])
    row = [ln for ln in out.read_text().splitlines() if ln.startswith("| `w`")][0].split("|")
    cells = [c.strip() for c in row[1:-1]]
    assert cells[1] == "2 x 20000" and cells[2] == "2 x 2" and cells[3] == "2"
    assert float(cells[4]) == 3.0                       # median of 4 and 2 us (timestamps in ns)
    logits = rows * V * 2
    read = 40.0 * 1024 / 0.5                            # FETCH calibrated by 0.5
    assert abs(float(cells[5]) - logits / 1e6) < 0.05
    assert abs(float(cells[8]) - read / logits) < 1e-3


def test_counter_summary_keys_by_kernel_and_launch(tmp_path):
    hdr = ["Dispatch_Id", "Kernel_Name", "Grid_Size", "Workgroup_Size", "Counter_Name", "Counter_Value"]
    rows = []
    for d, (kern, grid) in enumerate((("void wedlm::k_a<1>(int)", 256 * 10),
                                      ("void wedlm::k_a<2>(int)", 256 * 10))):
        rows.append([d, f'"{kern}"', grid, 256, "SQ_WAVES", 40 * (d + 1)])
    _write_csv(tmp_path / "p" / "run_counter_collection.csv", hdr, rows)
    out = tmp_path / "c.md"
    profiling.summarize_counters([str(tmp_path / "p" / "run_counter_collection.csv")], str(out), "t",
                                 "", [])
    text = out.read_text()
    # same launch size, different instantiations: two columns
    assert "`k_a<1>`, 10 workgroups" in text and "`k_a<2>`, 10 workgroups" in text
    assert "| `SQ_WAVES` | 40 | 80 |" in text
