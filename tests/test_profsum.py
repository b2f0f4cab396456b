"""The per-config traffic summarizer on synthetic counter files (CPU): the
copy kernel sets the scale, dispatches are assigned to configs in launch
order with other kernels skipped, and a step's kernels are summed."""
import csv
import json

from weight_streaming_gemv_decode_amd import profsum


def _csv(path, counter, rows):
    cols = ["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"]
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, cols)
        w.writeheader()
        for d, (name, v) in enumerate(rows, 1):
            # rocprofv3 writes one row per counter instance; the summarizer adds them
            w.writerow({"Dispatch_Id": d, "Kernel_Name": name, "Counter_Name": counter, "Counter_Value": v / 2})
            w.writerow({"Dispatch_Id": d, "Kernel_Name": name, "Counter_Name": counter, "Counter_Value": v / 2})
            w.writerow({"Dispatch_Id": d, "Kernel_Name": name, "Counter_Name": "OTHER", "Counter_Value": 1e9})


def test_summary(tmp_path):
    cal = ("void at::native::elementwise<AUnaryFunctor<float>>", 0)
    # FETCH reads half the bytes (KiB), WRITE all of them
    fetch = [(cal[0], 524288.0)] * 2 + [("fill", 7.0), ("dense_grouped_kernel<0, 2, 2, true, false>", 1000.0),
             ("copyBuffer", 5.0), ("dense_grouped_kernel<0, 2, 2, true, false>", 1002.0),
             ("dense_gemv_kernel<0, 8, 1, true, false>", 300.0), ("dense_reduce_kernel<0>", 10.0),
             ("dense_gemv_kernel<0, 8, 1, true, false>", 300.0), ("dense_reduce_kernel<0>", 12.0)]
    write = [(cal[0], 1048576.0)] * 2 + [("fill", 7.0), ("dense_grouped_kernel<0, 2, 2, true, false>", 4.0),
             ("copyBuffer", 5.0), ("dense_grouped_kernel<0, 2, 2, true, false>", 4.0),
             ("dense_gemv_kernel<0, 8, 1, true, false>", 8.0), ("dense_reduce_kernel<0>", 1.0),
             ("dense_gemv_kernel<0, 8, 1, true, false>", 8.0), ("dense_reduce_kernel<0>", 1.0)]
    _csv(tmp_path / "f.csv", "FETCH_SIZE", fetch)
    _csv(tmp_path / "w.csv", "WRITE_SIZE", write)
    man = {"calibration": {"label": "calibration", "read_bytes": 1 << 30, "write_bytes": 1 << 30},
           "configs": [{"label": "calibration", "workload": "copy", "kernels": ["AUnaryFunctor"], "steps": 2,
                        "algorithmic_bytes": 2 << 30},
                       {"label": "c3", "workload": "step", "kernels": ["dense_grouped_kernel<0, 2, 2"], "steps": 2,
                        "algorithmic_bytes": 2 * 1001 * 1024 + 4 * 1024},
                       {"label": "c2", "workload": "split", "kernels": ["dense_gemv_kernel<0, 8, 1",
                                                                         "dense_reduce_kernel<0>"], "steps": 2,
                        "algorithmic_bytes": 1000}]}
    (tmp_path / "m.json").write_text(json.dumps(man))
    recs, calrec = profsum.summarize(str(tmp_path / "f.csv"), str(tmp_path / "w.csv"), str(tmp_path / "m.json"))
    assert abs(calrec["fetch_scale"] - 2.0) < 1e-12 and abs(calrec["write_scale"] - 1.0) < 1e-12
    c3, c2 = recs
    assert c3["read_bytes"] == round(1001 * 1024 * 2.0) and c3["write_bytes"] == 4 * 1024
    assert c3["ratio_to_algorithmic"] == 1.0
    # one step of c2 is a GEMV and a reduce: (300 + 11) KiB read on average, scaled by 2
    assert c2["read_bytes"] == round(311 * 1024 * 2.0) and c2["write_bytes"] == 9 * 1024
    text = profsum.render(recs, calrec, ["cmd"])
    assert text.count(profsum.JSON_TAG) == 2


def test_shader_counter_summary(tmp_path):
    """SQ pass: counters summed over a dispatch's rows, dispatches of other
    kernels skipped, averages per (config, kernel), and the derived
    occupancy and busy fractions from hand-computed values."""
    cols = ["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value", "Start_Timestamp", "End_Timestamp",
            "VGPR_Count", "Accum_VGPR_Count", "SGPR_Count", "LDS_Block_Size"]
    # one die busy g = 8000 cycles; 1024 SIMDs; 10 us dispatch
    g = 8000.0
    want = {"GRBM_GUI_ACTIVE": 8 * g, "SQ_WAVE_CYCLES": 2.5 * g * 1024 / 4, "SQ_ACTIVE_INST_VALU": 0.4 * g * 1024 / 4,
            "SQ_VALU_MFMA_BUSY_CYCLES": 0.1 * g * 1024, "SQ_WAVES": 1000.0, "SQ_INSTS_VALU": 50000.0,
            "SQ_INSTS_MFMA": 3000.0, "SQ_INSTS_LDS": 7000.0}
    with open(tmp_path / "sq.csv", "w", newline="") as f:
        w = csv.DictWriter(f, cols)
        w.writeheader()
        disp = [("noise_kernel", 0.5), ("w4_grouped_kernel<2, 4, true, 1, false>", 1.0),
                ("w4_grouped_kernel<2, 4, true, 1, false>", 1.0), ("noise_kernel", 3.0)]
        for d, (name, f_) in enumerate(disp, 1):
            for c, v in want.items():
                for half in (0, 1):   # two rows per counter, added
                    w.writerow({"Dispatch_Id": d, "Kernel_Name": name, "Counter_Name": c,
                                "Counter_Value": f_ * v / 2, "Start_Timestamp": 1000, "End_Timestamp": 11000,
                                "VGPR_Count": 152, "Accum_VGPR_Count": 0, "SGPR_Count": 96, "LDS_Block_Size": 25088})
    man = {"configs": [{"label": "c5_M4", "workload": "W4A16 step, M = 4", "kernels": ["w4_grouped_kernel<2, 4"],
                        "steps": 2, "algorithmic_bytes": 10 << 20}]}
    with open(tmp_path / "man.json", "w") as f:
        json.dump(man, f)
    recs = profsum.sq_per_config(str(tmp_path / "sq.csv"), man["configs"])
    assert len(recs) == 1 and recs[0]["dispatches"] == 2 and recs[0]["vgpr"] == 152
    d = profsum.sq_derived(recs[0])
    assert abs(d["waves_per_simd"] - 2.5) < 1e-9
    assert abs(d["valu_busy"] - 0.4) < 1e-9 and abs(d["mfma_busy"] - 0.1) < 1e-9
    assert abs(d["valu_per_wave"] - 50.0) < 1e-9 and abs(d["mfma_per_wave"] - 3.0) < 1e-9
    assert abs(d["grbm_per_ns"] - 6.4) < 1e-9          # 64000 cycles over 10000 ns
    assert abs(d["valu_per_kib"] - 50000 / 10240) < 1e-9 and abs(d["mfma_per_kib"] - 3000 / 10240) < 1e-9
    profsum.main(["--sq", str(tmp_path / "sq.csv"), "--manifest", str(tmp_path / "man.json"),
                  "--out", str(tmp_path / "out.md"), "--command", "rocprofv3 ..."])
    text = (tmp_path / "out.md").read_text()
    assert "| W4A16 step, M = 4 | `w4_grouped_kernel<2, 4` | 2 | 10.0 | 6.4 | 152/0/96 | 2.50 | 40% | 10% " \
           "| 4.88 | 0.293 | 50 | 7 |" in text


def test_memory_unit_pass(tmp_path):
    """The memory-unit pass joins the shader pass by (config, kernel): busy
    fractions over the same die-busy cycles, from hand-computed values."""
    g = 10000.0
    cols = ["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value", "Start_Timestamp", "End_Timestamp",
            "VGPR_Count", "Accum_VGPR_Count", "SGPR_Count", "LDS_Block_Size"]

    def write(path, values):
        with open(path, "w", newline="") as f:
            w = csv.DictWriter(f, cols)
            w.writeheader()
            for c, v in values.items():
                w.writerow({"Dispatch_Id": 1, "Kernel_Name": "dense_grouped_kernel<0, 2, 2, true, false>",
                            "Counter_Name": c, "Counter_Value": v, "Start_Timestamp": 0, "End_Timestamp": 4000,
                            "VGPR_Count": 28, "Accum_VGPR_Count": 0, "SGPR_Count": 96, "LDS_Block_Size": 512})
    write(tmp_path / "sq.csv", {c: 8 * g if c == "GRBM_GUI_ACTIVE" else 1000.0 for c in profsum.SQ_COUNTERS})
    write(tmp_path / "mem.csv", {"TA_BUSY_avr": 0.7 * g, "TCP_TCP_TA_DATA_STALL_CYCLES_max": 0.25 * g,
                                 "TCC_BUSY_avr": 0.5 * g, "GRBM_GUI_ACTIVE": 8 * g})
    man = {"configs": [{"label": "c3", "workload": "step", "kernels": ["dense_grouped_kernel<0, 2, 2"], "steps": 1,
                        "algorithmic_bytes": 1 << 20}]}
    with open(tmp_path / "man.json", "w") as f:
        json.dump(man, f)
    mem = profsum.sq_per_config(str(tmp_path / "mem.csv"), man["configs"], profsum.MEM_COUNTERS)
    d = profsum.mem_derived(mem[0])
    assert abs(d["ta_busy"] - 0.7) < 1e-9 and abs(d["tcp_stall"] - 0.25) < 1e-9 and abs(d["tcc_busy"] - 0.5) < 1e-9
    profsum.main(["--sq", str(tmp_path / "sq.csv"), "--mem", str(tmp_path / "mem.csv"), "--manifest",
                  str(tmp_path / "man.json"), "--out", str(tmp_path / "out.md")])
    text = (tmp_path / "out.md").read_text()
    assert "| 70% | 25% | 50% |" in text and "TA busy | TCP stalled on TA | TCC busy |" in text


def test_source_hash_ignores_comments(tmp_path, monkeypatch):
    """The traffic records stay attached across comment edits, and detach on
    a code change."""
    src = tmp_path / "k.hip"
    src.write_text("int f(int x) { return x + 1; }  // one\n")
    monkeypatch.setattr(profsum, "SOURCES", ["k.hip"])
    h0 = profsum.source_sha256(str(tmp_path))
    src.write_text("/* a comment\n spanning lines */ int f(int x) {\n    return x + 1;   // two\n}\n")
    assert profsum.source_sha256(str(tmp_path)) == h0
    src.write_text("int f(int x) { return x + 2; }\n")
    assert profsum.source_sha256(str(tmp_path)) != h0


def test_chain_trace_stats_parts_of_a_stage():
    """Three linears of two units each, timestamps in 100 MHz ticks: every
    part of a stage follows from the per-unit records by hand."""
    w = []
    for t0, t1, t2, lin, wg in ((0, 100, 150, 0, 0), (0, 120, 160, 0, 1), (10, 300, 330, 1, 0),
                                (10, 350, 400, 1, 1), (20, 500, 600, 2, 0), (20, 520, 700, 2, 1)):
        w += [t0, t1, t2, lin | (wg << 32)]
    s = profsum.chain_trace_stats(w)
    assert s["units"] == 6 and s["linears"] == 3 and abs(s["span_us"] - 7.0) < 1e-9
    l1 = s["per_linear"][1]
    # linear 0 ends at 1.6 us; linear 1's inputs arrive at 3.0 and 3.5, it ends at 4.0
    assert abs(l1["detect_us"] - 1.4) < 1e-9 and abs(l1["spread_us"] - 0.5) < 1e-9
    assert abs(l1["tail_us"] - 0.5) < 1e-9 and abs(l1["stage_us"] - 2.4) < 1e-9
    assert abs(l1["compute_median_us"] - 0.4) < 1e-9
    # only the middle linear is a layer stage here
    assert abs(s["median_stage"]["stage_us"] - 2.4) < 1e-9
    md = profsum.render_chain_trace(s, ["a", "b", "c"], "cmd", 7.0, 7.1)
    assert "| 1 | b | 2 |" in md and "cmd" in md
