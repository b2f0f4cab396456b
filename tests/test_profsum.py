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
