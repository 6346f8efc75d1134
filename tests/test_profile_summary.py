"""Host-side checks of the rocprofv3 summary tool (relative_bias_amd/profile_summary.py)
on synthetic CSV files laid out like rocprofv3's: the timed-step mean, the median, the
copy-calibrated traffic. No GPU."""
import csv
import json
import os

from relative_bias_amd import profile_summary as ps

KN = "void rpa::(anonymous namespace)::attn_kernel<128, false, false, 0>(rpa::AttnParams)"


def _write(path, rows, fields):
    os.makedirs(os.path.dirname(path), exist_ok=True)
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=fields)
        w.writeheader()
        for r in rows:
            w.writerow(r)


def test_trace_timed_mean_covers_the_timed_calls(tmp_path):
    rows = []
    for i in range(30):  # 30 dispatches of 1000 .. 1029 ns, and an unrelated kernel in between
        rows.append({"Dispatch_Id": 2 * i, "Kernel_Name": KN, "Start_Timestamp": 10_000 * i,
                     "End_Timestamp": 10_000 * i + 1000 + i})
        rows.append({"Dispatch_Id": 2 * i + 1, "Kernel_Name": "void at::copy_kernel()", "Start_Timestamp": 0,
                     "End_Timestamp": 5})
    _write(str(tmp_path / "in" / "x" / "w_kernel_trace.csv"), rows,
           ["Dispatch_Id", "Kernel_Name", "Start_Timestamp", "End_Timestamp"])
    out = tmp_path / "out"
    out.mkdir()
    path = ps.trace("chunked_prefill", str(tmp_path / "in"), 20, out_dir=str(out))
    text = open(path).read()
    # bench.py times max(5, 20 // 2) = 10 calls of the chunked prefill: the last 10 dispatches.
    row = [l for l in text.splitlines() if l.startswith("| attn_kernel<128, false, false, 0>")]
    assert row == ["| attn_kernel<128, false, false, 0> | 30 | 1014 | 1024 | 1000 | 1029 |"], text
    assert "last 10 dispatches" in text and "copy_kernel" not in text
    assert ps.timed_steps("batched_decode", 20) == 20 and ps.timed_steps("long_decode", 4) == 5


def test_traffic_scales_by_the_copy_calibration(tmp_path):
    f = ["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"]
    gib = 1 << 30
    # The copy reads and writes 1 GiB: FETCH_SIZE reports half of it (factor 2), WRITE_SIZE all (factor 1).
    _write(str(tmp_path / "fc" / "c_counter_collection.csv"),
           [{"Dispatch_Id": 1, "Kernel_Name": "copyBuffer", "Counter_Name": "FETCH_SIZE",
             "Counter_Value": gib / 1024 / 2}], f)
    _write(str(tmp_path / "wc" / "c_counter_collection.csv"),
           [{"Dispatch_Id": 1, "Kernel_Name": "copyBuffer", "Counter_Name": "WRITE_SIZE",
             "Counter_Value": gib / 1024}], f)
    # Three dispatches; a counter split over two rows of one dispatch is summed.
    fetch = [{"Dispatch_Id": 5, "Kernel_Name": KN, "Counter_Name": "FETCH_SIZE", "Counter_Value": 60},
             {"Dispatch_Id": 5, "Kernel_Name": KN, "Counter_Name": "FETCH_SIZE", "Counter_Value": 40},
             {"Dispatch_Id": 6, "Kernel_Name": KN, "Counter_Name": "FETCH_SIZE", "Counter_Value": 200},
             {"Dispatch_Id": 7, "Kernel_Name": KN, "Counter_Name": "FETCH_SIZE", "Counter_Value": 300}]
    write = [{"Dispatch_Id": 5, "Kernel_Name": KN, "Counter_Name": "WRITE_SIZE", "Counter_Value": 10},
             {"Dispatch_Id": 6, "Kernel_Name": KN, "Counter_Name": "WRITE_SIZE", "Counter_Value": 30}]
    _write(str(tmp_path / "fk" / "k_counter_collection.csv"), fetch, f)
    _write(str(tmp_path / "wk" / "k_counter_collection.csv"), write, f)
    out = tmp_path / "out"
    out.mkdir()
    path = ps.traffic("chunked_prefill", str(tmp_path / "fk"), str(tmp_path / "wk"), str(tmp_path / "fc"),
                      str(tmp_path / "wc"), out_dir=str(out))
    j = json.load(open(path))
    assert j["copy_calibration"]["fetch_factor"] == 2.0 and j["copy_calibration"]["write_factor"] == 1.0
    assert j["fetch_size_kib_per_dispatch"] == 200 and j["write_size_kib_per_dispatch"] == 20
    assert j["hbm_read_bytes_per_launch"] == 200 * 1024 * 2
    assert j["hbm_write_bytes_per_launch"] == 20 * 1024
    assert j["hbm_bytes_per_launch"] == 200 * 1024 * 2 + 20 * 1024
    assert j["kernel"] == "attn_kernel<128, false, false, 0>"


def test_l2_summary_sums_channels_and_takes_the_median(tmp_path):
    f = ["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"]
    rows = []
    for d, (hit, miss) in {3: (700, 300), 4: (800, 200), 5: (900, 100)}.items():
        # each counter arrives split over two rows of the dispatch (summed), plus another kernel's rows
        for c, v in (("TCC_HIT_sum", hit), ("TCC_MISS_sum", miss), ("TCC_READ_sum", hit + miss - 50),
                     ("TCC_REQ_sum", hit + miss)):
            rows.append({"Dispatch_Id": d, "Kernel_Name": KN, "Counter_Name": c, "Counter_Value": v / 2})
            rows.append({"Dispatch_Id": d, "Kernel_Name": KN, "Counter_Name": c, "Counter_Value": v / 2})
        rows.append({"Dispatch_Id": d + 10, "Kernel_Name": "copyBuffer", "Counter_Name": "TCC_HIT_sum",
                     "Counter_Value": 1e9})
    _write(str(tmp_path / "l2" / "k_counter_collection.csv"), rows, f)
    out = tmp_path / "out"
    out.mkdir()
    path = ps.l2("chunked_prefill", str(tmp_path / "l2"), out_dir=str(out), algorithmic_bytes=128 * 500)
    j = json.load(open(path))
    assert j["counters_per_dispatch"] == {"TCC_HIT_sum": 800, "TCC_MISS_sum": 200, "TCC_READ_sum": 950,
                                          "TCC_REQ_sum": 1000}
    assert j["hit_fraction"] == 0.8 and j["algorithmic_lines_128b"] == 500
    assert j["requests_per_algorithmic_line"] == 2.0
    assert os.path.basename(path) == "attn_kernel_chunked_prefill_l2.json"
