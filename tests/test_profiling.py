"""Host logic of the rocprofv3 summaries (decoder_only_forward_amd.profiling) on small
hand-written CSV files shaped like rocprofv3's output."""
import csv
import json
import os

import pytest

from decoder_only_forward_amd import profiling

GEMM = "void gemm::gemm_kernel<gemm::Tile<256, 256, 2, 4, 64, 2>, true, 2, 5, false>(gemm::Args)"
DEC = "void q3::(anonymous namespace)::decode_gemm_kernel<1, 6, false>(gemm::Args)"
COPY = "void at::native::elementwise_kernel<128, 4>(int, Fn)"


def _write(path, header, rows):
    os.makedirs(os.path.dirname(path), exist_ok=True)
    with open(path, "w", newline="") as fh:
        w = csv.writer(fh)
        w.writerow(header)
        w.writerows(rows)


def _counters(d, rows):
    # rows: (dispatch, kernel, counter, value, start_ns, end_ns)
    _write(os.path.join(d, "host", "run_counter_collection.csv"),
           ["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value", "Start_Timestamp",
            "End_Timestamp"], rows)
    _write(os.path.join(d, "host", "run_agent_info.csv"),
           ["Agent_Type", "Simd_Count", "Num_Xcc"], [["CPU", 0, 0], ["GPU", 1024, 8]])


def test_short_name_drops_arguments_and_anonymous_namespaces():
    assert profiling.short_name(DEC) == "q3::decode_gemm_kernel<1, 6, false>"
    assert profiling.short_name(GEMM).endswith("true, 2, 5, false>")


def test_decode_tags_select_only_their_instantiation():
    disp = [(GEMM, 1.0), (DEC, 2.0),
            ("void q3::(anonymous namespace)::decode_gemm_kernel<2, 5, false>(gemm::Args)", 3.0)]
    assert profiling._select(disp, "decode_qkv_gemm") == [2.0]
    assert profiling._select(disp, "decode_gate_up_gemm") == [3.0]
    # the tiled gate|up signature does not pick up the decode kernels
    assert profiling._select(disp, "gate_up_gemm") == [1.0]


def test_traffic_scales_by_the_calibration_copy(tmp_path):
    f, w = str(tmp_path / "f"), str(tmp_path / "w")
    # a 1 GiB copy that the fetch counter reports as 0.5 GiB: scale 2; the GEMM's two
    # dispatches read 100 and 300 KiB raw (mean 200 -> 400 KiB real)
    _counters(f, [(1, COPY, "FETCH_SIZE", 512 * 1024, 0, 10), (2, GEMM, "FETCH_SIZE", 100, 0, 1),
                  (3, GEMM, "FETCH_SIZE", 300, 0, 1)])
    _counters(w, [(1, COPY, "WRITE_SIZE", 1024 * 1024, 0, 10), (2, GEMM, "WRITE_SIZE", 50, 0, 1),
                  (3, GEMM, "WRITE_SIZE", 50, 0, 1)])
    t = profiling.traffic_json(f, w, "wl", 1.0, "cf", "cw", ["gate_up_gemm"])
    e = t["wl/gate_up_gemm"]
    assert e["fetch_scale"] == pytest.approx(2.0) and e["write_scale"] == pytest.approx(1.0)
    assert e["bytes_per_launch"] == (200 * 2 + 50) * 1024
    assert e["dispatches"] == [2, 2]
    path = tmp_path / "traffic.json"
    path.write_text(json.dumps(t))
    assert profiling.traffic_for("wl", "gate_up_gemm", str(path)) == (200 * 2 + 50) * 1024
    # a table taken from other sources is not used
    t["wl/gate_up_gemm"]["source_sha"] = "0" * 16
    path.write_text(json.dumps(t))
    assert profiling.traffic_for("wl", "gate_up_gemm", str(path)) is None


def test_counter_rows_average_per_dispatch_and_sum_instances(tmp_path):
    d = str(tmp_path / "c")
    # dispatch 1 reports its counter from two instances (summed); dispatch 2 from one
    _counters(d, [(1, DEC, "TCC_HIT_sum", 10, 0, 4000), (1, DEC, "TCC_HIT_sum", 30, 0, 4000),
                  (2, DEC, "TCC_HIT_sum", 20, 0, 6000), (3, GEMM, "TCC_HIT_sum", 5, 0, 100)])
    rows = profiling.counter_rows(d)
    assert [r["kernel"] for r in rows] == ["q3::decode_gemm_kernel<1, 6, false>",
                                           profiling.short_name(GEMM)]
    assert rows[0]["dispatches"] == 2
    assert rows[0]["avg_us"] == pytest.approx(5.0)
    assert rows[0]["counters"]["TCC_HIT_sum"] == pytest.approx(30.0)
    md = profiling.counters_markdown([("wl", rows)], "cmd")
    assert "| `q3::decode_gemm_kernel<1, 6, false>` | 2 | 5.0 | 30 |" in md


def test_mfma_rows_flops_busy_share_and_clock(tmp_path):
    d = str(tmp_path / "m")
    # one dispatch of 1 us: 1000 MOPS units (512 flops each; fp16 and bf16 work add up),
    # 8 XCDs of 2000 active cycles
    _counters(d, [(1, GEMM, "SQ_INSTS_VALU_MFMA_MOPS_F16", 600, 0, 1000),
                  (1, GEMM, "SQ_INSTS_VALU_MFMA_MOPS_BF16", 400, 0, 1000),
                  (1, GEMM, "SQ_VALU_MFMA_BUSY_CYCLES", 1024 * 1000, 0, 1000),
                  (1, GEMM, "GRBM_GUI_ACTIVE", 8 * 2000, 0, 1000)])
    (r,) = profiling.mfma_rows(d)
    assert r["gflop"] == pytest.approx(512e3 / 1e9)
    assert r["busy_pct"] == pytest.approx(50.0)
    assert r["clock_ghz"] == pytest.approx(2.0)
    assert r["kernel"].endswith("(gate_up_gemm)")
