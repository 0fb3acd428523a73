"""Host checks of the rocprofv3 summaries (synthetic CSV input, no GPU)."""
import csv

from tensor_model_transformer_tmp_amd import rocprof_summary as rs

GEMM = "gemm_bf16_kernel<64, 64, 2, 2, 4, 64, (oases::Layout)0, (oases::Layout)0, 0>(oases::GemmArgs)"
SUM = "void oases::allreduce_bf16_kernel<3>(uint4 const*)"


def _write(path, fields, rows):
    with open(path, "w", newline="") as fh:
        w = csv.DictWriter(fh, fieldnames=fields)
        w.writeheader()
        w.writerows(rows)


def test_union_len():
    assert rs._union_len([]) == 0
    assert rs._union_len([(0, 5), (3, 8), (10, 12)]) == 10
    assert rs._union_len([(2, 3), (0, 10)]) == 10


def test_timeline_hidden_fraction(tmp_path):
    # a warm-up step, the timed step (a sum on queue 2 of which 10 of 40 ns
    # run beside GEMMs on queue 1), then the step with events
    rows = [(0, 10, 1, GEMM), (20, 30, 2, SUM), (40, 50, 1, GEMM),
            (10_000, 10_050, 1, GEMM), (10_040, 10_080, 2, SUM), (10_090, 10_100, 1, GEMM),
            (20_000, 20_050, 1, GEMM), (20_000, 20_050, 2, SUM), (20_090, 20_100, 1, GEMM)]
    p = tmp_path / "kt.csv"
    _write(p, ["Kernel_Name", "Queue_Id", "Start_Timestamp", "End_Timestamp"],
           [{"Kernel_Name": n, "Queue_Id": q, "Start_Timestamp": a, "End_Timestamp": b}
            for a, b, q, n in rows])
    out = rs.timeline(str(p), steps=1, warmup=1, width=10)
    assert "hidden fraction 0.250" in out
    assert "queue   1 |" in out and "queue   2 |" in out


def test_mfma_weighted_by_active_cycles(tmp_path):
    fields = ["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"]
    rows = []
    for d, util, act in ((1, 10.0, 100.0), (2, 40.0, 300.0)):
        rows += [{"Dispatch_Id": d, "Kernel_Name": GEMM, "Counter_Name": "MfmaUtil", "Counter_Value": util},
                 {"Dispatch_Id": d, "Kernel_Name": GEMM, "Counter_Name": "GRBM_GUI_ACTIVE", "Counter_Value": act},
                 {"Dispatch_Id": d, "Kernel_Name": GEMM, "Counter_Name": "SQ_INSTS_VALU_MFMA_MOPS_BF16",
                  "Counter_Value": 2.0e6}]
    p = tmp_path / "cc.csv"
    _write(p, fields, rows)
    out = rs.mfma_table(str(p), {"gemm_fwd": 1.024e9})
    line = [ln for ln in out.splitlines() if ln.startswith("gemm_fwd")][0].split(" | ")
    assert line[1] == "2"
    assert abs(float(line[2]) - 32.5) < 1e-9           # (10*100 + 40*300) / 400
    assert abs(float(line[3]) - 1.024) < 1e-9          # 2e6 * 512 FLOP
    assert abs(float(line[5]) - 1.0) < 1e-9


def test_util_table_weights_and_raw_fractions(tmp_path):
    fields = ["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"]
    rows = []
    for d, lds, mf, act, conf in ((1, 50.0, 20.0, 100.0, 512.0), (2, 80.0, 60.0, 300.0, 0.0)):
        for name, v in (("LdsUtil", lds), ("MfmaUtil", mf), ("GRBM_GUI_ACTIVE", act),
                        ("SQ_LDS_BANK_CONFLICT", conf), ("CU_NUM", 256.0)):
            rows.append({"Dispatch_Id": d, "Kernel_Name": GEMM, "Counter_Name": name, "Counter_Value": v})
    p = tmp_path / "u.csv"
    _write(p, fields, rows)
    out = rs.util_table(str(p)).splitlines()
    assert out[0] == "class | class launches | LdsUtil % | MfmaUtil % | SQ_LDS_BANK_CONFLICT per launch"
    line = [ln for ln in out if ln.startswith("gemm_fwd")][0].split(" | ")
    assert line[1] == "2"
    assert abs(float(line[2]) - 72.5) < 1e-9    # (50*100 + 80*300) / 400
    assert abs(float(line[3]) - 50.0) < 1e-9    # (20*100 + 60*300) / 400
    assert abs(float(line[4]) - 256.0) < 1e-9   # (512 + 0) / 2 launches
