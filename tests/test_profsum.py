"""The profile summary reader (host only): kernel stats and counter tables of rocprofv3 in, per
launch averages and calibrated HBM bytes out."""
import csv
import json

from moe_routed_expert_route_amd import profsum


def _write(path, header, rows):
    with open(path, "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(header)
        w.writerows(rows)


def test_kernel_stats_and_summary(tmp_path, monkeypatch):
    p = tmp_path / "run_kernel_stats.csv"
    _write(p, ["Name", "Calls", "TotalDurationNs", "AverageNs", "Percentage", "MinNs", "MaxNs", "StdDev"],
           [["void moe::k_gate_up<2, 2, 2>(float const*, signed char const*, int, int, moe::GuArgs)",
             480, 480 * 12000, 12000, 60, 11000, 15000, 1],
            ["void moe::k_down<2, 0>(moe::DnArgs)", 480, 480 * 8000, 8000, 40, 7000, 9000, 1]])
    monkeypatch.setattr(profsum, "PROFILES", str(tmp_path))
    doc = profsum.write_kernels(str(p), "w", "cmd")
    assert doc["kernels"]["gate_up"]["avg_ns"] == 12000 and doc["kernels"]["down"]["calls"] == 480
    assert json.load(open(tmp_path / "kernels_w.json"))["source_sha256"] == profsum.source_digest()
    assert "cmd" in open(tmp_path / "kernels_w.md").read()


def test_traffic_calibration(tmp_path, monkeypatch):
    hdr = ["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"]
    gu = "void moe::k_gate_up<2, 2, 2>(x)"
    # two dimension rows per dispatch; the copy reads half of its true KiB on this counter
    # (small copies of the run besides the calibration copy must not count as it)
    f_rows = [[1, "__amd_rocclr_copyBuffer", "FETCH_SIZE", 65536], [1, "__amd_rocclr_copyBuffer", "FETCH_SIZE", 65536],
              [4, "__amd_rocclr_copyBuffer", "FETCH_SIZE", 8], [5, "__amd_rocclr_copyBuffer", "FETCH_SIZE", 8],
              [2, gu, "FETCH_SIZE", 4000], [2, gu, "FETCH_SIZE", 5000], [3, gu, "FETCH_SIZE", 9000]]
    w_rows = [[1, "__amd_rocclr_copyBuffer", "WRITE_SIZE", 262144], [4, "__amd_rocclr_copyBuffer", "WRITE_SIZE", 16],
              [2, gu, "WRITE_SIZE", 16], [3, gu, "WRITE_SIZE", 16]]
    _write(tmp_path / "f.csv", hdr, f_rows)
    _write(tmp_path / "w.csv", hdr, w_rows)
    monkeypatch.setattr(profsum, "PROFILES", str(tmp_path))
    doc = profsum.write_traffic(str(tmp_path / "f.csv"), str(tmp_path / "w.csv"), "w", "cmd",
                                algorithmic={"gate_up": 18 * 1024 * 1024})
    k = doc["kernels"]["gate_up"]
    assert doc["calibration"]["fetch_scale"] == 2.0 and doc["calibration"]["write_scale"] == 1.0
    assert k["fetch_kib"] == 9000 and k["dispatches"] == 2
    assert k["hbm_bytes_per_launch"] == (9000 * 2 + 16) * 1024


def test_sq_summary(tmp_path, monkeypatch):
    hdr = ["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"]
    gu, dn = "void moe::k_gate_up<2, 2, 2, true>(x)", "void moe::k_down<2, 0>(moe::DnArgs)"
    rows = []
    for d, name, waves, valu in ((1, gu, 100, 64000), (2, gu, 100, 64000), (3, dn, 50, 10000)):
        for c in profsum.SQ:
            v = {"SQ_WAVES": waves, "SQ_INSTS_VALU": valu}.get(c, 10)
            rows.append([d, name, c, v])
    _write(tmp_path / "sq.csv", hdr, rows)
    monkeypatch.setattr(profsum, "PROFILES", str(tmp_path))
    got = profsum.write_sq(str(tmp_path / "sq.csv"), "w", "t", "cmd", weights={"gate_up": 64000 * 64, "down": 1})
    assert got["gate_up"]["SQ_INSTS_VALU"] == 64000 and got["gate_up"]["dispatches"] == 2
    text = open(tmp_path / "sq_w.md").read()
    assert "| VALU instructions per wave | 640.000 | 200.000 |" in text
    assert "| VALU lane-instructions per weight (x 64) | 1.000 |" in text
