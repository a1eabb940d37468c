"""CPU tests of bench.py's readers of rocprofv3 output, on small hand-made
CSV files whose answers follow from their definitions: the traffic
calibration against the 1 GiB copy, and the matrix-core busy fraction and
clock from SQ_VALU_MFMA_BUSY_CYCLES and GRBM_GUI_ACTIVE."""

import csv
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402

COUNTER_FIELDS = ["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value",
                  "Start_Timestamp", "End_Timestamp"]


def _write(path, rows, fields=COUNTER_FIELDS):
    with open(path, "w", newline="") as fh:
        w = csv.DictWriter(fh, fieldnames=fields)
        w.writeheader()
        for r in rows:
            w.writerow(dict(zip(fields, r)))
    return str(path)


def test_mfma_busy_and_clock(tmp_path):
    name = "void attn::(anonymous namespace)::fwd_bf16_kernel<128, false, true>(attn::FwdArgs)"
    ns = 2_000_000                                   # 2 ms dispatches
    active = 3.6e6 * bench.N_XCD                     # 3.6e6 cycles per XCD -> 1.8 GHz
    rows = []
    for disp, busy in ((1, 0.5), (2, 0.7)):
        rows.append((disp, name, "GRBM_GUI_ACTIVE", active, 10 ** 9, 10 ** 9 + ns))
        rows.append((disp, name, "SQ_VALU_MFMA_BUSY_CYCLES", busy * 3.6e6 * bench.N_SIMD,
                     10 ** 9, 10 ** 9 + ns))
    rows.append((3, "void at::native::fill_kernel", "GRBM_GUI_ACTIVE", 1.0, 0, 10))  # not attention
    out = bench.summarize_mfma(_write(tmp_path / "c.csv", rows)).splitlines()
    assert len(out) == 2
    fields = out[1].split()
    assert fields[-4:] == ["2", "2.000", "60.0%", "1.800"]


def test_mfma_coissue_columns(tmp_path):
    """With SQ_ACTIVE_INST_VALU (quad-cycles) and SQ_VALU_MFMA_COEXEC_CYCLES:
    vector-active share of SIMD cycles and the co-issued share of it."""
    name = "void attn::(anonymous namespace)::bwd_dq_kernel<128, false, true>(attn::BwdArgs)"
    ns = 1_000_000
    per_xcd = 1.9e6
    cyc = per_xcd * bench.N_SIMD                     # SIMD cycles of the dispatch
    rows = [(1, name, "GRBM_GUI_ACTIVE", per_xcd * bench.N_XCD, 0, ns),
            (1, name, "SQ_VALU_MFMA_BUSY_CYCLES", 0.6 * cyc, 0, ns),
            (1, name, "SQ_ACTIVE_INST_VALU", 0.4 * cyc / 4, 0, ns),   # 40% of cycles, in quad-cycles
            (1, name, "SQ_VALU_MFMA_COEXEC_CYCLES", 0.3 * cyc, 0, ns)]  # 75% of those co-issued
    out = bench.summarize_mfma(_write(tmp_path / "c.csv", rows)).splitlines()
    assert "VALU active" in out[0] and "co-issued" in out[0]
    fields = out[1].split()
    assert fields[-6:] == ["1", "1.000", "60.0%", "1.900", "40.0%", "75.0%"]


def test_traffic_calibration(tmp_path):
    copy = "void at::native::vectorized_elementwise_kernel<4, copy>"
    kern = "void attn::fwd_bf16_kernel<128, false, true>(attn::FwdArgs)"
    # the copy reads and writes 1 GiB; the counters read half of the fetch
    cf = _write(tmp_path / "cf.csv", [(1, copy, "FETCH_SIZE", 524288, 0, 1)])
    cw = _write(tmp_path / "cw.csv", [(1, copy, "WRITE_SIZE", 1048576, 0, 1)])
    f = _write(tmp_path / "f.csv", [(1, kern, "FETCH_SIZE", 1000000, 0, 1),
                                    (2, kern, "FETCH_SIZE", 3000000, 0, 1)])
    w = _write(tmp_path / "w.csv", [(1, kern, "WRITE_SIZE", 500000, 0, 1),
                                    (2, kern, "WRITE_SIZE", 500000, 0, 1)])
    text = bench.summarize_traffic(f, w, cf, cw)[0]
    line = [x for x in text.splitlines() if "fwd_bf16_kernel" in x][0]
    # mean fetch 2e6 KiB x 2 + mean write 5e5 KiB x 1, in GB
    assert abs(float(line.split()[-1]) - (2e6 * 2 + 5e5) * 1024 / 1e9) < 1e-3


def test_counter_averages_and_per_wave(tmp_path):
    """Two passes of one command: each counter averaged over dispatches;
    SQ_ counters also per wave (divided by the dispatch's SQ_WAVES, counted
    in the first pass), GRBM_ ones not."""
    name = "void attn::(anonymous namespace)::fwd_bf16_kernel<128, false, true>(attn::FwdArgs)"
    p1 = _write(tmp_path / "p1.csv", [(1, name, "SQ_WAVES", 1000, 0, 1), (1, name, "SQ_INSTS_VALU", 150000, 0, 1),
                                      (2, name, "SQ_WAVES", 1000, 0, 1), (2, name, "SQ_INSTS_VALU", 170000, 0, 1),
                                      (3, "void at::native::fill_kernel", "SQ_WAVES", 7, 0, 1)])
    p2 = _write(tmp_path / "p2.csv", [(1, name, "SQ_INSTS_SALU", 50000, 0, 1), (1, name, "GRBM_GUI_ACTIVE", 8e6, 0, 1),
                                      (2, name, "SQ_INSTS_SALU", 60000, 0, 1), (2, name, "GRBM_GUI_ACTIVE", 8e6, 0, 1)])
    out = bench.summarize_counters([p1, p2]).splitlines()
    assert len(out) == 6 and "fwd_bf16_kernel" in out[0]
    rows = {ln.split()[0]: ln.split()[1:] for ln in out[2:]}
    assert rows["SQ_INSTS_VALU"] == ["1.6e+05", "160.0"]
    assert rows["SQ_INSTS_SALU"] == ["55000", "55.0"]
    assert rows["GRBM_GUI_ACTIVE"] == ["8e+06"]
    assert rows["SQ_WAVES"] == ["1000"]
