"""Host-side arithmetic of the profile summaries (block_sparse_long_02_amd.profiling)
on a synthetic rocprofv3 counter file: the clock of a dispatch is its
GRBM_GUI_ACTIVE count per XCD over its duration, and its MFMA-busy share is the
SIMD-averaged MFMA busy count over those cycles."""
import csv
import os

from block_sparse_long_02_amd import profiling as prof


def _write(path, rows):
    keys = ["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value", "Start_Timestamp", "End_Timestamp"]
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=keys)
        w.writeheader()
        for r in rows:
            w.writerow(dict(zip(keys, r)))


def test_clocks_from_grbm_and_duration(tmp_path):
    d = tmp_path / "run" / "host"
    os.makedirs(d)
    # dispatch 1: 10 ms, 1.7e7 cycles per XCD (1.7 GHz), MFMA busy 0.8 of them on every SIMD
    # dispatch 2: 20 ms at 1.5 GHz, MFMA busy 0.6
    rows = []
    for did, dur_ns, ghz, busy in ((1, 10_000_000, 1.7, 0.8), (2, 20_000_000, 1.5, 0.6)):
        cyc = ghz * 1e9 * dur_ns * 1e-9
        rows.append((did, "void k_main(int)", "GRBM_GUI_ACTIVE", cyc * prof.N_XCDS, 1000, 1000 + dur_ns))
        rows.append((did, "void k_main(int)", "SQ_VALU_MFMA_BUSY_CYCLES", busy * cyc * prof.N_SIMDS, 1000,
                     1000 + dur_ns))
    rows.append((3, "other_kernel", "GRBM_GUI_ACTIVE", 5.0, 0, 100))
    _write(d / "p_counter_collection.csv", rows)
    v = sorted(prof._dispatch_clocks(prof._counter_rows(str(tmp_path)), "k_main"))
    assert len(v) == 2
    assert abs(v[0][1] / v[0][0] - 1.7e9) < 1.0 and abs(v[1][1] / v[1][0] - 1.5e9) < 1.0
    assert abs(v[0][2] / v[0][1] - 0.8) < 1e-12 and abs(v[1][2] / v[1][1] - 0.6) < 1e-12
    md = prof.clocks_md(str(tmp_path), ["k_main"], "t", "c")
    line = [x for x in md.splitlines() if x.startswith("| k_main")][0]
    cells = [c.strip() for c in line.strip("|").split("|")]
    assert cells[1] == "2" and cells[2] == "15.000" and cells[3] == "1.600" and cells[4] == "0.700"
    assert abs(float(cells[5]) - 1.6e9 * 1024 * prof.N_SIMDS / 1e15) < 1e-3
