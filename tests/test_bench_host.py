"""Host-side checks of bench.py's own arithmetic (CPU only)."""

import os
import sys

import numpy as np
import pytest
import torch

import gen

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def bench():
    sys.path.insert(0, ROOT)
    import bench as b
    return b


@pytest.mark.parametrize("fmt,code", [("e4m3", 0), ("e4m3fnuz", 1)])
def test_repack_fidelity_matches_oracle_stats(bench, oracle, fmt, code):
    """The fidelity figures bench.py reports for the GPU repack (relative RMS
    error, max error over row max, fp64 with torch) equal the oracle's
    statistics on the same codes."""
    d = gen.linear_config(2, n=96, k=512)
    p, st, _ = oracle.repack_q4_0(d["w_bf16"])
    wq, ws = oracle.repack_fp8(p, st, 512, code)
    rr, mr = oracle.repack_stats(p, st, wq, ws, 512, code)
    steps = torch.from_numpy(st.view(np.int16)).view(torch.bfloat16)
    r2, m2 = bench.repack_fidelity(torch, torch.from_numpy(p), steps, torch.from_numpy(wq),
                                   torch.from_numpy(ws), fmt, rows_per=40)
    assert abs(r2 - rr) <= 1e-12 * rr and abs(m2 - mr) <= 1e-12 * mr
    # the per-row maximum stays within half a code step at the top of the
    # format's range over its largest value (reached on larger samples)
    assert mr <= (16 / 448 if code == 0 else 8 / 240) * (1 + 1e-6)


def _pmc_csv(path, disp, counter, values, copy_value):
    """A rocprofv3 counter_collection.csv of the given kernel-name sequence
    (one counter; `values` by short name, the copy kernel `copy_value`)."""
    import csv
    os.makedirs(os.path.dirname(path), exist_ok=True)
    with open(path, "w", newline="") as fh:
        w = csv.writer(fh)
        w.writerow(["Dispatch_Id", "Kernel_Name", "Grid_Size", "Workgroup_Size", "VGPR_Count",
                    "LDS_Block_Size", "Start_Timestamp", "End_Timestamp", "Counter_Name", "Counter_Value"])
        for i, k in enumerate(disp, 1):
            v = copy_value if k == "copy_kernel" else values.get(k, 1.0)
            w.writerow([i, f"void qlin::{k}(int)", 256, 256, 32, 0, 1000 * i, 1000 * i + 500, counter, v])


def test_pmc_summary_counts_kernels_per_call(bench, tmp_path):
    """Rows are cut at the marker dispatches and each call's kernels found
    from the repeating name sequence, also where a call launches fewer
    kernels than planned; the warm-up call of the next row and the fill
    before the next marker belong to no row."""
    import json
    launches = 3
    r1 = ["a_kernel", "b_kernel"]  # planned as 3 kernels per call
    r2 = ["c_kernel"]
    disp = (r1 + ["fill_kernel", "fp8_encode_kernel"] + r1 * launches + r2 + ["fill_kernel", "fp8_encode_kernel"]
            + r2 * launches + ["fill_kernel", "fp8_encode_kernel"] + ["copy_kernel"] * 4)
    kib = bench.COPY_BYTES / 1024
    d1, d2 = str(tmp_path / "p1"), str(tmp_path / "p2")
    _pmc_csv(os.path.join(d1, "run_counter_collection.csv"), disp, "FETCH_SIZE",
             {"a_kernel": 100.0, "b_kernel": 200.0, "c_kernel": 300.0}, kib / 2)
    _pmc_csv(os.path.join(d2, "run_counter_collection.csv"), disp, "WRITE_SIZE",
             {"a_kernel": 10.0, "b_kernel": 20.0, "c_kernel": 30.0}, kib)
    with open(os.path.join(d1, "pmc_plan_moe.json"), "w") as fh:
        json.dump({"rows": [["R1", 3, 0], ["R2", 1, 0]], "launches": launches, "copy_bytes": bench.COPY_BYTES,
                   "copies": 4, "sources_sha256": "0" * 64}, fh)
    out = str(tmp_path / "moe_summary.md")
    bench.summarize_pmc([d1, d2], out, ["cmd"])
    text = open(out).read()
    table = json.loads(text[text.index("```json") + 7:text.rindex("```")])
    assert abs(table["fetch_factor"] - 2.0) < 1e-12 and abs(table["write_factor"] - 1.0) < 1e-12
    k1 = table["rows"]["R1"]["kernels"]
    assert [k["kernel"] for k in k1] == r1
    assert [(k["fetch_kib"], k["write_kib"]) for k in k1] == [(100.0, 10.0), (200.0, 20.0)]
    assert table["rows"]["R1"]["hbm_bytes"] == round((200 + 10 + 400 + 20) * 1024)
    k2 = table["rows"]["R2"]["kernels"]
    assert [(k["kernel"], k["fetch_kib"], k["write_kib"]) for k in k2] == [("c_kernel", 300.0, 30.0)]


def test_pmc_summary_rejects_short_rows(bench, tmp_path):
    """A row with fewer repeated calls than planned launches is an error,
    not a silent shift of the following rows."""
    import json
    disp = (["fp8_encode_kernel", "a_kernel", "b_kernel", "fill_kernel", "fp8_encode_kernel"]
            + ["copy_kernel"] * 4)
    d1 = str(tmp_path / "p1")
    _pmc_csv(os.path.join(d1, "run_counter_collection.csv"), disp, "FETCH_SIZE", {}, 1.0)
    with open(os.path.join(d1, "pmc_plan_moe.json"), "w") as fh:
        json.dump({"rows": [["R1", 1, 0]], "launches": 2, "copy_bytes": bench.COPY_BYTES, "copies": 4,
                   "sources_sha256": "0" * 64}, fh)
    with pytest.raises(ValueError):
        bench.summarize_pmc([d1], str(tmp_path / "x.md"), [])


def test_clock_summary_bounds(bench, tmp_path, capsys):
    """--summarize-clock: per kernel and grid, the wave-lifetime clock (4 x
    SQ_WAVE_CYCLES / SQ_WAVES over the dispatch time) and the GRBM clock
    (GRBM_GUI_ACTIVE / 8 XCDs over it), medians over dispatches of at least
    20 us; shorter dispatches are left out."""
    import csv
    d = tmp_path / "clk"
    d.mkdir()
    rows = []
    # kernel a: 3 dispatches of 100 us; waves live 2.0 GHz x 100 us, GRBM 2.2 GHz x 8 XCDs
    for i, ns in enumerate((100_000, 100_000, 100_000), 1):
        rows.append((i, "void qlin::a(int)", ns, dict(SQ_WAVES=10.0, SQ_WAVE_CYCLES=10 * 2.0 * ns / 4,
                                                       GRBM_GUI_ACTIVE=8 * 2.2 * ns)))
    # kernel b: one 10 us dispatch (too short, left out)
    rows.append((4, "void qlin::b(int)", 10_000, dict(SQ_WAVES=4.0, SQ_WAVE_CYCLES=4 * 2.0 * 10_000 / 4,
                                                       GRBM_GUI_ACTIVE=8 * 3.0 * 10_000)))
    with open(d / "run_counter_collection.csv", "w", newline="") as fh:
        w = csv.writer(fh)
        w.writerow(["Dispatch_Id", "Kernel_Name", "Grid_Size", "Workgroup_Size", "VGPR_Count",
                    "LDS_Block_Size", "Start_Timestamp", "End_Timestamp", "Counter_Name", "Counter_Value"])
        for i, k, ns, ctr in rows:
            for n, v in ctr.items():
                w.writerow([i, k, 256, 256, 32, 0, 1000, 1000 + ns, n, v])
    bench.summarize_clock([str(d)])
    out = capsys.readouterr().out.splitlines()
    lines = [l.split() for l in out[1:]]
    assert len(lines) == 1 and lines[0][0] == "a"
    n, us, lo, hi = int(lines[0][2]), float(lines[0][3]), float(lines[0][4]), float(lines[0][5])
    assert n == 3 and us == 100.0 and lo == 2.0 and hi == 2.2
