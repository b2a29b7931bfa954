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
