"""The quantizers' reciprocal quotient equals IEEE division where it matters.

The per-token and per-channel quantizers divide every value of a row by the
row's scale s = absmax / FMAX with IEEE fp32 division (the plainest reading
of the absmax/FMAX scales: the MI300X Gemma 4 E2B article, "Step 3", and the
Gemma 4 31B-it FP8 model card). The GPU kernels compute a/s as a reciprocal
quotient with one fma correction and a's sign copied on. quotient_check.c
enumerates every input such a row can hold (every positive finite bf16
absmax, the three FMAX values, every bf16 value up to the absmax, both
signs: 3.1e9 pairs) and counts the pairs whose codes could differ. The
answer must be zero.
"""

import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
def test_reciprocal_quotient_matches_ieee_division(tmp_path):
    exe = str(tmp_path / "quotient_check")
    subprocess.run(["gcc", "-O2", "-march=native", "-fopenmp", "-ffp-contract=off",
                    os.path.join(HERE, "quotient_check.c"), "-o", exe, "-lm"], check=True)
    env = dict(os.environ)
    env.setdefault("OMP_NUM_THREADS", str(min(16, os.cpu_count() or 1)))
    out = subprocess.run([exe], capture_output=True, text=True, timeout=900, env=env)
    fields = out.stdout.split()
    got = dict(zip(fields[0::2], (int(v) for v in fields[1::2])))
    assert out.returncode == 0 and got["bad"] == 0, out.stdout
    # every pair of the three formats with a fast-path scale was compared
    assert got["checked"] > 3_000_000_000
    assert got["same_bits"] > 0.99 * got["checked"]
