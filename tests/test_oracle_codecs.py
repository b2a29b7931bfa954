"""Pins for the oracle's number formats (CPU only).

FP8 E4M3 (OCP) and E4M3FNUZ: same 3 mantissa bits; OCP tops out at 448,
FNUZ at 240 with no negative zero (MI300X Gemma 4 E2B article, "Tip: E4M3
or E4M3FNUZ"). The oracle's decoder is checked against torch's fp8 dtypes
(a library routine), its encoder against a brute-force nearest search over
the decoded table and against torch's in-range casts (which round to
nearest even but do not saturate), bf16 rounding against torch's bfloat16.
"""

import numpy as np
import pytest
import torch

OCP, FNUZ = 0, 1
FMAX = {OCP: 448.0, FNUZ: 240.0}
TORCH = {OCP: torch.float8_e4m3fn, FNUZ: torch.float8_e4m3fnuz}


def _torch_decode(fmt):
    return torch.arange(256, dtype=torch.uint8).view(TORCH[fmt]).to(torch.float64).numpy()


@pytest.mark.parametrize("fmt", [OCP, FNUZ])
def test_decode_all_256_codes_match_library(oracle, fmt):
    ours = oracle.fp8_decode_table(fmt)
    ref = _torch_decode(fmt)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan)
    assert np.array_equal(ours[~nan], ref[~nan])
    # signed zero bits too
    assert np.array_equal(np.signbit(ours[~nan]), np.signbit(ref[~nan]))


def test_format_facts(oracle):
    assert oracle.fp8_value(0x7E, OCP) == 448.0
    assert np.isnan(oracle.fp8_value(0x7F, OCP)) and np.isnan(oracle.fp8_value(0xFF, OCP))
    assert oracle.fp8_value(0x7F, FNUZ) == 240.0
    assert np.isnan(oracle.fp8_value(0x80, FNUZ))
    assert oracle.fp8_value(0x01, OCP) == 2.0 ** -9 and oracle.fp8_value(0x01, FNUZ) == 2.0 ** -10
    assert oracle.fp8_value(0x38, OCP) == 1.0 and oracle.fp8_value(0x40, FNUZ) == 1.0
    # FNUZ has no negative zero: no code decodes to -0.0
    t = oracle.fp8_decode_table(FNUZ)
    z = t[t == 0.0]
    assert len(z) == 1 and not np.signbit(z[0])
    # same bits decode to exactly twice the value in OCP (bias 7 vs 8)
    to, tf = oracle.fp8_decode_table(OCP), oracle.fp8_decode_table(FNUZ)
    ok = ~np.isnan(to) & ~np.isnan(tf)
    assert np.array_equal(to[ok], 2.0 * tf[ok])


def _brute_encode(x, fmt, table):
    """Nearest finite code by exhaustive search; ties to the even code;
    |x| beyond the largest finite value saturates; sign from x."""
    top = 0x7E if fmt == OCP else 0x7F
    mags = table[: top + 1]  # codes 0..top, non-negative
    out = np.empty(x.shape, np.uint8)
    for i, v in enumerate(x):
        a = abs(float(v))
        if a >= mags[top]:
            c = top
        else:
            d = np.abs(mags - a)
            best = np.flatnonzero(d == d.min())
            c = int(best[0]) if len(best) == 1 else int(best[best % 2 == 0][0])
        neg = np.signbit(v)
        if c == 0:
            out[i] = 0x80 if (neg and fmt == OCP) else 0
        else:
            out[i] = c | (0x80 if neg else 0)
    return out


def _boundary_points(table, fmt):
    top = 0x7E if fmt == OCP else 0x7F
    mags = table[: top + 1].astype(np.float32)
    mids = ((table[:top] + table[1: top + 1]) / 2).astype(np.float32)  # exact in fp32
    pts = np.concatenate([mags, mids, np.nextafter(mids, np.float32(0)),
                          np.nextafter(mids, np.float32(1e9)), np.float32([FMAX[fmt] * 1.03, 1e6])])
    return np.concatenate([pts, -pts]).astype(np.float32)


@pytest.mark.parametrize("fmt", [OCP, FNUZ])
def test_encode_vs_bruteforce(oracle, fmt):
    table = oracle.fp8_decode_table(fmt)
    rng = np.random.default_rng(7)
    x = np.concatenate([_boundary_points(table, fmt),
                        (rng.standard_normal(3000) * 60).astype(np.float32),
                        (rng.standard_normal(2000) * 0.01).astype(np.float32),
                        np.float32([0.0, -0.0, 1e-30, -1e-30])])
    assert np.array_equal(oracle.fp8_encode_array(x, fmt), _brute_encode(x, fmt, table))


@pytest.mark.parametrize("fmt", [OCP, FNUZ])
def test_encode_vs_library_in_range(oracle, fmt):
    """Dense sweep of fp32 bit patterns below FMAX: the library cast rounds to
    nearest even exactly like the oracle (it differs only by not saturating)."""
    lim = np.float32(FMAX[fmt]).view(np.uint32)
    bits = np.arange(0, int(lim), 97, dtype=np.uint32)
    x = bits.view(np.float32)
    x = np.concatenate([x, -x, _boundary_points(oracle.fp8_decode_table(fmt), fmt)])
    x = x[np.abs(x) <= FMAX[fmt]]
    ref = torch.from_numpy(x).to(TORCH[fmt]).view(torch.uint8).numpy()
    ours = oracle.fp8_encode_array(x, fmt)
    assert np.array_equal(ours, ref)


@pytest.mark.parametrize("fmt", [OCP, FNUZ])
def test_encode_saturates_and_signed_zero(oracle, fmt):
    top = 0x7E if fmt == OCP else 0x7F
    for v in (FMAX[fmt], FMAX[fmt] * 1.01, 464.0, 1e30):
        assert oracle.fp8_encode(v, fmt) == top
        assert oracle.fp8_encode(-v, fmt) == top | 0x80
    assert oracle.fp8_encode(-0.0, fmt) == (0x80 if fmt == OCP else 0x00)
    assert oracle.fp8_encode(-1e-9, fmt) == (0x80 if fmt == OCP else 0x00)
    assert oracle.fp8_encode(0.0, fmt) == 0


def test_encode_round_trip_all_codes(oracle):
    for fmt in (OCP, FNUZ):
        t = oracle.fp8_decode_table(fmt)
        for b in range(256):
            if np.isnan(t[b]):
                continue
            if fmt == FNUZ and b == 0x00:
                assert oracle.fp8_encode(0.0, fmt) == 0
                continue
            assert oracle.fp8_encode(float(t[b]), fmt) == b, (fmt, b)


def test_bf16_nearest_vs_library(oracle):
    rng = np.random.default_rng(3)
    x = np.concatenate([rng.standard_normal(20000).astype(np.float32) * 10,
                        rng.standard_normal(2000).astype(np.float32) * 1e-3])
    # exact ties: low half-word 0x8000
    tie = (rng.integers(0x3F000000, 0x41000000, 500, dtype=np.uint32) & 0xFFFF0000) | 0x8000
    x = np.concatenate([x, tie.view(np.float32), -tie.view(np.float32)])
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(oracle.bf16_nearest_array(x), ref)
