"""Pins for the oracle's quantisers and GEMMs (CPU only).

* Per-token activation quantisation (31B model card: activations quantised
  to FP8 per token at run time; dev.to sizes article, format table: int8
  activations per token): brute force on small rows.
* FP8 GEMM: the decoded operands are exact, so an fp64 matmul is the exact
  sum; the oracle's fp32 k-ordered sum must lie within the recursive
  summation bound. One-hot activations pin indexing and transposition.
* int8 GEMM: int64 numpy matmul is the exact integer result.
* W4A16: bf16(c*step) equals the stored bf16 QAT weight, so the W4A16
  oracle equals the bf16 GEMM oracle on the stored weights bit for bit.
"""

import numpy as np
import pytest

import gen

OCP, FNUZ, INT8 = 0, 1, 2
U = 2.0 ** -24


def _bf(x):
    return gen.to_bf16_bits(np.asarray(x, np.float32))


def _f(b):
    return gen.bf16_bits_to_f32(b)


def _brute_quant_row(row_f32, fmt, table):
    fmax = {OCP: 448.0, FNUZ: 240.0, INT8: 127.0}[fmt]
    amax = np.float32(np.abs(row_f32).max())
    if amax == 0:
        return np.zeros(row_f32.shape, np.uint8), np.float32(0)
    s = amax / np.float32(fmax)
    v = row_f32 / s
    if fmt == INT8:
        return np.clip(np.rint(v), -127, 127).astype(np.int8).view(np.uint8), s
    top = 0x7E if fmt == OCP else 0x7F
    mags = table[: top + 1]
    out = np.empty(v.shape, np.uint8)
    for i, x in enumerate(v):
        d = np.abs(mags - abs(float(x)))
        best = np.flatnonzero(d == d.min())
        c = int(best[0]) if len(best) == 1 else int(best[best % 2 == 0][0])
        neg = np.signbit(x)
        out[i] = (0x80 if (neg and fmt == OCP) else 0) if c == 0 else (c | (0x80 if neg else 0))
    return out, s


@pytest.mark.parametrize("fmt", [OCP, FNUZ, INT8])
def test_quant_act_bruteforce(oracle, fmt):
    d = gen.linear_config(1)
    a = d["a"].copy()
    a = np.concatenate([a, np.zeros((1, a.shape[1]), np.uint16)])  # all-zero token
    a[-1, 3] = _bf([-1e-30])[0]  # a lone tiny negative: scale tiny, code saturates
    q, s = oracle.quant_act(a, fmt)
    table = oracle.fp8_decode_table(OCP if fmt == INT8 else fmt)
    for m in range(a.shape[0]):
        ref_q, ref_s = _brute_quant_row(_f(a[m]), fmt, table)
        assert s[m] == ref_s
        assert np.array_equal(q[m].view(np.uint8), ref_q), m
    # each non-zero token reaches the largest code
    if fmt == INT8:
        assert np.all(np.abs(q[:-1].astype(np.int32)).max(axis=1) == 127)
    else:
        top = 0x7E if fmt == OCP else 0x7F
        assert np.all((q[:-1] & 0x7F).max(axis=1) == top)


def test_quant_act_zero_row_and_negative_underflow(oracle):
    a = np.zeros((2, 64), np.uint16)
    a[1, 0] = _bf([448.0])[0]
    a[1, 1] = _bf([-1e-6])[0]  # rounds to zero, keeps its sign in OCP
    q, s = oracle.quant_act(a, OCP)
    assert s[0] == 0 and np.all(q[0] == 0)
    assert s[1] == 1.0 and q[1, 0] == 0x7E and q[1, 1] == 0x80
    q, s = oracle.quant_act(a, FNUZ)
    assert q[1, 1] == 0x00


def _fp8_case(oracle, M, N, K, seed):
    d = gen.linear_config(1, n=N, k=K, m=M)
    p, st, _ = oracle.repack_q4_0(d["w_bf16"])
    wq, ws = oracle.repack_fp8(p, st, K, OCP)
    aq, sa = oracle.quant_act(d["a"], OCP)
    return aq, sa, wq, ws


def test_fp8_gemm_within_summation_bound(oracle):
    aq, sa, wq, ws = _fp8_case(oracle, 8, 96, 512, 0)
    t = oracle.fp8_decode_table(OCP)
    A, W = t[aq], t[wq]
    exact = A @ W.T  # products exact, fp64 sum ~exact
    absum = np.abs(A) @ np.abs(W).T
    K = aq.shape[1]
    y32, y16 = oracle.gemm_fp8(aq, sa, wq, ws)
    scale = sa[:, None].astype(np.float64) * ws[None, :].astype(np.float64)
    bound = (K * U / (1 - K * U)) * absum * scale + 3 * U * np.abs(exact * scale) + 1e-30
    assert np.all(np.abs(y32 - exact * scale) <= bound)
    assert np.array_equal(y16, oracle.bf16_nearest_array(y32))


def test_fp8_gemm_one_hot_and_sign(oracle):
    """One-hot activation rows select single weight columns exactly:
    catches transposed operands, wrong indices and sign slips."""
    aq, sa, wq, ws = _fp8_case(oracle, 4, 40, 256, 1)
    K = aq.shape[1]
    t = oracle.fp8_decode_table(OCP)
    ks = [0, 7, 130, K - 1]
    oh = np.zeros((4, K), np.uint8)
    for i, k in enumerate(ks):
        oh[i, k] = 0x38 if i % 2 == 0 else 0xB8  # +1.0 / -1.0
    s1 = np.float32([1.0, 2.0, 0.5, 1.0])
    y32, _ = oracle.gemm_fp8(oh, s1, wq, ws)
    for i, k in enumerate(ks):
        sign = 1.0 if i % 2 == 0 else -1.0
        want = (np.float32(sign * t[wq[:, k]]) * s1[i]) * ws
        assert np.array_equal(y32[i], want.astype(np.float32))


def test_w8a8_gemm_exact(oracle):
    d = gen.linear_config(1, n=80, k=512, m=9)
    p, st, _ = oracle.repack_q4_0(d["w_bf16"])
    wq, ws = oracle.repack_int8(p, st, 512)
    aq, sa = oracle.quant_act(d["a"], INT8)
    acc, y32, y16 = oracle.gemm_w8a8(aq, sa, wq, ws)
    exact = aq.astype(np.int64) @ wq.astype(np.int64).T
    assert np.array_equal(acc, exact)
    ref = exact.astype(np.float64) * sa[:, None] * ws[None, :]
    assert np.all(np.abs(y32 - ref) <= 3 * U * np.abs(ref) + 1e-30)
    assert np.array_equal(y16, oracle.bf16_nearest_array(y32))
    # sampled entry points compute the same numbers
    mi = np.array([0, 8, 3]); ni = np.array([79, 0, 41])
    a2, y2 = oracle.gemm_w8a8_sample(aq, sa, wq, ws, mi, ni)
    assert np.array_equal(a2, acc[mi, ni]) and np.array_equal(y2, y32[mi, ni])


def test_w4a16_equals_bf16_gemm_on_stored_weights(oracle):
    d = gen.linear_config(1, n=72, k=384, m=5)
    p, st, _ = oracle.repack_q4_0(d["w_bf16"])
    y32, y16 = oracle.gemm_w4a16(d["a"], p, st)
    b32, b16 = oracle.gemm_bf16(d["a"], d["w_bf16"])
    assert np.array_equal(y32, b32) and np.array_equal(y16, b16)
    # bf16 GEMM within the summation bound of the exact fp64 result
    A, W = _f(d["a"]).astype(np.float64), _f(d["w_bf16"]).astype(np.float64)
    exact = A @ W.T
    bound = 384 * U / (1 - 384 * U) * (np.abs(A) @ np.abs(W).T) + 1e-30
    assert np.all(np.abs(b32 - exact) <= bound)
    mi, ni = np.array([4, 0]), np.array([0, 71])
    assert np.array_equal(oracle.gemm_w4a16_sample(d["a"], p, st, mi, ni), y32[mi, ni])


def test_w4a16_one_hot(oracle):
    d = gen.linear_config(1, n=48, k=256, m=2)
    p, st, _ = oracle.repack_q4_0(d["w_bf16"])
    a = np.zeros((2, 256), np.uint16)
    a[0, 33] = _bf([1.0])[0]
    a[1, 255] = _bf([-2.0])[0]
    y32, _ = oracle.gemm_w4a16(a, p, st)
    assert np.array_equal(y32[0], _f(d["w_bf16"][:, 33]))
    assert np.array_equal(y32[1], -2.0 * _f(d["w_bf16"][:, 255]))


def test_fp8_sample_matches_full(oracle):
    aq, sa, wq, ws = _fp8_case(oracle, 6, 64, 256, 2)
    y32, _ = oracle.gemm_fp8(aq, sa, wq, ws)
    mi, ni = np.array([0, 5, 2, 2]), np.array([63, 0, 17, 18])
    assert np.array_equal(oracle.gemm_fp8_sample(aq, sa, wq, ws, mi, ni), y32[mi, ni])
